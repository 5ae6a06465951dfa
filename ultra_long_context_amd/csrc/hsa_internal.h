// hsa_internal.h -- launch interface between the C ABI host code and the kernels.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hsa {

// Kernel stages that a caller may bracket with its own HIP events (the order of
// HSA_STAGE_* in hsa.h).
enum Stage { kStageScan = 0, kStageMerge = 1, kStageBucket = 2, kStageAttend = 3, kStageCombine = 4,
             kStages = 5 };

// Optional caller-owned events: ev[2*stage] is recorded on the launch stream
// before the stage's first kernel, ev[2*stage + 1] after its last.  Null
// entries (or a null array) record nothing.  The library keeps no reference.
struct Marks {
  void* const* ev = nullptr;
  hipError_t rec(int stage, int end, hipStream_t st) const {
    if (ev == nullptr || ev[2 * stage + end] == nullptr) return hipSuccess;
    return hipEventRecord(static_cast<hipEvent_t>(ev[2 * stage + end]), st);
  }
};

// Landmark scan + per-split top-K (Steps 1-2).
struct ScanArgs {
  const void* q_ret;      // [B, Lq, Hkv, D]
  const void* landmarks;  // [B, Hkv, Nc, D]
  int32_t* out_idx;       // [B, Lq, Hkv, K]
  float* out_score;       // [B, Lq, Hkv, K]
  uint64_t* lists;        // [B*Lq*Hkv, K, n_splits] per-split sorted candidates, entry-major (wide, n_splits > 1)
  int64_t Lq, q_pos0, Nc;
  int32_t Hkv, K;
  int32_t n_max;          // max eligible chunks over all rows
  int32_t split_len;      // chunks per split: 1024 (wide) or all eligible chunks
  int32_t n_splits;       // 1 for the one-wave scan
  float ret_scale;
};

// Merge of per-split sorted candidate lists into the final selection.
struct MergeArgs {
  const uint64_t* lists;  // [rows, K, n_splits] (entry-major)
  int32_t* out_idx;       // [rows, K]
  float* out_score;       // [rows, K]
  int64_t rows;
  int32_t n_splits, K;
  float ret_scale;
};

// Decode attend (few rows, bf16): merge in the prologue, MFMA per slot.
struct DecodeArgs {
  const void* q_attn;
  const void* k;
  const void* v;
  const uint64_t* lists;     // per-split sorted candidates [rows, K, n_splits], or nullptr
  const int32_t* idx_in;     // given selection when lists == nullptr
  const float* score_in;
  int32_t* idx_out;          // final selection written by slot block 0 (merged path; may be null)
  float* score_out;
  void* out;
  float* partials;           // [rows, n_blocks, G, D]
  uint32_t* counters;        // [rows], zero on entry
  int64_t Lq, Lkv, Nc;
  int32_t Hq, Hkv, K, n_splits, n_blocks;
  float ret_scale, attn_scale;
  int32_t qk_norm;
};

// Per-chunk attention + blend (Steps 3-4).
struct AttendArgs {
  const void* q_attn;     // [B, Lq, Hq, D]
  const void* k;          // [B, Hkv, Lkv, D]
  const void* v;          // [B, Hkv, Lkv, D]
  const int32_t* idx;     // [B, Lq, Hkv, K]
  const float* score;     // [B, Lq, Hkv, K]
  void* out;              // [B, Lq, Hq, D]
  float* partials;        // [B*Lq*Hkv, n_splits, G, D] when n_splits > 1
  uint32_t* counters;     // [B*Lq*Hkv] when n_splits > 1 (zero on entry)
  int64_t Lq, Lkv, Nc;
  int32_t Hq, Hkv, K;
  int32_t n_splits, slots_per_split;
  float attn_scale;
  int32_t qk_norm;
  int32_t mode;           // 0: wave per row (many rows); 1: workgroup per (row, slot)
};

// Chunk-major attend + blend (many rows, bf16): pairs bucketed by chunk.
struct ChunkArgs {
  const void* q_attn;     // [B, Lq, Hq, D] bf16
  const void* k;          // [B, Hkv, Lkv, D] bf16
  const void* v;          // [B, Hkv, Lkv, D] bf16
  const int32_t* idx;     // [rows, K]
  const float* score;     // [rows, K]
  void* out;              // [B, Lq, Hq, D] bf16
  uint32_t* counts;       // [n_bins]      pairs per (b, kv head, chunk)
  uint32_t* offsets;      // [n_bins + 1]  first pair of each bin
  uint32_t* cursor;       // [n_bins]      scatter positions
  uint64_t* items;        // [max_items]   bin | block << 32
  uint32_t* n_items;      // number of valid items
  uint32_t* seg_tot;      // [2 * chunk_scan_tiles(n_bins)] pairs and items per scan tile of bins
  uint32_t* item_start;   // [n_bins] first work item of each bin, or nullptr
  uint32_t* pairs;        // [rows * K]    pair ids (row * K + slot), grouped by bin
  float* wts;             // [rows * K]    blend weights
  uint16_t* partials;     // [rows * K, G, D] weighted per-chunk outputs (bf16)
  int64_t rows, Lq, Lkv, Nc, n_bins, max_items;
  int64_t band_rows, n_bands;   // bins split the query rows of a (batch, kv head) into bands
  int32_t pairs_per_item;       // work item size, at most 128 pairs
  int32_t bucket_rows;          // query rows per bucketing workgroup (set by launch_bucket)
  int32_t Hq, Hkv, K;
  float attn_scale;
  int32_t qk_norm;
};

// Backward for a given selection (bf16 inputs, fp32 gradients).  The pair
// bucketing of the chunk-major forward is reused through `c` (item_start set).
struct BwdArgs {
  ChunkArgs c;
  const void* q_ret;      // [B, Lq, Hkv, D]
  const void* landmarks;  // [B, Hkv, Nc, D]
  const void* dout;       // [B, Lq, Hq, D]
  float* dq_ret;          // [B, Lq, Hkv, D]
  float* dlandmarks;      // [B, Hkv, Nc, D]
  float* dq_attn;         // [B, Lq, Hq, D]
  float* dk;              // [B, Hkv, Lkv, D]
  float* dv;              // [B, Hkv, Lkv, D]
  float* wdw;             // [rows * K]   w_k * dL/dw_k per pair
  float* draw;            // [rows * K]   dL/d(q_ret . landmark) per pair
  uint16_t* dq_part;      // [rows * K, G, D]  per-pair gradient of the normalised query (bf16)
  float* item_part;       // [max_items, 2, 64, D]  per-item dV and dkhat of the chunk's keys
  float ret_scale;
};

hipError_t launch_backward(const BwdArgs& a, int D, int G, hipStream_t st, const Marks& mk);
int64_t bwd_pairs_per_item();

// Chunk-mean landmarks of chunks [c_begin, c_begin + n_chunks) of every (b, kv head).
struct LandmarkArgs {
  const void* k;          // [B, Hkv, Lkv, D]
  void* landmarks;        // [B, Hkv, Nc, D]
  int64_t Lkv, Nc, c_begin, n_chunks, jobs;   // jobs = B * Hkv * n_chunks
};

hipError_t launch_chunk_landmarks(const LandmarkArgs& a, bool bf16, int D, hipStream_t st);

// Top-K covering every eligible chunk: fused scores, in-chunk attention and
// online blend over all eligible chunks (bf16, G = 8 or 16).
struct GlobalArgs {
  const void* q_ret;      // [B, Lq, Hkv, D]
  const void* landmarks;  // [B, Hkv, Nc, D]
  const void* q_attn;     // [B, Lq, Hq, D]
  const void* k;          // [B, Hkv, Lkv, D]
  const void* v;
  void* k_hat;            // [B, Hkv, Nc * 64, D] normalised keys (bf16, workspace), with qk_norm
  void* out;              // [B, Lq, Hq, D]
  int64_t Lq, q_pos0, Lkv, Nc;
  int32_t Hq, Hkv;
  float ret_scale, attn_scale;
  int32_t qk_norm;
};

// Normalised keys of the complete chunks into a.k_hat, then the global kernel.
hipError_t launch_attend_global(const GlobalArgs& a, int64_t B, int D, int G, hipStream_t st);
hipError_t launch_scan(const ScanArgs& a, int64_t B, bool bf16, int D, hipStream_t st);
hipError_t launch_scan_wide(const ScanArgs& a, int64_t B, bool bf16, int D, hipStream_t st);
int scan_wide_chunks();
hipError_t launch_scan_block(const ScanArgs& a, int64_t B, int D, hipStream_t st);
int scan_block_max_k();
hipError_t launch_attend(const AttendArgs& a, int64_t B, bool bf16, int D, int G, hipStream_t st);
hipError_t launch_merge_lists(const MergeArgs& a, hipStream_t st);
hipError_t launch_attend_decode(const DecodeArgs& a, int64_t rows, int D, int G, hipStream_t st);
int decode_slots_per_block();
hipError_t launch_attend_chunk(const ChunkArgs& a, int D, int G, hipStream_t st, const Marks& mk);
// Pair bucketing alone: weights, bin counts and offsets, work items, pair ids.
hipError_t launch_bucket(const ChunkArgs& a, hipStream_t st);
int64_t chunk_pairs_per_item();   // forward work items of large problems (else 64)
int64_t chunk_band_rows();        // forward bins
int64_t chunk_scan_tiles(int64_t n_bins);   // tiles of the bin scan (entries of seg_tot / 2)
int64_t bwd_band_rows();          // backward bins (each bin sortable in LDS)
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t value, hipStream_t st);

}  // namespace hsa
