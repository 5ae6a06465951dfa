// hsa_internal.h -- launch interface between the C ABI host code and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hsa {

// Landmark scan + per-split top-K (Steps 1-2).
struct ScanArgs {
  const void* q_ret;      // [B, Lq, Hkv, D]
  const void* landmarks;  // [B, Hkv, Nc, D]
  int32_t* out_idx;       // [B, Lq, Hkv, K]
  float* out_score;       // [B, Lq, Hkv, K]
  uint64_t* lists;        // [B*Lq*Hkv, n_splits, K] per-split sorted candidates (wide, n_splits > 1)
  uint32_t* counters;     // one arrival counter per row block (wide, n_splits > 1), zero on entry
  int64_t Lq, q_pos0, Nc;
  int32_t Hkv, K;
  int32_t n_max;          // max eligible chunks over all rows
  int32_t split_len;      // chunks per split: 1024 (wide) or all eligible chunks
  int32_t n_splits;       // 1 for the one-wave scan
  float ret_scale;
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

hipError_t launch_scan(const ScanArgs& a, int64_t B, bool bf16, int D, hipStream_t st);
hipError_t launch_scan_wide(const ScanArgs& a, int64_t B, bool bf16, int D, hipStream_t st);
int scan_wide_chunks();
hipError_t launch_attend(const AttendArgs& a, int64_t B, bool bf16, int D, int G, hipStream_t st);
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t value, hipStream_t st);

}  // namespace hsa
