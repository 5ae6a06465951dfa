// hsa_api.hip -- C ABI of the HSA forward (see include/hsa.h): argument checks,
// work planning, workspace layout and kernel launch order.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "hsa.h"
#include "hsa_internal.h"

#define HSA_EXPORT extern "C" __attribute__((visibility("default")))

namespace hsa {
namespace {

constexpr int64_t kRowsPerWave = 16;
constexpr int64_t kMaxSplits = 512;    // wide scan: 1024 chunks x 512 splits
// the block scan pays off with many rows per (batch, kv head) over a long
// history (the wide scan re-reads the landmarks once per 16 rows)
constexpr int64_t kBlockScanMinRows = 512;
constexpr int64_t kBigItemPairs = INT64_C(1) << 22;   // (row, slot) pairs from which items hold 128
constexpr int64_t kBlockScanMinChunks = 128;
// The workspace starts with arrival counters that every call leaves at zero.
constexpr size_t kCounterBytes = 16384;
constexpr int64_t kWideMaxRowBlocks = 2048;   // wide scan: at most this many blocks of 16 rows
constexpr int64_t kAttendCounterBase = 2048;  // counters [2048, 4096): attend rows ([0, 2048) unused)
constexpr int64_t kAttendCounters = 2048;
static_assert((kAttendCounterBase + kAttendCounters) * 4 <= (int64_t)kCounterBytes, "counter region");

struct Plan {
  int64_t B, Lq, q_pos0, Lkv, Nc;
  int32_t Hq, Hkv, G, D, K;
  bool bf16, qk_norm;
  float ret_scale, attn_scale;
  int64_t rows;          // B * Lq * Hkv selection rows
  int32_t n_max;         // max eligible chunks over all query rows
  int32_t split_len, n_splits;
  bool wide;             // few-row scan: 16-wave workgroups, per-split lists
  bool block;            // many-row scan (bf16, K <= 32): 64 rows per workgroup
  bool global;           // K covers every eligible chunk (K > 64): fused dense kernel
  int32_t attn_splits, slots_per_split, attn_mode;
  int64_t n_bins, max_items, n_bands;   // chunk-major attend
  int32_t pairs_per_item;
  size_t off_idx, off_score, off_lists, off_partials, off_counters, total;
  size_t off_ccounts, off_coffsets, off_ccursor, off_citems, off_cnitems, off_cpairs, off_cwts,
      off_cparts, off_cseg;
  size_t off_khat = 0;   // global HSA with qk_norm: normalised keys
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool mul_ok(int64_t a, int64_t b, int64_t limit) { return a >= 0 && b >= 0 && (b == 0 || a <= limit / b); }

// check_positions: reject rows whose eligible chunks would reach past the
// history (not needed when the caller supplies the selection).  allow_global:
// a top_k above 64 that covers every row's eligible chunks is planned as
// global HSA (hsa_forward only).  big_selection: a given selection may have
// any number of slots (the backward, which takes the selection as an input).
hsa_status_t make_plan(const hsa_shape_t* s, Plan* p, bool check_positions, bool allow_global = false,
                       bool big_selection = false) {
  if (!s) return HSA_ERR_NULL_POINTER;
  if (s->batch < 1 || s->q_len < 1 || s->kv_len < 0 || s->q_pos0 < 0 || s->n_q_heads < 1 ||
      s->n_kv_heads < 1 || s->top_k < 1)
    return HSA_ERR_BAD_SHAPE;
  if (s->n_q_heads % s->n_kv_heads) return HSA_ERR_BAD_SHAPE;
  const int32_t G = s->n_q_heads / s->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return HSA_ERR_UNSUPPORTED;
  if (s->head_dim != 64 && s->head_dim != 128) return HSA_ERR_UNSUPPORTED;
  const bool big_k = s->top_k > HSA_MAX_TOP_K && !big_selection;
  if (big_k && !allow_global) return HSA_ERR_UNSUPPORTED;
  if (s->dtype != HSA_DTYPE_F32 && s->dtype != HSA_DTYPE_BF16) return HSA_ERR_UNSUPPORTED;
  if (s->flags & ~HSA_FLAG_QK_L2NORM) return HSA_ERR_UNSUPPORTED;
  if (!(std::isfinite(s->ret_scale) && std::isfinite(s->attn_scale))) return HSA_ERR_BAD_SHAPE;

  const int64_t lim = INT64_C(1) << 60;
  const int64_t Nc = s->kv_len / HSA_CHUNK_TOKENS;
  if (Nc > INT32_MAX - 1) return HSA_ERR_BAD_SHAPE;
  if (s->q_pos0 > lim - s->q_len) return HSA_ERR_BAD_SHAPE;
  const int64_t last_pos = s->q_pos0 + s->q_len - 1;
  if (check_positions && last_pos / HSA_CHUNK_TOKENS > Nc) return HSA_ERR_BAD_SHAPE;
  if (!mul_ok(s->batch, s->q_len, lim) || !mul_ok((int64_t)s->batch * s->q_len, s->n_q_heads, lim) ||
      !mul_ok((int64_t)s->batch * s->q_len * s->n_q_heads, s->head_dim, lim) ||
      !mul_ok((int64_t)s->batch * s->n_kv_heads, s->kv_len, lim) ||
      !mul_ok((int64_t)s->batch * s->n_kv_heads * s->kv_len, s->head_dim, lim))
    return HSA_ERR_BAD_SHAPE;

  p->B = s->batch; p->Lq = s->q_len; p->q_pos0 = s->q_pos0; p->Lkv = s->kv_len; p->Nc = Nc;
  p->Hq = s->n_q_heads; p->Hkv = s->n_kv_heads; p->G = G; p->D = s->head_dim; p->K = s->top_k;
  p->bf16 = s->dtype == HSA_DTYPE_BF16;
  p->qk_norm = (s->flags & HSA_FLAG_QK_L2NORM) != 0;
  const float dflt = 1.0f / std::sqrt((float)s->head_dim);
  p->ret_scale = s->ret_scale > 0.f ? s->ret_scale : dflt;
  p->attn_scale = s->attn_scale > 0.f ? s->attn_scale : dflt;
  p->rows = (int64_t)s->batch * s->q_len * s->n_kv_heads;
  if (p->rows > INT32_MAX) return HSA_ERR_BAD_SHAPE;  // one grid row per selection row

  const int64_t nmax = std::min<int64_t>(last_pos / HSA_CHUNK_TOKENS, Nc);
  p->n_max = (int32_t)nmax;
  p->global = false;
  if (big_k) {   // every eligible chunk selected: no top-K, no selection arrays
    if (!p->bf16 || s->top_k < nmax) return HSA_ERR_UNSUPPORTED;
    p->global = true;
    p->wide = p->block = false;
    p->n_splits = 1;
    p->attn_mode = 4;
    p->off_counters = 0;
    p->total = kCounterBytes;
    p->off_khat = 0;
    if (p->qk_norm && Nc > 0) {   // normalised keys of the complete chunks, staged once per call
      p->off_khat = align_up(p->total, 256);
      p->total = p->off_khat + (size_t)(s->batch * s->n_kv_heads) * (size_t)Nc * HSA_CHUNK_TOKENS * p->D * 2;
    }
    return HSA_OK;
  }
  // Scan plan.  bf16 with K <= 32, at least kBlockScanMinRows rows per
  // (batch, kv head) and kBlockScanMinChunks eligible chunks: the block kernel
  // (64 rows per workgroup over all their chunks).  Otherwise up to 2048 row blocks of 16 rows: the wide kernel (1024
  // chunks per workgroup; with several splits a merge combines the per-split
  // lists); beyond that the block kernel where it applies, else one wave per
  // 16 rows.
  const int64_t row_blocks = (s->q_len + kRowsPerWave - 1) / kRowsPerWave * s->batch * s->n_kv_heads;
  if (row_blocks > INT32_MAX) return HSA_ERR_BAD_SHAPE;
  const int64_t wchunks = 1024;
  const int64_t wsplits = std::max<int64_t>(1, (nmax + wchunks - 1) / wchunks);
  // many rows per (batch, kv head) in bf16 with K <= 32: the block scan (each
  // landmark tile read once per 64 rows); few rows: the wide scan
  const bool block_ok = p->bf16 && p->K <= scan_block_max_k();
  p->block = block_ok && s->q_len >= kBlockScanMinRows && nmax >= kBlockScanMinChunks;
  p->wide = !p->block && row_blocks <= kWideMaxRowBlocks && wsplits <= kMaxSplits;
  p->block = p->block || (!p->wide && block_ok);
  p->split_len = (int32_t)(p->wide ? wchunks : std::max<int64_t>(64, (nmax + 63) / 64 * 64));
  p->n_splits = (int32_t)(p->wide ? wsplits : 1);

  // Attend plan.  Few rows: one workgroup per (row, slot), partials combined by
  // the last slot to finish.  Many rows, bf16: pairs bucketed by chunk, one
  // MFMA workgroup per block of pairs of a chunk, then a slot-ordered combine.
  // Many rows, fp32: one wave per row.
  p->n_bands = (s->q_len + chunk_band_rows() - 1) / chunk_band_rows();
  p->n_bins = (int64_t)s->batch * s->n_kv_heads * p->n_bands * Nc;
  const int64_t n_pairs = p->rows * p->K;
  // large problems: 128-pair items (K and V staged half as often); smaller ones
  // keep 64-pair items so the items still fill the GPU
  p->pairs_per_item = n_pairs >= kBigItemPairs ? (int32_t)chunk_pairs_per_item() : 64;
  p->max_items = (n_pairs + p->pairs_per_item - 1) / p->pairs_per_item + p->n_bins;
  if (p->rows < 1024 && p->bf16) {
    p->attn_mode = 3;
    p->attn_splits = (p->K + decode_slots_per_block() - 1) / decode_slots_per_block();
    p->slots_per_split = decode_slots_per_block();
  } else if (p->rows < 1024) {
    p->attn_mode = 1;
    p->attn_splits = p->K;
    p->slots_per_split = 1;
  } else if (p->bf16 && n_pairs < INT32_MAX && p->n_bins + 1 < INT32_MAX && p->max_items < INT32_MAX) {
    p->attn_mode = 2;
    p->attn_splits = 1;
    p->slots_per_split = p->K;
  } else {
    p->attn_mode = 0;
    p->attn_splits = 1;
    p->slots_per_split = p->K;
  }

  size_t off = kCounterBytes;
  p->off_counters = 0;
  p->off_idx = off; off = align_up(off + (size_t)p->rows * p->K * 4, 256);
  p->off_score = off; off = align_up(off + (size_t)p->rows * p->K * 4, 256);
  p->off_lists = off;
  if (p->n_splits > 1) off = align_up(off + (size_t)p->rows * p->n_splits * p->K * 8, 256);
  p->off_partials = off;
  if (p->attn_splits > 1) off = align_up(off + (size_t)p->rows * p->attn_splits * G * p->D * 4, 256);
  p->off_ccounts = p->off_coffsets = p->off_ccursor = p->off_citems = p->off_cnitems = 0;
  p->off_cpairs = p->off_cwts = p->off_cparts = p->off_cseg = 0;
  if (p->attn_mode == 2) {
    const size_t nb = (size_t)p->n_bins, np = (size_t)n_pairs;
    p->off_ccounts = off; off = align_up(off + nb * 4, 256);
    p->off_coffsets = off; off = align_up(off + (nb + 1) * 4, 256);
    p->off_ccursor = off; off = align_up(off + nb * 4, 256);
    p->off_citems = off; off = align_up(off + (size_t)p->max_items * 8, 256);
    p->off_cnitems = off; off = align_up(off + 4, 256);
    p->off_cseg = off; off = align_up(off + (size_t)chunk_scan_tiles(p->n_bins) * 8, 256);
    p->off_cpairs = off; off = align_up(off + np * 4, 256);
    p->off_cwts = off; off = align_up(off + np * 4, 256);
    p->off_cparts = off; off = align_up(off + np * G * p->D * 2, 256);
  }
  p->total = off;
  return HSA_OK;
}

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

hsa_status_t check_ws(const Plan& p, void* ws, size_t ws_bytes) {
  if (!ws) return HSA_ERR_NULL_POINTER;
  if (!aligned(ws, 256)) return HSA_ERR_MISALIGNED;
  if (ws_bytes < p.total) return HSA_ERR_WORKSPACE_TOO_SMALL;
  return HSA_OK;
}

hsa_status_t check_ptrs(std::initializer_list<const void*> ptrs) {
  for (const void* q : ptrs)
    if (!q) return HSA_ERR_NULL_POINTER;
  for (const void* q : ptrs)
    if (!aligned(q, 16)) return HSA_ERR_MISALIGNED;
  return HSA_OK;
}

// Landmark scan; with several splits, the per-split lists are merged into the
// final selection unless the caller merges them itself (merge = false).
hsa_status_t launch_retrieve(const Plan& p, const void* q_ret, const void* landmarks,
                             int32_t* idx, float* score, void* ws, hipStream_t st, bool merge,
                             const Marks& mk) {
  char* w = static_cast<char*>(ws);
  ScanArgs a;
  a.q_ret = q_ret; a.landmarks = landmarks; a.out_idx = idx; a.out_score = score;
  a.lists = reinterpret_cast<uint64_t*>(w + p.off_lists);
  a.Lq = p.Lq; a.q_pos0 = p.q_pos0; a.Nc = p.Nc; a.Hkv = p.Hkv; a.K = p.K;
  a.n_max = p.n_max; a.split_len = p.split_len; a.n_splits = p.n_splits; a.ret_scale = p.ret_scale;
  if (mk.rec(kStageScan, 0, st) != hipSuccess) return HSA_ERR_DEVICE;
  const hipError_t e = p.wide    ? launch_scan_wide(a, p.B, p.bf16, p.D, st)
                       : p.block ? launch_scan_block(a, p.B, p.D, st)
                                 : launch_scan(a, p.B, p.bf16, p.D, st);
  if (e != hipSuccess || mk.rec(kStageScan, 1, st) != hipSuccess) return HSA_ERR_DEVICE;
  if (merge && p.n_splits > 1) {
    MergeArgs m;
    m.lists = a.lists; m.out_idx = idx; m.out_score = score; m.rows = p.rows;
    m.n_splits = p.n_splits; m.K = p.K; m.ret_scale = p.ret_scale;
    if (mk.rec(kStageMerge, 0, st) != hipSuccess || launch_merge_lists(m, st) != hipSuccess ||
        mk.rec(kStageMerge, 1, st) != hipSuccess)
      return HSA_ERR_DEVICE;
  }
  return HSA_OK;
}

// Decode attend: merges the scan's lists itself when `lists` is given.
hsa_status_t launch_decode(const Plan& p, const void* q_attn, const void* k, const void* v,
                           const uint64_t* lists, const int32_t* idx_in, const float* score_in,
                           int32_t* idx_out, float* score_out, void* out, void* ws, hipStream_t st,
                           const Marks& mk) {
  char* w = static_cast<char*>(ws);
  DecodeArgs a;
  a.q_attn = q_attn; a.k = k; a.v = v; a.lists = lists; a.idx_in = idx_in; a.score_in = score_in;
  a.idx_out = idx_out; a.score_out = score_out; a.out = out;
  a.partials = reinterpret_cast<float*>(w + p.off_partials);
  a.counters = reinterpret_cast<uint32_t*>(w + p.off_counters) + kAttendCounterBase;
  a.Lq = p.Lq; a.Lkv = p.Lkv; a.Nc = p.Nc; a.Hq = p.Hq; a.Hkv = p.Hkv; a.K = p.K;
  a.n_splits = p.n_splits; a.n_blocks = p.attn_splits;
  a.ret_scale = p.ret_scale; a.attn_scale = p.attn_scale; a.qk_norm = p.qk_norm ? 1 : 0;
  if (mk.rec(kStageAttend, 0, st) != hipSuccess || launch_attend_decode(a, p.rows, p.D, p.G, st) != hipSuccess ||
      mk.rec(kStageAttend, 1, st) != hipSuccess)
    return HSA_ERR_DEVICE;
  return HSA_OK;
}

hsa_status_t launch_attend_blend(const Plan& p, const void* q_attn, const void* k, const void* v,
                                 const int32_t* idx, const float* score, void* out, void* ws,
                                 hipStream_t st, const Marks& mk) {
  char* w = static_cast<char*>(ws);
  AttendArgs a;
  a.q_attn = q_attn; a.k = k; a.v = v; a.idx = idx; a.score = score; a.out = out;
  a.partials = reinterpret_cast<float*>(w + p.off_partials);
  a.counters = reinterpret_cast<uint32_t*>(w + p.off_counters) + kAttendCounterBase;
  a.Lq = p.Lq; a.Lkv = p.Lkv; a.Nc = p.Nc; a.Hq = p.Hq; a.Hkv = p.Hkv; a.K = p.K;
  a.n_splits = p.attn_splits; a.slots_per_split = p.slots_per_split;
  a.attn_scale = p.attn_scale; a.qk_norm = p.qk_norm ? 1 : 0; a.mode = p.attn_mode;
  if (p.attn_mode == 3)
    return launch_decode(p, q_attn, k, v, nullptr, idx, score, nullptr, nullptr, out, ws, st, mk);
  if (p.attn_mode == 2) {
    ChunkArgs c;
    c.q_attn = q_attn; c.k = k; c.v = v; c.idx = idx; c.score = score; c.out = out;
    c.counts = reinterpret_cast<uint32_t*>(w + p.off_ccounts);
    c.offsets = reinterpret_cast<uint32_t*>(w + p.off_coffsets);
    c.cursor = reinterpret_cast<uint32_t*>(w + p.off_ccursor);
    c.items = reinterpret_cast<uint64_t*>(w + p.off_citems);
    c.n_items = reinterpret_cast<uint32_t*>(w + p.off_cnitems);
    c.seg_tot = reinterpret_cast<uint32_t*>(w + p.off_cseg);
    c.item_start = nullptr;
    c.pairs = reinterpret_cast<uint32_t*>(w + p.off_cpairs);
    c.wts = reinterpret_cast<float*>(w + p.off_cwts);
    c.partials = reinterpret_cast<uint16_t*>(w + p.off_cparts);
    c.rows = p.rows; c.Lq = p.Lq; c.Lkv = p.Lkv; c.Nc = p.Nc; c.n_bins = p.n_bins;
    c.max_items = p.max_items; c.Hq = p.Hq; c.Hkv = p.Hkv; c.K = p.K;
    c.band_rows = chunk_band_rows(); c.n_bands = p.n_bands;
    c.pairs_per_item = p.pairs_per_item;
    c.attn_scale = p.attn_scale; c.qk_norm = p.qk_norm ? 1 : 0;
    return launch_attend_chunk(c, p.D, p.G, st, mk) == hipSuccess ? HSA_OK : HSA_ERR_DEVICE;
  }
  if (mk.rec(kStageAttend, 0, st) != hipSuccess || launch_attend(a, p.B, p.bf16, p.D, p.G, st) != hipSuccess ||
      mk.rec(kStageAttend, 1, st) != hipSuccess)
    return HSA_ERR_DEVICE;
  return HSA_OK;
}

}  // namespace
}  // namespace hsa

using hsa::Plan;

HSA_EXPORT hsa_status_t hsa_workspace_size(const hsa_shape_t* shape, size_t* bytes) {
  if (!bytes) return HSA_ERR_NULL_POINTER;
  Plan p;
  const hsa_status_t st = hsa::make_plan(shape, &p, false, true);
  if (st != HSA_OK) return st;
  *bytes = p.total;
  return HSA_OK;
}

HSA_EXPORT hsa_status_t hsa_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return HSA_ERR_NULL_POINTER;
  if (!hsa::aligned(ws, 256)) return HSA_ERR_MISALIGNED;
  if (ws_bytes < hsa::kCounterBytes) return HSA_ERR_WORKSPACE_TOO_SMALL;
  const hipError_t e = hsa::launch_fill_u32(static_cast<uint32_t*>(ws), hsa::kCounterBytes / 4, 0u,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? HSA_OK : HSA_ERR_DEVICE;
}

HSA_EXPORT hsa_status_t hsa_retrieve_topk(const hsa_shape_t* shape, const void* q_ret,
                                          const void* landmarks, int32_t* topk_idx,
                                          float* topk_score, void* ws, size_t ws_bytes,
                                          void* stream) {
  Plan p;
  hsa_status_t st = hsa::make_plan(shape, &p, true);
  if (st != HSA_OK) return st;
  const void* lm = p.Nc > 0 ? landmarks : q_ret;  // landmarks may be empty when Nc == 0
  if ((st = hsa::check_ptrs({q_ret, lm, topk_idx, topk_score})) != HSA_OK) return st;
  if ((st = hsa::check_ws(p, ws, ws_bytes)) != HSA_OK) return st;
  return hsa::launch_retrieve(p, q_ret, landmarks, topk_idx, topk_score, ws,
                              static_cast<hipStream_t>(stream), true, hsa::Marks{});
}

HSA_EXPORT hsa_status_t hsa_chunk_attend_blend(const hsa_shape_t* shape, const void* q_attn,
                                               const void* k, const void* v,
                                               const int32_t* topk_idx, const float* topk_score,
                                               void* out, void* ws, size_t ws_bytes,
                                               void* stream) {
  Plan p;
  hsa_status_t st = hsa::make_plan(shape, &p, false);
  if (st != HSA_OK) return st;
  const void* kk = p.Lkv > 0 ? k : q_attn;
  const void* vv = p.Lkv > 0 ? v : q_attn;
  if ((st = hsa::check_ptrs({q_attn, kk, vv, topk_idx, topk_score, out})) != HSA_OK) return st;
  if ((st = hsa::check_ws(p, ws, ws_bytes)) != HSA_OK) return st;
  return hsa::launch_attend_blend(p, q_attn, k, v, topk_idx, topk_score, out, ws,
                                  static_cast<hipStream_t>(stream), hsa::Marks{});
}

namespace hsa {
namespace {

hsa_status_t forward_impl(const hsa_shape_t* shape, const void* q_ret, const void* landmarks,
                          const void* q_attn, const void* k, const void* v, void* out,
                          int32_t* topk_idx, float* topk_score, void* ws, size_t ws_bytes,
                          void* stream, const Marks& mk) {
  Plan p;
  hsa_status_t st = make_plan(shape, &p, true, true);
  if (st != HSA_OK) return st;
  const void* lm = p.Nc > 0 ? landmarks : q_ret;
  const void* kk = p.Lkv > 0 ? k : q_attn;
  const void* vv = p.Lkv > 0 ? v : q_attn;
  if ((st = check_ptrs({q_ret, lm, q_attn, kk, vv, out})) != HSA_OK) return st;
  if ((topk_idx == nullptr) != (topk_score == nullptr)) return HSA_ERR_NULL_POINTER;
  if (topk_idx && p.global) return HSA_ERR_UNSUPPORTED;   // the selection is every eligible chunk
  if (topk_idx && (st = check_ptrs({topk_idx, topk_score})) != HSA_OK) return st;
  if ((st = check_ws(p, ws, ws_bytes)) != HSA_OK) return st;
  if (p.global) {
    GlobalArgs g;
    g.q_ret = q_ret; g.landmarks = lm; g.q_attn = q_attn; g.k = kk; g.v = vv; g.out = out;
    g.k_hat = p.off_khat ? static_cast<char*>(ws) + p.off_khat : nullptr;
    g.Lq = p.Lq; g.q_pos0 = p.q_pos0; g.Lkv = p.Lkv; g.Nc = p.Nc; g.Hq = p.Hq; g.Hkv = p.Hkv;
    g.ret_scale = p.ret_scale; g.attn_scale = p.attn_scale; g.qk_norm = p.qk_norm ? 1 : 0;
    const hipStream_t gs = static_cast<hipStream_t>(stream);
    if (mk.rec(kStageAttend, 0, gs) != hipSuccess || launch_attend_global(g, p.B, p.D, p.G, gs) != hipSuccess ||
        mk.rec(kStageAttend, 1, gs) != hipSuccess)
      return HSA_ERR_DEVICE;
    return HSA_OK;
  }
  char* w = static_cast<char*>(ws);
  int32_t* idx = topk_idx ? topk_idx : reinterpret_cast<int32_t*>(w + p.off_idx);
  float* score = topk_score ? topk_score : reinterpret_cast<float*>(w + p.off_score);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.attn_mode == 3 && p.n_splits > 1) {   // decode: the attend merges the lists
    if ((st = launch_retrieve(p, q_ret, landmarks, idx, score, ws, s, false, mk)) != HSA_OK) return st;
    return launch_decode(p, q_attn, k, v, reinterpret_cast<const uint64_t*>(w + p.off_lists), nullptr,
                         nullptr, topk_idx, topk_score, out, ws, s, mk);
  }
  if ((st = launch_retrieve(p, q_ret, landmarks, idx, score, ws, s, true, mk)) != HSA_OK) return st;
  return launch_attend_blend(p, q_attn, k, v, idx, score, out, ws, s, mk);
}

}  // namespace
}  // namespace hsa

HSA_EXPORT hsa_status_t hsa_forward(const hsa_shape_t* shape, const void* q_ret,
                                    const void* landmarks, const void* q_attn, const void* k,
                                    const void* v, void* out, int32_t* topk_idx,
                                    float* topk_score, void* ws, size_t ws_bytes, void* stream) {
  return hsa::forward_impl(shape, q_ret, landmarks, q_attn, k, v, out, topk_idx, topk_score, ws,
                           ws_bytes, stream, hsa::Marks{});
}

HSA_EXPORT hsa_status_t hsa_forward_profiled(const hsa_shape_t* shape, const void* q_ret,
                                             const void* landmarks, const void* q_attn,
                                             const void* k, const void* v, void* out,
                                             int32_t* topk_idx, float* topk_score, void* ws,
                                             size_t ws_bytes, void* stream,
                                             void* const* stage_events) {
  hsa::Marks mk;
  mk.ev = stage_events;
  return hsa::forward_impl(shape, q_ret, landmarks, q_attn, k, v, out, topk_idx, topk_score, ws,
                           ws_bytes, stream, mk);
}

HSA_EXPORT hsa_status_t hsa_chunk_landmarks(const hsa_shape_t* shape, const void* k, void* landmarks,
                                            int64_t chunk_begin, int64_t chunk_end, void* stream) {
  if (!shape) return HSA_ERR_NULL_POINTER;
  if (shape->batch < 1 || shape->n_kv_heads < 1 || shape->kv_len < 0) return HSA_ERR_BAD_SHAPE;
  if (shape->head_dim != 64 && shape->head_dim != 128) return HSA_ERR_UNSUPPORTED;
  if (shape->dtype != HSA_DTYPE_F32 && shape->dtype != HSA_DTYPE_BF16) return HSA_ERR_UNSUPPORTED;
  const int64_t Nc = shape->kv_len / HSA_CHUNK_TOKENS;
  if (chunk_begin < 0 || chunk_end < chunk_begin || chunk_end > Nc) return HSA_ERR_BAD_SHAPE;
  const int64_t lim = INT64_C(1) << 60;
  if (!hsa::mul_ok((int64_t)shape->batch * shape->n_kv_heads, shape->kv_len, lim) ||
      !hsa::mul_ok((int64_t)shape->batch * shape->n_kv_heads * shape->kv_len, shape->head_dim, lim))
    return HSA_ERR_BAD_SHAPE;
  hsa::LandmarkArgs a;
  a.k = k; a.landmarks = landmarks; a.Lkv = shape->kv_len; a.Nc = Nc;
  a.c_begin = chunk_begin; a.n_chunks = chunk_end - chunk_begin;
  a.jobs = (int64_t)shape->batch * shape->n_kv_heads * a.n_chunks;
  if (a.jobs == 0) return HSA_OK;
  if ((a.jobs + 3) / 4 > INT32_MAX) return HSA_ERR_BAD_SHAPE;
  hsa_status_t st;
  if ((st = hsa::check_ptrs({k, landmarks})) != HSA_OK) return st;
  return hsa::launch_chunk_landmarks(a, shape->dtype == HSA_DTYPE_BF16, shape->head_dim,
                                     static_cast<hipStream_t>(stream)) == hipSuccess
             ? HSA_OK : HSA_ERR_DEVICE;
}

namespace hsa {
namespace {

struct BwdPlan {
  Plan p;
  size_t off_counts, off_offsets, off_cursor, off_items, off_nitems, off_seg, off_istart, off_pairs,
      off_wts, off_wdw, off_draw, off_dqp, off_itemp, total;
};

hsa_status_t make_bwd_plan(const hsa_shape_t* s, BwdPlan* b) {
  hsa_status_t st = make_plan(s, &b->p, false, false, true);
  if (st != HSA_OK) return st;
  Plan& p = b->p;
  // backward bins and work items: smaller bands (every bin sortable in LDS)
  // and at most bwd_pairs_per_item() pairs per item
  p.n_bands = (p.Lq + bwd_band_rows() - 1) / bwd_band_rows();
  p.n_bins = p.rows / p.Lq * p.n_bands * p.Nc;
  p.max_items = (p.rows * p.K + bwd_pairs_per_item() - 1) / bwd_pairs_per_item() + p.n_bins;
  if (!p.bf16) return HSA_ERR_UNSUPPORTED;
  const int64_t n_pairs = p.rows * p.K, n_bg = p.rows / p.Lq;
  // grid sizes: per-row kernels take (rows * G + rows) / 8 workgroups at most,
  // per-chunk kernels 8 per chunk
  if (n_pairs >= INT32_MAX || p.n_bins + 1 >= INT32_MAX || p.max_items >= INT32_MAX ||
      n_bg * (p.Nc + 1) >= INT32_MAX / 8 || p.rows * (p.G + 1) / 8 >= INT32_MAX)
    return HSA_ERR_BAD_SHAPE;
  const size_t nb = (size_t)p.n_bins, np = (size_t)n_pairs, D = (size_t)p.D;
  size_t off = 0;
  b->off_counts = off; off = align_up(off + nb * 4, 256);
  b->off_offsets = off; off = align_up(off + (nb + 1) * 4, 256);
  b->off_cursor = off; off = align_up(off + nb * 4, 256);
  b->off_items = off; off = align_up(off + (size_t)p.max_items * 8, 256);
  b->off_nitems = off; off = align_up(off + 4, 256);
  b->off_seg = off; off = align_up(off + (size_t)chunk_scan_tiles(p.n_bins) * 8, 256);
  b->off_istart = off; off = align_up(off + nb * 4, 256);
  b->off_pairs = off; off = align_up(off + np * 4, 256);
  b->off_wts = off; off = align_up(off + np * 4, 256);
  b->off_wdw = off; off = align_up(off + np * 4, 256);
  b->off_draw = off; off = align_up(off + np * 4, 256);
  b->off_dqp = off; off = align_up(off + np * p.G * D * 2, 256);
  b->off_itemp = off; off = align_up(off + (size_t)p.max_items * 2 * HSA_CHUNK_TOKENS * D * 4, 256);
  b->total = std::max<size_t>(off, 256);
  return HSA_OK;
}

}  // namespace
}  // namespace hsa

HSA_EXPORT hsa_status_t hsa_backward_workspace_size(const hsa_shape_t* shape, size_t* bytes) {
  if (!bytes) return HSA_ERR_NULL_POINTER;
  hsa::BwdPlan b;
  const hsa_status_t st = hsa::make_bwd_plan(shape, &b);
  if (st != HSA_OK) return st;
  *bytes = b.total;
  return HSA_OK;
}

namespace hsa {
namespace {

hsa_status_t backward_impl(const hsa_shape_t* shape, const void* q_ret, const void* landmarks,
                           const void* q_attn, const void* k, const void* v, const int32_t* topk_idx,
                           const float* topk_score, const void* dout, float* dq_ret, float* dlandmarks,
                           float* dq_attn, float* dk, float* dv, void* ws, size_t ws_bytes, void* stream,
                           const Marks& mk) {
  hsa::BwdPlan b;
  hsa_status_t st = hsa::make_bwd_plan(shape, &b);
  if (st != HSA_OK) return st;
  const Plan& p = b.p;
  // empty tensors may come as NULL: stand in a pointer that is never read
  const void* lm = p.Nc > 0 ? landmarks : q_ret;
  const void* dlm = p.Nc > 0 ? static_cast<const void*>(dlandmarks) : dq_ret;
  const void* kk = p.Lkv > 0 ? k : q_attn;
  const void* vv = p.Lkv > 0 ? v : q_attn;
  const void* dkk = p.Lkv > 0 ? static_cast<const void*>(dk) : dq_attn;
  const void* dvv = p.Lkv > 0 ? static_cast<const void*>(dv) : dq_attn;
  if ((st = hsa::check_ptrs({q_ret, lm, q_attn, kk, vv, topk_idx, topk_score, dout, dq_ret, dlm, dq_attn,
                             dkk, dvv})) != HSA_OK)
    return st;
  if (!ws) return HSA_ERR_NULL_POINTER;
  if (!hsa::aligned(ws, 256)) return HSA_ERR_MISALIGNED;
  if (ws_bytes < b.total) return HSA_ERR_WORKSPACE_TOO_SMALL;
  char* w = static_cast<char*>(ws);
  hsa::BwdArgs a;
  hsa::ChunkArgs& c = a.c;
  c.q_attn = q_attn; c.k = kk; c.v = vv; c.idx = topk_idx; c.score = topk_score; c.out = nullptr;
  c.counts = reinterpret_cast<uint32_t*>(w + b.off_counts);
  c.offsets = reinterpret_cast<uint32_t*>(w + b.off_offsets);
  c.cursor = reinterpret_cast<uint32_t*>(w + b.off_cursor);
  c.items = reinterpret_cast<uint64_t*>(w + b.off_items);
  c.n_items = reinterpret_cast<uint32_t*>(w + b.off_nitems);
  c.seg_tot = reinterpret_cast<uint32_t*>(w + b.off_seg);
  c.item_start = reinterpret_cast<uint32_t*>(w + b.off_istart);
  c.pairs = reinterpret_cast<uint32_t*>(w + b.off_pairs);
  c.wts = reinterpret_cast<float*>(w + b.off_wts);
  // bucketing scratch (each pair's rank in its bin, 4 bytes per pair): the dq^
  // partial region, which the item kernel only writes after the bucketing
  c.partials = reinterpret_cast<uint16_t*>(w + b.off_dqp);
  c.rows = p.rows; c.Lq = p.Lq; c.Lkv = p.Lkv; c.Nc = p.Nc; c.n_bins = p.n_bins;
  c.max_items = p.max_items; c.Hq = p.Hq; c.Hkv = p.Hkv; c.K = p.K;
  c.band_rows = hsa::bwd_band_rows(); c.n_bands = p.n_bands;
  c.pairs_per_item = (int32_t)hsa::bwd_pairs_per_item();
  c.attn_scale = p.attn_scale; c.qk_norm = p.qk_norm ? 1 : 0;
  a.q_ret = q_ret; a.landmarks = lm; a.dout = dout;
  a.dq_ret = dq_ret; a.dlandmarks = dlandmarks; a.dq_attn = dq_attn; a.dk = dk; a.dv = dv;
  a.wdw = reinterpret_cast<float*>(w + b.off_wdw);
  a.draw = reinterpret_cast<float*>(w + b.off_draw);
  a.dq_part = reinterpret_cast<uint16_t*>(w + b.off_dqp);
  a.item_part = reinterpret_cast<float*>(w + b.off_itemp);
  a.ret_scale = p.ret_scale;
  return hsa::launch_backward(a, p.D, p.G, static_cast<hipStream_t>(stream), mk) == hipSuccess
             ? HSA_OK : HSA_ERR_DEVICE;
}

}  // namespace
}  // namespace hsa

HSA_EXPORT hsa_status_t hsa_backward(const hsa_shape_t* shape, const void* q_ret, const void* landmarks,
                                     const void* q_attn, const void* k, const void* v,
                                     const int32_t* topk_idx, const float* topk_score,
                                     const void* dout, float* dq_ret, float* dlandmarks,
                                     float* dq_attn, float* dk, float* dv, void* ws,
                                     size_t ws_bytes, void* stream) {
  return hsa::backward_impl(shape, q_ret, landmarks, q_attn, k, v, topk_idx, topk_score, dout, dq_ret,
                            dlandmarks, dq_attn, dk, dv, ws, ws_bytes, stream, hsa::Marks{});
}

HSA_EXPORT hsa_status_t hsa_backward_profiled(const hsa_shape_t* shape, const void* q_ret,
                                              const void* landmarks, const void* q_attn, const void* k,
                                              const void* v, const int32_t* topk_idx,
                                              const float* topk_score, const void* dout, float* dq_ret,
                                              float* dlandmarks, float* dq_attn, float* dk, float* dv,
                                              void* ws, size_t ws_bytes, void* stream,
                                              void* const* stage_events) {
  hsa::Marks mk;
  mk.ev = stage_events;
  return hsa::backward_impl(shape, q_ret, landmarks, q_attn, k, v, topk_idx, topk_score, dout, dq_ret,
                            dlandmarks, dq_attn, dk, dv, ws, ws_bytes, stream, mk);
}

// ---------------------------------------------------------------------------
// hsa_forward_noalloc: hsa_forward with the library's own static scratch as
// the workspace, for callers that cannot allocate device memory.
//
// `scratch` is one file-scope device array; every GPU the library runs on holds
// its own copy until the process ends.  In host code its name is only a
// stand-in for the symbol, so its device address is taken once per device with
// hipGetSymbolAddress (that device current) and only that pointer is ever
// passed to kernels.  The arrival counters at its start are zeroed once, by a
// fill kernel, when the pointer is first taken on a device; every completed
// call leaves them zero, and a call that fails on the device zeroes them again
// (enqueued on its stream).  All calls on one GPU share the array: calls that
// overlap on one GPU race.
// ---------------------------------------------------------------------------
namespace hsa {
namespace {

constexpr size_t kStaticScratchBytes = size_t(HSA_STATIC_SCRATCH_BYTES);
constexpr int kMaxScratchDevices = 64;
static_assert(kStaticScratchBytes >= kCounterBytes, "static scratch holds the counter region");

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the current device's scratch; on first use on a device
// also enqueues the zeroing of its counter region on `st`.
hsa_status_t static_scratch(hipStream_t st, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return HSA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return HSA_ERR_DEVICE;
    if (launch_fill_u32(static_cast<uint32_t*>(p), (int64_t)(kCounterBytes / 4), 0u, st) != hipSuccess)
      return HSA_ERR_DEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HSA_OK;
}

}  // namespace
}  // namespace hsa

HSA_EXPORT hsa_status_t hsa_forward_noalloc(const hsa_shape_t* shape, const void* q_ret,
                                            const void* landmarks, const void* q_attn, const void* k,
                                            const void* v, void* out, int32_t* topk_idx,
                                            float* topk_score, void* stream) {
  hsa::Plan p;
  hsa_status_t st = hsa::make_plan(shape, &p, true, true);
  if (st != HSA_OK) return st;
  if (p.total > hsa::kStaticScratchBytes) return HSA_ERR_SCRATCH_TOO_SMALL;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if ((st = hsa::static_scratch(s, &ws)) != HSA_OK) return st;
  st = hsa::forward_impl(shape, q_ret, landmarks, q_attn, k, v, out, topk_idx, topk_score, ws,
                         hsa::kStaticScratchBytes, stream, hsa::Marks{});
  if (st == HSA_ERR_DEVICE)   // a partly launched call may have left counters non-zero (best effort:
                              // the call's own error is what is reported)
    (void)hsa::launch_fill_u32(static_cast<uint32_t*>(ws), (int64_t)(hsa::kCounterBytes / 4), 0u, s);
  return st;
}

HSA_EXPORT const char* hsa_status_string(hsa_status_t status) {
  switch (status) {
    case HSA_OK: return "success";
    case HSA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case HSA_ERR_BAD_SHAPE: return "inconsistent or out-of-range shape";
    case HSA_ERR_UNSUPPORTED: return "unsupported head_dim, group size, top_k, dtype or flag";
    case HSA_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than hsa_workspace_size()";
    case HSA_ERR_DEVICE: return "HIP launch or runtime error";
    case HSA_ERR_MISALIGNED: return "pointer not 16-byte aligned (workspace: 256-byte)";
    case HSA_ERR_SCRATCH_TOO_SMALL:
      return "shape needs more workspace than the library's static scratch (HSA_STATIC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

HSA_EXPORT int32_t hsa_version(void) { return 100; }
