// attend_chunk.hip -- chunk-major per-chunk attention and blend for many query
// rows (Steps 3-4 of the HSA step in "Every Token Counts", agent-atlas
// explainer, "How It Works (Technically)").
//
// With many rows the same chunk is selected by many (row, slot) pairs, while the
// pairs of one row point at unrelated chunks.  Gathering per row would move a
// chunk's 2*64*d values once per pair; here the pairs are bucketed by chunk so a
// workgroup stages one chunk's K and V in LDS once and runs every pair that
// selected it on MFMA tiles:
//   count    per row: blend weights w_k (softmax of the selected scores) and a
//            histogram of pairs per (batch, kv head, chunk) bin;
//   scan     bin offsets and the list of work items (bin, block of pairs_per_item pairs);
//   scatter  pair ids into their bins;
//   attend   per work item: K and V (row-major) in LDS, key norms once; per
//            tile of 16 head-rows (16/G pairs x G heads): S = Q K^T on
//            v_mfma_f32_16x16x32_bf16, in-chunk softmax across the tile's rows,
//            P (times w_k, rounded to bf16) V on MFMA, bf16 partial per pair;
//   combine  per row: the partials of its slots summed in slot order.
// Results do not depend on the order of pairs inside a bin: every pair writes
// only its own partial, and the combine order is fixed.
#include "hsa_device.h"
#include "hsa_internal.h"

namespace hsa {
namespace {

constexpr int kMaxPairs = 128;   // pairs per work item at most (ChunkArgs::pairs_per_item)
constexpr int kFwdPairs = 128;   // forward work items: K and V staged once per 128 pairs
constexpr float kLog2e = 1.4426950408889634f;

// Bins are (batch, kv head, band of band_rows query rows, chunk): items of one
// band run close together in time, so the band's queries stay in the
// Infinity Cache while its pairs are processed.
__device__ __forceinline__ int64_t bin_of(int64_t row, int32_t c, const ChunkArgs& a) {
  const int64_t bg = (row / ((int64_t)a.Lq * a.Hkv)) * a.Hkv + row % a.Hkv;
  const int64_t band = ((row / a.Hkv) % a.Lq) / a.band_rows;
  return (bg * a.n_bands + band) * a.Nc + c;
}

// Rows are laid out on segments of S lanes (S = the smallest power of two
// >= K), so a wave holds 64 / S rows and a workgroup 256 / S.
__device__ __forceinline__ int seg_lanes(int K) { return K <= 1 ? 1 : 1 << (32 - __clz(K - 1)); }

// --- count: blend weights and pairs per bin (one lane per slot) ------------
// The count's returning atomic gives each pair its place in its bin, kept in
// the partial-output region (free until the attend writes it) so that the
// scatter needs no atomics: place = the bin's first slot + that rank.
__global__ __launch_bounds__(256) void chunk_count_kernel(ChunkArgs a) {
  const int K = a.K, S = seg_lanes(K);
  const int64_t row = (int64_t)blockIdx.x * (256 / S) + threadIdx.x / S;
  const int k = threadIdx.x & (S - 1);
  const bool active = row < a.rows && k < K;
  int32_t c = -1;
  float s = 0.f;
  if (active) {
    c = a.idx[row * K + k];
    s = a.score[row * K + k];
  }
  const bool valid = active && c >= 0 && (int64_t)c < a.Nc;
  // xor butterflies: every lane of a segment ends with the same (commutative) result
  float mx = valid ? s : -INFINITY;
  for (int o = 1; o < S; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
  const float ex = valid ? expf(s - mx) : 0.f;
  float den = ex;
  for (int o = 1; o < S; o <<= 1) den += __shfl_xor(den, o, kWave);
  if (active) a.wts[row * K + k] = valid ? ex / den : 0.f;
  if (valid) reinterpret_cast<uint32_t*>(a.partials)[row * K + k] = atomicAdd(&a.counts[bin_of(row, c, a)], 1u);
}

// --- more than 64 slots per row (a selection of every eligible chunk) ---------
// Blend weights with one wave per row (slots strided over the lanes; the
// maximum and the sum are reduced in a fixed order), and the bin histogram and
// scatter with one thread per (row, slot) pair.
__global__ __launch_bounds__(256) void chunk_wts_wide_kernel(ChunkArgs a) {
  const int K = a.K, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int32_t* idx = a.idx + row * K;
  const float* sc = a.score + row * K;
  float mx = -INFINITY;
  for (int k = lane; k < K; k += kWave) {
    const int32_t c = idx[k];
    if (c >= 0 && (int64_t)c < a.Nc) mx = fmaxf(mx, sc[k]);
  }
  mx = wave_max(mx);
  float den = 0.f;
  for (int k = lane; k < K; k += kWave) {
    const int32_t c = idx[k];
    if (c >= 0 && (int64_t)c < a.Nc) den += expf(sc[k] - mx);
  }
  den = wave_sum(den);
  for (int k = lane; k < K; k += kWave) {
    const int32_t c = idx[k];
    a.wts[row * K + k] = (c >= 0 && (int64_t)c < a.Nc) ? expf(sc[k] - mx) / den : 0.f;
  }
}

__global__ __launch_bounds__(256) void chunk_count_pairs_kernel(ChunkArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= a.rows * a.K) return;
  const int32_t c = a.idx[t];
  if (c >= 0 && (int64_t)c < a.Nc) atomicAdd(&a.counts[bin_of(t / a.K, c, a)], 1u);
}

__global__ __launch_bounds__(256) void chunk_scatter_pairs_kernel(ChunkArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= a.rows * a.K) return;
  const int32_t c = a.idx[t];
  if (c >= 0 && (int64_t)c < a.Nc) a.pairs[atomicAdd(&a.cursor[bin_of(t / a.K, c, a)], 1u)] = (uint32_t)t;
}

// --- bucketing through a workgroup histogram in LDS --------------------------
// A workgroup takes bucket_rows query rows of one (batch, kv head), counts its
// pairs per chunk in LDS and adds each nonzero count to the global bin once, so
// global atomics drop from one per pair to one per (workgroup, chunk).  Used
// when the chunks of one (batch, kv head) fit the LDS histogram.  bucket_rows
// is kBucketRows, halved (down to kBucketRowsMin) while the grid would have
// fewer than kBucketGrid workgroups: each workgroup's passes are a chain of
// dependent loads, so a small grid leaves the chip idle.
constexpr int kBucketRows = 1024;
constexpr int kBucketRowsMin = 64;
constexpr int kBucketGrid = 512;
constexpr int kBandRows = 16384;         // forward bins; a multiple of kBucketRows
constexpr int kHistMax = 16384;
constexpr int kBucketBatch = 4;          // row passes whose loads are issued together

struct BucketRange {
  int64_t bg, r0, r1;                    // (batch, kv head) and query rows [r0, r1)
  int b, g;
};
__device__ __forceinline__ BucketRange bucket_range(const ChunkArgs& a) {
  BucketRange br;
  const int64_t rbk = (a.Lq + a.bucket_rows - 1) / a.bucket_rows;
  br.bg = (int64_t)blockIdx.x / rbk;
  br.r0 = ((int64_t)blockIdx.x % rbk) * a.bucket_rows;
  br.r1 = min(br.r0 + a.bucket_rows, a.Lq);
  br.b = (int)(br.bg / a.Hkv);
  br.g = (int)(br.bg % a.Hkv);
  return br;
}

// Calls fn(row, slot, chunk, valid) for every slot of the range's rows; rows
// sit on segments of S lanes, kBucketBatch passes per load batch.  Every lane
// takes part in every call (the count uses segment shuffles).
template <class F>
__device__ __forceinline__ void for_range_slots(const ChunkArgs& a, const BucketRange& br, F&& fn) {
  const int K = a.K, S = seg_lanes(K), per = 256 / S;
  const int k = threadIdx.x & (S - 1);
  for (int64_t base = br.r0; base < br.r1; base += (int64_t)per * kBucketBatch) {
    int32_t c[kBucketBatch];
    int64_t row[kBucketBatch];
    bool act[kBucketBatch];
#pragma unroll
    for (int u = 0; u < kBucketBatch; ++u) {
      const int64_t r = base + (int64_t)u * per + threadIdx.x / S;
      act[u] = r < br.r1 && k < K;
      row[u] = ((int64_t)br.b * a.Lq + (act[u] ? r : br.r0)) * a.Hkv + br.g;
      c[u] = act[u] ? a.idx[row[u] * K + k] : -1;
    }
#pragma unroll
    for (int u = 0; u < kBucketBatch; ++u)
      fn(row[u], k, c[u], act[u], act[u] && c[u] >= 0 && (int64_t)c[u] < a.Nc);
  }
}

__global__ __launch_bounds__(256) void chunk_count_lds_kernel(ChunkArgs a) {
  extern __shared__ uint32_t hist[];
  const BucketRange br = bucket_range(a);
  for (int64_t i = threadIdx.x; i < a.Nc; i += 256) hist[i] = 0u;
  __syncthreads();
  const int S = seg_lanes(a.K);
  for_range_slots(a, br, [&](int64_t row, int k, int32_t c, bool active, bool valid) {
    const float s = active ? a.score[row * a.K + k] : 0.f;
    float mx = valid ? s : -INFINITY;
    for (int o = 1; o < S; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
    const float ex = valid ? expf(s - mx) : 0.f;
    float den = ex;
    for (int o = 1; o < S; o <<= 1) den += __shfl_xor(den, o, kWave);
    if (active) a.wts[row * a.K + k] = valid ? ex / den : 0.f;
    if (valid) atomicAdd(&hist[c], 1u);
  });
  __syncthreads();
  uint32_t* cnt = a.counts + (br.bg * a.n_bands + br.r0 / a.band_rows) * a.Nc;
  for (int64_t i = threadIdx.x; i < a.Nc; i += 256)
    if (hist[i] != 0u) atomicAdd(&cnt[i], hist[i]);
}

__global__ __launch_bounds__(256) void chunk_scatter_lds_kernel(ChunkArgs a) {
  extern __shared__ uint32_t hist[];
  const BucketRange br = bucket_range(a);
  for (int64_t i = threadIdx.x; i < a.Nc; i += 256) hist[i] = 0u;
  __syncthreads();
  for_range_slots(a, br, [&](int64_t, int, int32_t c, bool, bool valid) {
    if (valid) atomicAdd(&hist[c], 1u);
  });
  __syncthreads();
  // reserve this workgroup's run in every bin it touches
  uint32_t* cur = a.cursor + (br.bg * a.n_bands + br.r0 / a.band_rows) * a.Nc;
  for (int64_t i = threadIdx.x; i < a.Nc; i += 256)
    if (hist[i] != 0u) hist[i] = atomicAdd(&cur[i], hist[i]);
  __syncthreads();
  for_range_slots(a, br, [&](int64_t row, int k, int32_t c, bool, bool valid) {
    if (valid) a.pairs[atomicAdd(&hist[c], 1u)] = (uint32_t)(row * a.K + k);
  });
}

// --- scan: bin offsets, scatter cursors, work items ------------------------
// An exclusive scan of (pairs, items) over all bins in two kernels over tiles
// of kScanTile bins (kScanPer consecutive bins per thread): the first records
// each tile's totals; the second adds the totals of all earlier tiles, scans
// its tile, writes the bin offsets, the scatter cursors and the work items,
// and clears the counts for the next call.
constexpr int kScanThreads = 1024;
constexpr int kScanPer = 2;
constexpr int64_t kScanTile = (int64_t)kScanThreads * kScanPer;

__device__ __forceinline__ void block_exclusive_scan2(uint32_t& a, uint32_t& b, uint32_t* sa, uint32_t* sb,
                                                      uint32_t& tot_a, uint32_t& tot_b) {
  const int t = threadIdx.x;
  sa[t] = a;
  sb[t] = b;
  __syncthreads();
  for (int o = 1; o < kScanThreads; o <<= 1) {   // inclusive Hillis-Steele scan
    const uint32_t va = t >= o ? sa[t - o] : 0u, vb = t >= o ? sb[t - o] : 0u;
    __syncthreads();
    sa[t] += va;
    sb[t] += vb;
    __syncthreads();
  }
  tot_a = sa[kScanThreads - 1];
  tot_b = sb[kScanThreads - 1];
  a = sa[t] - a;
  b = sb[t] - b;
  __syncthreads();
}

__device__ __forceinline__ uint32_t items_of(uint32_t pairs, uint32_t ppi) { return (pairs + ppi - 1) / ppi; }

__global__ __launch_bounds__(kScanThreads) void chunk_tile_sum_kernel(ChunkArgs a) {
  const uint32_t ppi = (uint32_t)a.pairs_per_item;
  __shared__ uint32_t sp[kScanThreads / kWave], si[kScanThreads / kWave];
  const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
  const int64_t i0 = (int64_t)blockIdx.x * kScanTile + (int64_t)t * kScanPer;
  uint32_t tp = 0, ti = 0;
#pragma unroll
  for (int u = 0; u < kScanPer; ++u) {
    const uint32_t c = i0 + u < a.n_bins ? a.counts[i0 + u] : 0u;
    tp += c;
    ti += items_of(c, ppi);
  }
  for (int o = 32; o >= 1; o >>= 1) {
    tp += __shfl_xor(tp, o, kWave);
    ti += __shfl_xor(ti, o, kWave);
  }
  if (lane == 0) {
    sp[w] = tp;
    si[w] = ti;
  }
  __syncthreads();
  if (t == 0) {
    uint32_t p = 0, it = 0;
    for (int x = 0; x < kScanThreads / kWave; ++x) {
      p += sp[x];
      it += si[x];
    }
    a.seg_tot[2 * blockIdx.x] = p;
    a.seg_tot[2 * blockIdx.x + 1] = it;
  }
}

__global__ __launch_bounds__(kScanThreads) void chunk_tile_fix_kernel(ChunkArgs a) {
  const uint32_t ppi = (uint32_t)a.pairs_per_item;
  __shared__ uint32_t sp[kScanThreads], si[kScanThreads];
  const int t = threadIdx.x;
  const int64_t tile = blockIdx.x;
  uint32_t pb = 0, ib = 0;                       // totals of the earlier tiles
  for (int64_t x = t; x < tile; x += kScanThreads) {
    pb += a.seg_tot[2 * x];
    ib += a.seg_tot[2 * x + 1];
  }
  uint32_t tot_p, tot_i;
  block_exclusive_scan2(pb, ib, sp, si, tot_p, tot_i);
  const uint32_t base_p = tot_p, base_i = tot_i;
  // this thread's bins, then the tile's exclusive scan over threads
  const int64_t i0 = tile * kScanTile + (int64_t)t * kScanPer;
  uint32_t c[kScanPer];
  uint32_t lp = 0, li = 0;
#pragma unroll
  for (int u = 0; u < kScanPer; ++u) {
    c[u] = i0 + u < a.n_bins ? a.counts[i0 + u] : 0u;
    lp += c[u];
    li += items_of(c[u], ppi);
  }
  uint32_t tile_p, tile_i;
  block_exclusive_scan2(lp, li, sp, si, tile_p, tile_i);
  uint32_t op = base_p + lp, oi = base_i + li;
#pragma unroll
  for (int u = 0; u < kScanPer; ++u) {
    const int64_t i = i0 + u;
    if (i < a.n_bins) {
      a.offsets[i] = op;
      a.cursor[i] = op;
      a.counts[i] = 0u;                          // ready for the next call
      if (a.item_start != nullptr) a.item_start[i] = oi;
      const uint32_t ni = items_of(c[u], ppi);
      for (uint32_t jb = 0; jb < ni; ++jb) a.items[oi + jb] = (uint64_t)i | ((uint64_t)jb << 32);
      op += c[u];
      oi += ni;
    }
  }
  if (tile == (int64_t)gridDim.x - 1 && t == 0) {
    a.offsets[a.n_bins] = base_p + tile_p;
    *a.n_items = base_i + tile_i;
  }
}

// --- scatter: pair ids into bins (one lane per slot) -----------------------
__global__ __launch_bounds__(256) void chunk_scatter_kernel(ChunkArgs a) {
  const int K = a.K, S = seg_lanes(K);
  const int64_t row = (int64_t)blockIdx.x * (256 / S) + threadIdx.x / S;
  const int k = threadIdx.x & (S - 1);
  if (row >= a.rows || k >= K) return;
  const int32_t c = a.idx[row * K + k];
  if (c >= 0 && (int64_t)c < a.Nc) {
    const uint32_t pos = a.cursor[bin_of(row, c, a)] + reinterpret_cast<const uint32_t*>(a.partials)[row * K + k];
    a.pairs[pos] = (uint32_t)(row * K + k);
  }
}

// --- attend: one work item (a block of pairs of one chunk) per workgroup ----
// Loads the A operand (attention queries of one 16-row tile) of a wave.
template <int D, int G>
__device__ __forceinline__ void load_q_tile(const ChunkArgs& a, const int64_t* qoff_s, int n_pairs,
                                            int tile, int ma, int jg, bf16x8 (&qa)[D / 32]) {
  constexpr int PT = 16 / G;
  const int pa = tile * PT + ma / G, ha = ma % G;
  const bool va = pa < n_pairs;
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q_attn) + (va ? qoff_s[pa] : 0) + ha * D + 8 * jg;
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {      // unconditional load (element 0 when !va), then zero
    uint4 x = *reinterpret_cast<const uint4*>(qp + 32 * t);
    if (!va) x = make_uint4(0, 0, 0, 0);
    qa[t] = __builtin_bit_cast(bf16x8, x);
  }
}

// Sum of squares of 8 bf16 values (two-term bf16 dot products, fp32 accumulate).
__device__ __forceinline__ float sumsq8(uint4 x, float acc) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bf16x2 v = __builtin_bit_cast(bf16x2, w[q]);
    acc = __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
  }
  return acc;
}

template <int D, int G>
__global__ __launch_bounds__(256, 4) void chunk_attend_kernel(ChunkArgs a) {
  constexpr int KROW = D + 16;         // bf16 elements per K row in LDS (32-byte pad: no bank conflicts)
  constexpr int VROW = D + 16;         // bf16 elements per V row in LDS (read back transposed)
  constexpr int PT = 16 / G;           // pairs per MFMA tile (16 head-rows)
  constexpr int KSTEP = D / 32;        // MFMA K-steps over the head dimension
  constexpr int NT = D / 16;           // output dimension tiles
  __shared__ __align__(16) uint16_t ks[kChunk * KROW];
  __shared__ __align__(16) uint16_t vs[kChunk * VROW];
  __shared__ float rk[kChunk];
  __shared__ uint32_t pid_s[kMaxPairs];
  __shared__ float w_s[kMaxPairs];
  __shared__ int64_t qoff_s[kMaxPairs];   // element offset of the pair's G attention queries

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const uint32_t item_i = blockIdx.x;
  if (item_i >= *a.n_items) return;
  const uint64_t item = a.items[item_i];
  const int64_t bin = (int64_t)(item & 0xFFFFFFFFull);
  const uint32_t blk = (uint32_t)(item >> 32);
  const uint32_t p_begin = a.offsets[bin] + blk * (uint32_t)a.pairs_per_item;
  const uint32_t p_end = min(p_begin + (uint32_t)a.pairs_per_item, a.offsets[bin + 1]);
  const int n_pairs = (int)(p_end - p_begin);
  const int64_t bgb = bin / a.Nc;                // (batch, kv head) * n_bands + band
  const int64_t c = bin - bgb * a.Nc;
  const int64_t bg = bgb / a.n_bands;
  const int g = (int)(bg % a.Hkv);

  // pair ids and blend weights of the item; K and V (row-major) in LDS.  The
  // P.V operand is read from V with LDS transpose loads in the key order of
  // the S^T accumulators, so P^T feeds P.V from registers.
  if (tid < n_pairs) {
    const uint32_t pid = a.pairs[p_begin + tid];
    pid_s[tid] = pid;
    w_s[tid] = a.wts[pid];
    const int64_t qrow = (int64_t)(pid / (uint32_t)a.K) / a.Hkv;     // b * Lq + r
    qoff_s[tid] = (qrow * a.Hq + (int64_t)g * G) * D;
  }
  {
    const int64_t base = (bg * a.Lkv + c * kChunk) * D;
    const uint4* kp = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.k) + base);
    const uint16_t* vp = reinterpret_cast<const uint16_t*>(a.v) + base;
    constexpr int NK = kChunk * D / 8 / 256;          // 16-byte K pieces per thread
    const uint4* vp4 = reinterpret_cast<const uint4*>(vp);
    uint4 kx[NK], vx[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      kx[i] = kp[tid + 256 * i];
      vx[i] = vp4[tid + 256 * i];
    }
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int e = (tid + 256 * i) * 8;
      *reinterpret_cast<uint4*>(&ks[(e / D) * KROW + e % D]) = kx[i];
      *reinterpret_cast<uint4*>(&vs[(e / D) * VROW + e % D]) = vx[i];
    }
  }
  __syncthreads();
  const int n_tiles = (n_pairs + PT - 1) / PT;
  const int ma = lane & 15, jg = lane >> 4;        // head-row of the tile, lane group
  // this wave's first two tiles of queries in flight during the key norms
  bf16x8 qa[KSTEP], qn[KSTEP], qn2[KSTEP];
  if (w < n_tiles) load_q_tile<D, G>(a, qoff_s, n_pairs, w, ma, jg, qa);
  if (w + 4 < n_tiles) load_q_tile<D, G>(a, qoff_s, n_pairs, w + 4, ma, jg, qn);
  {  // key inverse norms: 4 threads per key
    const int key = tid >> 2, qd = tid & 3;
    float ss = 0.f;
#pragma unroll
    for (int x = 0; x < D / 4; x += 8)
      ss = sumsq8(*reinterpret_cast<const uint4*>(&ks[key * KROW + qd * (D / 4) + x]), ss);
    ss += __shfl_xor(ss, 1, kWave);
    ss += __shfl_xor(ss, 2, kWave);
    // logits are formed in base 2: log2(e) is folded into the key factor
    if (qd == 0) rk[key] = (a.qk_norm ? 1.0f / fmaxf(sqrtf(ss), 1e-6f) : 1.0f) * a.attn_scale * kLog2e;
  }
  __syncthreads();

  // S^T accumulators: lane holds keys 16*nt + 4*jg + i of head-row ma
  float rkl[4][4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) rkl[nt][i] = rk[16 * nt + 4 * jg + i];

  for (int tile = w; tile < n_tiles; tile += 4) {
    // queries two tiles ahead in flight while this one computes
    if (tile + 8 < n_tiles) load_q_tile<D, G>(a, qoff_s, n_pairs, tile + 8, ma, jg, qn2);
    float qss = 0.f;
#pragma unroll
    for (int t = 0; t < KSTEP; ++t) qss = sumsq8(__builtin_bit_cast(uint4, qa[t]), qss);
    qss = xrow_sum(qss);
    const float rq = a.qk_norm ? 1.0f / fmaxf(sqrtf(qss), 1e-6f) : 1.0f;
    // S^T = K Q^T on MFMA: A = keys from LDS, B = the tile's queries
    floatx4 s[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      s[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < KSTEP; ++t) {
        const uint4 kb = *reinterpret_cast<const uint4*>(&ks[(16 * nt + ma) * KROW + 32 * t + 8 * jg]);
        s[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb), qa[t], s[nt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // keep the P.V operand reads below the softmax
    // softmax over the 64 keys of head-row ma: 16 in this lane, the rest in
    // lanes ma + 16, ma + 32, ma + 48
    float mx = -INFINITY;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[nt][i] = s[nt][i] * rq * rkl[nt][i];
        mx = fmaxf(mx, s[nt][i]);
      }
    mx = xrow_max(mx);
    float sum = 0.f;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[nt][i] = __builtin_amdgcn_exp2f(s[nt][i] - mx);   // logits are in base 2
        sum += s[nt][i];
      }
    sum = xrow_sum(sum);
    const int pm = tile * PT + ma / G;
    const float scale = (pm < n_pairs ? w_s[pm] : 0.f) * __builtin_amdgcn_rcpf(sum);
    // P^T as the B operand of O^T = V^T P^T: step st takes keys of nt = 2st, 2st + 1
    bf16x8 pb[2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[st][e] = (__bf16)(s[2 * st + (e >> 2)][e & 3] * scale);
    // O^T: lane holds dims 16*nt + 4*jg + i of head-row ma; bf16 partial, 8-byte
    // stores.  bf16 keeps fp32's exponent range, so every finite partial
    // (|w O| <= max |V| of the chunk) stays finite and normal.
    const bool live = pm < n_pairs;
    uint16_t* dst = a.partials + (live ? ((int64_t)pid_s[pm] * G + (ma % G)) * D : 0) + 4 * jg;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      floatx4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        // A = V^T: dims 16nt.., keys 32st + 4jg + 0..3 and 32st + 16 + 4jg + 0..3
        const bf16x8 va = lds_operand_tr2(vs, VROW, 32 * st + 4 * jg, 32 * st + 16 + 4 * jg, 16 * nt, ma);
        o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[st], o, 0, 0, 0);
      }
      if (live) {
        const bf16x2 h01 = {(__bf16)o[0], (__bf16)o[1]}, h23 = {(__bf16)o[2], (__bf16)o[3]};
        *reinterpret_cast<uint2*>(dst + 16 * nt) =
            make_uint2(__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23));
      }
      if (nt % 2 == 1) __builtin_amdgcn_sched_barrier(0);   // two output tiles in flight
    }
#pragma unroll
    for (int t = 0; t < KSTEP; ++t) {
      qa[t] = qn[t];
      qn[t] = qn2[t];
    }
  }
}

template <int D, int G>
__global__ __launch_bounds__(256) void chunk_combine_kernel(ChunkArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  constexpr int J = D / 8;
  const int64_t total = a.rows * G * J;
  if (t >= total) return;
  const int64_t row = t / (G * J);
  const int h = (int)((t / J) % G), j = (int)(t % J);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int K = a.K;
  // slots in batches of 8 with every load in flight (indices clamped, unused
  // slots skipped when adding), added in slot order
  for (int k0 = 0; k0 < K; k0 += 8) {
    uint4 u[8];
    bool ok[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = k0 + e < K ? k0 + e : K - 1;
      const int32_t c = a.idx[row * K + k];
      ok[e] = k0 + e < K && c >= 0 && (int64_t)c < a.Nc;
      u[e] = load_stream(reinterpret_cast<const uint4*>(&a.partials[((row * K + k) * G + h) * D + 8 * j]));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (!ok[e]) continue;
      const uint32_t wd[4] = {u[e].x, u[e].y, u[e].z, u[e].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += __uint_as_float(wd[q] << 16);
        acc[2 * q + 1] += __uint_as_float(wd[q] & 0xFFFF0000u);
      }
    }
  }
  uint4 o;
  o.x = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
  o.y = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
  o.z = (uint32_t)f32_to_bf16(acc[4]) | ((uint32_t)f32_to_bf16(acc[5]) << 16);
  o.w = (uint32_t)f32_to_bf16(acc[6]) | ((uint32_t)f32_to_bf16(acc[7]) << 16);
  const int g = (int)(row % a.Hkv);
  *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.out) +
                            ((row / a.Hkv) * a.Hq + (int64_t)g * G + h) * D + 8 * j) = o;
}

template <int D, int G>
hipError_t launch_dg(const ChunkArgs& a, hipStream_t st, const Marks& mk) {
  hipError_t e;
  if ((e = mk.rec(kStageAttend, 0, st)) != hipSuccess) return e;
  hipLaunchKernelGGL((chunk_attend_kernel<D, G>), dim3((unsigned)a.max_items), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = mk.rec(kStageAttend, 1, st)) != hipSuccess) return e;
  if ((e = mk.rec(kStageCombine, 0, st)) != hipSuccess) return e;
  const int64_t total = a.rows * G * (D / 8);
  hipLaunchKernelGGL((chunk_combine_kernel<D, G>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return mk.rec(kStageCombine, 1, st);
}

}  // namespace

int64_t chunk_pairs_per_item() { return kFwdPairs; }
int64_t chunk_band_rows() { return kBandRows; }

int64_t chunk_scan_tiles(int64_t n_bins) { return (n_bins + kScanTile - 1) / kScanTile; }

hipError_t launch_bucket(const ChunkArgs& args, hipStream_t st) {
  hipError_t e;
  ChunkArgs a = args;
  const int64_t ranges = a.Lq > 0 ? a.rows / a.Lq : 0;   // (batch, kv head) pairs
  a.bucket_rows = kBucketRows;
  while (a.bucket_rows > kBucketRowsMin && (a.Lq + a.bucket_rows - 1) / a.bucket_rows * ranges < kBucketGrid)
    a.bucket_rows /= 2;
  if (a.band_rows % a.bucket_rows != 0) return hipErrorInvalidValue;   // a range lies in one band
  if ((e = launch_fill_u32(a.counts, a.n_bins, 0u, st)) != hipSuccess) return e;
  const bool wide = a.K > kWave;                 // more slots than lanes in a wave
  const bool lds = !wide && a.Nc <= kHistMax;
  // the global-histogram count keeps each pair's rank in its bin in the
  // partial-output region (4 bytes per pair) until the scatter reads it
  if (!wide && !lds && a.partials == nullptr) return hipErrorInvalidValue;
  const unsigned pair_blocks = (unsigned)((a.rows * a.K + 255) / 256);
  if (wide) {
    hipLaunchKernelGGL(chunk_wts_wide_kernel, dim3((unsigned)((a.rows + 3) / 4)), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // rows per 256-thread block of the one-lane-per-slot kernels (K <= 64 there)
  const int64_t seg = wide ? 64 : (a.K <= 1 ? 1 : (int64_t)1 << (32 - __builtin_clz((unsigned)a.K - 1)));
  const unsigned row_blocks = (unsigned)((a.rows + 256 / seg - 1) / (256 / seg));
  const unsigned range_blocks = (unsigned)((a.Lq + a.bucket_rows - 1) / a.bucket_rows * ranges);
  const size_t hist_bytes = (size_t)a.Nc * 4;
  if (wide) hipLaunchKernelGGL(chunk_count_pairs_kernel, dim3(pair_blocks), dim3(256), 0, st, a);
  else if (lds) hipLaunchKernelGGL(chunk_count_lds_kernel, dim3(range_blocks), dim3(256), hist_bytes, st, a);
  else hipLaunchKernelGGL(chunk_count_kernel, dim3(row_blocks), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t n_tiles = chunk_scan_tiles(a.n_bins);
  if (n_tiles > INT32_MAX) return hipErrorInvalidValue;
  if (n_tiles > 0) {
    if (n_tiles > 1) {   // one tile has no earlier tiles whose totals it needs
      hipLaunchKernelGGL(chunk_tile_sum_kernel, dim3((unsigned)n_tiles), dim3(kScanThreads), 0, st, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(chunk_tile_fix_kernel, dim3((unsigned)n_tiles), dim3(kScanThreads), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else if ((e = launch_fill_u32(a.n_items, 1, 0u, st)) != hipSuccess) {   // no bins: no work items
    return e;
  }
  if (wide) hipLaunchKernelGGL(chunk_scatter_pairs_kernel, dim3(pair_blocks), dim3(256), 0, st, a);
  else if (lds) hipLaunchKernelGGL(chunk_scatter_lds_kernel, dim3(range_blocks), dim3(256), hist_bytes, st, a);
  else hipLaunchKernelGGL(chunk_scatter_kernel, dim3(row_blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attend_chunk(const ChunkArgs& a, int D, int G, hipStream_t st, const Marks& mk) {
  hipError_t e;
  if ((e = mk.rec(kStageBucket, 0, st)) != hipSuccess) return e;
  if ((e = launch_bucket(a, st)) != hipSuccess) return e;
  if ((e = mk.rec(kStageBucket, 1, st)) != hipSuccess) return e;
#define HSA_CHUNK_CASE(DD, GG) \
  if (D == DD && G == GG) return launch_dg<DD, GG>(a, st, mk);
  HSA_CHUNK_CASE(128, 1) HSA_CHUNK_CASE(128, 2) HSA_CHUNK_CASE(128, 4) HSA_CHUNK_CASE(128, 8)
  HSA_CHUNK_CASE(128, 16) HSA_CHUNK_CASE(64, 1) HSA_CHUNK_CASE(64, 2) HSA_CHUNK_CASE(64, 4)
  HSA_CHUNK_CASE(64, 8) HSA_CHUNK_CASE(64, 16)
#undef HSA_CHUNK_CASE
  return hipErrorInvalidValue;
}

}  // namespace hsa
