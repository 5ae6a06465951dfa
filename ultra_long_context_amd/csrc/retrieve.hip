// retrieve.hip -- landmark scoring and causal top-K (Steps 1-2 of the HSA step in
// "Every Token Counts", agent-atlas explainer, "How It Works (Technically)").
//
// One wave scores 16 query rows of one (batch, kv head) against one range of
// chunks (a "split").  Scores come from MFMA tiles: the 16 landmarks of a tile
// are the A operand (M = chunks), the 16 retrieval queries the B operand
// (N = rows), so lane l holds row (l & 15) and chunks 4*(l >> 4) + i.  Each of
// the 4 lanes of a row therefore sees its own quarter of the row's chunks.
//
// Selection never materialises the score matrix:
//   pass 1  scores every tile and keeps, per lane, the running maximum of 16
//           disjoint chunk groups (64 groups per row).  The K-th largest group
//           maximum is a lower bound of the row's K-th largest score, because
//           K distinct chunks reach it.
//   pass 2  recomputes the tiles and appends every chunk at or above that bound
//           to a per-row LDS buffer.  If a buffer fills, it is cut back to its
//           exact top K and the bound is raised to the K-th key (exact, as keys
//           are unique), so the pass is correct for any input, ties included.
//   final   exact top K of the buffer by binary search on the packed 64-bit
//           key, then rank sort.
// With more than one split per row, each split writes its sorted list and a
// merge kernel combines them the same way.
#include "hsa_device.h"
#include "hsa_internal.h"

namespace hsa {
namespace {

constexpr int kRows = 16;              // query rows per wave (MFMA N)
constexpr int kCap = 96;               // candidate buffer entries per row
constexpr int kMaxSplits = 1024;

template <bool BF16, int D> struct QOperand;

// bf16: 16x16x32 MFMA; K-group j of step t covers dims 32t + 8j .. 32t + 8j + 7.
template <int D> struct QOperand<true, D> {
  bf16x8 v[D / 32];
  __device__ __forceinline__ void load(const uint16_t* row, bool ok, int j) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (ok) x = *reinterpret_cast<const uint4*>(row + 32 * t + 8 * j);
      v[t] = __builtin_bit_cast(bf16x8, x);
    }
  }
};

// fp32: 16x16x4 MFMA; step (u, e) with K-group j covers dim 16u + 4j + e.
template <int D> struct QOperand<false, D> {
  float4 v[D / 16];
  __device__ __forceinline__ void load(const float* row, bool ok, int j) {
#pragma unroll
    for (int u = 0; u < D / 16; ++u) {
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (ok) x = *reinterpret_cast<const float4*>(row + 16 * u + 4 * j);
      v[u] = x;
    }
  }
};

// Raw scores of chunks [cs, cs + 16) for the wave's 16 rows; chunks at or past
// c_stop contribute zeros (the caller masks them).
template <int D>
__device__ __forceinline__ floatx4 score_tile(const uint16_t* lm, int cs, int c_stop,
                                             const QOperand<true, D>& q, int lane) {
  const int cc = cs + (lane & 15);
  const bool ok = cc < c_stop;
  const uint16_t* p = lm + (int64_t)cc * D + 8 * (lane >> 4);
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    uint4 x = make_uint4(0, 0, 0, 0);
    if (ok) x = *reinterpret_cast<const uint4*>(p + 32 * t);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x), q.v[t], acc, 0, 0, 0);
  }
  return acc;
}

template <int D>
__device__ __forceinline__ floatx4 score_tile(const float* lm, int cs, int c_stop,
                                             const QOperand<false, D>& q, int lane) {
  const int cc = cs + (lane & 15);
  const bool ok = cc < c_stop;
  const float* p = lm + (int64_t)cc * D + 4 * (lane >> 4);
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < D / 16; ++u) {
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (ok) x = *reinterpret_cast<const float4*>(p + 16 * u);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.x, q.v[u].x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.y, q.v[u].y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.z, q.v[u].z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.w, q.v[u].w, acc, 0, 0, 0);
  }
  return acc;
}

__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
  return v;
}

// Sum over the 4 lanes (j = 0..3) that share a row.
__device__ __forceinline__ int row_sum(int v) {
  v += __shfl_xor(v, 16, kWave);
  v += __shfl_xor(v, 32, kWave);
  return v;
}

// Exact K-th largest packed candidate of each row's buffer (0 when the row has
// at most K entries).  All 64 lanes must call it; lane (row, j) visits buffer
// positions j, j + 4, ...
__device__ uint64_t row_kth(const uint64_t* rowbuf, int n, int K, int j) {
  const bool big = n > K;
  if (!__any(big)) return 0;
  uint32_t t32 = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = t32 | (1u << bit);
    int c = 0;
    for (int p = j; p < n; p += 4) c += cand_key(rowbuf[p]) >= cand;
    c = row_sum(c);
    if (c >= K) t32 = cand;
  }
  int above = 0, at = 0;
  for (int p = j; p < n; p += 4) {
    const uint32_t k = cand_key(rowbuf[p]);
    above += k > t32;
    at += k == t32;
  }
  above = row_sum(above);
  at = row_sum(at);
  const int need = K - above;
  uint32_t tl = 0;
  if (__any(big && at > need)) {          // a tie straddles the K-th place
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = tl | (1u << bit);
      int c = 0;
      for (int p = j; p < n; p += 4) {
        const uint64_t e = rowbuf[p];
        c += (cand_key(e) == t32) && ((uint32_t)e >= cand);
      }
      c = row_sum(c);
      if (c >= need) tl = cand;
    }
  }
  if (!big || at <= need) tl = 0;
  return big ? (((uint64_t)t32 << 32) | tl) : 0;
}

// Keep the exact top K of every row's buffer (unordered).  Returns the new
// count of the caller's row; `lo` becomes the bound for later appends.
__device__ int row_compact(uint64_t (*buf)[kCap], uint64_t (*stg)[kMaxTopK], int* cnt,
                           uint64_t& lo, int K, int qrow, int j) {
  __syncthreads();
  const int n = cnt[qrow];
  const uint64_t t = row_kth(buf[qrow], n, K, j);
  int kept = 0;
  for (int p = j; p < n; p += 4) kept += buf[qrow][p] >= t;
  int ex = 0;
#pragma unroll
  for (int jj = 0; jj < 3; ++jj) {
    const int o = __shfl(kept, qrow + 16 * jj, kWave);
    if (jj < j) ex += o;
  }
  for (int p = j; p < n; p += 4) {
    const uint64_t e = buf[qrow][p];
    if (e >= t) stg[qrow][ex++] = e;
  }
  __syncthreads();
  const int m = n > K ? K : n;
  for (int p = j; p < m; p += 4) buf[qrow][p] = stg[qrow][p];
  if (j == 0) cnt[qrow] = m;
  if (n > K) lo = t + 1;
  __syncthreads();
  return m;
}

template <bool BF16, int D>
__global__ __launch_bounds__(64) void scan_topk_kernel(ScanArgs a) {
  using T = typename Elem<BF16>::T;
  __shared__ uint64_t buf[kRows][kCap];
  __shared__ uint64_t stg[kRows][kMaxTopK];
  __shared__ int cnt[kRows];

  const int lane = threadIdx.x, qrow = lane & 15, j = lane >> 4;
  const int s = blockIdx.y;
  const int64_t rbk = (a.Lq + kRows - 1) / kRows;
  const int64_t rb = (int64_t)blockIdx.x % rbk;
  const int bg = (int)((int64_t)blockIdx.x / rbk);
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int64_t r = rb * kRows + qrow;
  const bool row_ok = r < a.Lq;
  int n_row = 0;
  if (row_ok) {
    const int64_t n = (a.q_pos0 + r) / kChunk;
    n_row = (int)(n < a.Nc ? n : a.Nc);
  }
  const int c_begin = s * a.split_len;
  const int c_end = min(c_begin + a.split_len, a.n_max);
  const int lim = min(n_row, c_end);                 // this row scores chunks [c_begin, lim)
  const int c_stop = wave_max_i(lim);

  const T* lm = reinterpret_cast<const T*>(a.landmarks) + (int64_t)bg * a.Nc * D;
  QOperand<BF16, D> q;
  q.load(reinterpret_cast<const T*>(a.q_ret) + ((b * a.Lq + (row_ok ? r : 0)) * a.Hkv + g) * D,
         row_ok, j);

  // pass 1: group maxima -> lower bound of the K-th score
  uint32_t gk[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) gk[i] = 0;
  for (int c0 = c_begin; c0 < c_stop; c0 += 64) {
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const int cs = c0 + sub * 16;
      if (cs < c_stop) {
        const floatx4 acc = score_tile<D>(lm, cs, c_stop, q, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = cs + 4 * j + i;
          if (c < lim) gk[sub * 4 + i] = max(gk[sub * 4 + i], score_key(acc[i]));
        }
      }
    }
  }
  uint32_t tau = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = tau | (1u << bit);
    int c = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) c += gk[i] >= cand;
    if (row_sum(c) >= a.K) tau = cand;
  }
  uint64_t lo = (uint64_t)tau << 32;

  // pass 2: collect candidates at or above the bound
  if (lane < kRows) cnt[lane] = 0;
  __syncthreads();
  for (int c0 = c_begin; c0 < c_stop; c0 += 64) {
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const int cs = c0 + sub * 16;
      if (cs < c_stop) {
        const floatx4 acc = score_tile<D>(lm, cs, c_stop, q, lane);
        if (__any(cnt[qrow] > kCap - 16)) row_compact(buf, stg, cnt, lo, a.K, qrow, j);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = cs + 4 * j + i;
          if (c < lim) {
            const uint64_t pk = pack_cand(score_key(acc[i]), (uint32_t)c);
            if (pk >= lo) {
              const int pos = atomicAdd(&cnt[qrow], 1);
              buf[qrow][pos] = pk;
            }
          }
        }
      }
    }
  }

  // final: exact top K of the buffer, rank-sorted
  const int m = row_compact(buf, stg, cnt, lo, a.K, qrow, j);
  if (!row_ok) return;
  const int64_t row_flat = (b * a.Lq + r) * a.Hkv + g;
  for (int p = j; p < m; p += 4) {
    const uint64_t e = buf[qrow][p];
    int rank = 0;
    for (int o = 0; o < m; ++o) rank += buf[qrow][o] > e;
    if (a.n_splits == 1) {
      a.out_idx[row_flat * a.K + rank] = (int32_t)cand_chunk(e);
      a.out_score[row_flat * a.K + rank] = key_score(cand_key(e)) * a.ret_scale;
    } else {
      a.lists[(row_flat * a.n_splits + s) * a.K + rank] = e;
    }
  }
  for (int k = m + ((j - m) & 3); k < a.K; k += 4) {
    if (a.n_splits == 1) {
      a.out_idx[row_flat * a.K + k] = -1;
      a.out_score[row_flat * a.K + k] = -INFINITY;
    } else {
      a.lists[(row_flat * a.n_splits + s) * a.K + k] = 0;
    }
  }
}

// K-th largest of arr[0..n) (unique packed keys) with the whole wave; 0 if n <= K.
__device__ uint64_t wave_kth(const uint64_t* arr, int n, int K, int lane) {
  if (n <= K) return 0;
  uint32_t t32 = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = t32 | (1u << bit);
    int c = 0;
    for (int p = lane; p < n; p += kWave) c += cand_key(arr[p]) >= cand;
    if (wave_sum_i(c) >= K) t32 = cand;
  }
  int above = 0, at = 0;
  for (int p = lane; p < n; p += kWave) {
    const uint32_t k = cand_key(arr[p]);
    above += k > t32;
    at += k == t32;
  }
  above = wave_sum_i(above);
  at = wave_sum_i(at);
  const int need = K - above;
  uint32_t tl = 0;
  if (at > need) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = tl | (1u << bit);
      int c = 0;
      for (int p = lane; p < n; p += kWave) {
        const uint64_t e = arr[p];
        c += (cand_key(e) == t32) && ((uint32_t)e >= cand);
      }
      if (wave_sum_i(c) >= need) tl = cand;
    }
  }
  return ((uint64_t)t32 << 32) | tl;
}

__global__ __launch_bounds__(64) void merge_topk_kernel(MergeArgs a) {
  __shared__ uint64_t heads[kMaxSplits];
  __shared__ uint64_t pool[kMaxTopK * kMaxTopK];
  __shared__ uint64_t top[kMaxTopK];
  __shared__ int n_pool;

  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int S = a.n_splits, K = a.K;
  const uint64_t* L = a.lists + row * S * K;

  for (int s = lane; s < S; s += kWave) heads[s] = L[(int64_t)s * K];
  if (lane == 0) n_pool = 0;
  __syncthreads();
  // Only lists whose head reaches the K-th largest head can hold a top-K entry;
  // at most K such lists exist, so the pool holds at most K*K entries.
  const uint64_t th = wave_kth(heads, S, K, lane);
  for (int s = lane; s < S; s += kWave) {
    if (heads[s] == 0 || heads[s] < th) continue;
    for (int k = 0; k < K; ++k) {
      const uint64_t e = L[(int64_t)s * K + k];
      if (e == 0 || e < th) break;
      pool[atomicAdd(&n_pool, 1)] = e;
    }
  }
  __syncthreads();
  const int n = n_pool;
  const uint64_t t = wave_kth(pool, n, K, lane);
  int off = 0;
  for (int base = 0; base < n; base += kWave) {
    const int p = base + lane;
    const uint64_t e = p < n ? pool[p] : 0;
    const bool keep = p < n && e >= t && e != 0;
    const uint64_t mask = __ballot(keep);
    if (keep) top[off + __popcll(mask & ((1ull << lane) - 1))] = e;
    off += __popcll(mask);
  }
  __syncthreads();
  const int m = off;
  if (lane < K) {
    const int64_t o = row * K;
    if (lane < m) {
      const uint64_t e = top[lane];
      int rank = 0;
      for (int i = 0; i < m; ++i) rank += top[i] > e;
      a.out_idx[o + rank] = (int32_t)cand_chunk(e);
      a.out_score[o + rank] = key_score(cand_key(e)) * a.ret_scale;
    } else {
      a.out_idx[o + lane] = -1;
      a.out_score[o + lane] = -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_scan(const ScanArgs& a, int64_t B, bool bf16, int D, hipStream_t st) {
  const int64_t rbk = (a.Lq + kRows - 1) / kRows;
  const dim3 grid((unsigned)(rbk * B * a.Hkv), (unsigned)a.n_splits, 1);
  const dim3 block(64, 1, 1);
  if (bf16) {
    if (D == 128) hipLaunchKernelGGL((scan_topk_kernel<true, 128>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((scan_topk_kernel<true, 64>), grid, block, 0, st, a);
  } else {
    if (D == 128) hipLaunchKernelGGL((scan_topk_kernel<false, 128>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((scan_topk_kernel<false, 64>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t st) {
  if (a.n_splits > kMaxSplits) return hipErrorInvalidValue;
  hipLaunchKernelGGL(merge_topk_kernel, dim3((unsigned)a.rows), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace hsa
