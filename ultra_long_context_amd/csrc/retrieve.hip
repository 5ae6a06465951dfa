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
constexpr int kMaxSplits = 512;       // wide-scan splits per row block (8 list heads per lane in the merge)

template <bool BF16, int D> struct QOperand;

// bf16: 16x16x32 MFMA; K-group j of step t covers dims 32t + 8j .. 32t + 8j + 7.
template <int D> struct QOperand<true, D> {
  bf16x8 v[D / 32];
  // row must be a valid address even when !ok (the load is unconditional so
  // that it never waits on earlier loads)
  __device__ __forceinline__ void load(const uint16_t* row, bool ok, int j) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      uint4 x = *reinterpret_cast<const uint4*>(row + 32 * t + 8 * j);
      if (!ok) x = make_uint4(0, 0, 0, 0);
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
      float4 x = *reinterpret_cast<const float4*>(row + 16 * u + 4 * j);
      if (!ok) x = make_float4(0.f, 0.f, 0.f, 0.f);
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
    a.out_idx[row_flat * a.K + rank] = (int32_t)cand_chunk(e);
    a.out_score[row_flat * a.K + rank] = key_score(cand_key(e)) * a.ret_scale;
  }
  for (int k = m + ((j - m) & 3); k < a.K; k += 4) {
    a.out_idx[row_flat * a.K + k] = -1;
    a.out_score[row_flat * a.K + k] = -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Wide scan: few query rows over a long history (decode, appended rows).
//
// A workgroup of 16 waves scores one block of 16 rows against 1024 chunks.
// Every wave issues the loads of its 64 landmarks up front; the chunks are then
// taken in four quarters (sub-tile q of every wave, 256 chunks), so the
// selection of one quarter runs while the next quarters' landmarks are still
// in flight.  Per quarter: the waves run their MFMA tiles and park the 16x256
// score keys in LDS (double-buffered); wave w then owns row w and folds the
// quarter's keys into the row's candidates: a key enters only if it reaches
// the K-th largest of the lanes' running maxima (K distinct chunks reach that
// bound, so it never excludes a top-K key); the bound rises with every quarter
// and the exact top K of the few survivors is taken once, after the last.
// With one split the workgroup writes the final selection; otherwise it writes
// one sorted list per row and split, which a merge (merge_lists_kernel, or the
// decode attend's prologue) combines.  The lists of a row are stored
// entry-major ([entry][split]), so the first entries of every split are
// contiguous.
// ---------------------------------------------------------------------------
constexpr int kWideWaves = 16;
constexpr int kWideChunksPerWave = 64;
constexpr int kWideChunks = kWideWaves * kWideChunksPerWave;
constexpr int kWideQuarter = kWideChunks / 4;      // chunks per quarter
constexpr int kWideKeyWords = kWideQuarter + 4;    // padded LDS row of a quarter's u32 keys
constexpr int kWideTmpCap = kMaxTopK + kWideQuarter;   // running list + one quarter's candidates

// Ranks of a and b among arr[0..n) in LDS (unique nonzero keys, n
// wave-uniform): the number of entries above each.  Every lane reads the same
// addresses (broadcast), eight entries in flight per step.
__device__ __forceinline__ void lds_rank2(const uint64_t* arr, int n, uint64_t a, uint64_t b, int& ra, int& rb) {
  ra = 0;
  rb = 0;
  for (int i0 = 0; i0 < n; i0 += 8) {
    uint64_t x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = arr[i0 + u < n ? i0 + u : n - 1];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool in = i0 + u < n;
      ra += (in && x[u] > a) ? 1 : 0;
      rb += (in && x[u] > b) ? 1 : 0;
    }
  }
}

__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o, kWave), hi = __shfl_xor((uint32_t)(v >> 32), o, kWave);
    const uint64_t u = ((uint64_t)hi << 32) | lo;
    v = u < v ? u : v;
  }
  return v;
}

// Running candidate set of one row over the quarters of a split (whole wave).
// Admission: key >= tau, where tau is the upper 16 bits of the K-th largest
// running lane maximum (K lanes, i.e. K distinct chunks, reach it, so it
// bounds the row's K-th largest key from below and only rises), and packed
// candidate > thr (0, or the exact K-th candidate after a cut).  T holds the
// admitted candidates, n of them; entries that fall below a raised bound are
// dropped when the buffer runs low, and if that is not enough the buffer is
// cut to its exact top K.
struct RowCands {
  uint32_t lmx = 0;      // this lane's running maximum key
  uint32_t tau = 0;
  uint64_t thr = 0;
  int n = 0;
};

// Keeps the entries of T[0..n) that can still be in the top K; returns their count.
__device__ __forceinline__ int filter_cands(uint64_t* T, int n, uint32_t tau, uint64_t thr, int lane) {
  int off = 0;
  for (int p0 = 0; p0 < n; p0 += kWave) {
    const int p = p0 + lane;
    const uint64_t e = p < n ? T[p] : 0ull;
    const bool keep = p < n && cand_key(e) >= tau && e >= thr;
    const uint64_t mask = __ballot(keep);
    // every lane has read its entry before any lane writes (same wave, in order)
    if (keep) T[off + __popcll(mask & lanemask_lt())] = e;
    off += __popcll(mask);
  }
  return off;
}

template <class ChunkOf>
__device__ __forceinline__ void collect_quarter(const uint32_t (&v)[4], ChunkOf chunk_of, RowCands& rc, uint64_t* T,
                                                int K, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) rc.lmx = max(rc.lmx, v[i]);
  const uint32_t m16 = rc.lmx >> 16;
  uint32_t t16 = 0;
  for (int bit = 15; bit >= 0; --bit) {
    const uint32_t cand = t16 | (1u << bit);
    if (wave_count(m16 >= cand) >= K) t16 = cand;
  }
  rc.tau = max(rc.tau, t16 << 16);
  uint64_t e[4];
  bool keep[4];
  int nn = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    e[i] = pack_cand(v[i], (uint32_t)chunk_of(lane + kWave * i));
    keep[i] = v[i] != 0u && v[i] >= rc.tau && e[i] > rc.thr;
    nn += wave_count(keep[i]);
  }
  if (nn == 0) return;
  if (rc.n + nn > kWideTmpCap) {
    rc.n = filter_cands(T, rc.n, rc.tau, rc.thr, lane);
    if (rc.n + nn > kWideTmpCap) {
      // exact cut to the top K; later candidates must beat its K-th entry
      rc.n = wave_keep_top<kWideTmpCap / kWave>(T, rc.n, K, lane);
      uint64_t mn = ~0ull;
      for (int p = lane; p < rc.n; p += kWave) mn = T[p] < mn ? T[p] : mn;
      rc.thr = wave_min_u64(mn);
      nn = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        keep[i] = keep[i] && e[i] > rc.thr;
        nn += wave_count(keep[i]);
      }
    }
  }
  int off = rc.n;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint64_t mask = __ballot(keep[i]);
    if (keep[i]) T[off + __popcll(mask & lanemask_lt())] = e[i];
    off += __popcll(mask);
  }
  rc.n = off;
}

// Exact top K of the row's candidates, sorted best first into L; returns m.
__device__ __forceinline__ int finish_cands(RowCands& rc, uint64_t* T, uint64_t* L, int K, int lane) {
  const int n = filter_cands(T, rc.n, rc.tau, rc.thr, lane);
  if (n <= 2 * kWave) {
    const uint64_t a = lane < n ? T[lane] : 0ull;
    const uint64_t b = lane + kWave < n ? T[lane + kWave] : 0ull;
    int ra = 0, rb = 0;
    if (n <= kWave) ra = lds_rank(T, n, a);
    else lds_rank2(T, n, a, b, ra, rb);
    if (lane < n && ra < K) L[ra] = a;
    if (lane + kWave < n && rb < K) L[rb] = b;
    return n < K ? n : K;
  }
  const int mm = wave_keep_top<kWideTmpCap / kWave>(T, n, K, lane);
  wave_rank_sort(T, mm, L, lane);
  return mm;
}

// Writes a row's final selection (sorted top[0..m), padding after it).
__device__ __forceinline__ void write_selection(const uint64_t* top, int m, int K, int lane,
                                                int32_t* idx, float* score, float ret_scale) {
  if (lane < K) {
    if (lane < m) {
      const uint64_t e = top[lane];
      idx[lane] = (int32_t)cand_chunk(e);
      score[lane] = key_score(cand_key(e)) * ret_scale;
    } else {
      idx[lane] = -1;
      score[lane] = -INFINITY;
    }
  }
}

template <bool BF16, int D>
__global__ __launch_bounds__(1024) void scan_wide_kernel(ScanArgs a) {
  using T = typename Elem<BF16>::T;
  constexpr int LOADS = BF16 ? D / 32 : D / 16;
  // sub-tiles whose landmark loads are in flight ahead of their use (bf16: all
  // four, the wave's whole 16 KiB; fp32: as many as the registers allow)
  constexpr int PF = BF16 ? 4 : (D == 128 ? 1 : 2);
  __shared__ __align__(16) uint32_t S[2][kWideWaves][kWideKeyWords];
  __shared__ uint64_t lst[kWideWaves][kMaxTopK];
  __shared__ uint64_t tmp[kWideWaves][kWideTmpCap];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, qrow = lane & 15, j = lane >> 4;
  const int s = blockIdx.y;
  const int64_t rbk = (a.Lq + kRows - 1) / kRows;
  const int64_t rb = (int64_t)blockIdx.x % rbk;
  const int bg = (int)((int64_t)blockIdx.x / rbk);
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int c_begin = s * kWideChunks;
  const int c_end = min(c_begin + kWideChunks, a.n_max);
  const int K = a.K;

  const int64_t r = rb * kRows + qrow;
  const bool row_ok = r < a.Lq;
  int lim = 0;
  if (row_ok) {
    const int64_t n = (a.q_pos0 + r) / kChunk;
    lim = min((int)(n < a.Nc ? n : a.Nc), c_end);
  }
  // with no eligible chunk at all (then c_begin == c_end == 0) the loads read
  // the first query row instead: an address that is always valid
  const T* lm = c_begin < c_end ? reinterpret_cast<const T*>(a.landmarks) + (int64_t)bg * a.Nc * D
                                : reinterpret_cast<const T*>(a.q_ret);
  const int cw = c_begin + w * kWideChunksPerWave;
  uint4 x[4][LOADS];
  auto issue = [&](int sub) {
    // chunks past c_end load chunk c_begin instead (their keys are masked):
    // unconditional loads are all in flight at once
    const int cc0 = cw + sub * 16 + qrow;
    const int cc = cc0 < c_end ? cc0 : c_begin;
    const T* p = lm + (int64_t)cc * D + (BF16 ? 8 : 4) * j;
#pragma unroll
    for (int t = 0; t < LOADS; ++t) x[sub][t] = *reinterpret_cast<const uint4*>(p + (BF16 ? 32 : 16) * t);
  };
  // the retrieval queries first (loads complete in order, and the first
  // quarter needs them), unconditionally: rows past Lq have lim = 0, so all
  // their keys are masked and their query values never matter
  QOperand<BF16, D> q;
  q.load(reinterpret_cast<const T*>(a.q_ret) + ((b * a.Lq + (row_ok ? r : 0)) * a.Hkv + g) * D, true, j);
#pragma unroll
  for (int sub = 0; sub < PF; ++sub) issue(sub);
  __builtin_amdgcn_sched_barrier(0);

  // candidates of row w (wave w)
  const int64_t rw = rb * kRows + w;
  const bool rw_ok = rw < a.Lq;
  RowCands rc;
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    if (qt + PF < 4) issue(qt + PF);
    // --- scores of quarter qt: sub-tile qt of every wave --------------------
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < LOADS; ++t) {
      if constexpr (BF16) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x[qt][t]), q.v[t], acc, 0, 0, 0);
      } else {
        const float4 f = __builtin_bit_cast(float4, x[qt][t]);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(f.x, q.v[t].x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(f.y, q.v[t].y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(f.z, q.v[t].z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(f.w, q.v[t].w, acc, 0, 0, 0);
      }
    }
    uint4 kv;
    const int c0 = cw + qt * 16 + 4 * j;
    kv.x = c0 + 0 < lim ? score_key(acc[0]) : 0u;
    kv.y = c0 + 1 < lim ? score_key(acc[1]) : 0u;
    kv.z = c0 + 2 < lim ? score_key(acc[2]) : 0u;
    kv.w = c0 + 3 < lim ? score_key(acc[3]) : 0u;
    // quarter entry w*16 + 4j + i <-> chunk c_begin + w*64 + qt*16 + 4j + i
    *reinterpret_cast<uint4*>(&S[qt & 1][qrow][w * 16 + 4 * j]) = kv;
    // one barrier per quarter: the other buffer was last read before it
    __syncthreads();
    // --- wave w adds the quarter's candidates of row w -----------------------
    uint32_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = S[qt & 1][w][lane + kWave * i];
    collect_quarter(v, [&](int xq) { return c_begin + (xq >> 4) * kWideChunksPerWave + qt * 16 + (xq & 15); },
                    rc, tmp[w], K, lane);
  }
  const int m = finish_cands(rc, tmp[w], lst[w], K, lane);

  if (!rw_ok) return;
  const int64_t row_flat = (b * a.Lq + rw) * a.Hkv + g;
  if (a.n_splits == 1) {
    write_selection(lst[w], m, K, lane, a.out_idx + row_flat * K, a.out_score + row_flat * K, a.ret_scale);
    return;
  }
  // entry-major lists: entry j of split s at [row][j][s]
  if (lane < K) a.lists[row_flat * a.n_splits * K + (int64_t)lane * a.n_splits + s] = lane < m ? lst[w][lane] : 0ull;
}

// ---------------------------------------------------------------------------
// Block scan: many query rows (prefill), bf16, K <= 32.
//
// A workgroup of 4 waves takes 64 consecutive query rows of one (batch, kv
// head); they share their eligible chunk range up to one chunk.  Landmark tiles
// of 64 chunks go through LDS (double-buffered: the next tile's global loads
// are in flight while the current one is scored), so a landmark leaves L2 once
// per 64 rows and pass.  Wave w scores its 16 rows with
// v_mfma_f32_16x16x32_bf16 (A = landmarks from LDS, B = the rows' retrieval
// queries): lane l holds row l & 15 and chunks 4*(l >> 4) + i of each
// 16-chunk sub-tile.
//   pass 1  keeps, per lane, the running maximum of 16 chunk groups (64 groups
//           per row).  K distinct chunks reach the K-th largest group maximum,
//           so it bounds the row's K-th score from below; the bound is taken
//           on the upper 16 bits of the ordering key (still a lower bound).
//   pass 2  rescores and appends each chunk at or above the bound to the row's
//           LDS slots as (score, chunk); each lane of a row owns every 4th slot
//           past the row's kept entries, so appends need no cross-lane count.
//           If slots run low, the row is cut to its exact top K and, since
//           later chunks lose ties, the bound rises strictly above the K-th.
//   final   exact top K per row, rank sort, write.
// Cuts work in a quad layout (lane l holds row l >> 2, slots (l & 3) + 4s), so
// per-row counts are two DPP adds.  Rows are wave-local: the selection needs
// no workgroup barrier.
// ---------------------------------------------------------------------------
constexpr int kBlkWaves = 4;
constexpr int kBlkRows = kBlkWaves * kRows;     // query rows per workgroup
constexpr int kTileMax = 64;                    // chunks per LDS tile: 64, or 32 with 3 workgroups per CU
constexpr int kBlkCap = 64;                     // candidate slots per row
constexpr int kBlkStride = kBlkCap + 1;         // padded: a wave's 16 rows start on different banks
constexpr int kBlkMaxK = 32;                    // a cut leaves >= 32 free slots
constexpr uint64_t kEmpty = ~0ull;              // free slot: chunk field 0xFFFFFFFF

// Sum over the 4 lanes of a quad (DPP, no LDS).
__device__ __forceinline__ int quad_total(int v) {
  v += dpp_i<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_i<0x4E>(v);    // quad_perm [2,3,0,1]
  return v;
}
// Value of quad lane q (0..3) in every lane of the quad.
template <int Q>
__device__ __forceinline__ int quad_get(int v) {
  return dpp_i<Q * 0x55>(v);   // quad_perm [Q,Q,Q,Q]
}
// Sum over the 4 lanes (j = 0..3) that hold a row in the MFMA layout.
__device__ __forceinline__ int row_total(int v) {
  v += __shfl_xor(v, 16, kWave);
  v += __shfl_xor(v, 32, kWave);
  return v;
}

// Smallest float above x (x not NaN; +inf stays +inf): one step along the
// IEEE-754 ordering of the bit patterns.
__device__ __forceinline__ float float_above(float x) {
  const uint32_t b = __float_as_uint(x);
  if (x == 0.0f) return __uint_as_float(1u);
  if (b == 0x7F800000u) return x;
  return __uint_as_float((b & 0x80000000u) ? b - 1u : b + 1u);
}

// A slot holds (score bits << 32) | chunk; its ordering key is the packed candidate.
__device__ __forceinline__ uint64_t slot_cand(uint64_t s) {
  return s == kEmpty ? 0ull : pack_cand(score_key(__uint_as_float((uint32_t)(s >> 32))), (uint32_t)s);
}
__device__ __forceinline__ uint64_t make_slot(float score, uint32_t chunk) {
  return ((uint64_t)__float_as_uint(score) << 32) | chunk;
}

// Exact K-th largest of each quad row's register-held candidates e[0..16)
// (unique nonzero keys, zeros ignored); 0 when the row holds at most K.
__device__ __forceinline__ uint64_t quad_kth(const uint64_t (&e)[16], int n, int K) {
  if (!__any(n > K)) return 0ull;
  uint32_t t32 = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = t32 | (1u << bit);
    int c = 0;
#pragma unroll
    for (int s = 0; s < 16; ++s) c += cand_key(e[s]) >= cand;
    if (quad_total(c) >= K) t32 = cand;
  }
  int above = 0, at = 0;
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    above += cand_key(e[s]) > t32;
    at += e[s] != 0ull && cand_key(e[s]) == t32;
  }
  above = quad_total(above);
  at = quad_total(at);
  const int need = K - above;            // candidates taken at key t32 (<= at)
  uint32_t tl = 0;
  if (__any(n > K && at > need)) {       // ties at the K-th key: lower chunk index first
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = tl | (1u << bit);
      int c = 0;
#pragma unroll
      for (int s = 0; s < 16; ++s) c += e[s] != 0ull && cand_key(e[s]) == t32 && (uint32_t)e[s] >= cand;
      if (quad_total(c) >= need) tl = cand;
    }
  }
  if (at <= need) tl = 0;
  return n > K ? (((uint64_t)t32 << 32) | tl) : 0ull;
}

// Cuts every row of the wave (quad layout: rows[rq]) to its exact top K.
// Rewrites the row as kept slots [0, m) and free slots after; returns m.  kth
// receives the row's K-th candidate (0 if the row held at most K).
__device__ __forceinline__ int block_cut(uint64_t* row, int K, int jq, uint64_t& kth, bool packed_out) {
  uint64_t e[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) e[s] = slot_cand(row[jq + 4 * s]);
  int nz = 0;
#pragma unroll
  for (int s = 0; s < 16; ++s) nz += e[s] != 0ull;
  const int n = quad_total(nz);
  kth = quad_kth(e, n, K);
  const uint64_t t = kth != 0ull ? kth : 1ull;
  int kept = 0;
#pragma unroll
  for (int s = 0; s < 16; ++s) kept += e[s] >= t;
  const int k0 = quad_get<0>(kept), k1 = quad_get<1>(kept), k2 = quad_get<2>(kept);
  int off = (jq > 0 ? k0 : 0) + (jq > 1 ? k1 : 0) + (jq > 2 ? k2 : 0);
  const int m = n > K ? K : n;
  // every slot of the row is in registers: free the tail, then write the kept
#pragma unroll
  for (int s = 0; s < 16; ++s)
    if (jq + 4 * s >= m) row[jq + 4 * s] = kEmpty;
#pragma unroll
  for (int s = 0; s < 16; ++s)
    if (e[s] >= t)
      row[off++] = packed_out ? e[s]
                              : make_slot(key_score(cand_key(e[s])), cand_chunk(e[s]));
  return m;
}

// Landmark tile (TILE chunks from c_first) into LDS with direct global->LDS
// loads (global_load_lds_dwordx4): one wave operation moves 64 x 16 bytes to
// 1 KiB of consecutive LDS, so rows are unpadded and their 16-byte units are
// XOR-swizzled by row (unit u of row r sits in slot u ^ (r % RU)), which keeps
// the MFMA operand reads of 16 consecutive rows on distinct banks.  Chunks at
// or past c_stop load chunk 0 (scores masked by the caller).
template <int D, int TILE>
__device__ __forceinline__ void tile_to_lds(const uint16_t* lm, int c_first, int c_stop, uint16_t* dst,
                                            int w, int lane) {
  constexpr int RU = D / 8;                       // 16-byte units per landmark
  constexpr int OPS = TILE * RU / kWave / kBlkWaves;    // wave operations per wave
#pragma unroll
  for (int i = 0; i < OPS; ++i) {
    const int op = w * OPS + i;
    const int r = op * (kWave / RU) + lane / RU;  // tile row
    const int u = (lane % RU) ^ (r % RU);         // global unit stored in this lane's slot
    const int c = c_first + r;
    const uint16_t* src = lm + (int64_t)(c < c_stop ? c : 0) * D + 8 * u;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)(dst + op * (kWave * 8)),
                                     16, 0, 0);
  }
}

// s_waitcnt vmcnt(0): this wave's direct-to-LDS loads have landed.
__device__ __forceinline__ void wait_tile() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// One pass of a block-scan workgroup over its landmark tiles.  Two LDS tile
// buffers (distinct arrays, so the compiler can tell the in-flight copy into
// one from the reads of the other): tile t + 1 streams into the idle buffer
// while tile t is scored.  fn(sub-tile scores, sub-tile, first chunk, whole
// sub-tile eligible for every row of the wave).
template <int D, int TILE, class F>
__device__ __forceinline__ void block_sweep(const uint16_t* lm, int c_stop, int n_tiles, int w_stop,
                                            int w_min, uint16_t* lmA, uint16_t* lmB,
                                            const QOperand<true, D>& q, int w, int lane, int qrow, int j,
                                            F&& fn) {
  constexpr int RU = D / 8;
  constexpr int KSTEP = D / 32;
  if (n_tiles <= 0) return;                       // uniform over the workgroup
  // vbase: with 32-chunk tiles the sub-tiles of odd tiles are numbered 2, 3,
  // so fn always sees the four 16-chunk sub-tiles of 64 chunks as 0..3
  auto score = [&](const uint16_t* L, int t, int vbase) __attribute__((always_inline)) {
    auto sub_tile = [&](int sub) __attribute__((always_inline)) {
      const int cs = t * TILE + 16 * sub;
      const int r = 16 * sub + qrow;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KSTEP; ++k) {
        const uint4 x = *reinterpret_cast<const uint4*>(L + r * D + 8 * ((4 * k + j) ^ (r % RU)));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x), q.v[k], acc, 0, 0, 0);
      }
      fn(acc, vbase + sub, cs, cs + 16 <= w_min);
    };
    // unrolled: fn indexes registers by sub-tile, and the sub-tiles' load ->
    // MFMA -> compare chains overlap (a rolled loop that kept one copy of pass
    // 2's step ran each chain in turn: the 1M chunked prefill's scan 0.75
    // against 0.69 ms)
#pragma unroll
    for (int sub = 0; sub < TILE / 16; ++sub) {
      if (t * TILE + 16 * sub >= w_stop) break;
      sub_tile(sub);
    }
  };
  tile_to_lds<D, TILE>(lm, 0, c_stop, lmA, w, lane);
  wait_tile();
  __syncthreads();
  for (int t = 0; t < n_tiles; t += 2) {
    tile_to_lds<D, TILE>(lm, (t + 1) * TILE, c_stop, lmB, w, lane);   // past the end: chunk 0, unused
    score(lmA, t, 0);
    wait_tile();
    __syncthreads();
    if (t + 1 >= n_tiles) break;
    tile_to_lds<D, TILE>(lm, (t + 2) * TILE, c_stop, lmA, w, lane);
    score(lmB, t + 1, (kTileMax - TILE) / 16);   // 32-chunk tiles: sub-tiles 2, 3 of the pair
    wait_tile();
    __syncthreads();
  }
}

template <int D, int TILE>
__global__ __launch_bounds__(256, TILE == 32 ? 3 : 2) void scan_block_kernel(ScanArgs a) {
  __shared__ __align__(16) uint16_t lmA[TILE * D];   // landmark tiles (swizzled rows)
  __shared__ __align__(16) uint16_t lmB[TILE * D];
  __shared__ uint64_t buf[kBlkWaves][kRows * kBlkStride];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int wu = __builtin_amdgcn_readfirstlane(w);   // wave index as a scalar (LDS copy base)
  const int qrow = lane & 15, j = lane >> 4;     // MFMA layout
  const int rq = lane >> 2, jq = lane & 3;       // quad layout
  // consecutive workgroups: the same row block of successive (batch, kv head)
  // pairs (each XCD keeps to the landmarks of one pair), latest rows first
  const int64_t rbk = (a.Lq + kBlkRows - 1) / kBlkRows;
  const int64_t nbg = (int64_t)gridDim.x / rbk;
  const int bg = (int)((int64_t)blockIdx.x % nbg);
  const int64_t rb = rbk - 1 - (int64_t)blockIdx.x / nbg;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int64_t r0 = rb * kBlkRows, rw0 = r0 + w * kRows;
  auto limit = [&](int64_t r) -> int __attribute__((always_inline)) {   // chunks [0, limit) are eligible for row r
    if (r >= a.Lq) return 0;
    const int64_t n = (a.q_pos0 + r) / kChunk;
    return (int)(n < a.Nc ? n : a.Nc);
  };
  const int64_t r = rw0 + qrow;
  const int lim = limit(r);
  const int c_stop = limit(min(r0 + kBlkRows - 1, a.Lq - 1));   // the block's last row sees the most
  const int w_stop = rw0 < a.Lq ? limit(min(rw0 + kRows - 1, a.Lq - 1)) : 0;
  const int w_min = rw0 + kRows <= a.Lq ? limit(rw0) : 0;       // every row of the wave sees [0, w_min)

  QOperand<true, D> q;
  q.load(reinterpret_cast<const uint16_t*>(a.q_ret) + ((b * a.Lq + (r < a.Lq ? r : 0)) * a.Hkv + g) * D,
         r < a.Lq, j);
  const uint16_t* lm = reinterpret_cast<const uint16_t*>(a.landmarks) + (int64_t)bg * a.Nc * D;
  const int n_tiles = (c_stop + TILE - 1) / TILE;
  const int K = a.K;

  auto sweep = [&](auto&& fn) __attribute__((always_inline)) {
    block_sweep<D, TILE>(lm, c_stop, n_tiles, w_stop, w_min, lmA, lmB, q, wu, lane, qrow, j, fn);
  };

  // --- pass 1: group maxima, then a lower bound of each row's K-th key -------
  float gm[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) gm[x] = -INFINITY;
  sweep([&](const floatx4& acc, int sub, int cs, bool all) __attribute__((always_inline)) {
    floatx4 v = acc;
    if (!all) {                         // a sub-tile past some row's last eligible chunk
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (cs + 4 * j + i >= lim) v[i] = -INFINITY;
    }
    // max(a, b) as the median of (a, b, +inf): one instruction, scores are finite
#pragma unroll
    for (int i = 0; i < 4; ++i) gm[4 * sub + i] = __builtin_amdgcn_fmed3f(gm[4 * sub + i], v[i], INFINITY);
  });
  uint32_t t16 = 0;
  {
    uint32_t hk[16];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub)
#pragma unroll
      for (int i = 0; i < 4; ++i)   // group (sub, i) is empty unless its first chunk is eligible
        hk[4 * sub + i] = 16 * sub + 4 * j + i < lim ? score_key(gm[4 * sub + i]) >> 16 : 0u;
    for (int bit = 15; bit >= 0; --bit) {
      const uint32_t cand = t16 | (1u << bit);
      int c = 0;
#pragma unroll
      for (int x = 0; x < 16; ++x) c += hk[x] >= cand;
      if (row_total(c) >= K) t16 = cand;
    }
  }
  // keys at or above t16 << 16 are the scores at or above lo (keys up to that
  // of -inf: every score)
  float lo = t16 <= 0x7Fu ? -INFINITY : key_score(t16 << 16);

  // --- pass 2: candidates at or above the bound -----------------------------
  uint64_t* rows = &buf[w][0];
  uint64_t* qrowbuf = rows + rq * kBlkStride;    // quad layout row
  uint64_t* mrowbuf = rows + qrow * kBlkStride;  // MFMA layout row
#pragma unroll
  for (int s = 0; s < 16; ++s) qrowbuf[jq + 4 * s] = kEmpty;
  int m = 0, cj = 0;     // kept entries of the row; this lane's appends after them
  sweep([&](const floatx4& acc, int sub, int cs, bool all) __attribute__((always_inline)) {
    // this lane's eligible scores at or above the bound, as a 4-bit mask; the
    // rest of the step runs only when some lane of the wave has one
    unsigned vm = 0xFu;
    if (!all) {
      vm = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) vm |= (unsigned)(cs + 4 * j + i < lim) << i;
    }
    auto reach = [&]() __attribute__((always_inline)) {
      unsigned qm = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) qm |= (unsigned)(acc[i] >= lo) << i;
      return qm & vm;
    };
    unsigned qm = reach();
    if (!__any(qm != 0u)) return;
    if (__any(m + j + 4 * cj + 12 >= kBlkCap)) {   // room for four more appends per lane
      uint64_t kth;
      const int mq = block_cut(qrowbuf, K, jq, kth, false);
      // later chunks lose ties with the row's K-th: the bound becomes strict
      const float loq = kth != 0ull ? float_above(key_score(cand_key(kth))) : -INFINITY;
      m = __shfl(mq, 4 * qrow, kWave);
      lo = fmaxf(lo, __shfl(loq, 4 * qrow, kWave));
      cj = 0;
      qm = reach();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if ((qm >> i) & 1u) {
        mrowbuf[m + j + 4 * cj] = make_slot(acc[i], (uint32_t)(cs + 4 * j + i));
        ++cj;
      }
    }
  });

  // --- final: exact top K, rank sort, write ---------------------------------
  uint64_t kth;
  const int mq = block_cut(qrowbuf, K, jq, kth, true);
  const int64_t rrow = rw0 + rq;
  if (rrow >= a.Lq) return;
  const int64_t row_flat = (b * a.Lq + rrow) * a.Hkv + g;
  for (int p = jq; p < mq; p += 4) {
    const uint64_t e = qrowbuf[p];
    int rank = 0;
    for (int o = 0; o < mq; ++o) rank += qrowbuf[o] > e;
    a.out_idx[row_flat * K + rank] = (int32_t)cand_chunk(e);
    a.out_score[row_flat * K + rank] = key_score(cand_key(e)) * a.ret_scale;
  }
  for (int k = mq + ((jq - mq) & 3); k < K; k += 4) {
    a.out_idx[row_flat * K + k] = -1;
    a.out_score[row_flat * K + k] = -INFINITY;
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


hipError_t launch_scan_wide(const ScanArgs& a, int64_t B, bool bf16, int D, hipStream_t st) {
  if (a.split_len != kWideChunks || a.n_splits > kMaxSplits) return hipErrorInvalidValue;
  const int64_t rbk = (a.Lq + kRows - 1) / kRows;
  const dim3 grid((unsigned)(rbk * B * a.Hkv), (unsigned)a.n_splits, 1);
  const dim3 block(kWideWaves * 64, 1, 1);
  if (bf16) {
    if (D == 128) hipLaunchKernelGGL((scan_wide_kernel<true, 128>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((scan_wide_kernel<true, 64>), grid, block, 0, st, a);
  } else {
    if (D == 128) hipLaunchKernelGGL((scan_wide_kernel<false, 128>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((scan_wide_kernel<false, 64>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

int scan_wide_chunks() { return kWideChunks; }

int scan_block_max_k() { return kBlkMaxK; }

hipError_t launch_scan_block(const ScanArgs& a, int64_t B, int D, hipStream_t st) {
  if (a.K > kBlkMaxK) return hipErrorInvalidValue;
  const int64_t rbk = (a.Lq + kBlkRows - 1) / kBlkRows;
  const dim3 grid((unsigned)(rbk * B * a.Hkv), 1, 1), block(kBlkWaves * 64, 1, 1);
  // 32-chunk tiles fit three workgroups per CU (better latency hiding) when
  // the grid fills them; with fewer workgroups 64-chunk tiles halve the steps
  const bool small_tiles = grid.x >= 4 * 3 * 256;
  if (D == 128) {
    if (small_tiles) hipLaunchKernelGGL((scan_block_kernel<128, 32>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((scan_block_kernel<128, 64>), grid, block, 0, st, a);
  } else {
    if (small_tiles) hipLaunchKernelGGL((scan_block_kernel<64, 32>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((scan_block_kernel<64, 64>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}


}  // namespace hsa
