// backward.hip -- HSA backward for a given selection (bf16): the gradients of
// sum(out * dout) with respect to q_ret, landmarks, q_attn, k and v.  The
// selection carries no gradient; the gradient reaches the retrieval path
// through the blend weights w = softmax(s) (Step 4 of the HSA step in "Every
// Token Counts", agent-atlas explainer, "How It Works (Technically)") and
// s = ret_scale (q_ret . landmark) (Step 2), and the attention path through
// each chunk's softmax attention with the query-key normalisation (Step 3).
//
// Pairs (row, slot) are bucketed by chunk exactly as for the chunk-major
// forward, and each bin's pair list is then sorted, so every sum below runs
// in a fixed order (bit-identical results run to run).
//   item     per work item (<= 64 pairs of one chunk): K, K^T, V and the key
//            norms in LDS; per 16-head-row tile (one wave): S^T = K Q^T and
//            dP^T = V dO_w^T on MFMA (dO_w = w dout), P, w dw = sum P dP,
//            dz = P (dP - sum P dP); dqhat^T = K^T g^T (g = attn dz / |k|)
//            stored per pair in bf16; P^T, h^T (h = attn dz / |q|), dO_w^T and
//            q^T staged in LDS, then each wave accumulates 16 keys of
//            dV = P^T dO_w and dkhat = h^T q over the item's head-rows.
//   slot     per (row, slot): ds = w dw - w sum(w dw), times ret_scale.
//   dq       per (row, head): dq = normalisation's gradient of the summed
//            dqhat; per row: dq_ret = sum over slots of ds landmark.
//   chunk    per chunk: the items' dV and dkhat summed in order; dk is the
//            normalisation's gradient of dkhat.
//   landmark per chunk: dlandmark = sum over its pairs of ds q_ret.
#include "hsa_device.h"
#include "hsa_internal.h"

namespace hsa {
namespace {

constexpr int kBP = 64;                     // pairs per work item (as the forward)
constexpr float kLog2eB = 1.4426950408889634f;
// 1 / max(sqrt(ss), 1e-6) for a sum of squares ss >= 0, by the hardware
// reciprocal square root (within about 1 ulp)
__device__ __forceinline__ float inv_norm(float ss) { return __builtin_amdgcn_rsqf(fmaxf(ss, 1e-12f)); }

// --- sort each bin's pair ids ascending (bitonic in LDS) --------------------
constexpr int kSortCap = 8192;

__global__ __launch_bounds__(256) void bin_sort_kernel(BwdArgs a) {
  __shared__ uint32_t v[kSortCap];
  const int64_t bin = blockIdx.x;
  const uint32_t o0 = a.c.offsets[bin], n = a.c.offsets[bin + 1] - o0;
  if (n <= 1 || n > kSortCap) return;       // larger bins keep their order (not expected)
  if (n <= 256) {                           // rank sort: pair ids in a bin are distinct
    const uint32_t x = threadIdx.x < n ? a.c.pairs[o0 + threadIdx.x] : 0xFFFFFFFFu;
    v[threadIdx.x] = x;
    __syncthreads();
    if (threadIdx.x < n) {
      uint32_t r = 0;
      for (uint32_t j = 0; j < n; ++j) r += v[j] < x;
      a.c.pairs[o0 + r] = x;
    }
    return;
  }
  // larger bins: place every pair at its query row's offset inside the band
  // (the pair ids of one bin differ in their row unless a row names the chunk
  // in two slots), then compact in row order; a repeated row falls back to a
  // bitonic sort
  __shared__ uint32_t cnt[256];
  __shared__ int dup;
  const int64_t band = (bin / a.c.Nc) % a.c.n_bands, r0 = band * a.c.band_rows;
  if (a.c.band_rows <= kSortCap) {
    for (int i = threadIdx.x; i < kSortCap; i += 256) v[i] = 0xFFFFFFFFu;
    if (threadIdx.x == 0) dup = 0;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < n; i += 256) {
      const uint32_t pid = a.c.pairs[o0 + i];
      const int64_t r = ((int64_t)(pid / (uint32_t)a.c.K) / a.c.Hkv) % a.c.Lq;
      if (atomicCAS(&v[r - r0], 0xFFFFFFFFu, pid) != 0xFFFFFFFFu) dup = 1;
    }
    __syncthreads();
    if (!dup) {
      constexpr int PER = kSortCap / 256;
      uint32_t c = 0;
#pragma unroll 8
      for (int j = 0; j < PER; ++j) c += v[threadIdx.x * PER + j] != 0xFFFFFFFFu;
      cnt[threadIdx.x] = c;
      __syncthreads();
      uint32_t base = 0;
      for (uint32_t t = 0; t < threadIdx.x; ++t) base += cnt[t];
      for (int j = 0; j < PER; ++j) {
        const uint32_t x = v[threadIdx.x * PER + j];
        if (x != 0xFFFFFFFFu) a.c.pairs[o0 + base++] = x;
      }
      return;
    }
    __syncthreads();
  }
  int np = 1;
  while (np < (int)n) np <<= 1;
  for (int i = threadIdx.x; i < np; i += 256) v[i] = i < (int)n ? a.c.pairs[o0 + i] : 0xFFFFFFFFu;
  __syncthreads();
  for (int k = 2; k <= np; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < np; i += 256) {
        const int l = i ^ j;
        if (l > i) {
          const bool up = (i & k) == 0;
          const uint32_t x = v[i], y = v[l];
          if ((x > y) == up) {
            v[i] = y;
            v[l] = x;
          }
        }
      }
      __syncthreads();
    }
  for (int i = threadIdx.x; i < (int)n; i += 256) a.c.pairs[o0 + i] = v[i];
}

// --- per work item ------------------------------------------------------------
template <int D, int G>
__global__ __launch_bounds__(256, 2) void bwd_item_kernel(BwdArgs a) {
  constexpr int KROW = D + 16;              // K, V rows (bf16; 32-byte pad: no bank conflicts)
  constexpr int PT = 16 / G;                // pairs per 16-head-row tile
  constexpr int KSTEP = D / 32, NT = D / 16;
  // about 67 KiB of LDS: two workgroups per CU.  ks holds the normalised keys
  // khat (k itself without query-key normalisation).
  __shared__ __align__(16) uint16_t ks[kChunk * KROW];
  __shared__ __align__(16) uint16_t vs[kChunk * KROW];
  // phase B operands of 32 head-rows (2 tiles), row-major (read back
  // transposed): P and h [hr][key], dO and q [hr][dim], stored as four 8-row
  // blocks whose stride is 8 padded rows plus 128 bytes.  A transpose load's
  // lane groups jg = 0, 1 (and 2, 3) are served in the same cycle (64 banks of
  // 4 bytes, 32 lanes of 8 bytes) and read blocks jg; with a plain row stride
  // 8 rows span a multiple of 256 bytes for both row widths and the two groups
  // fell on the same banks (37 % of the kernel's LDS-active cycles were bank
  // conflicts, nearly all in these loads).
  constexpr int PROW = kChunk + 16, QROW = D + 16;
  constexpr int PBLK = 8 * PROW + 64, QBLK = 8 * QROW + 64;
  __shared__ __align__(16) uint16_t ps[4 * PBLK];
  __shared__ __align__(16) uint16_t hs[4 * PBLK];
  __shared__ __align__(16) uint16_t ds_[4 * QBLK];
  __shared__ __align__(16) uint16_t qs[4 * QBLK];
  __shared__ uint32_t pid_s[kBP];
  __shared__ float w_s[kBP];
  __shared__ int64_t qoff_s[kBP];

  const ChunkArgs& c = a.c;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, ma = lane & 15, jg = lane >> 4;
  const uint32_t item_i = blockIdx.x;
  if (item_i >= *c.n_items) return;
  const uint64_t item = c.items[item_i];
  const int64_t bin = (int64_t)(item & 0xFFFFFFFFull);
  const uint32_t blk = (uint32_t)(item >> 32);
  const uint32_t p_begin = c.offsets[bin] + blk * kBP;
  const uint32_t p_end = min(p_begin + (uint32_t)kBP, c.offsets[bin + 1]);
  const int n_pairs = (int)(p_end - p_begin);
  const int64_t bgb = bin / c.Nc, chunk = bin - bgb * c.Nc, bg = bgb / c.n_bands;
  const int g = (int)(bg % c.Hkv);
  if (tid < n_pairs) {
    const uint32_t pid = c.pairs[p_begin + tid];
    pid_s[tid] = pid;
    w_s[tid] = c.wts[pid];
    const int64_t qrow = (int64_t)(pid / (uint32_t)c.K) / c.Hkv;
    qoff_s[tid] = (qrow * c.Hq + (int64_t)g * G) * D;
  }
  {  // K and V row-major, key norms
    const int64_t base = (bg * c.Lkv + chunk * kChunk) * D;
    const uint16_t* kp = reinterpret_cast<const uint16_t*>(c.k) + base;
    const uint16_t* vp = reinterpret_cast<const uint16_t*>(c.v) + base;
    constexpr int NU = kChunk * D / 8 / 256;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int e = (tid + 256 * u) * 8, key = e / D, d0 = e % D;
      const uint4 kx = *reinterpret_cast<const uint4*>(kp + e);
      const uint4 vx = *reinterpret_cast<const uint4*>(vp + e);
      *reinterpret_cast<uint4*>(&ks[key * KROW + d0]) = kx;
      *reinterpret_cast<uint4*>(&vs[key * KROW + d0]) = vx;
    }
  }
  __syncthreads();
  if (c.qk_norm) {  // khat = k / max(|k|, 1e-6), each key's D dims over 4 threads
    const int key = tid >> 2, qd = tid & 3;
    uint4 u[D / 32];
    float ss = 0.f;
#pragma unroll
    for (int x = 0; x < D / 32; ++x) {
      u[x] = *reinterpret_cast<const uint4*>(&ks[key * KROW + qd * (D / 4) + 8 * x]);
      const uint32_t wd[4] = {u[x].x, u[x].y, u[x].z, u[x].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x2 v2 = __builtin_bit_cast(bf16x2, wd[q]);
        ss = __builtin_amdgcn_fdot2_f32_bf16(v2, v2, ss, false);
      }
    }
    ss += __shfl_xor(ss, 1, kWave);
    ss += __shfl_xor(ss, 2, kWave);
    const float r = inv_norm(ss);
#pragma unroll
    for (int x = 0; x < D / 32; ++x) {
      uint32_t wd[4] = {u[x].x, u[x].y, u[x].z, u[x].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x2 o2 = {(__bf16)(__uint_as_float(wd[q] << 16) * r),
                           (__bf16)(__uint_as_float(wd[q] & 0xFFFF0000u) * r)};
        wd[q] = __builtin_bit_cast(uint32_t, o2);
      }
      *reinterpret_cast<uint4*>(&ks[key * KROW + qd * (D / 4) + 8 * x]) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
    __syncthreads();
  }

  floatx4 dv[NT], dk[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    dv[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    dk[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  const float as = c.attn_scale;
  const int n_tiles = (n_pairs + PT - 1) / PT;
  // q and dout rows of this wave's tile (16 head-rows), loaded one tile ahead.
  // Head-rows past the item's pairs read the first pair's rows (finite data
  // of this item) and carry weight 0, which zeroes everything they add.
  uint4 xr[KSTEP], yr[KSTEP];
  auto tile_off = [&](int tile) -> int64_t {
    const int pm = tile * PT + ma / G;
    return (tile < n_tiles && pm < n_pairs ? qoff_s[pm] : qoff_s[0]) + (int64_t)(ma % G) * D;
  };
  {
    const int64_t off = tile_off(w);
#pragma unroll
    for (int t = 0; t < KSTEP; ++t) {
      xr[t] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(c.q_attn) + off + 8 * jg + 32 * t);
      yr[t] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.dout) + off + 8 * jg + 32 * t);
    }
  }
  for (int t0 = 0; t0 < n_tiles; t0 += 4) {
    // ---- phase A: this wave's tile of 16 head-rows -------------------------
    const int tile = t0 + w;
    const int pm = tile * PT + ma / G, hd = ma % G;
    const bool live = tile < n_tiles && pm < n_pairs;
    const float wp = live ? w_s[pm] : 0.f;
    // The pair's blend weight w scales its output gradient dO = w dout, and
    // dP, dz and dV are linear in dO: the products below use dout itself and
    // w enters once, in dz's factor and in the staged P (w P for dV).
    bf16x8 qa[KSTEP], da[KSTEP];
    uint4 qst[KSTEP], dst[KSTEP];             // this tile's q and dout rows for phase B
    float qss = 0.f;
#pragma unroll
    for (int t = 0; t < KSTEP; ++t) {
      const uint4 x = xr[t], y = yr[t];
      qa[t] = __builtin_bit_cast(bf16x8, x);
      da[t] = __builtin_bit_cast(bf16x8, y);
      const uint32_t qw[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x2 v2 = __builtin_bit_cast(bf16x2, qw[q]);
        qss = __builtin_amdgcn_fdot2_f32_bf16(v2, v2, qss, false);
      }
      qst[t] = x;
      dst[t] = y;
    }
    if (t0 + 4 < n_tiles) {   // next tile's rows, in flight during this one
      const int64_t off = tile_off(t0 + 4 + w);
#pragma unroll
      for (int t = 0; t < KSTEP; ++t) {
        xr[t] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(c.q_attn) + off + 8 * jg + 32 * t);
        yr[t] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.dout) + off + 8 * jg + 32 * t);
      }
    }
    qss = xrow_sum(qss);
    const float rq = c.qk_norm ? inv_norm(qss) : 1.0f;
    // S^T = khat Q^T and dP'^T = V dout^T: lane holds keys 16*nt + 4*jg + i of head-row ma
    floatx4 sv[4], dp[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      sv[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
      dp[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < KSTEP; ++t) {
        const uint4 kb = *reinterpret_cast<const uint4*>(&ks[(16 * nt + ma) * KROW + 32 * t + 8 * jg]);
        const uint4 vb = *reinterpret_cast<const uint4*>(&vs[(16 * nt + ma) * KROW + 32 * t + 8 * jg]);
        sv[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb), qa[t], sv[nt], 0, 0, 0);
        dp[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vb), da[t], dp[nt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // softmax over the chunk's keys in base 2: the logit factor cs > 0, so the
    // largest raw product gives the largest logit
    const float cs = rq * as * kLog2eB;
    float mx = -INFINITY;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sv[nt][i]);
    mx = xrow_max(mx);
    const float mxs = mx * cs;
    float sum = 0.f, edp = 0.f;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[nt][i] = __builtin_amdgcn_exp2f(fmaf(sv[nt][i], cs, -mxs));   // e, unnormalised
        sum += sv[nt][i];
        edp = fmaf(sv[nt][i], dp[nt][i], edp);
      }
    sum = xrow_sum(sum);
    edp = xrow_sum(edp);
    const float inv = __builtin_amdgcn_rcpf(sum);
    const float pdp = edp * inv;                            // sum_j P dP' = dout . O
    {  // w dw of the pair: its G head-rows are lanes ma with equal ma / G
      float wdw = pdp;
#pragma unroll
      for (int o = 1; o < G; o <<= 1) wdw += __shfl_xor(wdw, o, kWave);
      if (live && jg == 0 && hd == 0) a.wdw[pid_s[pm]] = wp * wdw;
    }
    // dz = w P (dP' - pdp) attn (the score gradient), g = dz (for dqhat, khat
    // staged), h = dz |q|^-1 (for dkhat); the staged P is w P (for dV)
    const float pw = inv * wp, ez = pw * as;
    bf16x8 gb[2];
    uint2 pst[4], hst[4];                     // this tile's w P and h rows for phase B
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      float hv[4], pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float dz = sv[nt][i] * ez * (dp[nt][i] - pdp);
        hv[i] = dz * rq;
        pv[i] = sv[nt][i] * pw;
        gb[nt >> 1][4 * (nt & 1) + i] = (__bf16)dz;
      }
      // w P and h of head-row ma, keys 16nt + 4jg .. +3
      const bf16x2 p01 = {(__bf16)pv[0], (__bf16)pv[1]}, p23 = {(__bf16)pv[2], (__bf16)pv[3]};
      const bf16x2 h01 = {(__bf16)hv[0], (__bf16)hv[1]}, h23 = {(__bf16)hv[2], (__bf16)hv[3]};
      pst[nt] = make_uint2(__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23));
      hst[nt] = make_uint2(__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23));
    }
    // dqhat^T = khat^T g^T: lane holds dims 16*nt + 4*jg + i of head-row ma.  The
    // A operand khat^T comes from the row-major keys by transpose loads, in the
    // key order of g (keys 32st + 4jg + 0..3 and 32st + 16 + 4jg + 0..3)
    uint16_t* dq = a.dq_part + (live ? ((int64_t)pid_s[pm] * G + hd) * D : 0) + 4 * jg;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      floatx4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8 ka = lds_operand_tr2(ks, KROW, 32 * st + 4 * jg, 32 * st + 16 + 4 * jg, 16 * nt, ma);
        o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, gb[st], o, 0, 0, 0);
      }
      if (live) {
        const bf16x2 lo = {(__bf16)o[0], (__bf16)o[1]}, hi = {(__bf16)o[2], (__bf16)o[3]};
        *reinterpret_cast<uint2*>(dq + 16 * nt) =
            make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
      }
      if (nt % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
    // ---- phase B: keys 16w .. 16w+15 over the 4 tiles' head-rows, two tiles
    // (32 head-rows) per round.  A = P^T / h^T (key x head-row), B = dO_w / q
    // (head-row x dim), both read transposed from the row-major staging.
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if ((w >> 1) == half) {
        const int r = 16 * (w & 1) + ma, qr = (r >> 3) * QBLK + (r & 7) * QROW,
                  pr = (r >> 3) * PBLK + (r & 7) * PROW;
#pragma unroll
        for (int t = 0; t < KSTEP; ++t) {
          *reinterpret_cast<uint4*>(&qs[qr + 32 * t + 8 * jg]) = qst[t];
          *reinterpret_cast<uint4*>(&ds_[qr + 32 * t + 8 * jg]) = dst[t];
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          *reinterpret_cast<uint2*>(&ps[pr + 16 * nt + 4 * jg]) = pst[nt];
          *reinterpret_cast<uint2*>(&hs[pr + 16 * nt + 4 * jg]) = hst[nt];
        }
      }
      __syncthreads();
      // lane group jg reads head-rows 8 jg .. 8 jg + 7: block jg
      const bf16x8 pa = lds_operand_tr(ps + jg * PBLK, PROW, 0, 16 * w, ma);
      const bf16x8 ha = lds_operand_tr(hs + jg * PBLK, PROW, 0, 16 * w, ma);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const bf16x8 db = lds_operand_tr(ds_ + jg * QBLK, QROW, 0, 16 * nt, ma);
        const bf16x8 qb = lds_operand_tr(qs + jg * QBLK, QROW, 0, 16 * nt, ma);
        dv[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, db, dv[nt], 0, 0, 0);
        dk[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ha, qb, dk[nt], 0, 0, 0);
        if (nt % 2 == 1) __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();
    }
  }
  // item partials: lane holds keys 16w + 4*jg + i, dims 16*nt + ma
  float* pv = a.item_part + (int64_t)item_i * 2 * kChunk * D;
  float* pk = pv + kChunk * D;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = 16 * w + 4 * jg + i;
      pv[key * D + 16 * nt + ma] = dv[nt][i];
      pk[key * D + 16 * nt + ma] = dk[nt][i];
    }
}

// --- per chunk: dV, dK --------------------------------------------------------
// A key's D / 4 threads each own 4 dims; a workgroup takes 256 / (D / 4) keys
// of one chunk and sums the items of the chunk's bins (band by band, item by
// item) for them.
template <int D>
__global__ __launch_bounds__(256) void bwd_chunk_kernel(BwdArgs a) {
  const ChunkArgs& c = a.c;
  constexpr int TPK = D / 4, KPB = 256 / TPK, BPC = kChunk / KPB;
  const int64_t blk = blockIdx.x, bgc = blk / BPC, bg = bgc / c.Nc, chunk = bgc % c.Nc;
  const int tid = threadIdx.x, kl = (int)(blk % BPC) * KPB + tid / TPK, x4 = 4 * (tid % TPK);
  float4 sv = make_float4(0.f, 0.f, 0.f, 0.f), sk = sv;
  const int64_t poff = (int64_t)kl * D + x4;
  for (int64_t band = 0; band < c.n_bands; ++band) {
    const int64_t bin = (bg * c.n_bands + band) * c.Nc + chunk;
    const uint32_t n = c.offsets[bin + 1] - c.offsets[bin];
    const uint32_t i0 = c.item_start[bin], i1 = i0 + (n + kBP - 1) / kBP;
    for (uint32_t it = i0; it < i1; it += 4) {     // 4 items in flight, summed in item order
      float4 v4[4], k4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float* pv = a.item_part + (int64_t)min(it + u, i1 - 1) * 2 * kChunk * D + poff;
        v4[u] = load_stream(reinterpret_cast<const float4*>(pv));
        k4[u] = load_stream(reinterpret_cast<const float4*>(pv + kChunk * D));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (it + u < i1) {
          sv.x += v4[u].x; sv.y += v4[u].y; sv.z += v4[u].z; sv.w += v4[u].w;
          sk.x += k4[u].x; sk.y += k4[u].y; sk.z += k4[u].z; sk.w += k4[u].w;
        }
    }
  }
  const int64_t row = bg * c.Lkv + chunk * kChunk + kl;
  const uint2 kr = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(c.k) + row * D + x4);
  const float kx[4] = {__uint_as_float(kr.x << 16), __uint_as_float(kr.x & 0xFFFF0000u),
                       __uint_as_float(kr.y << 16), __uint_as_float(kr.y & 0xFFFF0000u)};
  const float dk4[4] = {sk.x, sk.y, sk.z, sk.w};
  float ss = 0.f, dot = 0.f;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    ss += kx[x] * kx[x];
    dot += kx[x] * dk4[x];
  }
#pragma unroll
  for (int o = 1; o < TPK; o <<= 1) {
    ss += __shfl_xor(ss, o, kWave);
    dot += __shfl_xor(dot, o, kWave);
  }
  // dkhat -> dk: (dkh - khat (khat . dkh)) / |k|, or dkh / eps below eps
  const float n = sqrtf(ss);
  float g[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    g[x] = dk4[x];
    if (c.qk_norm) g[x] = n > 1e-6f ? (dk4[x] - kx[x] * (dot / (n * n))) / n : dk4[x] * 1e6f;
  }
  *reinterpret_cast<float4*>(a.dk + row * D + x4) = make_float4(g[0], g[1], g[2], g[3]);
  *reinterpret_cast<float4*>(a.dv + row * D + x4) = sv;
}

// Keys of the trailing partial chunk take no part (no landmark): zero.
__global__ __launch_bounds__(256) void bwd_tail_kernel(BwdArgs a, int D) {
  const ChunkArgs& c = a.c;
  const int64_t bg = blockIdx.y, n = (c.Lkv - c.Nc * kChunk) * D;
  const int64_t base = (bg * c.Lkv + c.Nc * kChunk) * D;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    a.dk[base + i] = 0.f;
    a.dv[base + i] = 0.f;
  }
}

// --- per slot: dL/ds --------------------------------------------------------------
// One lane per slot (segments of a power of two >= K lanes per row):
// draw_k = ret_scale (w_k dw_k - w_k sum_j w_j dw_j), zero for unused slots.
__global__ __launch_bounds__(256) void bwd_slot_kernel(BwdArgs a) {
  const ChunkArgs& c = a.c;
  const int K = c.K, S = K <= 1 ? 1 : 1 << (32 - __clz(K - 1));
  const int64_t row = (int64_t)blockIdx.x * (256 / S) + threadIdx.x / S;
  const int k = threadIdx.x & (S - 1);
  const bool active = row < c.rows && k < K;
  int32_t ci = -1;
  if (active) ci = c.idx[row * K + k];
  const bool valid = active && ci >= 0 && (int64_t)ci < c.Nc;
  const float wdw = valid ? a.wdw[row * K + k] : 0.f;
  const float wk = valid ? c.wts[row * K + k] : 0.f;
  float sum = wdw;
  for (int o = 1; o < S; o <<= 1) sum += __shfl_xor(sum, o, kWave);
  if (active) a.draw[row * K + k] = valid ? a.ret_scale * (wdw - wk * sum) : 0.f;
}

// More than 64 slots per row: one wave per row, the sum over slots reduced in
// a fixed order (lane-strided partial sums, then the wave reduction).
__global__ __launch_bounds__(256) void bwd_slot_wide_kernel(BwdArgs a) {
  const ChunkArgs& c = a.c;
  const int K = c.K, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= c.rows) return;
  float sum = 0.f;
  for (int k = lane; k < K; k += kWave) {
    const int32_t ci = c.idx[row * K + k];
    if (ci >= 0 && (int64_t)ci < c.Nc) sum += a.wdw[row * K + k];
  }
  sum = wave_sum(sum);
  for (int k = lane; k < K; k += kWave) {
    const int32_t ci = c.idx[row * K + k];
    const bool valid = ci >= 0 && (int64_t)ci < c.Nc;
    a.draw[row * K + k] = valid ? a.ret_scale * (a.wdw[row * K + k] - c.wts[row * K + k] * sum) : 0.f;
  }
}

// --- per row: dq_attn and dq_ret -----------------------------------------------
// D / 4 threads per output row, each owning 4 dims.  Blocks [0, n_attn) take
// the head-rows (row, head) of dq_attn: the pairs' dqhat summed in slot order,
// then the normalisation's gradient; the rest take the rows of dq_ret:
// sum over slots of draw_k * landmark[c_k].
template <int D, int G>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdArgs a, uint32_t n_attn) {
  const ChunkArgs& c = a.c;
  constexpr int TPH = D / 4, HPB = 256 / TPH;
  const int K = c.K, tid = threadIdx.x, x4 = 4 * (tid % TPH);
  if (blockIdx.x < n_attn) {
    const int64_t u = (int64_t)blockIdx.x * HPB + tid / TPH;     // (row, head)
    const bool in = u < c.rows * G;
    const int64_t row = in ? u / G : 0;
    const int hd = (int)(u % G);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k0 = 0; k0 < K; k0 += 8) {
      uint2 v[8];
      bool ok[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = min(k0 + e, K - 1);
        const int32_t ci = c.idx[row * K + k];
        ok[e] = k0 + e < K && ci >= 0 && (int64_t)ci < c.Nc;
        v[e] = load_stream(reinterpret_cast<const uint2*>(a.dq_part + ((row * K + k) * G + hd) * D + x4));
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (ok[e]) {
          acc.x += __uint_as_float(v[e].x << 16);
          acc.y += __uint_as_float(v[e].x & 0xFFFF0000u);
          acc.z += __uint_as_float(v[e].y << 16);
          acc.w += __uint_as_float(v[e].y & 0xFFFF0000u);
        }
    }
    const int64_t qrow = (row / c.Hkv) * c.Hq + (int64_t)(row % c.Hkv) * G + hd;
    const uint2 qr = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(c.q_attn) + qrow * D + x4);
    const float qx[4] = {__uint_as_float(qr.x << 16), __uint_as_float(qr.x & 0xFFFF0000u),
                         __uint_as_float(qr.y << 16), __uint_as_float(qr.y & 0xFFFF0000u)};
    const float dq4[4] = {acc.x, acc.y, acc.z, acc.w};
    float ss = 0.f, dot = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      ss += qx[x] * qx[x];
      dot += qx[x] * dq4[x];
    }
#pragma unroll
    for (int o = 1; o < TPH; o <<= 1) {
      ss += __shfl_xor(ss, o, kWave);
      dot += __shfl_xor(dot, o, kWave);
    }
    const float n = sqrtf(ss);
    float g[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      g[x] = dq4[x];
      if (c.qk_norm) g[x] = n > 1e-6f ? (dq4[x] - qx[x] * (dot / (n * n))) / n : dq4[x] * 1e6f;
    }
    if (in) *reinterpret_cast<float4*>(a.dq_attn + qrow * D + x4) = make_float4(g[0], g[1], g[2], g[3]);
    return;
  }
  const int64_t row = (int64_t)(blockIdx.x - n_attn) * HPB + tid / TPH;   // (b*Lq + r)*Hkv + g
  if (row >= c.rows) return;
  const int g = (int)(row % c.Hkv);
  const int64_t b = row / c.Hkv / c.Lq;
  const uint16_t* lmb = reinterpret_cast<const uint16_t*>(a.landmarks) + (b * c.Hkv + g) * c.Nc * D + x4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = 0; k0 < K; k0 += 8) {
    uint2 l[8];
    float dr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = min(k0 + e, K - 1);
      const int32_t ci = c.idx[row * K + k];
      const bool ok = k0 + e < K && ci >= 0 && (int64_t)ci < c.Nc;
      dr[e] = ok ? a.draw[row * K + k] : 0.f;
      l[e] = *reinterpret_cast<const uint2*>(lmb + (int64_t)(ok ? ci : 0) * D);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc.x += dr[e] * __uint_as_float(l[e].x << 16);
      acc.y += dr[e] * __uint_as_float(l[e].x & 0xFFFF0000u);
      acc.z += dr[e] * __uint_as_float(l[e].y << 16);
      acc.w += dr[e] * __uint_as_float(l[e].y & 0xFFFF0000u);
    }
  }
  *reinterpret_cast<float4*>(a.dq_ret + row * D + x4) = acc;
}

// --- dlandmark ------------------------------------------------------------------
// dlandmarks = sum over the pairs that chose a chunk of draw(pair) * q_ret(row),
// in two passes so that no workgroup walks the pairs of a whole chunk (early
// chunks are chosen by many more rows than late ones).  First, per work item
// (at most kBP pairs of one bin): each of NG lane groups adds its pairs in
// order, then the groups are added in order; the item's D sums go to the first
// D floats of its item_part slot, which bwd_chunk_kernel has finished reading.
template <int D>
__global__ __launch_bounds__(256) void bwd_lm_item_kernel(BwdArgs a) {
  const ChunkArgs& c = a.c;
  constexpr int TPP = D / 8, NG = 256 / TPP;
  __shared__ float red[NG][D + 4];
  const uint32_t item_i = blockIdx.x;
  if (item_i >= *c.n_items) return;
  const uint64_t item = c.items[item_i];
  const int64_t bin = (int64_t)(item & 0xFFFFFFFFull);
  const uint32_t p0 = c.offsets[bin] + (uint32_t)(item >> 32) * kBP;
  const uint32_t p1 = min(p0 + (uint32_t)kBP, c.offsets[bin + 1]);
  const int tid = threadIdx.x, grp = tid / TPP, x8 = 8 * (tid % TPP);
  const uint16_t* qr = reinterpret_cast<const uint16_t*>(a.q_ret) + x8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (uint32_t p = p0 + grp; p < p1; p += 4 * NG) {   // four pairs in flight, in order
    uint32_t pid[4];
    float dr[4];
    uint4 q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) pid[u] = c.pairs[min(p + u * NG, p1 - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      dr[u] = p + u * NG < p1 ? a.draw[pid[u]] : 0.f;
      q[u] = *reinterpret_cast<const uint4*>(qr + (int64_t)(pid[u] / (uint32_t)c.K) * D);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t wq[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += dr[u] * __uint_as_float(wq[e] << 16);
        acc[2 * e + 1] += dr[u] * __uint_as_float(wq[e] & 0xFFFF0000u);
      }
    }
  }
#pragma unroll
  for (int x = 0; x < 8; ++x) red[grp][x8 + x] = acc[x];
  __syncthreads();
  if (tid < D) {
    float sum = 0.f;
    for (int gi = 0; gi < NG; ++gi) sum += red[gi][tid];
    a.item_part[(int64_t)item_i * 2 * kChunk * D + tid] = sum;
  }
}

// Second pass: per (batch, kv head, chunk), the item sums of the chunk's bins
// (band by band, item by item) added in that order; thread t owns dim t.
template <int D>
__global__ __launch_bounds__(D) void bwd_landmark_kernel(BwdArgs a) {
  const ChunkArgs& c = a.c;
  const int64_t bg = blockIdx.x / c.Nc, chunk = blockIdx.x % c.Nc;
  const int x = threadIdx.x;
  float sum = 0.f;
  for (int64_t band = 0; band < c.n_bands; ++band) {
    const int64_t bin = (bg * c.n_bands + band) * c.Nc + chunk;
    const uint32_t n = c.offsets[bin + 1] - c.offsets[bin];
    const uint32_t i0 = c.item_start[bin], i1 = i0 + (n + kBP - 1) / kBP;
    for (uint32_t it = i0; it < i1; it += 4) {     // 4 items in flight, added in item order
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = a.item_part[(int64_t)min(it + u, i1 - 1) * 2 * kChunk * D + x];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (it + u < i1) sum += v[u];
    }
  }
  a.dlandmarks[(bg * c.Nc + chunk) * D + x] = sum;
}

}  // namespace

int64_t bwd_pairs_per_item() { return kBP; }
int64_t bwd_band_rows() { return 8192; }   // a bin holds <= 8192 pairs: sortable in LDS

namespace {

template <int D, int G>
hipError_t launch_bwd_dg(const BwdArgs& a, hipStream_t st, const Marks& mk) {
  hipError_t e;
  const int64_t n_bg = a.c.rows / a.c.Lq;
  if ((e = mk.rec(kStageAttend, 0, st)) != hipSuccess) return e;
  if (a.c.max_items > 0) {
    hipLaunchKernelGGL((bwd_item_kernel<D, G>), dim3((unsigned)a.c.max_items), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = mk.rec(kStageAttend, 1, st)) != hipSuccess) return e;
  if ((e = mk.rec(kStageCombine, 0, st)) != hipSuccess) return e;
  if (a.c.K > kWave) {
    hipLaunchKernelGGL(bwd_slot_wide_kernel, dim3((unsigned)((a.c.rows + 3) / 4)), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else {
    const int64_t S = a.c.K <= 1 ? 1 : (int64_t)1 << (32 - __builtin_clz((unsigned)a.c.K - 1));
    hipLaunchKernelGGL(bwd_slot_kernel, dim3((unsigned)((a.c.rows + 256 / S - 1) / (256 / S))), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {
    constexpr int64_t HPB = 256 / (D / 4);
    const int64_t n_attn = (a.c.rows * G + HPB - 1) / HPB, n_ret = (a.c.rows + HPB - 1) / HPB;
    hipLaunchKernelGGL((bwd_dq_kernel<D, G>), dim3((unsigned)(n_attn + n_ret)), dim3(256), 0, st, a,
                       (uint32_t)n_attn);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.c.Nc > 0) {
    constexpr int64_t BPC = kChunk / (256 / (D / 4));
    hipLaunchKernelGGL((bwd_chunk_kernel<D>), dim3((unsigned)(n_bg * a.c.Nc * BPC)), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // after bwd_chunk_kernel: the landmark item sums reuse the item partials' memory
    if (a.c.max_items > 0) {
      hipLaunchKernelGGL((bwd_lm_item_kernel<D>), dim3((unsigned)a.c.max_items), dim3(256), 0, st, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL((bwd_landmark_kernel<D>), dim3((unsigned)(n_bg * a.c.Nc)), dim3(D), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.c.Lkv > a.c.Nc * kChunk) {
    hipLaunchKernelGGL(bwd_tail_kernel, dim3(8, (unsigned)n_bg), dim3(256), 0, st, a, D);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return mk.rec(kStageCombine, 1, st);
}

}  // namespace

// bucket (+ per-bin sort) | per-item MFMA kernel | row, chunk and landmark reductions
hipError_t launch_backward(const BwdArgs& a, int D, int G, hipStream_t st, const Marks& mk) {
  hipError_t e;
  if ((e = mk.rec(kStageBucket, 0, st)) != hipSuccess) return e;
  if ((e = launch_bucket(a.c, st)) != hipSuccess) return e;
  if (a.c.n_bins > 0) {
    hipLaunchKernelGGL(bin_sort_kernel, dim3((unsigned)a.c.n_bins), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = mk.rec(kStageBucket, 1, st)) != hipSuccess) return e;
#define HSA_BWD_CASE(DD, GG) \
  if (D == DD && G == GG) return launch_bwd_dg<DD, GG>(a, st, mk);
  HSA_BWD_CASE(128, 1) HSA_BWD_CASE(128, 2) HSA_BWD_CASE(128, 4) HSA_BWD_CASE(128, 8)
  HSA_BWD_CASE(128, 16) HSA_BWD_CASE(64, 1) HSA_BWD_CASE(64, 2) HSA_BWD_CASE(64, 4)
  HSA_BWD_CASE(64, 8) HSA_BWD_CASE(64, 16)
#undef HSA_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace hsa
