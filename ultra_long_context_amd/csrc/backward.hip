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
//            written per pair; P^T, h^T (h = attn dz / |q|), dO_w^T and q^T
//            staged in LDS, then each wave accumulates 16 keys of
//            dV = P^T dO_w and dkhat = h^T q over the item's head-rows.
//   chunk    per chunk: the items' dV and dkhat summed in order; dk is the
//            normalisation's gradient of dkhat.
//   row      per row: dq = normalisation's gradient of the summed dqhat;
//            ds = w dw - w sum(w dw); dq_ret = ret_scale sum ds landmark.
//   lm       per chunk: dlandmark = ret_scale sum over its pairs ds q_ret.
#include "hsa_device.h"
#include "hsa_internal.h"

namespace hsa {
namespace {

constexpr int kBP = 64;                     // pairs per work item (as the forward)
constexpr float kLog2eB = 1.4426950408889634f;

// --- sort each bin's pair ids ascending (bitonic in LDS) --------------------
constexpr int kSortCap = 8192;

__global__ __launch_bounds__(256) void bin_sort_kernel(BwdArgs a) {
  __shared__ uint32_t v[kSortCap];
  const int64_t bin = blockIdx.x;
  const uint32_t o0 = a.c.offsets[bin], n = a.c.offsets[bin + 1] - o0;
  if (n <= 1 || n > kSortCap) return;       // larger bins keep their order (not expected)
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
__global__ __launch_bounds__(256) void bwd_item_kernel(BwdArgs a) {
  constexpr int KROW = D + 8;               // K, V rows (bf16)
  constexpr int TROW = kChunk + 8;          // K^T rows (permuted keys)
  constexpr int HROW = 64 + 8;              // staged [key or dim][64 head-rows]
  constexpr int PT = 16 / G;                // pairs per 16-head-row tile
  constexpr int KSTEP = D / 32, NT = D / 16;
  __shared__ __align__(16) uint16_t ks[kChunk * KROW];
  __shared__ __align__(16) uint16_t vs[kChunk * KROW];
  __shared__ __align__(16) uint16_t kt[D * TROW];
  __shared__ float rk[kChunk];
  __shared__ __align__(16) uint16_t ps[kChunk * HROW];   // P^T   [key][hr]
  __shared__ __align__(16) uint16_t hs[kChunk * HROW];   // h^T   [key][hr]
  __shared__ __align__(16) uint16_t dt[D * HROW];        // dO_w^T [dim][hr]
  __shared__ __align__(16) uint16_t qt[D * HROW];        // q^T   [dim][hr]
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
  {  // K and V row-major, K^T with keys permuted inside 32-key blocks, key norms
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
      const int kq = key & 31;
      const int col = 32 * (key >> 5) + 8 * ((kq & 15) >> 2) + 4 * (kq >> 4) + (kq & 3);
      const uint32_t wd[4] = {kx.x, kx.y, kx.z, kx.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        kt[(d0 + 2 * q) * TROW + col] = (uint16_t)(wd[q] & 0xFFFFu);
        kt[(d0 + 2 * q + 1) * TROW + col] = (uint16_t)(wd[q] >> 16);
      }
    }
  }
  __syncthreads();
  {
    const int key = tid >> 2, qd = tid & 3;
    float ss = 0.f;
#pragma unroll
    for (int x = 0; x < D / 4; x += 8) {
      const uint4 u = *reinterpret_cast<const uint4*>(&ks[key * KROW + qd * (D / 4) + x]);
      const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x2 v2 = __builtin_bit_cast(bf16x2, wd[q]);
        ss = __builtin_amdgcn_fdot2_f32_bf16(v2, v2, ss, false);
      }
    }
    ss += __shfl_xor(ss, 1, kWave);
    ss += __shfl_xor(ss, 2, kWave);
    if (qd == 0) rk[key] = c.qk_norm ? 1.0f / fmaxf(sqrtf(ss), 1e-6f) : 1.0f;
  }
  __syncthreads();

  floatx4 dv[NT], dk[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    dv[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    dk[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  const float as = c.attn_scale;
  const int n_tiles = (n_pairs + PT - 1) / PT;
  for (int t0 = 0; t0 < n_tiles; t0 += 4) {
    // ---- phase A: this wave's tile of 16 head-rows -------------------------
    const int tile = t0 + w;
    const int pm = tile * PT + ma / G, hd = ma % G;
    const bool live = tile < n_tiles && pm < n_pairs;
    const int64_t off = live ? qoff_s[pm] + (int64_t)hd * D : 0;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(c.q_attn) + off + 8 * jg;
    const uint16_t* op = reinterpret_cast<const uint16_t*>(a.dout) + off + 8 * jg;
    const float wp = live ? w_s[pm] : 0.f;
    bf16x8 qa[KSTEP], da[KSTEP];
    float qss = 0.f;
#pragma unroll
    for (int t = 0; t < KSTEP; ++t) {
      uint4 x = *reinterpret_cast<const uint4*>(qp + 32 * t);
      uint4 y = *reinterpret_cast<const uint4*>(op + 32 * t);
      if (!live) x = y = make_uint4(0, 0, 0, 0);
      qa[t] = __builtin_bit_cast(bf16x8, x);
      const uint32_t qw[4] = {x.x, x.y, x.z, x.w}, yw[4] = {y.x, y.y, y.z, y.w};
      uint32_t dw4[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x2 v2 = __builtin_bit_cast(bf16x2, qw[q]);
        qss = __builtin_amdgcn_fdot2_f32_bf16(v2, v2, qss, false);
        const bf16x2 o2 = {(__bf16)(__uint_as_float(yw[q] << 16) * wp),
                           (__bf16)(__uint_as_float(yw[q] & 0xFFFF0000u) * wp)};
        dw4[q] = __builtin_bit_cast(uint32_t, o2);
      }
      da[t] = __builtin_bit_cast(bf16x8, make_uint4(dw4[0], dw4[1], dw4[2], dw4[3]));
      // stage q^T and dO_w^T for phase B: [dim][head-row]
      const uint16_t* qe = reinterpret_cast<const uint16_t*>(&qa[t]);
      const uint16_t* de = reinterpret_cast<const uint16_t*>(&da[t]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qt[(32 * t + 8 * jg + e) * HROW + 16 * w + ma] = qe[e];
        dt[(32 * t + 8 * jg + e) * HROW + 16 * w + ma] = de[e];
      }
    }
    qss += __shfl_xor(qss, 16, kWave);
    qss += __shfl_xor(qss, 32, kWave);
    const float rq = c.qk_norm ? 1.0f / fmaxf(sqrtf(qss), 1e-6f) : 1.0f;
    // S^T = K Q^T and dP^T = V dO_w^T: lane holds keys 16*nt + 4*jg + i of head-row ma
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
    float rkl[4][4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const float4 r4 = *reinterpret_cast<const float4*>(&rk[16 * nt + 4 * jg]);
      rkl[nt][0] = r4.x; rkl[nt][1] = r4.y; rkl[nt][2] = r4.z; rkl[nt][3] = r4.w;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[nt][i] = sv[nt][i] * (rq * as * kLog2eB) * rkl[nt][i];
        mx = fmaxf(mx, sv[nt][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    float sum = 0.f;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[nt][i] = __builtin_amdgcn_exp2f(sv[nt][i] - mx);
        sum += sv[nt][i];
      }
    sum += __shfl_xor(sum, 16, kWave);
    sum += __shfl_xor(sum, 32, kWave);
    const float inv = __builtin_amdgcn_rcpf(sum);
    float pdp = 0.f;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[nt][i] *= inv;                                   // P
        pdp += sv[nt][i] * dp[nt][i];
      }
    pdp += __shfl_xor(pdp, 16, kWave);
    pdp += __shfl_xor(pdp, 32, kWave);                      // sum_j P dP = w dout . O
    {  // w dw of the pair: its G head-rows are lanes ma with equal ma / G
      float wdw = pdp;
#pragma unroll
      for (int o = 1; o < G; o <<= 1) wdw += __shfl_xor(wdw, o, kWave);
      if (live && jg == 0 && hd == 0) a.wdw[pid_s[pm]] = wdw;
    }
    // g = attn dz |k|^-1 (for dqhat), h = attn dz |q|^-1 (for dkhat), dz = P (dP - pdp)
    bf16x8 gb[2];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float dz = sv[nt][i] * (dp[nt][i] - pdp) * as;
        const int key = 16 * nt + 4 * jg + i;
        ps[key * HROW + 16 * w + ma] = __builtin_bit_cast(uint16_t, (__bf16)sv[nt][i]);
        hs[key * HROW + 16 * w + ma] = __builtin_bit_cast(uint16_t, (__bf16)(dz * rq));
        gb[nt >> 1][4 * (nt & 1) + i] = (__bf16)(dz * rkl[nt][i]);
      }
    // dqhat^T = K^T g^T: lane holds dims 16*nt + 4*jg + i of head-row ma
    float* dq = a.dq_part + (live ? ((int64_t)pid_s[pm] * G + hd) * D : 0) + 4 * jg;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      floatx4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const uint4 ka = *reinterpret_cast<const uint4*>(&kt[(16 * nt + ma) * TROW + 32 * st + 8 * jg]);
        o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka), gb[st], o, 0, 0, 0);
      }
      if (live) *reinterpret_cast<float4*>(dq + 16 * nt) = make_float4(o[0], o[1], o[2], o[3]);
      if (nt % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    // ---- phase B: keys 16w .. 16w+15 over the 64 staged head-rows ----------
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const uint4 pa = *reinterpret_cast<const uint4*>(&ps[(16 * w + ma) * HROW + 32 * st + 8 * jg]);
        const uint4 ha = *reinterpret_cast<const uint4*>(&hs[(16 * w + ma) * HROW + 32 * st + 8 * jg]);
        const uint4 db = *reinterpret_cast<const uint4*>(&dt[(16 * nt + ma) * HROW + 32 * st + 8 * jg]);
        const uint4 qb = *reinterpret_cast<const uint4*>(&qt[(16 * nt + ma) * HROW + 32 * st + 8 * jg]);
        dv[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pa), __builtin_bit_cast(bf16x8, db),
                                                         dv[nt], 0, 0, 0);
        dk[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ha), __builtin_bit_cast(bf16x8, qb),
                                                         dk[nt], 0, 0, 0);
      }
      if (nt % 2 == 1) __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
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
// One workgroup per (batch, kv head, chunk); thread t owns key t / 4 and 32
// dims.  Chunk index Nc stands for the trailing partial chunk (zero).
template <int D>
__global__ __launch_bounds__(256) void bwd_chunk_kernel(BwdArgs a) {
  const ChunkArgs& c = a.c;
  constexpr int DPT = D / 4;                 // dims per thread
  const int64_t bg = blockIdx.x / (c.Nc + 1), chunk = blockIdx.x % (c.Nc + 1);
  const int tid = threadIdx.x, key = tid >> 2, d0 = (tid & 3) * DPT;
  if (chunk == c.Nc) {                       // tail tokens without a landmark
    for (int64_t t = c.Nc * kChunk + key; t < c.Lkv; t += 64)
      for (int x = 0; x < DPT; ++x) {
        a.dk[(bg * c.Lkv + t) * D + d0 + x] = 0.f;
        a.dv[(bg * c.Lkv + t) * D + d0 + x] = 0.f;
      }
    return;
  }
  float sv[DPT], sk[DPT];
#pragma unroll
  for (int x = 0; x < DPT; ++x) sv[x] = sk[x] = 0.f;
  for (int64_t band = 0; band < c.n_bands; ++band) {
    const int64_t bin = (bg * c.n_bands + band) * c.Nc + chunk;
    const uint32_t n = c.offsets[bin + 1] - c.offsets[bin];
    const uint32_t i0 = c.item_start[bin], ni = (n + kBP - 1) / kBP;
    for (uint32_t it = i0; it < i0 + ni; ++it) {
      const float* pv = a.item_part + (int64_t)it * 2 * kChunk * D + key * D + d0;
      const float* pk = pv + kChunk * D;
#pragma unroll
      for (int x = 0; x < DPT; x += 4) {
        const float4 v4 = *reinterpret_cast<const float4*>(pv + x);
        const float4 k4 = *reinterpret_cast<const float4*>(pk + x);
        sv[x] += v4.x; sv[x + 1] += v4.y; sv[x + 2] += v4.z; sv[x + 3] += v4.w;
        sk[x] += k4.x; sk[x + 1] += k4.y; sk[x + 2] += k4.z; sk[x + 3] += k4.w;
      }
    }
  }
  const int64_t row = bg * c.Lkv + chunk * kChunk + key;
  const uint16_t* kp = reinterpret_cast<const uint16_t*>(c.k) + row * D + d0;
  float kx[DPT], ss = 0.f, dot = 0.f;
#pragma unroll
  for (int x = 0; x < DPT; ++x) {
    kx[x] = bf16_to_f32(kp[x]);
    ss += kx[x] * kx[x];
    dot += kx[x] * sk[x];
  }
  ss += __shfl_xor(ss, 1, kWave);
  ss += __shfl_xor(ss, 2, kWave);
  dot += __shfl_xor(dot, 1, kWave);
  dot += __shfl_xor(dot, 2, kWave);
  // dkhat -> dk: (dkh - khat (khat . dkh)) / |k|, or dkh / eps below eps
  const float n = sqrtf(ss);
  float* dko = a.dk + row * D + d0;
  float* dvo = a.dv + row * D + d0;
#pragma unroll
  for (int x = 0; x < DPT; ++x) {
    float g = sk[x];
    if (c.qk_norm) g = n > 1e-6f ? (sk[x] - kx[x] * (dot / (n * n))) / n : sk[x] * 1e6f;
    dko[x] = g;
    dvo[x] = sv[x];
  }
}

// --- per row: dq_attn, ds, dq_ret ---------------------------------------------
// One wave per (row, kv head); lane k < K holds slot k.
template <int D, int G>
__global__ __launch_bounds__(64) void bwd_row_kernel(BwdArgs a) {
  const ChunkArgs& c = a.c;
  const int64_t row = blockIdx.x;            // (b*Lq + r)*Hkv + g
  const int lane = threadIdx.x, K = c.K;
  const int g = (int)(row % c.Hkv);
  const int64_t br = row / c.Hkv;
  const int32_t ci = lane < K ? c.idx[row * K + lane] : -1;
  const bool valid = ci >= 0 && (int64_t)ci < c.Nc;
  const float wk = valid ? c.wts[row * K + lane] : 0.f;
  const float wdw = valid ? a.wdw[row * K + lane] : 0.f;
  const float swdw = wave_sum(wdw);
  const float dr = valid ? a.ret_scale * (wdw - wk * swdw) : 0.f;   // ret_scale * ds_k
  if (lane < K) a.draw[row * K + lane] = dr;
  const uint64_t vmask = __ballot(valid);
  // dq_ret = sum_k dr_k landmark[c_k] (slot order); lanes split the dims
  const uint16_t* lmb = reinterpret_cast<const uint16_t*>(a.landmarks) + ((br / c.Lq) * c.Hkv + g) * c.Nc * D;
  float* dqr = a.dq_ret + row * D;
  for (int x = lane; x < D; x += 64) {
    float acc = 0.f;
    for (int k = 0; k < K; ++k) {
      if (!((vmask >> k) & 1ull)) continue;
      const int32_t ck = __shfl(ci, k, kWave);
      const float drk = __shfl(dr, k, kWave);
      acc += drk * bf16_to_f32(lmb[(int64_t)ck * D + x]);
    }
    dqr[x] = acc;
  }
  // dq_attn per head: normalisation's gradient of sum_k dqhat_k (slot order)
  for (int hd = 0; hd < G; ++hd) {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(c.q_attn) + (br * c.Hq + (int64_t)g * G + hd) * D;
    float dqh[D / 64 > 0 ? D / 64 : 1], qv[D / 64 > 0 ? D / 64 : 1];
    float ss = 0.f, dot = 0.f;
#pragma unroll
    for (int u = 0; u < D / 64; ++u) {
      const int x = lane + 64 * u;
      float acc = 0.f;
      for (int k = 0; k < K; ++k)
        if ((vmask >> k) & 1ull) acc += a.dq_part[((row * K + k) * G + hd) * D + x];
      dqh[u] = acc;
      qv[u] = bf16_to_f32(qp[x]);
      ss += qv[u] * qv[u];
      dot += qv[u] * acc;
    }
    ss = wave_sum(ss);
    dot = wave_sum(dot);
    const float n = sqrtf(ss);
    float* dqo = a.dq_attn + (br * c.Hq + (int64_t)g * G + hd) * D;
#pragma unroll
    for (int u = 0; u < D / 64; ++u) {
      float gq = dqh[u];
      if (c.qk_norm) gq = n > 1e-6f ? (dqh[u] - qv[u] * (dot / (n * n))) / n : dqh[u] * 1e6f;
      dqo[lane + 64 * u] = vmask ? gq : 0.f;
    }
  }
}

// --- per chunk: dlandmark -------------------------------------------------------
template <int D>
__global__ __launch_bounds__(D) void bwd_landmark_kernel(BwdArgs a) {
  const ChunkArgs& c = a.c;
  const int64_t bg = blockIdx.x / c.Nc, chunk = blockIdx.x % c.Nc;
  const int x = threadIdx.x;
  const uint16_t* qr = reinterpret_cast<const uint16_t*>(a.q_ret) + x;
  float acc = 0.f;
  for (int64_t band = 0; band < c.n_bands; ++band) {
    const int64_t bin = (bg * c.n_bands + band) * c.Nc + chunk;
    const uint32_t p0 = c.offsets[bin], p1 = c.offsets[bin + 1];
    for (uint32_t p = p0; p < p1; p += 8) {   // 8 pairs in flight, summed in pair order
      uint32_t pid[8];
      float dr[8], qv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) pid[u] = c.pairs[min(p + u, p1 - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        dr[u] = a.draw[pid[u]];
        qv[u] = bf16_to_f32(qr[(int64_t)(pid[u] / (uint32_t)c.K) * D]);   // row (b*Lq + r)*Hkv + g
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (p + u < p1) acc += dr[u] * qv[u];
    }
  }
  a.dlandmarks[(bg * c.Nc + chunk) * D + x] = acc;
}

}  // namespace

int64_t bwd_pairs_per_item() { return kBP; }

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
  hipLaunchKernelGGL((bwd_row_kernel<D, G>), dim3((unsigned)a.c.rows), dim3(64), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_chunk_kernel<D>), dim3((unsigned)(n_bg * (a.c.Nc + 1))), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.c.Nc > 0) {
    hipLaunchKernelGGL((bwd_landmark_kernel<D>), dim3((unsigned)(n_bg * a.c.Nc)), dim3(D), 0, st, a);
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
