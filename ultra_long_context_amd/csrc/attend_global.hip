// attend_global.hip -- HSA with a top-K that covers every eligible chunk (the
// "global HSA" of the warm-up stage in "Every Token Counts", agent-atlas
// explainer, "Build Your Own" step 5, where the top-K spans every eligible
// chunk), bf16, G = 1, 2, 4, 8 or 16 query heads per kv head.
//
// With every eligible chunk selected, Steps 2-4 reduce to: for each chunk c
// before the query's own chunk, the in-chunk attention output O_c (Step 3)
// weighted by softmax_c(s_c) over all of them (Step 4).  No top-K is needed;
// the blend runs as an online softmax over the chunks:
//   m' = max(m, s_c),  l' = l 2^(m-m') + 2^(s_c-m'),  acc' = acc 2^(m-m') + 2^(s_c-m') O_c,
// out = acc / l (scores in base 2).  A workgroup owns 256/G consecutive query
// rows of one (batch, kv head), 256 head-rows in tiles of 16 (16/G rows of G
// heads), one tile per wave over 16 waves or two per wave over 8 (TW below),
// and streams their eligible chunks: each chunk's K (normalised once per call by
// key_norm_kernel when query-key normalisation is on) and V (row-major) are
// staged in LDS once for all 256 head-rows, double-buffered so the next chunk's loads are
// in flight during the current one; S^T = K Q^T and O^T += V^T P^T run on
// v_mfma_f32_16x16x32_bf16, V^T read with LDS transpose loads, with P (times
// the chunk's blend factor, over the in-chunk sum, rounded to bf16) fed from
// registers.  Retrieval scores of the block's rows come 64 chunks at a
// time (32 when G <= 2, the block then holding 128 or 256 rows) from the same
// MFMA, landmarks as the A operand, 16 rows x 16 chunks per wave task.
#include "hsa_device.h"
#include "hsa_internal.h"

namespace hsa {
namespace {

constexpr float kLog2eG = 1.4426950408889634f;

// Normalised keys khat = k / max(|k|, 1e-6) (bf16) of the complete chunks,
// written once per call for every workgroup of the global kernel to stage
// (each would otherwise normalise every chunk again).  Thread t takes 16-byte
// piece t (8 dims of one key; a key's D/8 pieces sit in consecutive lanes of
// one DPP row): the same lane layout and reduction order as a staging pass,
// so the rounded keys do not depend on which kernel normalised them.
template <int D>
__global__ __launch_bounds__(256) void key_norm_kernel(GlobalArgs a, int64_t n_pieces) {
  constexpr int PPK = D / 8;                                 // pieces per key
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t tc = t < n_pieces ? t : 0;
  const int64_t per_bg = a.Nc * kChunk * PPK;                // pieces per (batch, kv head)
  const int64_t bg = tc / per_bg, pc = tc % per_bg;
  const uint4 x = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.k) +
                                                  bg * a.Lkv * D + pc * 8);
  float ss = 0.f;
  const uint32_t kw[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bf16x2 v2 = __builtin_bit_cast(bf16x2, kw[q]);
    ss = __builtin_amdgcn_fdot2_f32_bf16(v2, v2, ss, false);
  }
  ss += dpp_f<0xB1>(ss);           // xor 1
  ss += dpp_f<0x4E>(ss);           // xor 2
  ss += dpp_f<0x141>(ss);          // half-row mirror: 8 lanes
  if constexpr (D == 128) ss += dpp_f<0x140>(ss);   // row mirror: 16 lanes
  const float rk = 1.0f / fmaxf(sqrtf(ss), 1e-6f);
  bf16x8 kb = __builtin_bit_cast(bf16x8, x);
#pragma unroll
  for (int e = 0; e < 8; ++e) kb[e] = (__bf16)((float)kb[e] * rk);
  if (t < n_pieces)
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.k_hat) + bg * per_bg * 8 + pc * 8) =
        __builtin_bit_cast(uint4, kb);
}

// TW: 16-head-row tiles per wave.  The workgroup always holds 256 head-rows
// (16 / TW waves); with TW = 2 every K and V^T operand read from LDS feeds two
// MFMAs, halving the LDS operand traffic per chunk, but leaves two waves per
// SIMD instead of four.  Measured on the 32K window (G = 8), with the row
// reductions on the row-swap permutes: TW = 2 1.3-1.5 % faster than TW = 1 in
// three interleaved rounds (2.35-2.38 against 2.39-2.41 ms per call); with the
// LDS-shuffle reductions they were equal at d = 128, and at d = 64 TW = 2 ran
// 0.44 against 0.40 ms.  So d = 128 launches TW = 2, d = 64 TW = 1.
template <int D, int G, int TW>
__global__ __launch_bounds__(64 * 16 / TW) void attend_global_kernel(GlobalArgs a) {
  constexpr int NW = 16 / TW;                  // waves per workgroup
  constexpr int NTHR = 64 * NW;
  constexpr int R = 256 / G;                   // query rows per workgroup
  // landmarks (chunks) per score tile: the scores of R rows x kGTile chunks sit in LDS
  constexpr int kGTile = G <= 2 ? 32 : 64;
  constexpr int kScoreTasks = (R / 16) * (kGTile / 16);   // 16 rows x 16 chunks each
  constexpr int KROW = D + 16, VROW = D + 16, LROW = D + 16;   // 288-byte rows: no LDS bank conflicts
  constexpr int KSTEP = D / 32, NT = D / 16;
  constexpr int TPR = 16 / G;                  // rows per 16-head-row tile (G = 8: 2, G = 16: 1)
  constexpr int NKP = kChunk * D / 8;          // 16-byte pieces of K (and of V) per chunk
  constexpr int PPT = (NKP + NTHR - 1) / NTHR; // pieces staged per thread
  __shared__ __align__(16) uint16_t ks[2][kChunk * KROW];
  __shared__ __align__(16) uint16_t vs[2][kChunk * VROW];   // V rows, read back transposed
  __shared__ __align__(16) uint16_t lt[kGTile * LROW];
  __shared__ float sc[R][kGTile + 1];          // base-2 retrieval scores, -inf past the row's chunks

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int ma = lane & 15, jg = lane >> 4;
  // latest (longest) row blocks first, the (batch, kv head) pairs interleaved
  const int64_t rbk = (a.Lq + R - 1) / R;
  const int64_t nbg = (int64_t)gridDim.x / rbk;
  const int64_t bg = (int64_t)blockIdx.x % nbg;
  const int64_t r0 = (rbk - 1 - (int64_t)blockIdx.x / nbg) * R;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  auto n_of = [&](int64_t r) -> int {          // eligible chunks of query row r
    if (r >= a.Lq) return 0;
    const int64_t n = (a.q_pos0 + r) / kChunk;
    return (int)(n < a.Nc ? n : a.Nc);
  };
  const int c_stop = n_of(min(r0 + R - 1, a.Lq - 1));

  // tile u of this wave: 16 head-rows, rows r0 + TPR*(TW*w + u) + ma/G, heads g*G + ma%G;
  // the query factor (normalisation, attention scale, log2 e) is folded into
  // the query operand once: S comes out of the MFMA as base-2 logits
  int rloc[TW];
  bool row_ok[TW];
  bf16x8 qa[TW][KSTEP];
#pragma unroll
  for (int u = 0; u < TW; ++u) {
    rloc[u] = TPR * (TW * w + u) + ma / G;
    const int64_t row = r0 + rloc[u];
    row_ok[u] = row < a.Lq;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q_attn) +
                         (((int64_t)b * a.Lq + (row_ok[u] ? row : 0)) * a.Hq + (int64_t)g * G + ma % G) * D + 8 * jg;
    float qss = 0.f;
#pragma unroll
    for (int t = 0; t < KSTEP; ++t) {
      uint4 x = *reinterpret_cast<const uint4*>(qp + 32 * t);
      if (!row_ok[u]) x = make_uint4(0, 0, 0, 0);
      qa[u][t] = __builtin_bit_cast(bf16x8, x);
      const uint32_t wd[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x2 v2 = __builtin_bit_cast(bf16x2, wd[q]);
        qss = __builtin_amdgcn_fdot2_f32_bf16(v2, v2, qss, false);
      }
    }
    qss = xrow_sum(qss);
    const float rq = (a.qk_norm ? 1.0f / fmaxf(sqrtf(qss), 1e-6f) : 1.0f) * a.attn_scale * kLog2eG;
#pragma unroll
    for (int t = 0; t < KSTEP; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) qa[u][t][e] = (__bf16)((float)qa[u][t][e] * rq);
  }
  // With query-key normalisation every logit is at most attn_scale * log2 e in
  // magnitude, so exp2 cannot overflow without subtracting the maximum (the
  // softmax is shift-invariant); otherwise the in-chunk maximum is subtracted.
  const bool bounded = a.qk_norm && a.attn_scale * kLog2eG <= 64.0f;

  // keys as staged: the normalised copy (with query-key normalisation) or K itself
  const uint16_t* kbase = a.qk_norm ? reinterpret_cast<const uint16_t*>(a.k_hat) + bg * a.Nc * kChunk * D
                                    : reinterpret_cast<const uint16_t*>(a.k) + bg * a.Lkv * D;
  const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.v) + bg * a.Lkv * D;
  // K / V staging: thread tid takes pieces tid + NTHR*i (8 dims of one key),
  // both row-major; the P.V operand is read from V with LDS transpose loads in
  // the key order of the S^T accumulators, so P^T feeds P.V from registers
  uint4 kx[PPT], vx[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i) kx[i] = vx[i] = make_uint4(0, 0, 0, 0);
  auto load_kv = [&](int c) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int pc = tid + NTHR * i;
      if (pc < NKP) {
        kx[i] = *reinterpret_cast<const uint4*>(kbase + (int64_t)c * kChunk * D + pc * 8);
        vx[i] = *reinterpret_cast<const uint4*>(vbase + (int64_t)c * kChunk * D + pc * 8);
      }
    }
  };
  auto store_kv = [&](int bi) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int pc = tid + NTHR * i;
      if (pc < NKP) {
        const int key = pc * 8 / D, d0 = (pc * 8) % D;
        *reinterpret_cast<uint4*>(&ks[bi][key * KROW + d0]) = kx[i];
        *reinterpret_cast<uint4*>(&vs[bi][key * VROW + d0]) = vx[i];
      }
    }
  };
  floatx4 acc[TW][NT];
  float m[TW], l[TW];                          // online blend state of each tile's row
#pragma unroll
  for (int u = 0; u < TW; ++u) {
    m[u] = -INFINITY;
    l[u] = 0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[u][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  if (c_stop > 0) {
    load_kv(0);
    store_kv(0);
  }
  __syncthreads();
  const uint16_t* lmb = reinterpret_cast<const uint16_t*>(a.landmarks) + bg * a.Nc * D;
  for (int c = 0; c < c_stop; ++c) {
    const int cb = c & 1;
    if (c % kGTile == 0) {                     // retrieval scores of the next kGTile chunks
      for (int qi = tid; qi < kGTile * D / 8; qi += NTHR) {
        const int cl = qi / (D / 8), u = qi % (D / 8);
        const int cc = c + cl < c_stop ? c + cl : c;
        *reinterpret_cast<uint4*>(&lt[cl * LROW + u * 8]) =
            *reinterpret_cast<const uint4*>(lmb + (int64_t)cc * D + u * 8);
      }
      __syncthreads();
      for (int task = w; task < kScoreTasks; task += NW) {   // 16 rows x 16 chunks
        const int rt = task / (kGTile / 16), ct = task % (kGTile / 16);
        const int64_t qr = r0 + 16 * rt + ma;
        const bool ok = qr < a.Lq;
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q_ret) +
                             (((int64_t)b * a.Lq + (ok ? qr : 0)) * a.Hkv + g) * D + 8 * jg;
        floatx4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < KSTEP; ++t) {
          uint4 x = *reinterpret_cast<const uint4*>(qp + 32 * t);
          if (!ok) x = make_uint4(0, 0, 0, 0);
          const uint4 lx = *reinterpret_cast<const uint4*>(&lt[(16 * ct + ma) * LROW + 32 * t + 8 * jg]);
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, lx), __builtin_bit_cast(bf16x8, x),
                                                      s, 0, 0, 0);
        }
        // lane holds chunks 16*ct + 4*jg + i of row 16*rt + ma
        const int nq = n_of(qr);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int cl = 16 * ct + 4 * jg + i;
          sc[16 * rt + ma][cl] = c + cl < nq ? s[i] * (a.ret_scale * kLog2eG) : -INFINITY;
        }
      }
      __syncthreads();
    }
    if (c + 1 < c_stop) load_kv(c + 1);       // next chunk in flight during this one
    // --- S^T = K Q^T: lane holds keys 16*nt + 4*jg + i of head-row ma ---------
    floatx4 s4[TW][4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
      for (int u = 0; u < TW; ++u) s4[u][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < KSTEP; ++t) {
        const uint4 kb = *reinterpret_cast<const uint4*>(&ks[cb][(16 * nt + ma) * KROW + 32 * t + 8 * jg]);
#pragma unroll
        for (int u = 0; u < TW; ++u)
          s4[u][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb), qa[u][t], s4[u][nt],
                                                              0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 pb[TW][2];
    float al[TW];
#pragma unroll
    for (int u = 0; u < TW; ++u) {
      if (bounded) {                           // uniform branch: no maximum to subtract
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) s4[u][nt][i] = __builtin_amdgcn_exp2f(s4[u][nt][i]);
      } else {
        float mx = -INFINITY;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s4[u][nt][i]);
        mx = xrow_max(mx);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) s4[u][nt][i] = __builtin_amdgcn_exp2f(s4[u][nt][i] - mx);
      }
      float sum = 0.f;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sum += s4[u][nt][i];
      sum = xrow_sum(sum);
      // --- online blend over chunks (Step 4) ---------------------------------
      const float sr = sc[rloc[u]][c % kGTile];
      float f = 0.f;                           // this chunk's factor on O_c
      al[u] = 1.0f;                            // rescale of the running sum
      if (sr != -INFINITY) {
        const float mn = fmaxf(m[u], sr);
        al[u] = __builtin_amdgcn_exp2f(m[u] - mn);   // m = -inf first: 0
        f = __builtin_amdgcn_exp2f(sr - mn);
        l[u] = l[u] * al[u] + f;
        m[u] = mn;
      }
      const float scale = f * __builtin_amdgcn_rcpf(sum);
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[u][st][e] = (__bf16)(s4[u][2 * st + (e >> 2)][e & 3] * scale);
    }
#pragma unroll
    for (int u = 0; u < TW; ++u) {
      if (__any(al[u] != 1.0f)) {              // the running maximum rose for some row
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[u][nt][i] *= al[u];
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        // A = V^T: dims 16nt.., keys 32st + 4jg + 0..3 and 32st + 16 + 4jg + 0..3
        const bf16x8 va = lds_operand_tr2(vs[cb], VROW, 32 * st + 4 * jg, 32 * st + 16 + 4 * jg, 16 * nt, ma);
#pragma unroll
        for (int u = 0; u < TW; ++u)
          acc[u][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[u][st], acc[u][nt], 0, 0, 0);
      }
      if (nt % 4 == 3) __builtin_amdgcn_sched_barrier(0);   // bound the V^T operands in flight
    }
    if (c + 1 < c_stop) store_kv(cb ^ 1);
    __syncthreads();
  }
  // --- out = acc / l; lane holds dims 16*nt + 4*jg + i of head-row ma --------
#pragma unroll
  for (int u = 0; u < TW; ++u) {
    if (!row_ok[u]) continue;
    const int64_t row = r0 + rloc[u];
    const float inv = l[u] > 0.f ? 1.0f / l[u] : 0.f;   // no eligible chunk: 0
    uint16_t* op = reinterpret_cast<uint16_t*>(a.out) +
                   (((int64_t)b * a.Lq + row) * a.Hq + (int64_t)g * G + ma % G) * D + 4 * jg;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint32_t lo =
          (uint32_t)f32_to_bf16(acc[u][nt][0] * inv) | ((uint32_t)f32_to_bf16(acc[u][nt][1] * inv) << 16);
      const uint32_t hi =
          (uint32_t)f32_to_bf16(acc[u][nt][2] * inv) | ((uint32_t)f32_to_bf16(acc[u][nt][3] * inv) << 16);
      *reinterpret_cast<uint2*>(op + 16 * nt) = make_uint2(lo, hi);
    }
  }
}

}  // namespace

int global_rows_per_block(int G) { return 256 / G; }

// Tiles per wave (measured: see the kernel's comment).
template <int D> constexpr int global_tw() { return D == 128 ? 2 : 1; }

hipError_t launch_attend_global(const GlobalArgs& a, int64_t B, int D, int G, hipStream_t st) {
  const int64_t R = 256 / G;
  const int64_t blocks = (a.Lq + R - 1) / R * B * a.Hkv;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (a.qk_norm && a.Nc > 0) {
    if (a.k_hat == nullptr) return hipErrorInvalidValue;
    const int64_t n_pieces = B * a.Hkv * a.Nc * kChunk * (D / 8);
    const int64_t nb = (n_pieces + 255) / 256;
    if (nb > INT32_MAX) return hipErrorInvalidValue;
    if (D == 128) hipLaunchKernelGGL(key_norm_kernel<128>, dim3((unsigned)nb), dim3(256), 0, st, a, n_pieces);
    else hipLaunchKernelGGL(key_norm_kernel<64>, dim3((unsigned)nb), dim3(256), 0, st, a, n_pieces);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
#define HSA_GLOBAL_CASE(DD, GG)                                                                  \
  if (D == DD && G == GG) {                                                                      \
    constexpr int TW = global_tw<DD>();                                                          \
    hipLaunchKernelGGL((attend_global_kernel<DD, GG, TW>), dim3((unsigned)blocks), dim3(64 * 16 / TW), 0, st, a); \
    return hipGetLastError();                                                                    \
  }
  HSA_GLOBAL_CASE(128, 1) HSA_GLOBAL_CASE(128, 2) HSA_GLOBAL_CASE(128, 4) HSA_GLOBAL_CASE(128, 8)
  HSA_GLOBAL_CASE(128, 16) HSA_GLOBAL_CASE(64, 1) HSA_GLOBAL_CASE(64, 2) HSA_GLOBAL_CASE(64, 4)
  HSA_GLOBAL_CASE(64, 8) HSA_GLOBAL_CASE(64, 16)
#undef HSA_GLOBAL_CASE
  return hipErrorInvalidValue;
}

}  // namespace hsa
