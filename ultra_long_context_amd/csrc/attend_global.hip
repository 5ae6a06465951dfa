// attend_global.hip -- HSA with a top-K that covers every eligible chunk (the
// "global HSA" of the warm-up stage in "Every Token Counts", agent-atlas
// explainer, "Build Your Own" step 5: a large top-K covering the whole
// sequence), bf16, G = 8 or 16 query heads per kv head.
//
// With every eligible chunk selected, Steps 2-4 reduce to: for each chunk c
// before the query's own chunk, the in-chunk attention output O_c (Step 3)
// weighted by softmax_c(s_c) over all of them (Step 4).  No top-K is needed;
// the blend runs as an online softmax over the chunks:
//   m' = max(m, s_c),  l' = l 2^(m-m') + 2^(s_c-m'),  acc' = acc 2^(m-m') + 2^(s_c-m') O_c,
// out = acc / l (scores in base 2).  A workgroup of 16 waves owns 256/G
// consecutive query rows of one (batch, kv head) (16 head-rows per wave) and
// streams their eligible chunks: each chunk's K and V (row-major) are staged in
// LDS once for all 256 head-rows, double-buffered so the next chunk's loads are
// in flight during the current one; S^T = K Q^T and O^T += V^T P^T run on
// v_mfma_f32_16x16x32_bf16, V^T read with LDS transpose loads, with P (times
// the chunk's blend factor, over the in-chunk sum, rounded to bf16) fed from
// registers.  Retrieval scores of the block's rows come 64 chunks at a
// time from the same MFMA, landmarks as the A operand.
#include "hsa_device.h"
#include "hsa_internal.h"

namespace hsa {
namespace {

constexpr int kGWaves = 16;
constexpr int kGThreads = kGWaves * 64;
constexpr int kGTile = 64;                     // landmarks (chunks) per score tile
constexpr float kLog2eG = 1.4426950408889634f;

template <int D, int G>
__global__ __launch_bounds__(kGThreads) void attend_global_kernel(GlobalArgs a) {
  constexpr int R = 256 / G;                   // query rows per workgroup
  constexpr int KROW = D + 16, VROW = D + 16, LROW = D + 16;   // 288-byte rows: no LDS bank conflicts
  constexpr int KSTEP = D / 32, NT = D / 16;
  constexpr int TPR = 16 / G;                  // rows per 16-head-row tile (G = 8: 2, G = 16: 1)
  __shared__ __align__(16) uint16_t ks[2][kChunk * KROW];
  __shared__ __align__(16) uint16_t vs[2][kChunk * VROW];   // V rows, read back transposed
  __shared__ float rk[2][kChunk];
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

  // this wave's 16 head-rows: rows r0 + TPR*w + ma/G, heads g*G + ma%G
  const int rloc = TPR * w + ma / G;
  const int64_t row = r0 + rloc;
  const bool row_ok = row < a.Lq;
  const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k) + bg * a.Lkv * D;
  const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.v) + bg * a.Lkv * D;
  bf16x8 qa[KSTEP];
  float qss = 0.f;
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q_attn) +
                         (((int64_t)b * a.Lq + (row_ok ? row : 0)) * a.Hq + (int64_t)g * G + ma % G) * D + 8 * jg;
#pragma unroll
    for (int t = 0; t < KSTEP; ++t) {
      uint4 x = *reinterpret_cast<const uint4*>(qp + 32 * t);
      if (!row_ok) x = make_uint4(0, 0, 0, 0);
      qa[t] = __builtin_bit_cast(bf16x8, x);
      const uint32_t wd[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x2 v2 = __builtin_bit_cast(bf16x2, wd[q]);
        qss = __builtin_amdgcn_fdot2_f32_bf16(v2, v2, qss, false);
      }
    }
  }
  qss += __shfl_xor(qss, 16, kWave);
  qss += __shfl_xor(qss, 32, kWave);
  const float rq = (a.qk_norm ? 1.0f / fmaxf(sqrtf(qss), 1e-6f) : 1.0f) * a.attn_scale * kLog2eG;

  // K / V staging: each thread one 16-byte piece of K and one of V (8 dims of
  // one key), both row-major; the P.V operand is read from V with LDS
  // transpose loads in the key order of the S^T accumulators, so P^T feeds
  // P.V from registers
  constexpr int NKP = kChunk * D / 8;          // 16-byte pieces per chunk
  uint4 kx = make_uint4(0, 0, 0, 0), vx = make_uint4(0, 0, 0, 0);
  auto load_kv = [&](int c) {
    if (tid < NKP) {
      kx = *reinterpret_cast<const uint4*>(kbase + (int64_t)c * kChunk * D + tid * 8);
      vx = *reinterpret_cast<const uint4*>(vbase + (int64_t)c * kChunk * D + tid * 8);
    }
  };
  auto store_kv = [&](int bi) {
    if (tid < NKP) {
      const int key = tid * 8 / D, d0 = (tid * 8) % D;
      *reinterpret_cast<uint4*>(&ks[bi][key * KROW + d0]) = kx;
      // key norm: the D/8 consecutive lanes holding this key add their squares
      float ss = 0.f;
      {
        const uint32_t kw[4] = {kx.x, kx.y, kx.z, kx.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bf16x2 v2 = __builtin_bit_cast(bf16x2, kw[q]);
          ss = __builtin_amdgcn_fdot2_f32_bf16(v2, v2, ss, false);
        }
      }
      ss += dpp_f<0xB1>(ss);               // xor 1
      ss += dpp_f<0x4E>(ss);               // xor 2
      ss += dpp_f<0x141>(ss);              // half-row mirror: 8 lanes
      if constexpr (D == 128) ss += dpp_f<0x140>(ss);   // row mirror: 16 lanes
      if (d0 == 0) rk[bi][key] = a.qk_norm ? 1.0f / fmaxf(sqrtf(ss), 1e-6f) : 1.0f;
      *reinterpret_cast<uint4*>(&vs[bi][key * VROW + d0]) = vx;
    }
  };
  floatx4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;                // online blend state of this lane's row

  if (c_stop > 0) {
    load_kv(0);
    store_kv(0);
  }
  __syncthreads();
  const uint16_t* lmb = reinterpret_cast<const uint16_t*>(a.landmarks) + bg * a.Nc * D;
  for (int c = 0; c < c_stop; ++c) {
    const int cb = c & 1;
    if (c % kGTile == 0) {                     // retrieval scores of the next 64 chunks
      {
        const int qi = tid, cl = qi / (D / 8), u = qi % (D / 8);
        if (qi < kGTile * D / 8) {
          const int cc = c + cl < c_stop ? c + cl : c;
          *reinterpret_cast<uint4*>(&lt[cl * LROW + u * 8]) =
              *reinterpret_cast<const uint4*>(lmb + (int64_t)cc * D + u * 8);
        }
      }
      __syncthreads();
      if (w < (R / 16) * 4) {                  // wave: 16 rows x 16 chunks
        const int rt = w >> 2, ct = w & 3;
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
    floatx4 s4[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      s4[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < KSTEP; ++t) {
        const uint4 kb = *reinterpret_cast<const uint4*>(&ks[cb][(16 * nt + ma) * KROW + 32 * t + 8 * jg]);
        s4[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb), qa[t], s4[nt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    float mx = -INFINITY;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const float4 r4 = *reinterpret_cast<const float4*>(&rk[cb][16 * nt + 4 * jg]);
      const float rr[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s4[nt][i] = s4[nt][i] * rq * rr[i];
        mx = fmaxf(mx, s4[nt][i]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    float sum = 0.f;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s4[nt][i] = __builtin_amdgcn_exp2f(s4[nt][i] - mx);
        sum += s4[nt][i];
      }
    sum += __shfl_xor(sum, 16, kWave);
    sum += __shfl_xor(sum, 32, kWave);
    // --- online blend over chunks (Step 4) -----------------------------------
    const float sr = sc[rloc][c % kGTile];
    float f = 0.f;                             // this chunk's factor on O_c
    float al = 1.0f;                           // rescale of the running sum
    if (sr != -INFINITY) {
      const float mn = fmaxf(m, sr);
      al = __builtin_amdgcn_exp2f(m - mn);     // m = -inf first: 0
      f = __builtin_amdgcn_exp2f(sr - mn);
      l = l * al + f;
      m = mn;
    }
    if (__any(al != 1.0f)) {                   // the running maximum rose for some row
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[nt][i] *= al;
    }
    const float scale = f * __builtin_amdgcn_rcpf(sum);
    bf16x8 pb[2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[st][e] = (__bf16)(s4[2 * st + (e >> 2)][e & 3] * scale);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        // A = V^T: dims 16nt.., keys 32st + 4jg + 0..3 and 32st + 16 + 4jg + 0..3
        const bf16x8 va = lds_operand_tr2(vs[cb], VROW, 32 * st + 4 * jg, 32 * st + 16 + 4 * jg, 16 * nt, ma);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[st], acc[nt], 0, 0, 0);
      }
      if (nt % 4 == 3) __builtin_amdgcn_sched_barrier(0);   // bound the V^T operands in flight
    }
    if (c + 1 < c_stop) store_kv(cb ^ 1);
    __syncthreads();
  }
  // --- out = acc / l; lane holds dims 16*nt + 4*jg + i of head-row ma --------
  if (!row_ok) return;
  const float inv = l > 0.f ? 1.0f / l : 0.f;  // no eligible chunk: 0
  uint16_t* op = reinterpret_cast<uint16_t*>(a.out) +
                 (((int64_t)b * a.Lq + row) * a.Hq + (int64_t)g * G + ma % G) * D + 4 * jg;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const uint32_t lo = (uint32_t)f32_to_bf16(acc[nt][0] * inv) | ((uint32_t)f32_to_bf16(acc[nt][1] * inv) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(acc[nt][2] * inv) | ((uint32_t)f32_to_bf16(acc[nt][3] * inv) << 16);
    *reinterpret_cast<uint2*>(op + 16 * nt) = make_uint2(lo, hi);
  }
}

}  // namespace

int global_rows_per_block(int G) { return 256 / G; }

hipError_t launch_attend_global(const GlobalArgs& a, int64_t B, int D, int G, hipStream_t st) {
  const int64_t R = 256 / G;
  const int64_t blocks = (a.Lq + R - 1) / R * B * a.Hkv;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(kGThreads);
#define HSA_GLOBAL_CASE(DD, GG)                                                  \
  if (D == DD && G == GG) {                                                      \
    hipLaunchKernelGGL((attend_global_kernel<DD, GG>), grid, block, 0, st, a);   \
    return hipGetLastError();                                                    \
  }
  HSA_GLOBAL_CASE(128, 8) HSA_GLOBAL_CASE(128, 16) HSA_GLOBAL_CASE(64, 8) HSA_GLOBAL_CASE(64, 16)
#undef HSA_GLOBAL_CASE
  return hipErrorInvalidValue;
}

}  // namespace hsa
