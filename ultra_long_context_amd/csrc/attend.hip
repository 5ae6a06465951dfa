// attend.hip -- per-chunk attention and retrieval-weighted blend (Steps 3-4 of
// the HSA step in "Every Token Counts", agent-atlas explainer, "How It Works
// (Technically)").
//
// General path: one wave per (query row, kv head) and slot range.  Lane t owns
// key t of the selected chunk (one lane per token of a 64-token chunk), so the
// key norms, logits and the in-chunk softmax of all G q heads of the group are
// lane-parallel; P (already multiplied by the blend weight w_k) goes through LDS
// and P.V is computed with lane = output dimension.  The blend is folded into
// the accumulation: out = sum_k (w_k * P_k) V_k.
//
// (Few rows use attend_slot_kernel below instead.)
#include "hsa_device.h"
#include "hsa_internal.h"

namespace hsa {
namespace {

template <bool BF16, int N>
__device__ __forceinline__ void load_vec(const typename Elem<BF16>::T* p, float* out);

template <>
__device__ __forceinline__ void load_vec<true, 8>(const uint16_t* p, float* out) {
  const uint4 x = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

template <>
__device__ __forceinline__ void load_vec<false, 8>(const float* p, float* out) {
  const float4 x = *reinterpret_cast<const float4*>(p);
  const float4 y = *reinterpret_cast<const float4*>(p + 4);
  out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
  out[4] = y.x; out[5] = y.y; out[6] = y.z; out[7] = y.w;
}

template <bool BF16, int D, int G>
__global__ __launch_bounds__(64) void attend_blend_kernel(AttendArgs a) {
  using E = Elem<BF16>;
  using T = typename E::T;
  constexpr int XD = D / kWave;                 // output dims per lane
  __shared__ float qs[G][D];
  __shared__ float ps[kChunk][G];

  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;               // (b*Lq + r)*Hkv + g
  const int g = (int)(row % a.Hkv);
  const int64_t br = row / a.Hkv;               // b*Lq + r
  const int64_t b = br / a.Lq;
  const int K = a.K;

  // Step 4 weights: lane k holds slot k
  const int32_t my_idx = lane < K ? a.idx[row * K + lane] : -1;
  const float my_s = lane < K ? a.score[row * K + lane] : 0.f;
  const bool valid = my_idx >= 0 && (int64_t)my_idx < a.Nc;
  const float mx = wave_max(valid ? my_s : -INFINITY);
  const float ex = valid ? expf(my_s - mx) : 0.f;
  const float den = wave_sum(ex);
  const float w = valid ? ex / den : 0.f;

  // attention queries of the group's G heads
  const T* qp = reinterpret_cast<const T*>(a.q_attn) + (br * a.Hq + (int64_t)g * G) * D;
  for (int i = lane; i < G * D; i += kWave) qs[i / D][i % D] = E::load(qp + i);
  __syncthreads();
  float rq[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float ss = 0.f;
#pragma unroll
    for (int xi = 0; xi < XD; ++xi) {
      const float x = qs[h][lane + kWave * xi];
      ss += x * x;
    }
    ss = wave_sum(ss);
    rq[h] = a.qk_norm ? 1.0f / fmaxf(sqrtf(ss), 1e-6f) : 1.0f;
  }

  float acc[G][XD];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int xi = 0; xi < XD; ++xi) acc[h][xi] = 0.f;

  const int k_lo = 0, k_hi = K;
  const T* kbase = reinterpret_cast<const T*>(a.k) + (b * a.Hkv + g) * a.Lkv * D;
  const T* vbase = reinterpret_cast<const T*>(a.v) + (b * a.Hkv + g) * a.Lkv * D;
  for (int k = k_lo; k < k_hi; ++k) {
    const int c = __shfl(my_idx, k, kWave);
    const float wk = __shfl(w, k, kWave);
    if (c < 0 || (int64_t)c >= a.Nc) continue;
    // logits of key `lane` for every head of the group
    const T* kr = kbase + ((int64_t)c * kChunk + lane) * D;
    float dot[G];
#pragma unroll
    for (int h = 0; h < G; ++h) dot[h] = 0.f;
    float ss = 0.f;
#pragma unroll 1
    for (int x0 = 0; x0 < D; x0 += 8) {
      float kv[8];
      load_vec<BF16, 8>(kr + x0, kv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ss += kv[e] * kv[e];
#pragma unroll
        for (int h = 0; h < G; ++h) dot[h] += qs[h][x0 + e] * kv[e];
      }
    }
    const float rk = a.qk_norm ? 1.0f / fmaxf(sqrtf(ss), 1e-6f) : 1.0f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float logit = dot[h] * rq[h] * rk * a.attn_scale;
      const float m = wave_max(logit);
      const float p = expf(logit - m);
      const float sp = wave_sum(p);
      ps[lane][h] = p / sp * wk;
    }
    __syncthreads();
    const T* vr = vbase + (int64_t)c * kChunk * D;
#pragma unroll 4
    for (int t = 0; t < kChunk; ++t) {
      float vv[XD];
#pragma unroll
      for (int xi = 0; xi < XD; ++xi) vv[xi] = E::load(vr + (int64_t)t * D + lane + kWave * xi);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pt = ps[t][h];
#pragma unroll
        for (int xi = 0; xi < XD; ++xi) acc[h][xi] += pt * vv[xi];
      }
    }
    __syncthreads();
  }

  T* op = reinterpret_cast<T*>(a.out) + (br * a.Hq + (int64_t)g * G) * D;
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int xi = 0; xi < XD; ++xi) E::store(op + h * D + lane + kWave * xi, acc[h][xi]);
}

// ---------------------------------------------------------------------------
template <bool BF16, int D, int G>
__global__ __launch_bounds__(256) void attend_slot_kernel(AttendArgs a) {
  using E = Elem<BF16>;
  using T = typename E::T;
  constexpr int VEC = 16 / (int)sizeof(T);             // elements per 16-byte load
  constexpr int KROW = D + VEC;                        // padded key row in LDS
  constexpr int NV = kChunk * D / VEC / 256;           // 16-byte loads per thread per tensor
  constexpr int HPW = (G + 3) / 4;                     // q heads per wave
  constexpr int XD = D / kWave;                        // output dims per lane
  __shared__ __align__(16) T ks[kChunk * KROW];
  __shared__ __align__(16) T vs[kChunk * D];
  __shared__ float qs[G][D];
  __shared__ float ps[G][kChunk];
  __shared__ int last;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int64_t row = blockIdx.x;
  const int sk = blockIdx.y;
  const int g = (int)(row % a.Hkv);
  const int64_t br = row / a.Hkv;
  const int64_t b = br / a.Lq;
  const int K = a.K;

  const int32_t my_idx = lane < K ? a.idx[row * K + lane] : -1;
  const float my_s = lane < K ? a.score[row * K + lane] : 0.f;
  const bool valid = my_idx >= 0 && (int64_t)my_idx < a.Nc;
  const float mxs = wave_max(valid ? my_s : -INFINITY);
  const float ex = valid ? expf(my_s - mxs) : 0.f;
  const float den = wave_sum(ex);
  const int c = __shfl(my_idx, sk, kWave);
  const float wk = __shfl(valid ? ex / den : 0.f, sk, kWave);
  const bool use = c >= 0 && (int64_t)c < a.Nc;

  float acc[HPW][XD];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
    for (int xi = 0; xi < XD; ++xi) acc[hh][xi] = 0.f;

  if (use) {
    const int64_t base = ((b * a.Hkv + g) * a.Lkv + (int64_t)c * kChunk) * D;
    const uint4* kp = reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(a.k) + base);
    const uint4* vp = reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(a.v) + base);
    uint4 kx[NV], vx[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      kx[i] = kp[tid + 256 * i];
      vx[i] = vp[tid + 256 * i];
    }
    const T* qp = reinterpret_cast<const T*>(a.q_attn) + (br * a.Hq + (int64_t)g * G) * D;
    for (int i = tid; i < G * D; i += 256) qs[i / D][i % D] = E::load(qp + i);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = (tid + 256 * i) * VEC;
      *reinterpret_cast<uint4*>(&ks[(e / D) * KROW + e % D]) = kx[i];
      *reinterpret_cast<uint4*>(&vs[e]) = vx[i];
    }
  }
  __syncthreads();
  if (use) {
    // logits of key `lane` for this wave's heads
    float dot[HPW], rq[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      dot[hh] = 0.f;
      const int h = w + 4 * hh;
      float ss = 0.f;
      if (h < G) {
#pragma unroll
        for (int xi = 0; xi < XD; ++xi) ss += qs[h][lane + kWave * xi] * qs[h][lane + kWave * xi];
      }
      ss = wave_sum(ss);
      rq[hh] = a.qk_norm ? 1.0f / fmaxf(sqrtf(ss), 1e-6f) : 1.0f;
    }
    float kss = 0.f;
    const T* kr = &ks[lane * KROW];
#pragma unroll 4
    for (int x0 = 0; x0 < D; x0 += VEC) {
      float kv[VEC];
      const uint4 u = *reinterpret_cast<const uint4*>(kr + x0);
      if constexpr (BF16) {
        const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kv[2 * i] = __uint_as_float(wd[i] << 16);
          kv[2 * i + 1] = __uint_as_float(wd[i] & 0xFFFF0000u);
        }
      } else {
        const float4 f = __builtin_bit_cast(float4, u);
        kv[0] = f.x; kv[1] = f.y; kv[2] = f.z; kv[3] = f.w;
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        kss += kv[e] * kv[e];
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh)
          if (w + 4 * hh < G) dot[hh] += qs[w + 4 * hh][x0 + e] * kv[e];
      }
    }
    const float rk = a.qk_norm ? 1.0f / fmaxf(sqrtf(kss), 1e-6f) : 1.0f;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int h = w + 4 * hh;
      const float logit = dot[hh] * rq[hh] * rk * a.attn_scale;
      const float m = wave_max(logit);
      const float p = expf(logit - m);
      const float sp = wave_sum(p);
      if (h < G) ps[h][lane] = p / sp * wk;
    }
    // P.V (the wave reads back only its own heads' P)
#pragma unroll 4
    for (int t = 0; t < kChunk; ++t) {
      float vv[XD];
      if constexpr (BF16 && XD == 2) {
        const uint32_t u = *reinterpret_cast<const uint32_t*>(&vs[t * D + 2 * lane]);
        vv[0] = __uint_as_float(u << 16);
        vv[1] = __uint_as_float(u & 0xFFFF0000u);
      } else {
#pragma unroll
        for (int xi = 0; xi < XD; ++xi) vv[xi] = E::load(&vs[t * D + XD * lane + xi]);
      }
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        const int h = w + 4 * hh;
        if (h < G) {
          const float pt = ps[h][t];
#pragma unroll
          for (int xi = 0; xi < XD; ++xi) acc[hh][xi] += pt * vv[xi];
        }
      }
    }
  }

  T* op = reinterpret_cast<T*>(a.out) + (br * a.Hq + (int64_t)g * G) * D;
  if (a.n_splits == 1) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int h = w + 4 * hh;
      if (h < G)
#pragma unroll
        for (int xi = 0; xi < XD; ++xi) E::store(op + h * D + XD * lane + xi, acc[hh][xi]);
    }
    return;
  }
  float* part = a.partials + (row * a.n_splits + sk) * (int64_t)(G * D);
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const int h = w + 4 * hh;
    if (h < G)
#pragma unroll
      for (int xi = 0; xi < XD; ++xi) publish(&part[h * D + XD * lane + xi], acc[hh][xi]);
  }
  wait_stores();
  __syncthreads();
  if (tid == 0) last = arrive(&a.counters[row]) == (uint32_t)(a.n_splits - 1);
  __syncthreads();
  if (!last) return;
  // every thread sums its outputs over the partials; 16 partials per batch of
  // loads, all outputs of the thread in flight together
  const float* pb = a.partials + row * a.n_splits * (int64_t)(G * D);
  constexpr int OPT = (G * D + 255) / 256;
  float sum[OPT];
#pragma unroll
  for (int u = 0; u < OPT; ++u) sum[u] = 0.f;
  for (int p0 = 0; p0 < a.n_splits; p0 += 16) {
    float x[16][OPT];
#pragma unroll
    for (int q = 0; q < 16; ++q)
#pragma unroll
      for (int u = 0; u < OPT; ++u) {
        const int o = tid + 256 * u;
        x[q][u] = (p0 + q < a.n_splits && o < G * D) ? fetch(&pb[(int64_t)(p0 + q) * G * D + o]) : 0.f;
      }
#pragma unroll
    for (int q = 0; q < 16; ++q)
#pragma unroll
      for (int u = 0; u < OPT; ++u) sum[u] += x[q][u];
  }
#pragma unroll
  for (int u = 0; u < OPT; ++u)
    if (tid + 256 * u < G * D) E::store(op + tid + 256 * u, sum[u]);
  if (tid == 0) reset_counter(&a.counters[row]);
}

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

template <bool BF16, int D>
hipError_t launch_g(const AttendArgs& a, int G, dim3 grid, hipStream_t st) {
  const bool slot = a.mode == 1;
  const dim3 block(slot ? 256 : 64);
#define HSA_ATTEND_CASE(GG)                                                              \
  case GG:                                                                               \
    if (slot) hipLaunchKernelGGL((attend_slot_kernel<BF16, D, GG>), grid, block, 0, st, a); \
    else hipLaunchKernelGGL((attend_blend_kernel<BF16, D, GG>), grid, block, 0, st, a);     \
    break;
  switch (G) {
    HSA_ATTEND_CASE(1)
    HSA_ATTEND_CASE(2)
    HSA_ATTEND_CASE(4)
    HSA_ATTEND_CASE(8)
    HSA_ATTEND_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef HSA_ATTEND_CASE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attend(const AttendArgs& a, int64_t B, bool bf16, int D, int G, hipStream_t st) {
  const dim3 grid((unsigned)(B * a.Lq * a.Hkv), (unsigned)a.n_splits, 1);
  if (bf16) return D == 128 ? launch_g<true, 128>(a, G, grid, st) : launch_g<true, 64>(a, G, grid, st);
  return D == 128 ? launch_g<false, 128>(a, G, grid, st) : launch_g<false, 64>(a, G, grid, st);
}

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t value, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n, value);
  return hipGetLastError();
}

}  // namespace hsa
