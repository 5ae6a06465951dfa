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
// When a row's slots are spread over several waves (few rows, e.g. decode),
// each wave writes its fp32 partial sum and the last wave to finish -- found
// with a per-row arrival counter -- adds the partials in slot order, so the
// result does not depend on timing.
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
  __shared__ int last;

  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;               // (b*Lq + r)*Hkv + g
  const int sk = blockIdx.y;
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

  const int k_lo = sk * a.slots_per_split;
  const int k_hi = min(K, k_lo + a.slots_per_split);
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
  if (a.n_splits == 1) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int xi = 0; xi < XD; ++xi) E::store(op + h * D + lane + kWave * xi, acc[h][xi]);
    return;
  }
  float* part = a.partials + (row * a.n_splits + sk) * (int64_t)(G * D);
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int xi = 0; xi < XD; ++xi) part[h * D + lane + kWave * xi] = acc[h][xi];
  __threadfence();
  __syncthreads();
  if (lane == 0) last = atomicAdd(&a.counters[row], 1u) == (uint32_t)(a.n_splits - 1);
  __syncthreads();
  if (!last) return;
  __threadfence();
  const float* base = a.partials + row * a.n_splits * (int64_t)(G * D);
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int xi = 0; xi < XD; ++xi) {
      const int o = h * D + lane + kWave * xi;
      float s = 0.f;
      for (int p = 0; p < a.n_splits; ++p) s += base[(int64_t)p * G * D + o];
      E::store(op + o, s);
    }
  if (lane == 0) a.counters[row] = 0;
}

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

template <bool BF16, int D>
hipError_t launch_g(const AttendArgs& a, int G, dim3 grid, hipStream_t st) {
  const dim3 block(64);
  switch (G) {
    case 1: hipLaunchKernelGGL((attend_blend_kernel<BF16, D, 1>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((attend_blend_kernel<BF16, D, 2>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((attend_blend_kernel<BF16, D, 4>), grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL((attend_blend_kernel<BF16, D, 8>), grid, block, 0, st, a); break;
    case 16: hipLaunchKernelGGL((attend_blend_kernel<BF16, D, 16>), grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
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
