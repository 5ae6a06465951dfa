// landmarks.hip -- one landmark per 64-token chunk from the keys (Step 1 of the
// HSA step in "Every Token Counts", agent-atlas explainer, "How It Works
// (Technically)").  The page's landmark comes from a learned encoder; without
// trained weights the stand-in is the mean of the chunk's 64 keys, which is
// also how a KV cache keeps its landmarks current: after an append, the chunks
// the append completed get their landmark.
//
// One wave per chunk: every lane issues all of its 16-byte loads of the
// chunk's keys at once (the chunk is one contiguous 64 x d block; streaming
// loads, since every key is read once: 6.26 against 5.9 TB/s with cached
// loads over the 16M history), adds its
// rows in fp32, the lanes holding the same columns are combined with xor
// shuffles, and the lanes of the first row store the mean in the input dtype.
// HBM-bound: 64 * d * e bytes read and d * e written per chunk.
#include "hsa_device.h"
#include "hsa_internal.h"

namespace hsa {
namespace {

template <bool BF16, int D>
__global__ __launch_bounds__(256) void chunk_landmark_kernel(LandmarkArgs a) {
  using T = typename Elem<BF16>::T;
  constexpr int EPU = BF16 ? 8 : 4;          // elements per 16-byte unit
  constexpr int UPR = D / EPU;               // units per key row
  constexpr int RPI = kWave / UPR;           // key rows covered by one wave-wide load
  constexpr int ITER = kChunk / RPI;         // loads per lane
  constexpr int BATCH = ITER < 16 ? ITER : 16;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t job = (int64_t)blockIdx.x * 4 + w;
  if (job >= a.jobs) return;
  const int64_t bg = job / a.n_chunks, c = a.c_begin + job % a.n_chunks;
  const int col = lane % UPR, r0 = lane / UPR;
  const T* base = reinterpret_cast<const T*>(a.k) + (bg * a.Lkv + c * kChunk) * D + col * EPU;
  float acc[EPU];
#pragma unroll
  for (int e = 0; e < EPU; ++e) acc[e] = 0.f;
#pragma unroll
  for (int i0 = 0; i0 < ITER; i0 += BATCH) {
    uint4 x[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) x[i] = load_stream(reinterpret_cast<const uint4*>(base + (r0 + RPI * (i0 + i)) * D));
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const uint32_t wd[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
      if constexpr (BF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += __uint_as_float(wd[q] << 16);
          acc[2 * q + 1] += __uint_as_float(wd[q] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] += __uint_as_float(wd[q]);
      }
    }
  }
#pragma unroll
  for (int o = UPR; o < kWave; o <<= 1)
#pragma unroll
    for (int e = 0; e < EPU; ++e) acc[e] += __shfl_xor(acc[e], o, kWave);
  if (r0 != 0) return;
  T* dst = reinterpret_cast<T*>(a.landmarks) + (bg * a.Nc + c) * D + col * EPU;
  constexpr float kInv = 1.0f / kChunk;      // exact (power of two)
  if constexpr (BF16) {
    uint4 y;
    uint32_t* yw = reinterpret_cast<uint32_t*>(&y);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      yw[q] = (uint32_t)f32_to_bf16(acc[2 * q] * kInv) | ((uint32_t)f32_to_bf16(acc[2 * q + 1] * kInv) << 16);
    *reinterpret_cast<uint4*>(dst) = y;
  } else {
    *reinterpret_cast<float4*>(dst) = make_float4(acc[0] * kInv, acc[1] * kInv, acc[2] * kInv, acc[3] * kInv);
  }
}

}  // namespace

hipError_t launch_chunk_landmarks(const LandmarkArgs& a, bool bf16, int D, hipStream_t st) {
  if (a.jobs <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.jobs + 3) / 4)), block(256);
  if (bf16) {
    if (D == 128) hipLaunchKernelGGL((chunk_landmark_kernel<true, 128>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((chunk_landmark_kernel<true, 64>), grid, block, 0, st, a);
  } else {
    if (D == 128) hipLaunchKernelGGL((chunk_landmark_kernel<false, 128>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((chunk_landmark_kernel<false, 64>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace hsa
