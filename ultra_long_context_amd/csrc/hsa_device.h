// hsa_device.h -- device-side helpers shared by the HSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hsa {

constexpr int kChunk = 64;     // tokens per chunk (Step 1 of the method)
constexpr int kWave = 64;      // CDNA4 wavefront width
constexpr int kMaxTopK = 64;

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// element conversion
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// round to nearest even; inputs are finite
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <bool BF16> struct Elem;
template <> struct Elem<true> {
  using T = uint16_t;
  static __device__ __forceinline__ float load(const T* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(T* p, float v) { *p = f32_to_bf16(v); }
};
template <> struct Elem<false> {
  using T = float;
  static __device__ __forceinline__ float load(const T* p) { return *p; }
  static __device__ __forceinline__ void store(T* p, float v) { *p = v; }
};

// ---------------------------------------------------------------------------
// ordering keys
//
// A score maps to an unsigned key whose integer order equals the float order,
// with -0.0 and +0.0 mapping to the same key.  Key 0 is below every finite
// score and marks "no candidate".  A candidate is packed as
//   (key << 32) | (0xFFFFFFFF - chunk)
// so one unsigned compare gives the selection order: score descending, then
// chunk index ascending.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_key(float f) {
  f = (f == 0.0f) ? 0.0f : f;
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  const uint32_t b = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(b);
}
__device__ __forceinline__ uint64_t pack_cand(uint32_t key, uint32_t chunk) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - chunk);
}
__device__ __forceinline__ uint32_t cand_chunk(uint64_t c) { return 0xFFFFFFFFu - (uint32_t)c; }
__device__ __forceinline__ uint32_t cand_key(uint64_t c) { return (uint32_t)(c >> 32); }

// ---------------------------------------------------------------------------
// wave reductions (64 lanes)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  uint32_t lo = __shfl((uint32_t)v, src, kWave), hi = __shfl((uint32_t)(v >> 32), src, kWave);
  return ((uint64_t)hi << 32) | lo;
}

}  // namespace hsa
