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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming loads for data read exactly once (partials of a reduction): the
// lines are not kept in the caches for reuse.
__device__ __forceinline__ uint2 load_stream(const uint2* p) {
  const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(x[0], x[1]);
}
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ float4 load_stream(const float4* p) {
  const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]), __uint_as_float(x[3]));
}

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
//
// Within each 16-lane row, DPP butterflies (xor 1, xor 2, half-row mirror, row
// mirror) leave the row's result in every lane; the four row results are then
// combined with v_readlane, so nothing goes through the LDS crossbar.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));   // row_half_mirror
  v = fmaxf(v, dpp_f<0x140>(v));   // row_mirror
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}
__device__ __forceinline__ int wave_sum_i(int v) {
  v += dpp_i<0xB1>(v);
  v += dpp_i<0x4E>(v);
  v += dpp_i<0x141>(v);
  v += dpp_i<0x140>(v);
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}
// Sum / maximum over the four 16-lane rows (lanes l, l ^ 16, l ^ 32, l ^ 48),
// result in every lane, with gfx950's row-swap permutes: a VALU op per step
// instead of an LDS crossbar round trip.  permlane16_swap(v, v) leaves rows
// (0, 0, 2, 2) in its first result and (1, 1, 3, 3) in its second, so their
// sum is v[l] + v[l ^ 16] in every lane; permlane32_swap(v, v) does the same
// for the two halves (v[l] + v[l ^ 32]).  Each step adds the same two values
// as x + shfl_xor(x, 16 or 32) does, so the results are identical.
__device__ __forceinline__ float xrow_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float xrow_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// number of lanes whose predicate holds
__device__ __forceinline__ int wave_count(bool p) { return __popcll(__ballot(p)); }
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  uint32_t lo = __shfl((uint32_t)v, src, kWave), hi = __shfl((uint32_t)(v >> 32), src, kWave);
  return ((uint64_t)hi << 32) | lo;
}

}  // namespace hsa

namespace hsa {

// ---------------------------------------------------------------------------
// hand-off between workgroups of one kernel
//
// Pattern: every thread of a producer workgroup stores its part with publish,
// calls wait_stores, and the workgroup meets at a barrier; one thread then
// calls arrive on the row's counter; the workgroup that sees the last count
// meets at a barrier again and reads every part with fetch, then resets the
// counter for the next call.
//
// Why the parts are complete when the last workgroup reads them:
//  * In the HIP (scoped C++) memory model, the parts are relaxed device-scope
//    atomics; the barrier makes each thread's store happen before the arriving
//    thread's release (arrive is an acq_rel device-scope read-modify-write);
//    the counter's modification order makes that release synchronise with the
//    last workgroup's acquire (the same arrive), and its barrier makes the
//    acquire happen before every fetch.  So every store happens before every
//    fetch, and the fetches see the stored values.
//  * On gfx950 this compiles to: publish = global_store ... sc1, which writes
//    through the XCD's L2 to the device coherence point; wait_stores =
//    s_waitcnt vmcnt(0), so each store has completed there before the barrier
//    (a workgroup-scope barrier alone does not wait for global stores);
//    arrive = buffer_wbl2 sc1 (L2 write-back; nothing of the hand-off is dirty
//    in the L2, since the parts were written through) + atomic + buffer_inv
//    sc1 (drops stale L2 lines); fetch = global_load ... sc1, which is served
//    from the coherence point, not from a possibly stale line of this XCD's
//    L2.  The L2s of different XCDs are not coherent with each other, which is
//    why neither side may use plain cached accesses for the parts.
// ---------------------------------------------------------------------------
template <class T>
__device__ __forceinline__ void publish(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T fetch(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// s_waitcnt vmcnt(0): every global store of this thread has completed.
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ uint32_t arrive(uint32_t* ctr) {
  return __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void reset_counter(uint32_t* ctr) {
  __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// wave-level selection over packed candidates held in LDS
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t lanemask_lt() {
  return (1ull << (threadIdx.x & (kWave - 1))) - 1ull;
}

// K-th largest of the register-held packed candidates e[0..nlive) of the wave
// (slot i of every lane; unique nonzero keys, zeros ignored; nlive <= N is
// wave-uniform); 0 when at most K are nonzero.  Counts come from ballots, so a
// bisection step costs a few scalar operations per live slot.
template <int N>
__device__ __forceinline__ uint64_t wave_kth_regs(const uint64_t (&e)[N], int nlive, int K) {
  int nz = 0;
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (i < nlive) nz += wave_count(e[i] != 0ull);
  if (nz <= K) return 0ull;
  uint32_t t32 = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = t32 | (1u << bit);
    int c = 0;
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (i < nlive) c += wave_count(cand_key(e[i]) >= cand);
    if (c >= K) t32 = cand;
  }
  int above = 0, at = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i < nlive) {
      above += wave_count(cand_key(e[i]) > t32);
      at += wave_count(e[i] != 0ull && cand_key(e[i]) == t32);
    }
  }
  const int need = K - above;
  uint32_t tl = 0;
  if (at > need) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = tl | (1u << bit);
      int c = 0;
#pragma unroll
      for (int i = 0; i < N; ++i)
        if (i < nlive) c += wave_count(e[i] != 0ull && cand_key(e[i]) == t32 && (uint32_t)e[i] >= cand);
      if (c >= need) tl = cand;
    }
  }
  return ((uint64_t)t32 << 32) | tl;
}

// Largest key value t such that at least K of the register-held candidates
// have key >= t (0 if fewer than K are nonzero).  A lower bound of the K-th
// largest candidate's key that skips tie resolution.
template <int N>
__device__ __forceinline__ uint32_t wave_kth_key(const uint64_t (&e)[N], int nlive, int K) {
  uint32_t t32 = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = t32 | (1u << bit);
    int c = 0;
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (i < nlive) c += wave_count(cand_key(e[i]) >= cand);
    if (c >= K) t32 = cand;
  }
  return t32;
}

// Keeps the top min(n, K) entries of arr[0..n) at arr[0..m), unordered, and
// returns m.  n <= kPerLane * 64.
template <int kPerLane>
__device__ __forceinline__ int wave_keep_top(uint64_t* arr, int n, int K, int lane) {
  if (n <= K) return n;
  const int nlive = (n + kWave - 1) / kWave;
  uint64_t e[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int p = lane + kWave * i;
    e[i] = (i < nlive && p < n) ? arr[p] : 0ull;
  }
  const uint64_t t = wave_kth_regs<kPerLane>(e, nlive, K);
  int off = 0;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    if (i >= nlive) break;
    const bool keep = e[i] != 0ull && e[i] >= t;
    const uint64_t mask = __ballot(keep);
    if (keep) arr[off + __popcll(mask & lanemask_lt())] = e[i];
    off += __popcll(mask);
  }
  return off;
}

// Rank of e among arr[0..n) in LDS (unique nonzero keys, n wave-uniform): the
// number of entries above it.  Every lane reads the same addresses (broadcast),
// eight entries in flight per step.
__device__ __forceinline__ int lds_rank(const uint64_t* arr, int n, uint64_t e) {
  int rank = 0;
  for (int i0 = 0; i0 < n; i0 += 8) {
    uint64_t x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = arr[i0 + u < n ? i0 + u : n - 1];
#pragma unroll
    for (int u = 0; u < 8; ++u) rank += (i0 + u < n && x[u] > e) ? 1 : 0;
  }
  return rank;
}

// Rank-sorts arr[0..m) (m <= 64, unique keys) into dst[0..m), best first.
// dst must not alias arr.
__device__ __forceinline__ void wave_rank_sort(const uint64_t* arr, int m, uint64_t* dst, int lane) {
  const uint64_t e = lane < m ? arr[lane] : 0ull;
  const int rank = lds_rank(arr, m, e);
  if (lane < m) dst[rank] = e;
}

// LDS transpose load (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane j passes the address of X[r0 + j / 4][c0 + 4 (j % 4)] (8 bytes of a
// row-major bf16 array) and lane t receives X[r0 + e][c0 + t], e = 0..3: four
// consecutive rows of one column, the k-run of an MFMA operand.
typedef short short4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_tr4(const uint16_t* p) {
  const short4v x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)(p));
  return __builtin_bit_cast(uint2, x);
}

// MFMA operand (v_mfma_f32_16x16x32_bf16, A or B) at column c0 + lane % 16 of
// a row-major [k][n] bf16 array in LDS with row stride `ld` elements: its
// eight k entries are rows ra..ra+3 then rb..rb+3 (two transpose loads; each
// lane group lane / 16 passes its own ra, rb).  lds_operand_tr: rows r0..r0+7.
__device__ __forceinline__ bf16x8 lds_operand_tr2(const uint16_t* base, int ld, int ra, int rb, int c0, int ma) {
  const int off = (ma >> 2) * ld + c0 + 4 * (ma & 3);
  const uint2 lo = lds_tr4(base + ra * ld + off), hi = lds_tr4(base + rb * ld + off);
  return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}
__device__ __forceinline__ bf16x8 lds_operand_tr(const uint16_t* base, int ld, int r0, int c0, int ma) {
  return lds_operand_tr2(base, ld, r0, r0 + 4, c0, ma);
}

}  // namespace hsa
