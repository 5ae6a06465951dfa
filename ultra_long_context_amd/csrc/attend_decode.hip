// attend_decode.hip -- per-chunk attention and blend for few query rows over a
// long history (decode), bf16 (Steps 2-4 of the HSA step in "Every Token
// Counts", agent-atlas explainer, "How It Works (Technically)").
//
// One workgroup of 4 waves serves 4 selected slots of one query row:
//   selection  when the landmark scan left one sorted candidate list per chunk
//              range, the waves merge them (only lists whose head reaches the
//              K-th largest head key can contribute); every wave ends with the
//              ranked selection in its lanes and takes its own slot's chunk and
//              blend weight from it, and the workgroup of slot block 0 writes
//              the row's final topk_idx / topk_score;
//   attend     each wave takes one slot: the chunk's keys are the B operand of
//              v_mfma_f32_16x16x32_bf16 straight from HBM, the G attention
//              queries the A operand (16 rows, G of them used), V is staged
//              transposed in LDS for the P.V product;
//   blend      the 4 waves' weighted outputs are summed in LDS, published as the
//              workgroup's partial, and the last workgroup of the row adds the
//              partials in slot order.
#include "hsa_device.h"
#include "hsa_internal.h"

namespace hsa {
namespace {

constexpr int kSlotsPerBlock = 4;       // one wave per slot
constexpr int kThreads = 64 * kSlotsPerBlock;
constexpr int kMergeCap = 512;
constexpr int kMaxHeads = 8;          // list heads per lane: up to 512 splits
constexpr int kMaxBlocks = kMaxTopK / kSlotsPerBlock;   // slot blocks of a row

// Exact top K of one row from its per-split lists, entry-major: entry j of
// split s at L[j * n_splits + s], each list sorted best first and zero-padded;
// whole wave.  Leaves the sorted selection in top[0..m) and returns m.
//
// Fast path (one round of loads): the first kFirst entries of every list are
// loaded together; the heads bound the K-th largest key from below (the K-th
// largest of the lanes' largest heads: K lanes hold a key there), the loaded
// entries at or above the bound are ranked, and the result is exact unless
// some list's last loaded entry still reaches the K-th selected key (then a
// later entry of that list could belong to the top K).  In that case the full
// merge below runs: a list can only contribute if its head reaches the K-th
// largest head, and then only entries at or above that head; those lists are
// read in batches and the surviving candidates ranked.  Loads are
// unconditional (indices clamped) so they are all in flight together.
constexpr int kFirst = 4;

template <int NH>
__device__ __forceinline__ int merge_row_lists_nh(const uint64_t* L, int n_splits, int K, uint64_t* C,
                                                  uint64_t* top, int* act, int lane) {
  constexpr int kMaxHeadSlots = NH;                  // list heads per lane
  const int nh = (n_splits + kWave - 1) / kWave;      // <= NH
  const int ne = K < kFirst ? K : kFirst;
  uint64_t f[kFirst][kMaxHeadSlots];
#pragma unroll
  for (int j = 0; j < kFirst; ++j)
#pragma unroll
    for (int i = 0; i < kMaxHeadSlots; ++i) {
      const int sp = lane + kWave * i;
      const uint64_t v = L[(int64_t)(j < ne ? j : 0) * n_splits + (sp < n_splits ? sp : 0)];
      f[j][i] = (j < ne && i < nh && sp < n_splits) ? v : 0ull;
    }
  // the K-th largest lane maximum of the heads: K lanes hold a key at or above
  // it, so it bounds the row's K-th largest key from below (0 if fewer)
  uint64_t hmax = f[0][0];
#pragma unroll
  for (int i = 1; i < kMaxHeadSlots; ++i) hmax = f[0][i] > hmax ? f[0][i] : hmax;
  C[lane] = hmax;
  const int hrank = lds_rank(C, kWave, hmax);
  const uint64_t kmask_h = __ballot(hmax != 0ull && hrank == K - 1);
  const uint64_t lo_heads = kmask_h != 0ull ? shfl_u64(hmax, (int)__builtin_ctzll(kmask_h)) : 0ull;
  {
    uint64_t lo = lo_heads;
    int n_on = 0;
#pragma unroll
    for (int j = 0; j < kFirst; ++j)
#pragma unroll
      for (int i = 0; i < kMaxHeadSlots; ++i) n_on += wave_count(f[j][i] != 0ull && f[j][i] >= lo);
    if (n_on > kWave) {                 // exact K-th of the loaded entries: K survive
      uint64_t flat[kFirst * kMaxHeadSlots];
#pragma unroll
      for (int j = 0; j < kFirst; ++j)
#pragma unroll
        for (int i = 0; i < kMaxHeadSlots; ++i) flat[j * kMaxHeadSlots + i] = f[j][i];
      lo = wave_kth_regs<kFirst * kMaxHeadSlots>(flat, kFirst * kMaxHeadSlots, K);
    }
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < kFirst; ++j)
#pragma unroll
      for (int i = 0; i < kMaxHeadSlots; ++i) {
        const bool keep = f[j][i] != 0ull && f[j][i] >= lo;
        const uint64_t mask = __ballot(keep);
        if (keep) C[cnt + __popcll(mask & lanemask_lt())] = f[j][i];
        cnt += __popcll(mask);
      }
    if (cnt <= kWave) {
      const uint64_t mine = lane < cnt ? C[lane] : 0ull;
      const int rank = lds_rank(C, cnt, mine);
      const int m = cnt < K ? cnt : K;
      // K-th selected key (with fewer than K, any nonzero entry would still enter)
      const uint64_t kmask = __ballot(lane < cnt && rank == K - 1);
      const uint64_t kth = (m == K && kmask != 0ull) ? shfl_u64(mine, (int)__builtin_ctzll(kmask)) : 1ull;
      bool open = false;
#pragma unroll
      for (int i = 0; i < kMaxHeadSlots; ++i) open = open || f[kFirst - 1][i] >= kth;
      if (ne == K || !__any(open)) {
        if (lane < cnt && rank < K) top[rank] = mine;
        return m;
      }
    }
  }
  // ---- full merge ------------------------------------------------------------
  uint64_t h[kMaxHeadSlots];
#pragma unroll
  for (int i = 0; i < kMaxHeadSlots; ++i) h[i] = f[0][i];
  uint64_t lo = lo_heads;
  int n_on = 0;
#pragma unroll
  for (int i = 0; i < kMaxHeadSlots; ++i)
    if (i < nh) n_on += wave_count(h[i] != 0ull && h[i] >= lo);
  if (n_on > kWave) lo = wave_kth_regs<kMaxHeadSlots>(h, nh, K);   // exactly K heads remain
  int na = 0;
#pragma unroll
  for (int i = 0; i < kMaxHeadSlots; ++i) {
    if (i >= nh) break;
    const bool on = h[i] != 0ull && h[i] >= lo;
    const uint64_t mask = __ballot(on);
    if (on) act[na + __popcll(mask & lanemask_lt())] = lane + kWave * i;
    na += __popcll(mask);
  }
  const int my_list = lane < na ? act[lane] : -1;
  const uint64_t* lp = L + (my_list >= 0 ? my_list : 0);
  int cnt = 0;
  for (int q0 = 0; q0 < K; q0 += 16) {
    uint64_t e[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) e[q] = lp[(int64_t)(q0 + q < K ? q0 + q : K - 1) * n_splits];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (my_list < 0 || q0 + q >= K) e[q] = 0ull;
      if (cnt + kWave > kMergeCap) {
        cnt = wave_keep_top<kMergeCap / kWave>(C, cnt, K, lane);
        if (cnt >= K) {
          uint64_t mn = ~0ull;
          for (int p = 0; p < cnt; ++p) mn = C[p] < mn ? C[p] : mn;
          lo = mn + 1;
        }
      }
      const bool keep = e[q] != 0ull && e[q] >= lo;
      const uint64_t mask = __ballot(keep);
      if (keep) C[cnt + __popcll(mask & lanemask_lt())] = e[q];
      cnt += __popcll(mask);
    }
    // lists are sorted: one whose last entry here is below the bound is done
    if (!__any(e[15] != 0ull && e[15] >= lo)) break;
  }
  if (cnt <= kWave) {                    // one candidate per lane
    const uint64_t mine = lane < cnt ? C[lane] : 0ull;
    const int rank = lds_rank(C, cnt, mine);
    if (lane < cnt && rank < K) top[rank] = mine;
    return cnt < K ? cnt : K;
  }
  const int m = wave_keep_top<kMergeCap / kWave>(C, cnt, K, lane);
  wave_rank_sort(C, m, top, lane);
  return m;
}

__device__ __forceinline__ int merge_row_lists(const uint64_t* L, int n_splits, int K, uint64_t* C, uint64_t* top,
                                               int* act, int lane) {
  if (n_splits <= kWave) return merge_row_lists_nh<1>(L, n_splits, K, C, top, act, lane);
  if (n_splits <= 2 * kWave) return merge_row_lists_nh<2>(L, n_splits, K, C, top, act, lane);
  if (n_splits <= 4 * kWave) return merge_row_lists_nh<4>(L, n_splits, K, C, top, act, lane);
  return merge_row_lists_nh<kMaxHeads>(L, n_splits, K, C, top, act, lane);
}

// The fast path of merge_row_lists with the workgroup's waves sharing the
// work: wave w loads entry w of every list, wave 0 derives the bound from the
// heads, the waves compact their entries at or above it side by side into C
// and rank the candidates against a quarter of C each.  Whenever the one-round
// result is not exact (more than 64 candidates, or a list whose last loaded
// entry reaches the K-th selected key) wave 0 runs merge_row_lists instead.
// Called by every wave of the workgroup; every wave ends with the selection
// spread over its lanes: lane p holds a candidate e with rank r (the r-th
// largest key; valid if p < n and r < K), n returned.
struct MergeShared {
  uint64_t lo;                        // bound from the heads
  int cnt[kSlotsPerBlock];            // entries at or above it, per wave
  int prank[kSlotsPerBlock][kWave];   // partial ranks of the candidates
  uint64_t lastmax[kWave];            // per lane: largest last loaded entry
  int m;                              // size of the one-wave merge's selection
};
static_assert(kSlotsPerBlock == kFirst, "one wave per first entry of the lists");

template <int NH>
__device__ __forceinline__ int merge_row_lists_waves(const uint64_t* L, int n_splits, int K, uint64_t* C,
                                                     uint64_t* top, int* act, MergeShared& sh, int w, int lane,
                                                     uint64_t& e_out, int& rank_out) {
  const int nh = (n_splits + kWave - 1) / kWave;      // <= NH
  const int ne = K < kFirst ? K : kFirst;
  uint64_t f[NH];                                     // entry w of lists lane + 64 i
#pragma unroll
  for (int i = 0; i < NH; ++i) {
    const int sp = lane + kWave * i;
    const uint64_t v = L[(int64_t)(w < ne ? w : 0) * n_splits + (sp < n_splits ? sp : 0)];
    f[i] = (w < ne && i < nh && sp < n_splits) ? v : 0ull;
  }
  if (w == 0) {
    // the K-th largest lane maximum of the heads: K lanes hold a key at or
    // above it, so it bounds the row's K-th largest key from below (0 if fewer)
    uint64_t hmax = f[0];
#pragma unroll
    for (int i = 1; i < NH; ++i) hmax = f[i] > hmax ? f[i] : hmax;
    C[lane] = hmax;
    const int hrank = lds_rank(C, kWave, hmax);
    const uint64_t kmask_h = __ballot(hmax != 0ull && hrank == K - 1);
    const uint64_t lo_heads = kmask_h != 0ull ? shfl_u64(hmax, (int)__builtin_ctzll(kmask_h)) : 0ull;
    if (lane == 0) sh.lo = lo_heads;
  }
  if (w == kFirst - 1) {
    uint64_t lm = f[0];
#pragma unroll
    for (int i = 1; i < NH; ++i) lm = f[i] > lm ? f[i] : lm;
    sh.lastmax[lane] = lm;
  }
  __syncthreads();
  const uint64_t lo = sh.lo;
  int n = 0;
#pragma unroll
  for (int i = 0; i < NH; ++i) n += wave_count(f[i] != 0ull && f[i] >= lo);
  if (lane == 0) sh.cnt[w] = n;
  __syncthreads();
  int off = 0, total = 0;
#pragma unroll
  for (int v = 0; v < kSlotsPerBlock; ++v) {
    off += v < w ? sh.cnt[v] : 0;
    total += sh.cnt[v];
  }
  if (total <= kWave) {
#pragma unroll
    for (int i = 0; i < NH; ++i) {
      const bool keep = f[i] != 0ull && f[i] >= lo;
      const uint64_t mask = __ballot(keep);
      if (keep) C[off + __popcll(mask & lanemask_lt())] = f[i];
      off += __popcll(mask);
    }
  }
  __syncthreads();
  if (total <= kWave) {                   // partial ranks against C[16 w, 16 w + 16)
    const uint64_t mine = lane < total ? C[lane] : 0ull;
    constexpr int Q = kWave / kSlotsPerBlock;
    const int q0 = Q * w;
    uint64_t x[Q];
#pragma unroll
    for (int u = 0; u < Q; ++u) x[u] = C[q0 + u < total ? q0 + u : 0];
    int pr = 0;
#pragma unroll
    for (int u = 0; u < Q; ++u) pr += (q0 + u < total && x[u] > mine) ? 1 : 0;
    sh.prank[w][lane] = pr;
  }
  __syncthreads();
  // every wave: full ranks and the exactness test (same data, same outcome)
  bool exact = false;
  if (total <= kWave) {
    const uint64_t mine = lane < total ? C[lane] : 0ull;
    int rank = 0;
#pragma unroll
    for (int v = 0; v < kSlotsPerBlock; ++v) rank += sh.prank[v][lane];
    const int m = total < K ? total : K;
    // K-th selected key (with fewer than K, any nonzero entry would still enter)
    const uint64_t kmask = __ballot(lane < total && rank == K - 1);
    const uint64_t kth = (m == K && kmask != 0ull) ? shfl_u64(mine, (int)__builtin_ctzll(kmask)) : 1ull;
    exact = ne == K || !__any(sh.lastmax[lane] >= kth);
    e_out = mine;
    rank_out = rank;
  }
  if (exact) return total;
  // not exact (uniform over the workgroup): the one-wave merge on wave 0
  if (w == 0) {
    const int m = merge_row_lists_nh<NH>(L, n_splits, K, C, top, act, lane);
    if (lane == 0) sh.m = m;
  }
  __syncthreads();
  const int m = sh.m;
  e_out = lane < m ? top[lane] : 0ull;
  rank_out = lane;
  return m;
}

// Dispatch on the list-head slots per lane; called by every wave.
__device__ __forceinline__ int merge_row_lists_wg(const uint64_t* L, int n_splits, int K, uint64_t* C,
                                                  uint64_t* top, int* act, MergeShared& sh, int w, int lane,
                                                  uint64_t& e, int& rank) {
  if (n_splits <= kWave) return merge_row_lists_waves<1>(L, n_splits, K, C, top, act, sh, w, lane, e, rank);
  if (n_splits <= 2 * kWave) return merge_row_lists_waves<2>(L, n_splits, K, C, top, act, sh, w, lane, e, rank);
  if (n_splits <= 4 * kWave) return merge_row_lists_waves<4>(L, n_splits, K, C, top, act, sh, w, lane, e, rank);
  return merge_row_lists_waves<kMaxHeads>(L, n_splits, K, C, top, act, sh, w, lane, e, rank);
}

template <int D, int G>
__global__ __launch_bounds__(kThreads) void attend_decode_kernel(DecodeArgs a) {
  constexpr int KSTEP = D / 32;
  constexpr int NT = D / 16;
  constexpr int VROW = D + 16;         // bf16 elements per staged V row (row-major)
  constexpr int PROW = kChunk + 8;
  __shared__ __align__(16) uint16_t vs[kSlotsPerBlock][kChunk * VROW];
  __shared__ __align__(16) uint16_t ps[kSlotsPerBlock][16 * PROW];
  __shared__ uint64_t cand[kMergeCap];
  __shared__ uint64_t top[kMaxTopK];
  __shared__ int act[kWave];
  __shared__ float osum[kSlotsPerBlock][G * D];
  __shared__ int last;
  __shared__ MergeShared msh;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int64_t row = blockIdx.x;                     // (b*Lq + r)*Hkv + g
  const int blk = blockIdx.y;
  const int g = (int)(row % a.Hkv);
  const int64_t br = row / a.Hkv;
  const int64_t b = br / a.Lq;
  const int K = a.K;

  // --- the row's selection and blend weights -------------------------------
  // every wave holds the whole selection, lane p: chunk, score and rank (the
  // merged selection's order, or the slot order of a given one), and takes its
  // own slot's chunk and weight from it
  const int slot = blk * kSlotsPerBlock + w;
  int32_t chunk = -1, rank = lane;
  float s = -INFINITY;
  bool valid;
  if (a.lists != nullptr) {                // uniform: every wave takes part in the merge
    uint64_t e = 0ull;
    const int n = merge_row_lists_wg(a.lists + row * a.n_splits * K, a.n_splits, K, cand, top, act, msh, w, lane,
                                     e, rank);
    valid = lane < n && rank < K;
    if (valid) {
      chunk = (int32_t)cand_chunk(e);
      s = key_score(cand_key(e)) * a.ret_scale;
    }
    if (blk == 0 && w == 0 && a.idx_out != nullptr) {
      const int m = n < K ? n : K;
      if (valid) {
        a.idx_out[row * K + rank] = chunk;
        a.score_out[row * K + rank] = s;
      }
      if (lane >= m && lane < K) {
        a.idx_out[row * K + lane] = -1;
        a.score_out[row * K + lane] = -INFINITY;
      }
    }
  } else {                                 // given selection: kept as is (slot order)
    const int32_t ci = lane < K ? a.idx_in[row * K + lane] : -1;
    valid = ci >= 0 && (int64_t)ci < a.Nc;
    if (valid) {
      chunk = ci;
      s = a.score_in[row * K + lane];
    }
  }
  const float mx = wave_max(valid ? s : -INFINITY);
  const float ex = valid ? expf(s - mx) : 0.f;
  const float den = wave_sum(ex);
  const uint64_t hit = __ballot(valid && rank == slot);
  const int src = hit != 0ull ? (int)__builtin_ctzll(hit) : 0;
  const int c = hit != 0ull ? __shfl(chunk, src, kWave) : -1;
  const float wk = hit != 0ull ? __shfl(ex, src, kWave) / den : 0.f;

  // --- one slot per wave ----------------------------------------------------
  const int ma = lane & 15, jg = lane >> 4;
  floatx4 o[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) o[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  if (c >= 0) {
    const int64_t base = ((b * a.Hkv + g) * a.Lkv + (int64_t)c * kChunk) * D;
    const uint16_t* kp = reinterpret_cast<const uint16_t*>(a.k) + base;
    const uint16_t* vp = reinterpret_cast<const uint16_t*>(a.v) + base;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q_attn) + (br * a.Hq + (int64_t)g * G) * D;
    // all loads first: keys as B operands, queries as A operands, V rows
    uint4 kb[4][KSTEP], qa[KSTEP], vx[D / 8];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int t = 0; t < KSTEP; ++t)
        kb[nt][t] = *reinterpret_cast<const uint4*>(kp + (16 * nt + ma) * D + 32 * t + 8 * jg);
#pragma unroll
    for (int t = 0; t < KSTEP; ++t) {    // rows >= G load row 0 (unconditional), then zero
      qa[t] = *reinterpret_cast<const uint4*>(qp + (ma < G ? ma : 0) * D + 32 * t + 8 * jg);
      if (ma >= G) qa[t] = make_uint4(0, 0, 0, 0);
    }
    // V: consecutive lanes take consecutive 16-byte pieces of the chunk
#pragma unroll
    for (int dg = 0; dg < D / 8; ++dg) vx[dg] = *reinterpret_cast<const uint4*>(vp + (dg * kWave + lane) * 8);
    // V rows into LDS (read back transposed as the B operand of P V)
#pragma unroll
    for (int dg = 0; dg < D / 8; ++dg) {
      const int e = (dg * kWave + lane) * 8;
      *reinterpret_cast<uint4*>(&vs[w][(e / D) * VROW + e % D]) = vx[dg];
    }
    // norms: lane holds 32 dims of query row ma and of key 16*nt + ma
    float qss = 0.f, kss[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < KSTEP; ++t) {
      const uint32_t qw[4] = {qa[t].x, qa[t].y, qa[t].z, qa[t].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = __uint_as_float(qw[q] << 16), hi = __uint_as_float(qw[q] & 0xFFFF0000u);
        qss += lo * lo + hi * hi;
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const uint32_t kw[4] = {kb[nt][t].x, kb[nt][t].y, kb[nt][t].z, kb[nt][t].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = __uint_as_float(kw[q] << 16), hi = __uint_as_float(kw[q] & 0xFFFF0000u);
          kss[nt] += lo * lo + hi * hi;
        }
      }
    }
    qss = xrow_sum(qss);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      kss[nt] = xrow_sum(kss[nt]);
    }
    const float rq_mine = a.qk_norm ? 1.0f / fmaxf(sqrtf(qss), 1e-6f) : 1.0f;
    float rk[4];
#pragma unroll
    // logits in base 2: log2(e) folded into the key factor
    for (int nt = 0; nt < 4; ++nt)
      rk[nt] = (a.qk_norm ? 1.0f / fmaxf(sqrtf(kss[nt]), 1e-6f) : 1.0f) * a.attn_scale * 1.4426950408889634f;
    // S = Q K^T: lane holds S[4*jg + i][16*nt + ma]
    floatx4 s[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      s[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < KSTEP; ++t)
        s[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[t]),
                                                        __builtin_bit_cast(bf16x8, kb[nt][t]), s[nt], 0, 0, 0);
    }
    // softmax per query row over the 64 keys
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * jg + i;
      const float rq = __shfl(rq_mine, m, kWave);
      float x[4], mx = -INFINITY;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        x[nt] = s[nt][i] * rq * rk[nt];
        mx = fmaxf(mx, x[nt]);
      }
      mx = fmaxf(mx, dpp_f<0xB1>(mx));
      mx = fmaxf(mx, dpp_f<0x4E>(mx));
      mx = fmaxf(mx, dpp_f<0x141>(mx));
      mx = fmaxf(mx, dpp_f<0x140>(mx));
      float sum = 0.f;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        x[nt] = __builtin_amdgcn_exp2f(x[nt] - mx);
        sum += x[nt];
      }
      sum += dpp_f<0xB1>(sum);
      sum += dpp_f<0x4E>(sum);
      sum += dpp_f<0x141>(sum);
      sum += dpp_f<0x140>(sum);
      const float scale = (m < G ? wk : 0.f) / sum;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) ps[w][m * PROW + 16 * nt + ma] = f32_to_bf16(x[nt] * scale);
    }
    // O = P V
    bf16x8 pa8[2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
      pa8[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&ps[w][ma * PROW + 32 * st + 8 * jg]));
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8 bv = lds_operand_tr(vs[w], VROW, 32 * st + 8 * jg, 16 * nt, ma);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa8[st], bv, o[nt], 0, 0, 0);
      }
  }
  // --- sum the 4 waves' outputs; lane holds O[4*jg + i][16*nt + ma] ----------
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * jg + i;
      if (m < G) osum[w][m * D + 16 * nt + ma] = o[nt][i];
    }
  __syncthreads();
  const int n_blk = a.n_blocks;
  uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + (br * a.Hq + (int64_t)g * G) * D;
  float* part = a.partials + (row * n_blk + blk) * (int64_t)(G * D);
  for (int e = tid; e < G * D; e += kThreads) {
    float v = osum[0][e];
#pragma unroll
    for (int x = 1; x < kSlotsPerBlock; ++x) v += osum[x][e];
    if (n_blk == 1) op[e] = f32_to_bf16(v);
    else publish(&part[e], v);
  }
  if (n_blk == 1) return;
  wait_stores();
  __syncthreads();
  if (tid == 0) last = arrive(&a.counters[row]) == (uint32_t)(n_blk - 1);
  __syncthreads();
  if (!last) return;
  // each thread adds 4 consecutive outputs over the blocks, in block order,
  // with every block's 16 bytes in flight at once
  const float* pb = a.partials + row * n_blk * (int64_t)(G * D);
  for (int e0 = 4 * tid; e0 < G * D; e0 += 4 * kThreads) {
    uint64_t lo[kMaxBlocks], hi[kMaxBlocks];
#pragma unroll
    for (int p = 0; p < kMaxBlocks; ++p) {
      const uint64_t* q = reinterpret_cast<const uint64_t*>(pb + (int64_t)(p < n_blk ? p : 0) * G * D + e0);
      lo[p] = fetch(q);
      hi[p] = fetch(q + 1);
    }
    float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < kMaxBlocks; ++p)
      if (p < n_blk) {
        v[0] += __uint_as_float((uint32_t)lo[p]);
        v[1] += __uint_as_float((uint32_t)(lo[p] >> 32));
        v[2] += __uint_as_float((uint32_t)hi[p]);
        v[3] += __uint_as_float((uint32_t)(hi[p] >> 32));
      }
    const uint32_t b01 = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    const uint32_t b23 = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    *reinterpret_cast<uint2*>(op + e0) = make_uint2(b01, b23);
  }
  if (tid == 0) reset_counter(&a.counters[row]);
}

// One wave per row: merge the per-split lists into the final selection.
__global__ __launch_bounds__(64) void merge_lists_kernel(MergeArgs a) {
  __shared__ uint64_t cand[kMergeCap];
  __shared__ uint64_t top[kMaxTopK];
  __shared__ int act[kWave];
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int K = a.K;
  const int m = merge_row_lists(a.lists + row * a.n_splits * K, a.n_splits, K, cand, top, act, lane);
  if (lane < K) {
    if (lane < m) {
      a.out_idx[row * K + lane] = (int32_t)cand_chunk(top[lane]);
      a.out_score[row * K + lane] = key_score(cand_key(top[lane])) * a.ret_scale;
    } else {
      a.out_idx[row * K + lane] = -1;
      a.out_score[row * K + lane] = -INFINITY;
    }
  }
}

}  // namespace

int decode_slots_per_block() { return kSlotsPerBlock; }

hipError_t launch_merge_lists(const MergeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(merge_lists_kernel, dim3((unsigned)a.rows), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attend_decode(const DecodeArgs& a, int64_t rows, int D, int G, hipStream_t st) {
  const dim3 grid((unsigned)rows, (unsigned)a.n_blocks, 1), block(kThreads);
#define HSA_DEC_CASE(DD, GG)                                                                  \
  if (D == DD && G == GG) {                                                                   \
    hipLaunchKernelGGL((attend_decode_kernel<DD, GG>), grid, block, 0, st, a);                 \
    return hipGetLastError();                                                                 \
  }
  HSA_DEC_CASE(128, 1) HSA_DEC_CASE(128, 2) HSA_DEC_CASE(128, 4) HSA_DEC_CASE(128, 8)
  HSA_DEC_CASE(128, 16) HSA_DEC_CASE(64, 1) HSA_DEC_CASE(64, 2) HSA_DEC_CASE(64, 4)
  HSA_DEC_CASE(64, 8) HSA_DEC_CASE(64, 16)
#undef HSA_DEC_CASE
  return hipErrorInvalidValue;
}

}  // namespace hsa
