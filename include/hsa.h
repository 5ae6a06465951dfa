/*
 * hsa.h -- C ABI of the MI355X (gfx950) Hierarchical Sparse Attention forward.
 *
 * The operation is the HSA step of "Every Token Counts: Generalizing 16M
 * Ultra-Long Context in LLMs" (agent-atlas explainer, section "How It Works
 * (Technically)", Steps 1-4, and the hsa_step sketch under "The algorithm,
 * simplified"):
 *
 *   Step 1  the KV history is cut into chunks of 64 tokens; chunk i owns
 *           tokens [64 i, 64 i + 64) and one landmark vector.
 *   Step 2  score  s[t,i] = (q_ret[t] . landmark[i]) * ret_scale  for every chunk
 *           that lies entirely before the query's own chunk; keep the top_k
 *           chunks (ties go to the lower chunk index).
 *   Step 3  for each kept chunk, softmax attention of every q head of the kv
 *           group over the chunk's 64 keys, with query-key L2 normalisation
 *           when HSA_FLAG_QK_L2NORM is set:  O[t,i] = softmax(qhat khat^T *
 *           attn_scale) V[i],  xhat = x / max(||x||_2, 1e-6).
 *   Step 4  w[t,i] = softmax of s over the kept chunks;  out[t] = sum_i w O.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout: dense row-major, no strides.  B = batch, Lq = q_len, Lkv = kv_len,
 * Hq/Hkv = q/kv heads, G = Hq/Hkv (q head h uses kv head h/G), d = head_dim,
 * K = top_k, Nc = floor(Lkv/64).
 *     q_ret      [B, Lq,  Hkv, d]   dtype      retrieval query, one per kv head
 *     landmarks  [B, Hkv, Nc,  d]   dtype      one per complete chunk
 *     q_attn     [B, Lq,  Hq,  d]   dtype      attention query
 *     k, v       [B, Hkv, Lkv, d]   dtype
 *     out        [B, Lq,  Hq,  d]   dtype
 *     topk_idx   [B, Lq,  Hkv, K]   int32      chunk indices, best first
 *     topk_score [B, Lq,  Hkv, K]   float32    s of each kept chunk
 * Query row r has absolute position p = q_pos0 + r; its eligible chunks are
 * 0 .. min(floor(p/64), Nc) - 1.  Slots beyond the number of eligible chunks
 * hold index -1 and score -inf; a row with no eligible chunk outputs 0.
 *
 * Ownership: every pointer is a caller-owned device pointer on the current HIP
 * device, 16-byte aligned; outputs must not alias inputs.  The library keeps
 * no state and allocates nothing (hsa_forward_noalloc's static scratch array
 * aside): scratch memory is the caller's workspace
 * (at least hsa_workspace_size() bytes, 256-byte aligned), which may be reused
 * by calls on the same stream, for any shape.  Its first 16 KiB hold arrival
 * counters that must be zero when a call starts: zero them once after
 * allocating (hsa_workspace_init); every completed call leaves them zero.
 * `stream` is a hipStream_t (NULL: the default stream); calls only enqueue
 * work.  Concurrent calls on different streams need different workspaces.
 * A call that returns HSA_ERR_DEVICE may have launched part of its kernels
 * and left the counters non-zero: run hsa_workspace_init on the workspace
 * again before its next use.
 *
 * Errors: all argument checks run on the host before any launch.  On any error
 * nothing is launched and no output is written.  HSA_ERR_DEVICE reports a
 * failed launch.  Results are bit-identical from run to run (no floating-point
 * atomics).
 */
#ifndef HSA_H_
#define HSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HSA_OK = 0,
  HSA_ERR_NULL_POINTER = 1,        /* a required pointer is NULL */
  HSA_ERR_BAD_SHAPE = 2,           /* sizes inconsistent or out of range */
  HSA_ERR_UNSUPPORTED = 3,         /* valid but not implemented (d, G, K, dtype, flags) */
  HSA_ERR_WORKSPACE_TOO_SMALL = 4, /* ws_bytes < hsa_workspace_size() */
  HSA_ERR_DEVICE = 5,              /* a HIP launch or runtime call failed */
  HSA_ERR_MISALIGNED = 6,          /* a pointer breaks the alignment rule */
  HSA_ERR_SCRATCH_TOO_SMALL = 7    /* hsa_forward_noalloc: shape needs more than the static scratch */
} hsa_status_t;

typedef enum { HSA_DTYPE_F32 = 0, HSA_DTYPE_BF16 = 1 } hsa_dtype_t;

/* Query-key L2 normalisation of Step 3 (the paper's stability ingredient). */
#define HSA_FLAG_QK_L2NORM 0x1u

#define HSA_CHUNK_TOKENS 64 /* Step 1: fixed chunk size */
#define HSA_MAX_TOP_K 64

typedef struct {
  int32_t batch;       /* B >= 1 */
  int32_t q_len;       /* Lq >= 1 */
  int64_t kv_len;      /* Lkv >= 0 */
  int64_t q_pos0;      /* absolute position of query row 0, >= 0 */
  int32_t n_q_heads;   /* Hq */
  int32_t n_kv_heads;  /* Hkv; G = Hq/Hkv must be 1, 2, 4, 8 or 16 */
  int32_t head_dim;    /* d: 64 or 128 */
  int32_t top_k;       /* K: 1 .. 64; larger only as described at hsa_forward and hsa_backward */
  float ret_scale;     /* Step 2 scale; <= 0 means 1/sqrt(d) */
  float attn_scale;    /* Step 3 scale; <= 0 means 1/sqrt(d) */
  uint32_t flags;      /* HSA_FLAG_* */
  int32_t dtype;       /* hsa_dtype_t of q_ret, landmarks, q_attn, k, v and out */
} hsa_shape_t;

/* Validates `shape` and stores in *bytes the workspace size that
 * hsa_forward, hsa_retrieve_topk and hsa_chunk_attend_blend need for it.
 * hsa_forward and hsa_retrieve_topk also require
 * floor((q_pos0 + Lq - 1)/64) <= Nc: no row may need a chunk the history does
 * not hold (HSA_ERR_BAD_SHAPE otherwise). */
hsa_status_t hsa_workspace_size(const hsa_shape_t* shape, size_t* bytes);

/* Enqueues the zeroing of the workspace's counter region (its first 16 KiB) on
 * `stream`.  Call once per newly allocated workspace; ws_bytes >= 16384. */
hsa_status_t hsa_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Steps 1-2 (landmark scoring, causal eligibility, top-K).
 * Inputs q_ret, landmarks; outputs topk_idx, topk_score (both required).
 * Ranking uses the fp32 dot product before scaling; the order is
 * (dot product descending, chunk index ascending); -0.0 ranks equal to +0.0. */
hsa_status_t hsa_retrieve_topk(const hsa_shape_t* shape, const void* q_ret, const void* landmarks,
                               int32_t* topk_idx, float* topk_score, void* ws, size_t ws_bytes,
                               void* stream);

/* Steps 3-4 for a given selection (e.g. from hsa_retrieve_topk, or a caller's
 * own ranking).  Slot k of row (b, r, g) is used when 0 <= topk_idx < Nc;
 * other slots are skipped; a row with no used slot outputs 0.  topk_score
 * need not be sorted.  q_pos0 is not used (no causal check on a given
 * selection). */
hsa_status_t hsa_chunk_attend_blend(const hsa_shape_t* shape, const void* q_attn, const void* k,
                                    const void* v, const int32_t* topk_idx,
                                    const float* topk_score, void* out, void* ws, size_t ws_bytes,
                                    void* stream);

/* Steps 1-4.  topk_idx / topk_score may be NULL (the selection then stays in
 * the workspace) or receive the selection as hsa_retrieve_topk writes it.
 * A top_k above 64 is accepted when it covers every row's eligible chunks
 * (top_k >= min(floor((q_pos0 + Lq - 1)/64), Nc)): every eligible chunk is
 * then selected, the warm-up stage's global HSA ("Every Token Counts",
 * agent-atlas explainer, "Build Your Own" step 5).  bf16 only, and
 * topk_idx / topk_score must be NULL (HSA_ERR_UNSUPPORTED otherwise); with
 * HSA_FLAG_QK_L2NORM its workspace also holds the normalised keys of the
 * complete chunks (B * Hkv * Nc * 64 * d * 2 bytes). */
hsa_status_t hsa_forward(const hsa_shape_t* shape, const void* q_ret, const void* landmarks,
                         const void* q_attn, const void* k, const void* v, void* out,
                         int32_t* topk_idx, float* topk_score, void* ws, size_t ws_bytes,
                         void* stream);

/* hsa_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Arguments and results are those of hsa_forward; the
 * workspace is a static device array inside the library, HSA_STATIC_SCRATCH_BYTES
 * (16 MiB) per GPU, held until the process ends.  Shapes whose
 * hsa_workspace_size() exceeds it are rejected with HSA_ERR_SCRATCH_TOO_SMALL
 * before any launch (decode-sized calls fit: 16 query rows over a 16M-token
 * history with top_k 32 need about 1.6 MiB; many-row prefills do not).  The
 * call allocates nothing: on its first call on a device it takes the array's
 * address and enqueues the zeroing of its counters on `stream`.  Every call on
 * one GPU shares that GPU's array, so calls that overlap on one GPU (e.g. on
 * two streams) race; serialise them. */
#define HSA_STATIC_SCRATCH_BYTES (16u << 20)
hsa_status_t hsa_forward_noalloc(const hsa_shape_t* shape, const void* q_ret, const void* landmarks,
                                 const void* q_attn, const void* k, const void* v, void* out,
                                 int32_t* topk_idx, float* topk_score, void* stream);

/* Backward of Steps 2-4 for a given selection: the gradients of
 * sum(out * dout) with respect to q_ret, landmarks, q_attn, k and v, where out
 * is what hsa_chunk_attend_blend computes from the same selection.  The
 * selection (Step 2's top-K) is piecewise constant and carries no gradient;
 * the gradient reaches q_ret and the landmarks through the softmax blend
 * weights of the retrieval scores (Steps 2 and 4 of "How It Works
 * (Technically)"), and q_attn, k, v through each chunk's softmax attention
 * (Step 3), including the query-key L2 normalisation when the flag is set
 * (gradient of x / max(|x|, 1e-6)).
 * bf16 inputs only (HSA_ERR_UNSUPPORTED otherwise).  top_k may exceed 64:
 * the warm-up stage's global HSA (top-K spanning every eligible chunk) is
 * differentiated by passing the selection of every eligible chunk.
 *   topk_idx, topk_score [B, Lq, Hkv, top_k] as for hsa_chunk_attend_blend
 *                (slots outside [0, Nc) are unused).
 *   dout         [B, Lq, Hq, d] bf16.
 *   dq_ret       [B, Lq, Hkv, d] fp32, written.
 *   dlandmarks   [B, Hkv, Nc, d] fp32, written (zero for unselected chunks).
 *   dq_attn      [B, Lq, Hq, d] fp32, written (zero for rows with no used slot).
 *   dk, dv       [B, Hkv, kv_len, d] fp32, written (zero for unselected chunks
 *                and the trailing partial chunk).
 * Every sum runs in a fixed order, so results repeat bit for bit.  Pointers
 * 16-byte aligned, workspace 256-byte aligned and at least
 * hsa_backward_workspace_size() bytes; asynchronous on `stream`. */
hsa_status_t hsa_backward_workspace_size(const hsa_shape_t* shape, size_t* bytes);
hsa_status_t hsa_backward(const hsa_shape_t* shape, const void* q_ret, const void* landmarks,
                          const void* q_attn, const void* k, const void* v,
                          const int32_t* topk_idx, const float* topk_score, const void* dout,
                          float* dq_ret, float* dlandmarks, float* dq_attn, float* dk, float* dv,
                          void* ws, size_t ws_bytes, void* stream);

/* Landmarks of chunks [chunk_begin, chunk_end) of every (batch, kv head): the
 * mean of each chunk's 64 keys, accumulated in fp32 and stored in the shape's
 * dtype (bf16: round to nearest even).  Step 1 of "How It Works (Technically)"
 * gives every chunk one landmark from a learned encoder; without trained
 * weights this chunk mean is the stand-in.  It also keeps a KV cache's
 * landmarks current: after appending tokens to k, call it for the chunks the
 * append completed.
 * Uses shape->batch, n_kv_heads, kv_len, head_dim and dtype only.
 * k [B, Hkv, kv_len, d] is read; landmarks [B, Hkv, kv_len / 64, d] is written
 * for the chunks in the range only.  Requires 0 <= chunk_begin <= chunk_end <=
 * kv_len / 64 (HSA_ERR_BAD_SHAPE otherwise); an empty range launches nothing.
 * Pointers 16-byte aligned (HSA_ERR_MISALIGNED).  Asynchronous on `stream`. */
hsa_status_t hsa_chunk_landmarks(const hsa_shape_t* shape, const void* k, void* landmarks,
                                 int64_t chunk_begin, int64_t chunk_end, void* stream);

/* Kernel stages of a forward call, for hsa_forward_profiled.  A stage the
 * plan does not run records nothing (e.g. MERGE when the attend merges the
 * per-split candidate lists itself, BUCKET and COMBINE outside the chunk-major
 * attend). */
typedef enum {
  HSA_STAGE_SCAN = 0,     /* landmark scoring + per-split / per-row top-K        */
  HSA_STAGE_MERGE = 1,    /* merge of per-split candidate lists (separate kernel) */
  HSA_STAGE_BUCKET = 2,   /* chunk-major attend: bucketing of (row, slot) pairs   */
  HSA_STAGE_ATTEND = 3,   /* per-chunk attention (with the blend where fused)     */
  HSA_STAGE_COMBINE = 4,  /* chunk-major attend: slot-ordered blend of partials   */
  HSA_STAGE_COUNT = 5
} hsa_stage_t;

/* hsa_forward, with caller-owned HIP events (hipEvent_t, passed as void*)
 * recorded on `stream` around each kernel stage: stage_events[2*s] before the
 * stage's first kernel and stage_events[2*s + 1] after its last, for
 * s < HSA_STAGE_COUNT.  stage_events may be NULL and any entry may be NULL
 * (nothing recorded).  The library keeps no reference to the events.  An event
 * record failure returns HSA_ERR_DEVICE.  Diagnostics for per-kernel timing;
 * outputs are those of hsa_forward. */
hsa_status_t hsa_forward_profiled(const hsa_shape_t* shape, const void* q_ret,
                                  const void* landmarks, const void* q_attn, const void* k,
                                  const void* v, void* out, int32_t* topk_idx, float* topk_score,
                                  void* ws, size_t ws_bytes, void* stream,
                                  void* const* stage_events);

/* hsa_backward with stage events as for hsa_forward_profiled: BUCKET = pair
 * bucketing and the per-bin sort, ATTEND = the per-item MFMA kernel,
 * COMBINE = the per-row, per-chunk and per-landmark reductions (SCAN and MERGE
 * record nothing).  Outputs are those of hsa_backward. */
hsa_status_t hsa_backward_profiled(const hsa_shape_t* shape, const void* q_ret, const void* landmarks,
                                   const void* q_attn, const void* k, const void* v,
                                   const int32_t* topk_idx, const float* topk_score,
                                   const void* dout, float* dq_ret, float* dlandmarks,
                                   float* dq_attn, float* dk, float* dv, void* ws, size_t ws_bytes,
                                   void* stream, void* const* stage_events);

/* Static description of a status code. */
const char* hsa_status_string(hsa_status_t status);

/* Library version as major*10000 + minor*100 + patch. */
int32_t hsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HSA_H_ */
