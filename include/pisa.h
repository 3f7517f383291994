/*
 * pisa.h - C ABI of the MI355X (gfx950) PISA hot path: key pyramid, hierarchical
 * LogSumExp block selection, block-sparse attention and the decode step.
 *
 * The method is the one described on the paper-summary page "Block Sparse
 * Attention with Log-Linear Complexity" (Tang, Qin, Pan, Li, Liu).  Section
 * names below refer to that page: Prerequisites (block sparse attention,
 * LogSumExp, grouped-query attention), Core method (pyramid eq. 10-15,
 * routing eq. 16-20, LSE score eq. 21) and Method steps (pyramid mean,
 * Stage 1 head sum eq. 22, Stage 2 leaf LSE, final top-K, decode update,
 * attention on the selected leaves).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or keeps device memory and never synchronises the
 *    stream: every call only validates its arguments on the host and enqueues
 *    kernels on `stream` (a hipStream_t passed as void*; NULL = default
 *    stream).  Inputs must stay alive until the stream has passed the call.
 *  - Token-major tensors (Q, K, V, O, KV caches) are described by pisa_tensor:
 *    element [b][t][h][c] lives at ptr + b*stride_b + t*stride_t + h*stride_h + c
 *    (strides in ELEMENTS, the head_dim axis contiguous).  The pointer must be
 *    16-byte aligned and every stride a multiple of 8 elements.
 *  - GQA: query head h belongs to KV head h / G with G = n_q_heads / n_kv_heads
 *    (contiguous groups).
 *  - The pyramid is float32, [batch][n_kv_heads][nodes(capacity)][head_dim],
 *    levels stored leaf level first: level 1 (leaves, M_1 = ceil(cap / 64)
 *    nodes) at node offset 0, then level 2 (M_2 = ceil(M_1 / 2) nodes), ...,
 *    up to the level with one node.  For a current length n <= capacity only
 *    the first ceil(n / 64), ceil(ceil(n/64)/2), ... nodes of each level are
 *    meaningful; the root of length n is node 0 of level L(n).
 *  - Selections are int32 [batch][n_kv_heads][tokens][top_k]: leaf-block ids in
 *    ascending order, padded with -1.  Block j covers keys [64 j, 64 j + 64).
 *  - Errors: arguments are checked before anything is enqueued; a non-zero
 *    pisa_status means nothing was launched, except PISA_ERR_HIP, which means a
 *    launch failed (pisa_last_hip_error() then returns the hipError_t value of
 *    the calling thread's last failure).  No C++ exception crosses the ABI.
 *  - Debug mode: when the environment variable PISA_SYNC_LAUNCHES holds a value
 *    other than "0" at the library's first launch, every launch waits for its
 *    stream (hipStreamSynchronize), so an asynchronous fault or error of a kernel
 *    is returned as PISA_ERR_HIP by the entry point that launched it.  This is the
 *    one exception to "never synchronises"; do not use it under stream capture.
 *  - Thread safety: no global mutable state besides the thread-local error code,
 *    the thread-local stage events of pisa_stage_events and the per-device
 *    address of the fixed array behind pisa_sparse_attn_fwd_noalloc (set once,
 *    under a lock).
 */
#ifndef PISA_H_
#define PISA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PISA_ABI_VERSION 7

typedef enum {
  PISA_OK = 0,
  PISA_ERR_INVALID_ARG = 1,   /* null pointer, bad shape, misaligned pointer or stride */
  PISA_ERR_UNSUPPORTED = 2,   /* valid request outside the supported envelope */
  PISA_ERR_WORKSPACE = 3,     /* workspace pointer null or smaller than required */
  PISA_ERR_HIP = 4            /* a kernel launch failed */
} pisa_status;

typedef enum { PISA_F32 = 0, PISA_BF16 = 1 } pisa_dtype;
/* Fields and arguments that take a pisa_dtype or pisa_score value are declared int32_t, so any
 * value a caller passes is representable and an unknown one is rejected as
 * PISA_ERR_INVALID_ARG (an enum type cannot hold a value outside its enumerators in C++). */

/*
 * Problem description.  Supported envelope: block == 64 (C), fanout == 2 (g),
 * head_dim in {64, 128}, n_q_heads % n_kv_heads == 0 with G = n_q_heads /
 * n_kv_heads in {1, 2, 4, 8, 16}, 1 <= top_k <= 32, seq_len >= 1 and
 * seq_len * 2 * top_k < 2^31.  scale <= 0 selects 1/sqrt(head_dim), the scale
 * of the LSE score (Core method, eq. 21), also used by attention.
 */
/* Candidate score from the logits of a candidate's valid children (raw keys <= t
 * at the leaf level).  PISA_SCORE_LSE is the method's log-sum-exp (Core method
 * eq. 21); PISA_SCORE_MEAN and PISA_SCORE_MEAN_VAR are its first- and
 * second-order truncations from the Taylor expansion of the LSE (Core method; the
 * PISA-1 and PISA-2 variants): the mean, and the mean plus half the population
 * variance, of the valid children's logits, without the log(count) term.  Scores
 * are summed over the group's query heads in every case. */
typedef enum { PISA_SCORE_LSE = 0, PISA_SCORE_MEAN = 1, PISA_SCORE_MEAN_VAR = 2 } pisa_score;

typedef struct {
  int32_t batch;        /* B */
  int32_t seq_len;      /* N for prefill; KV-cache capacity for decode */
  int32_t n_q_heads;    /* H_q */
  int32_t n_kv_heads;   /* H_kv */
  int32_t head_dim;     /* d */
  int32_t block;        /* C, leaf block size: must be 64 */
  int32_t fanout;       /* g, children per node above the leaves: must be 2 */
  int32_t top_k;        /* K, leaf blocks kept per (token, KV head) */
  int32_t dtype;        /* a pisa_dtype: element type of Q, K, V, O and the KV caches */
  float scale;          /* logit scale; <= 0 means 1/sqrt(head_dim) */
  int32_t score;        /* a pisa_score: candidate score at every level (routing, leaves, decode) */
} pisa_cfg;

typedef struct { const void* ptr; int64_t stride_b, stride_t, stride_h; } pisa_tensor;
typedef struct { void* ptr; int64_t stride_b, stride_t, stride_h; } pisa_tensor_mut;

/* ABI version of the loaded library (PISA_ABI_VERSION). */
int pisa_abi_version(void);

/* Static description of a status code. */
const char* pisa_status_string(int32_t status);

/* hipError_t of the calling thread's last failed launch (0 if none). */
int pisa_last_hip_error(void);

/* Timing hook: hands the calling thread `count` hipEvent_t handles (as void*,
 * created by the caller) for its NEXT entry-point call, which records
 * events[i] on its stream right after enqueueing its i-th kernel (in launch
 * order; events beyond the kernels it launches stay unrecorded) and then drops
 * the list, also when it returns an error.  Recording the same event twice in
 * one call is the caller's choice.  The array must stay valid during that
 * call.  Kernels per call: build_pyramid 1 or 2 (leaves, then the top levels
 * above 8 leaves); select_blocks 5 or 6 (split summaries for bf16 inputs,
 * routing, clustering, packing of K for bf16 inputs, leaf LSE, top-K);
 * sparse_attn_fwd with bf16 inputs 1 + passes, or 8 + passes up to 16384 leaf
 * blocks (packing of K and V; the seven kernels of the passes' token order:
 * clear, adjacent-token share, block counts, keys, per-key prefix over chunks,
 * key starts, scatter; then one launch per pass), fp32 inputs 1; decode_step 1;
 * select_flat 3.  count = 0 clears the list.  Returns PISA_ERR_INVALID_ARG
 * for count < 0 or a null array or handle. */
pisa_status pisa_stage_events(void* const* events, int32_t count);

/* Nodes per (sequence, KV head) of a pyramid with room for `capacity` keys:
 * sum over levels of ceil(capacity / 64), then repeated ceil(/2) down to 1.
 * Returns 0 for capacity < 1. */
int64_t pisa_pyramid_nodes(int32_t capacity);

/* Bytes of a pyramid for cfg->batch * cfg->n_kv_heads sequences of `capacity` keys. */
size_t pisa_pyramid_bytes(const pisa_cfg* cfg, int32_t capacity);

/*
 * build_pyramid - mean-pooled key pyramid (Method steps, first step; Core
 * method eq. 10-15).  Leaf i of each (b, kvh) is the float32 mean of keys
 * [64 i, min(64 i + 64, n)) summed in key order; a node above is the mean of
 * its one or two children, (c0 + c1) * 0.5 (the unweighted mean, also for
 * partial nodes).  Writes levels for length n into `pyr`, laid out for
 * `capacity` (>= n) keys as described above.
 *   k    : [B][>= n][H_kv][d] keys, cfg->dtype
 *   pyr  : float32 output, pisa_pyramid_bytes(cfg, capacity) bytes
 */
pisa_status pisa_build_pyramid(const pisa_cfg* cfg, pisa_tensor k, int32_t n, int32_t capacity,
                               float* pyr, void* stream);

/* Workspace bytes needed by pisa_select_blocks for cfg (256-byte aligned pieces). */
size_t pisa_select_workspace_bytes(const pisa_cfg* cfg);

/*
 * select_blocks - hierarchical top-K leaf selection for every query token t
 * in [0, N) of every (b, kvh) (Core method eq. 16-21; Method steps eq. 22 and
 * the two selection stages).  From the root, each level with more than K
 * candidates scores every candidate by u = sum over the group's query heads of
 * the LSE of the head's scaled dot products with the candidate's causally
 * valid children (node (l, i) is valid for t when its first key
 * i * 64 * 2^(l-1) <= t), keeps K by (u descending, index ascending) and
 * expands the survivors to their valid children.  The leaf level scores the
 * at most 2K candidate leaves exactly over their raw keys at positions <= t.
 * Precision: products of raw inputs are exact with float32 sums.  For bf16
 * inputs the float32 summaries above the leaves enter the dot products as a
 * bf16 part plus a float16 remainder scaled by 2^10 (about 2^-20 relative
 * error per element); float32 inputs use the summaries as they are.  With
 * every score, bf16 routing first scores each level from a float16 copy of
 * the summaries with a bound on its distance to the split score, and scores
 * again from both split parts only the candidates the bound leaves
 * undecided; the kept sets are those of scoring every candidate from both
 * parts (which the environment variable PISA_ROUTE_EXACT=1 forces).
 *   q, k    : [B][N][H_q][d] and [B][N][H_kv][d], cfg->dtype
 *   pyr     : pyramid of k built with n = N (capacity N)
 *   sel     : int32 [B][H_kv][N][K] output, ascending, -1 padded
 *   sel_u   : optional float32 [B][H_kv][N][K] output (NULL to skip): the leaf
 *             score u of each selected block, -inf on padding
 *   ws      : workspace of >= pisa_select_workspace_bytes(cfg) bytes (for
 *             bf16 inputs it also holds the split summaries, their float16
 *             copy with two bounds per node, and packed copies of K and Q,
 *             about the size of q plus k); its first
 *             B*H_kv*N*2K int32 hold the leaf candidates of each token (-1
 *             padded) after the call
 * Returns PISA_ERR_UNSUPPORTED for N > 1000000 (the leaf clustering keeps a
 * counter per leaf block of the sequence in LDS).
 */
pisa_status pisa_select_blocks(const pisa_cfg* cfg, pisa_tensor q, pisa_tensor k, const float* pyr,
                               int32_t* sel, float* sel_u, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes needed by pisa_select_flat for cfg (summed query groups and leaf
 * means, both float32 in MFMA fragment order). */
size_t pisa_flat_workspace_bytes(const pisa_cfg* cfg);

/*
 * select_flat - the single-level block selection of the block-sparse framework
 * (Prerequisites: block sparse attention / top-K block selection and
 * grouped-query attention), the O(N^2 / C) scan that hierarchical routing
 * replaces; provided as the baseline to measure routing against.  Every leaf j
 * with 64 j <= t is scored by u = sum over the group's query heads of
 * q_h . k_bar_j * scale, k_bar_j the leaf mean of the pyramid (built over the
 * whole block), and K leaves are kept by (u descending, index ascending).
 *   q       : [B][N][H_q][d], cfg->dtype
 *   pyr     : pyramid of k built with n = N (capacity N); only the leaves are read
 *   sel     : int32 [B][H_kv][N][K] output, ascending, -1 padded
 *   sel_u   : optional float32 [B][H_kv][N][K] output (NULL to skip), -inf on padding
 *   ws      : workspace of >= pisa_flat_workspace_bytes(cfg) bytes
 * Returns PISA_ERR_UNSUPPORTED for K > 16.
 */
pisa_status pisa_select_flat(const pisa_cfg* cfg, pisa_tensor q, const float* pyr, int32_t* sel, float* sel_u,
                             void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes needed by pisa_sparse_attn_fwd for cfg: bf16 inputs stage K and
 * V as packed 64-key blocks, each fragment of the attention products one
 * contiguous run (2 * B * H_kv * ceil(N / 64) * 64 * d * 2 bytes, each half
 * rounded up to 256 bytes), followed by B * H_q * N * 8 bytes (rounded up to
 * 256) for the softmax state carried between the two passes of a float32-output
 * call (even block ids, then odd ones; the output rows hold the partial sums
 * between them), then, up to 16384 leaf blocks (N <= 1048576), the arrays that
 * order each pass's tokens: B * H_kv * ceil(N / 64) block counts, 2 * B * H_kv *
 * (ceil(N / 64) + 1) * ceil(N / 4096) key counts per chunk of 4096 tokens,
 * 2 * B * H_kv * (ceil(N / 64) + 1) key totals, two 64-bit statistics,
 * 2 * B * H_kv * N token keys and 2 * B * H_kv * N token positions (4 bytes
 * each, every array rounded up to 256); fp32 inputs need none (0). */
size_t pisa_attn_workspace_bytes(const pisa_cfg* cfg);

/*
 * sparse_attn_fwd - causal softmax attention of each query head over the raw
 * keys/values of its group's selected blocks (Prerequisites, block sparse
 * attention; Method steps, fourth step): the key set of token t is the union
 * of blocks in sel[b][kvh][t] cut to positions <= t; fp32 accumulation.
 *   q, k, v : cfg->dtype, shapes as in select_blocks (v like k)
 *   sel     : int32 [B][H_kv][N][K]; the key set of token t is the union of
 *             the listed blocks j with 0 <= j <= t / 64: entries < 0, entries
 *             past t / 64 and repeats of an id listed earlier in the row are
 *             skipped, so any int32 content is memory-safe (a token with no
 *             such block gets a zero row and row LSE -inf)
 *   o       : [B][N][H_q][d] output of element type o_dtype (float32 keeps the
 *             fp32 accumulator; bfloat16 rounds it to nearest-even).  With bf16
 *             inputs and a float32 output the call runs two passes, even then odd
 *             block ids, and the rows of o hold the first pass's unnormalised sums
 *             until the second pass writes the final values; o must not alias q,
 *             k, v or sel
 *   row_lse : optional float32 [B][H_q][N] output (NULL to skip): natural-log
 *             normaliser of each row's softmax
 *   ws      : workspace of >= pisa_attn_workspace_bytes(cfg) bytes (may be NULL
 *             when that is 0), 256-byte aligned
 * With bf16 inputs the passes visit tokens either in position order or, when
 * the selections' blocks are listed by the previous token less than a quarter
 * of the time (measured on the device, per call), sorted by each token's
 * smallest block of the pass selected at most 4 * 64 * K times (ties in
 * position order), in eight contiguous slices, one per XCD, so tokens sharing
 * such a block meet in one L2.
 * Either way every row is computed from its own selection alone: the outputs
 * are the same bit for bit.
 */
pisa_status pisa_sparse_attn_fwd(const pisa_cfg* cfg, pisa_tensor q, pisa_tensor k, pisa_tensor v,
                                 const int32_t* sel, pisa_tensor_mut o, int32_t o_dtype, float* row_lse,
                                 void* ws, size_t ws_bytes, void* stream);

/* Size of the device array behind pisa_sparse_attn_fwd_noalloc (one per GPU). */
#define PISA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/*
 * sparse_attn_fwd_noalloc - for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same computation, arguments and errors as sparse_attn_fwd, but
 * the workspace is a fixed array of PISA_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held from the first call on that GPU until the process
 * ends; nothing is allocated or freed.  Returns PISA_ERR_WORKSPACE, before
 * touching the device, when pisa_attn_workspace_bytes(cfg) exceeds
 * PISA_NOALLOC_SCRATCH_BYTES (128 MiB: e.g. bf16 inputs with d = 128, 16
 * query heads per KV head and B * H_kv * N up to about 200K tokens), and
 * PISA_ERR_HIP if the array's device address cannot be obtained.  Every call
 * on one GPU uses the same array and leaves its contents behind (each call
 * writes all it reads first, so no clearing is needed): calls that overlap on
 * one GPU (on several streams or threads) race and must be serialised by the
 * caller.
 */
pisa_status pisa_sparse_attn_fwd_noalloc(const pisa_cfg* cfg, pisa_tensor q, pisa_tensor k, pisa_tensor v,
                                         const int32_t* sel, pisa_tensor_mut o, int32_t o_dtype,
                                         float* row_lse, void* stream);

/* Workspace bytes needed by pisa_sparse_attn_bwd for cfg (0 for an unsupported
 * cfg): packed copies of K and V (2 * B * H_kv * ceil(N / 64) * 64 * d * 2
 * bytes), a record per token and KV head (its queries and upstream gradients
 * in bf16 and row statistics: 8320 bytes at d = 128, 4224 at d = 64), the
 * inverse of the selection lists, and per-item
 * dk / dv partial sums (about (B * H_kv * N * K / 512 + B * H_kv * ceil(N / 64))
 * * 64 * d * 8 bytes). */
size_t pisa_attn_bwd_workspace_bytes(const pisa_cfg* cfg);

/*
 * sparse_attn_bwd - gradients of sparse_attn_fwd (Prerequisites, block sparse
 * attention; Method steps, fourth step) with the selected sets held fixed: the
 * page calls the method trainable but states no gradient, and the selection is
 * piecewise constant in q and k, so only the softmax attention over the
 * selected keys is differentiated.  For token t, head h and selected key r:
 * P = softmax(scale q . k_r), dv_r += P dO, dS = P (dO . v_r - dO . O),
 * dq = scale sum_r dS k_r, dk_r += scale dS q.
 *   q, k, v  : bfloat16 (cfg->dtype must be PISA_BF16), as in sparse_attn_fwd
 *   sel      : int32 [B][H_kv][N][K] as given to sparse_attn_fwd; an entry takes
 *              part if 0 <= j <= t / 64 and no earlier slot of the row lists
 *              j (select_blocks rows always satisfy this)
 *   o, dout  : [B][N][H_q][d] forward output and its upstream gradient, both of
 *              element type grad_dtype (float32 or bfloat16); dout enters the
 *              products rounded to bfloat16
 *   row_lse  : float32 [B][H_q][N], the row LSE written by sparse_attn_fwd
 *   dq       : float32 [B][N][H_q][d] output (every row written; zero for a
 *              token with no block in use)
 *   dk, dv   : float32 [B][N][H_kv][d] outputs (every row written; zero for
 *              keys no token selects)
 *   ws       : workspace of >= pisa_attn_bwd_workspace_bytes(cfg) bytes,
 *              256-byte aligned
 * Products run on bf16 MFMA with fp32 accumulation; P and dS enter the second
 * products rounded to bfloat16.  Results are deterministic (no atomics).
 * Returns PISA_ERR_UNSUPPORTED for fp32 inputs, for ceil(N / 64) > 8192 and
 * when B * H_kv * N * K exceeds 2^31 - 1.
 */
pisa_status pisa_sparse_attn_bwd(const pisa_cfg* cfg, pisa_tensor q, pisa_tensor k, pisa_tensor v,
                                 const int32_t* sel, pisa_tensor o, pisa_tensor dout, int32_t grad_dtype,
                                 const float* row_lse, pisa_tensor_mut dq, pisa_tensor_mut dk, pisa_tensor_mut dv,
                                 void* ws, size_t ws_bytes, void* stream);

/*
 * decode_step - one autoregressive step for every sequence (Method steps,
 * third step): writes k_new / v_new at position n_ctx of the caches, updates
 * the leaf n_ctx / 64 and its ancestor path in `pyr` (same arithmetic and
 * order as build_pyramid, so the result equals a rebuild at length n_ctx + 1),
 * then routes the new query at t = n_ctx (every key valid) through all levels
 * with exact leaf LSE in one fused kernel and attends over the selected blocks.
 *   cfg->seq_len      : cache capacity; requires n_ctx + 1 <= capacity
 *   n_ctx             : keys already in the cache (same for every sequence)
 *   q                 : [B][H_q][d]    (stride_t ignored)
 *   k_new, v_new      : [B][H_kv][d]   (stride_t ignored)
 *   k_cache, v_cache  : [B][capacity][H_kv][d] by their strides, updated in place.  Any
 *                       strides with d contiguous; a head-major cache (stride_t = d,
 *                       stride_h = capacity * d) keeps each leaf's 64 keys in one
 *                       contiguous 16 KB run at d = 128 and bf16, which the leaf
 *                       scoring reads faster than rows 2 KB apart (token-major, 8 KV heads)
 *   pyr               : pyramid of the cache (capacity layout), updated in place
 *   sel_out           : optional int32 [B][H_kv][K] (NULL to skip)
 *   o                 : [B][H_q][d] output of element type o_dtype (stride_t ignored)
 * Requires G * 2K <= 256 (leaf logits are staged on chip).
 */
pisa_status pisa_decode_step(const pisa_cfg* cfg, int32_t n_ctx, pisa_tensor q, pisa_tensor k_new,
                             pisa_tensor v_new, pisa_tensor_mut k_cache, pisa_tensor_mut v_cache,
                             float* pyr, int32_t* sel_out, pisa_tensor_mut o, int32_t o_dtype,
                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PISA_H_ */
