/*
 * csa2.h -- C ABI of the MI355X (gfx950) CSA2 hot-path library, libcsa2.so.
 *
 * CSA2 (Compressed Sparse Attention 2) step of DeepSeek V4.1 Flash's global
 * attention branch: for each query token, score every compressed KV entry with
 * the lightning indexer, keep the top-k, gather those entries (optionally
 * decoding FP4 E2M1 values with one E4M3 scale per 16 channels) and run softmax
 * attention of every query head over that one shared entry set.  Layers run in
 * Full, Reindex or Reuse mode.
 *
 * Conventions for every entry point
 *  - Tensor arguments are DEVICE pointers owned by the caller, row-major and
 *    contiguous (last dimension fastest), 16-byte aligned.  The library never
 *    allocates, frees or keeps them after the call returns.
 *  - Temporary memory comes only from the caller's workspace (ws, ws_bytes),
 *    sized by the matching *_workspace_size function; NULL with 0 bytes is
 *    allowed when that function returns 0.  Workspace must be 256-byte aligned.
 *  - `stream` is the caller's hipStream_t passed as void * (so that this header
 *    needs no HIP include; NULL = the default stream).  Work is
 *    enqueued asynchronously on it; no call synchronises with the host, and no
 *    call records a memset node, so a call may be captured into a HIP graph.
 *  - Return value: CSA2_OK, or an error status.  Arguments are validated before
 *    anything is enqueued, so a call that fails validation has no effect.
 *    CSA2_EHIP means a launch failed (state of the outputs undefined).  The
 *    message of the last failure on the calling thread is csa2_last_error().
 *    No C++ exception crosses this interface.
 *  - Preconditions that are documented but not checked: floating inputs are
 *    finite; outputs do not alias inputs; candidate rows are strictly
 *    ascending over their non-negative entries; the stream is valid on the
 *    current device.
 *  - B * Q (query rows per call) is at most 65535; larger calls return
 *    CSA2_EUNSUPPORTED before anything is enqueued.
 *  - Calls that overlap on one stream are ordered by that stream; concurrent
 *    calls on different streams must use different workspaces.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_API __attribute__((visibility("default")))

typedef enum {
    CSA2_OK = 0,
    CSA2_EINVAL = 1,       /* bad argument (null pointer, size, alignment, mode/pointer mismatch) */
    CSA2_EUNSUPPORTED = 2, /* valid request with no kernel (e.g. dtype/shape combination) */
    CSA2_EWORKSPACE = 3,   /* workspace smaller than *_workspace_size */
    CSA2_EHIP = 4,         /* a HIP launch or runtime call failed */
    CSA2_EINTERNAL = 5     /* unexpected internal failure */
} csa2_status;

/* Element formats.
 * CSA2_F32, CSA2_BF16: plain rows of D elements.
 * CSA2_FP4: a row of D channels is D/2 + D/16 bytes: D/2 bytes of 4-bit E2M1
 *   codes (channel 2i in the low nibble of byte i, channel 2i+1 in the high
 *   nibble), then D/16 E4M3 ("FN", OCP 8-bit float) scale bytes, scale b
 *   covering channels 16b..16b+15.  Value = e2m1(code) * e4m3(scale), which
 *   is exactly representable in bf16.  ("Recall之王 祭出Reuse", section
 *   "把KV Cache压到极致的几把杀手锏": FP4 main KV cache, E2M1 with one E4M3
 *   scale per 16 channels.)  Every scale byte is accepted: zero and negative
 *   zero, subnormals and sign-set bytes are their E4M3 values; the E4M3 NaN
 *   code S.1111.111 (never written by csa2_quantize_fp4) saturates to +-448.
 *   Main KV, and indexer keys (csa2_index_score).
 *   CSA2_FP4E2M1_S16E4M3 is the same format under its descriptive name.
 * CSA2_FP4QK (indexer only): FP4 indexer queries and keys -- qI holds one FP4
 *   row of dI channels per head and kI one per entry, both in the CSA2_FP4
 *   layout.  "读完这篇，你就搞懂 DeepSeek v4 了", the passage on V4's FP4
 *   quantization-aware training: the lightning indexer's q and K are FP4. */
typedef enum { CSA2_F32 = 0, CSA2_BF16 = 1, CSA2_FP4 = 2, CSA2_FP4E2M1_S16E4M3 = 2, CSA2_FP4QK = 3 } csa2_dtype;

/* The value the layer's top-k ranks (csa2_layer_args.score_fmt).
 *   CSA2_SCORE_F64  -- the binary64 score of the indexer formula (default).
 *   CSA2_SCORE_BF16 -- that score rounded once to bfloat16 (nearest, ties to
 *                      the even significand, straight from binary64; past the
 *                      largest finite value it becomes infinite).  Same
 *                      passage: the indexer's score is quantized only down to
 *                      BF16, since top-k ranks it.  Equal rounded scores are
 *                      ordered by entry index like any tie, so the choice
 *                      differs from CSA2_SCORE_F64's where scores that round
 *                      alike straddle the cut. */
typedef enum { CSA2_SCORE_F64 = 0, CSA2_SCORE_BF16 = 1 } csa2_score_fmt;

/* Layer modes (V4.1 Flash video transcript on prism.simon-ai.net, the passage
 * introducing CSA2's three modes; "Recall之王 祭出Reuse", same section):
 *   CSA2_FULL    -- run the indexer over every visible entry, keep top-k (and
 *                   optionally the top-P candidate pool), attend.
 *   CSA2_REINDEX -- reuse the shared main KV and indexer keys; score only the
 *                   candidate pool with this layer's own indexer queries, keep
 *                   top-k of the pool, attend.
 *   CSA2_REUSE   -- reuse main KV and the previous top-k indices; no indexer,
 *                   attention only. */
typedef enum { CSA2_FULL = 0, CSA2_REINDEX = 1, CSA2_REUSE = 2 } csa2_mode;

/* ---------------------------------------------------------------------------
 * csa2_compress -- token compression into compressed entries.
 *
 * "读完这篇，你就搞懂 DeepSeek v4 了" (note.crab.center): the HCA "压缩机制"
 * paragraphs (eqs. 10, 11) define CSA's compression by contrast -- groups of m
 * tokens, two consecutive groups concatenated, a per-channel softmax weight
 * over a projection Z plus a learnable bias B.  Reading taken: entry i pools
 * the previous and its own group (2m tokens); for channel c and window
 * position r (0..2m-1, token t):
 *     l_r[c] = sum_d x_t[d] * wz[d][c] + bias[r][c]
 *     out_i[c] = sum_r softmax_r(l[c]) * x_t[c]
 * Window positions before token 0 are dropped.
 *
 * x:    [rows, D] in dt (CSA2_F32 or CSA2_BF16).  halo = 0: rows = n_out*m and
 *       x starts at token 0.  halo = 1: rows = (n_out+1)*m, the first m rows
 *       are the previous group of the first output entry.
 * wz:   [D, D] in dt.  bias: [2m, D] fp32.  out: [n_out, D] in dt (fp32 math,
 *       rounded to nearest even on store).
 * Limits: 1 <= m <= 16, D % 16 == 0, n_out >= 1.
 * ------------------------------------------------------------------------- */
CSA2_API size_t csa2_compress_workspace_size(int dt, int64_t n_out, int32_t D, int32_t m, int32_t halo);
CSA2_API int csa2_compress(const void *x, int dt, int64_t n_out, int32_t D, int32_t m, int32_t halo,
                           const void *wz, const float *bias, void *out, void *ws, size_t ws_bytes,
                           void *stream);

/* ---------------------------------------------------------------------------
 * csa2_quantize_fp4 -- FP4 rows for main-KV cache writes.
 *
 * "Recall之王 祭出Reuse", section "把KV Cache压到极致的几把杀手锏": the main KV
 * cache holds E2M1 values with one E4M3 scale per 16 channels.  Reading (the
 * pages give no recipe), per group of 16 channels: the scale is the smallest
 * non-negative E4M3 value s with 6 s >= the group's largest |x| (448 if none
 * is, then codes saturate at +-6); each code is the E2M1 value nearest to
 * x / s, ties to the even code, a zero stored as +0 (s = 0: all codes 0).
 * Typical use, decode-time append: csa2_compress of the last 2m tokens
 * (n_out = 1, halo = 1) into a bf16 row, then this call into the cache.
 *
 * x [n, D] in dt (CSA2_F32 or CSA2_BF16), finite, D % 16 == 0.
 * cache: FP4 rows of D/2 + D/16 bytes (layout as CSA2_FP4); row r of x is
 *   written to cache row dst_row[r] (int64 [n] on the device), or to row r
 *   when dst_row is NULL.  Destination rows must be distinct; other rows of
 *   the cache are not touched.  Bit-exact: the result does not depend on n.
 * ------------------------------------------------------------------------- */
CSA2_API int csa2_quantize_fp4(const void *x, int dt, int64_t n, int32_t D, void *cache, const int64_t *dst_row,
                               void *stream);

/* ---------------------------------------------------------------------------
 * csa2_index_score -- lightning-indexer scores.
 *
 * "读完这篇，你就搞懂 DeepSeek v4 了", section "闪电索引机制（对应步骤二）", eq. (8):
 * every compressed entry is scored against the query token per indexer head,
 * head scores are weighted and summed (DSA of V3.2, with its per-head ReLU):
 *     s(j) = sum_h w_h * ReLU(qI_h . kI_j)
 * One key row per entry is shared by all heads.
 *
 * qI [B,Q,HI,dI] and kI [B,N,dI] in dt (CSA2_F32 or CSA2_BF16); w [B,Q,HI] fp32.
 * dt = CSA2_FP4: FP4 indexer keys -- kI holds FP4 rows of dI/2 + dI/16 bytes
 *   (layout as CSA2_FP4, e.g. written by csa2_quantize_fp4) and qI is bf16.
 * dt = CSA2_FP4QK: FP4 queries too -- qI holds [B,Q,HI] FP4 rows of the same
 *   width, decoded exactly (into bf16, in the workspace) before scoring.
 *   Both FP4 forms need dI % 64 == 0 and a matrix-core shape.  Same page,
 *   the passage on V4's FP4 indexer q/K (the score is held at higher
 *   precision: here fp32 with the bound below; csa2_layer can rank it
 *   rounded to bf16, see csa2_score_fmt).
 * q_pos [B,Q] absolute token positions, or NULL: with q_pos, entry j is visible
 *   to the query only if (j+1)*m <= q_pos+1 (complete groups); without it all
 *   N entries are visible.
 * cand [B,Q,P] or NULL: with cand, slot p scores entry cand[p]; -1 = empty.
 * scores [B,Q,N] (or [B,Q,P]) fp32 out; invisible entries and empty slots get
 *   -inf.  Accumulation order is the kernel's (matrix cores for bf16).
 * err [B,Q] fp32 out or NULL: a rigorous per-query bound E with
 *   |scores - s_exact| <= E for every scored entry, where s_exact is the
 *   binary64 value of the formula in its sequential order.
 * ------------------------------------------------------------------------- */
CSA2_API size_t csa2_index_score_workspace_size(int dt, int32_t B, int32_t Q, int32_t HI, int32_t dI, int64_t N,
                                                int32_t P);
CSA2_API int csa2_index_score(const void *qI, const float *w, const void *kI, int dt, int32_t B, int32_t Q,
                              int32_t HI, int32_t dI, int64_t N, const int64_t *q_pos, int32_t m,
                              const int32_t *cand, int32_t P, float *scores, float *err, void *ws,
                              size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * csa2_topk -- exact top-k of given fp32 scores.
 *
 * Same section of the same page: keep the k highest-scoring entries.  Order is
 * (score descending, entry index ascending); slots scoring -inf, and slots
 * whose cand entry is -1, are never kept.  Output: the kept entry indices in
 * ascending order, then -1 padding; count = number kept = min(k, selectable).
 *
 * scores [B,Q,n] fp32; cand [B,Q,n] or NULL (entry index of slot p is cand[p],
 *   else p; cand rows must be strictly ascending over their non-negative
 *   entries, which the pool produced by csa2_layer is -- not checked).
 *   A slot a query may not select (past its visible count, or an empty
 *   candidate) is given as a -inf score, which is how csa2_index_score marks
 *   invisible entries; there is no separate per-query valid count.  Scores
 *   must not be NaN (a NaN has no place in the order; the result is then
 *   unspecified).
 * idx [B,Q,k] int32 out; count [B,Q] int32 out or NULL.  1 <= k.
 * The result is bit-exact (pure comparison, no arithmetic on the scores).
 * ------------------------------------------------------------------------- */
CSA2_API size_t csa2_topk_workspace_size(int32_t B, int32_t Q, int64_t n, int32_t k);
CSA2_API int csa2_topk(const float *scores, int32_t B, int32_t Q, int64_t n, const int32_t *cand, int32_t k,
                       int32_t *idx, int32_t *count, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * csa2_sparse_attn -- gather + (FP4 decode) + shared-KV attention.
 *
 * Same page, section "注意力计算（对应步骤三）", eq. (9): standard attention
 * with shared KV -- the k entries kept by the indexer form one matrix C that
 * every query head uses as both keys and values:
 *     a_j = scale * q_h . C_j,  o_h = sum_j softmax(a)_j C_j,  lse_h = logsumexp(a)
 *
 * q [B,Q,H,D] in q_dt (CSA2_F32 or CSA2_BF16); kv [B,N,row] in kv_dt
 *   (CSA2_F32, CSA2_BF16 or CSA2_FP4; FP4 needs q_dt = CSA2_BF16).
 * idx [B,Q,k] int32 entry indices in [0, N) or -1 (skipped).
 * out [B,Q,H,D] in q_dt; lse [B,Q,H] fp32 or NULL.  A query with no listed
 *   entry gets out = 0 and lse = -inf.
 * The result for one query does not depend on B, Q or the other queries
 *   (fixed split of the k entries, fixed reduction order).
 * ------------------------------------------------------------------------- */
CSA2_API size_t csa2_sparse_attn_workspace_size(int q_dt, int kv_dt, int32_t B, int32_t Q, int32_t H, int32_t D,
                                                int32_t k);
CSA2_API int csa2_sparse_attn(const void *q, const void *kv, int q_dt, int kv_dt, int32_t B, int32_t Q, int32_t H,
                              int32_t D, int64_t N, const int32_t *idx, int32_t k, float scale, void *out,
                              float *lse, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * csa2_layer -- one CSA2 layer (FULL, REINDEX or REUSE), selection certified
 * bit-exact.
 *
 * FULL    = index score over all visible entries -> top-k (+ top-P pool) ->
 *           attention.
 * REINDEX = index score of the P pool slots (shared kI, own qI/w) -> top-k of
 *           the pool (ties by entry index) -> attention on the shared kv.
 *           "Recall之王 祭出Reuse", same section: the hierarchical indexer --
 *           the first Full layer picks a candidate pool of at most 16,384
 *           positions and later Reindex layers score only inside it.
 * REUSE   = attention with the given idx.
 * The selection (idx, pool, count) equals the top-k of the binary64 scores of
 * the formula in csa2_index_score, taken in sequential order, exactly: entries
 * whose fp32 score is within the error bound of the k-th are rescored in
 * binary64 on the GPU before the cut.  With score_fmt = CSA2_SCORE_BF16 the
 * ranked value is that binary64 score rounded to bfloat16 (the bound then
 * also covers the rounding, and rescored entries are rounded before the cut),
 * again exactly.
 * ------------------------------------------------------------------------- */
typedef struct {
    int32_t mode;         /* csa2_mode */
    int32_t B, Q;         /* sequences, query tokens per sequence */
    int64_t N;            /* compressed entries per sequence */
    int32_t m;            /* group size (for q_pos visibility) */
    int32_t HI, dI;       /* indexer heads and dim */
    int32_t idx_dt;       /* dtype of qI and kI (CSA2_F32 or CSA2_BF16), or CSA2_FP4: FP4 kI, bf16 qI,
                             or CSA2_FP4QK: FP4 qI and kI (as csa2_index_score; dI % 64 == 0,
                             dI <= 256) */
    int32_t k;            /* top-k (>= 1) */
    int32_t P;            /* FULL: pool size (0 = no pool); REINDEX: pool slots */
    int32_t H, D;         /* attention heads and dim (kv row width D) */
    int32_t q_dt, kv_dt;  /* dtype of q/out; format of kv */
    float scale;          /* softmax scale */
    const int64_t *q_pos; /* [B,Q] or NULL (decode: all N visible) */
    const void *qI;       /* [B,Q,HI,dI] (FULL, REINDEX) */
    const float *w;       /* [B,Q,HI]    (FULL, REINDEX) */
    const void *kI;       /* [B,N,dI]    (FULL: own; REINDEX: the Full layer's, shared) */
    int32_t *pool;        /* [B,Q,P] FULL out (if P > 0) / REINDEX in; ascending, -1 padded */
    int32_t *idx;         /* [B,Q,k] FULL/REINDEX out, REUSE in; ascending, -1 padded */
    int32_t *count;       /* [B,Q] out, or NULL (number of valid idx entries) */
    float *scores;        /* [B,Q,N] (FULL) or [B,Q,P] (REINDEX) fp32 out, or NULL */
    const void *q;        /* [B,Q,H,D] */
    const void *kv;       /* [B,N,row] (shared across layers of a group) */
    void *out;            /* [B,Q,H,D] in q_dt */
    float *lse;           /* [B,Q,H] or NULL */
    int32_t score_fmt;    /* csa2_score_fmt: the value top-k ranks (FULL, REINDEX); 0 = binary64 */
} csa2_layer_args;

CSA2_API size_t csa2_layer_workspace_size(const csa2_layer_args *a);
/* The same size under its short name. */
CSA2_API size_t csa2_workspace_size(const csa2_layer_args *a);
CSA2_API int csa2_layer(const csa2_layer_args *a, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * csa2_layer_noalloc -- csa2_layer without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).
 *
 * Same arguments, kernels and results as csa2_layer; the scratch comes from a
 * device array inside the library (one per GPU, CSA2_NOALLOC_SCRATCH_BYTES =
 * 64 MiB, held until the process ends) instead of the caller's workspace.  A
 * layer whose csa2_layer_workspace_size exceeds that returns
 * CSA2_EUNSUPPORTED before anything is enqueued.  The call itself allocates
 * nothing (the array's device address is looked up once per device, on the
 * first call with that device current).  Every call on one GPU shares its
 * array: calls that overlap on one GPU (different streams, or different host
 * threads) race on it and must be serialised by the caller.
 * ------------------------------------------------------------------------- */
#define CSA2_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
CSA2_API int csa2_layer_noalloc(const csa2_layer_args *a, void *stream);

/* ---------------------------------------------------------------------------
 * csa2_swa_attn -- the sliding-window (SWA) branch, optionally merged with the
 * CSA2 branch's result.
 *
 * Video transcript on V4.1 Flash (prism.simon-ai.net), passages on the SWA
 * branch: each layer keeps its own uncompressed KV of the most recent 128
 * tokens (not shared across layers) beside the shared global KV.  Readings
 * (the pages state neither): the window of a query at token position p is
 * the rows p - W + 1 .. p, its own token the newest; the rows have the form
 * of the global KV (one D-vector per token, key and value of every head);
 * the two branches combine as one softmax over the union of their entries.
 *
 * q [B,Q,H,D] in q_dt; swa_kv [B,T,row] in kv_dt (formats as csa2_sparse_attn);
 * q_pos [B,Q] int64 token positions (rows past T - 1 or below 0 are skipped);
 * W >= 1 window length.  Computes o_swa, lse_swa = attention over the window.
 * csa_out [B,Q,H,D] in q_dt and csa_lse [B,Q,H] fp32: the CSA2 branch's
 *   result (csa2_layer / csa2_sparse_attn with lse); both NULL for the window
 *   branch alone.  With them, out = (u csa_out + v o_swa) / (u + v) with
 *   u = exp(csa_lse - M), v = exp(lse_swa - M), M the larger lse, and
 *   lse = M + ln(u + v).  out may be csa_out (merged in place).
 * out [B,Q,H,D] in q_dt; lse [B,Q,H] fp32 or NULL.
 * ------------------------------------------------------------------------- */
CSA2_API size_t csa2_swa_attn_workspace_size(int q_dt, int kv_dt, int32_t B, int32_t Q, int32_t H, int32_t D,
                                             int32_t W);
CSA2_API int csa2_swa_attn(const void *q, const void *swa_kv, int q_dt, int kv_dt, int32_t B, int32_t Q, int32_t H,
                           int32_t D, int64_t T, const int64_t *q_pos, int32_t W, float scale, const void *csa_out,
                           const float *csa_lse, void *out, float *lse, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * csa2_merge_attn -- one softmax over the union of two disjoint entry sets
 * from each set's attention output and lse (the merge step of csa2_swa_attn
 * on its own; same reading).
 *
 * o_a, o_b, out [R,D] in dt (CSA2_F32 or CSA2_BF16), D % 8 == 0; lse_a, lse_b
 * [R] fp32; lse [R] fp32 or NULL.  A set with lse = -inf has weight 0; both
 * empty give out = 0, lse = -inf.  out may alias o_a or o_b.
 * ------------------------------------------------------------------------- */
CSA2_API int csa2_merge_attn(const void *o_a, const float *lse_a, const void *o_b, const float *lse_b, int dt,
                             int64_t R, int32_t D, void *out, float *lse, void *stream);

/* Message of the last non-OK status returned on the calling thread. */
CSA2_API const char *csa2_last_error(void);
/* Library version string. */
CSA2_API const char *csa2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
