/*
 * stdk.h — dynamic top-K sparse decode attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libstdk.so. Every pointer argument is a DEVICE pointer unless its
 * comment says "host". The caller allocates and owns every buffer (inputs,
 * outputs, workspace, ReTopK state); the library never allocates device
 * memory on these calls and keeps no device state between them.
 *
 * Conventions shared by every entry point
 *  - Return value: STDK_OK (0) or a negative STDK_E* code. Arguments are
 *    validated on the host before anything is enqueued, so a call that
 *    returns STDK_EINVAL / STDK_EUNSUPPORTED / STDK_EWORKSPACE has launched
 *    nothing. STDK_EHIP means a launch failed; stdk_last_error() (per host
 *    thread) holds the text. No C++ exception crosses the ABI.
 *  - Ordering: all work is enqueued on `stream` (a hipStream_t; NULL = the
 *    legacy default stream) and nothing is synchronised inside the library.
 *  - Determinism: identical inputs give bit-identical outputs. The chosen
 *    rows never depend on the batch; o and lse are summed in one of two
 *    fixed orders, chosen by the head count (B * n_q_heads at least the
 *    GPU's CU count folds softmax . V into the select launch), so the same
 *    sequence in a batch on the other side of that count may differ in the
 *    last bits of o and lse.
 *  - Concurrency: calls are reentrant; two calls that are in flight at the
 *    same time must not share a workspace buffer.
 *  - Workspace state: the first B * n_q_heads * 16448 bytes of a workspace
 *    hold counters (two radix histograms and an arrival counter per query
 *    head) that each call adds to and then clears again. They must be zero
 *    before the first call that uses the buffer (fill the new buffer with
 *    zeros once, e.g. hipMemset). Every call that
 *    returns STDK_OK leaves them zero, so the buffer can be reused by later
 *    calls with the same stdk_layout (topk_attn_decode, its _static and
 *    _int8 variants, retopk_step, and topk_multi_query, which leaves that
 *    region untouched) without clearing. A call that returns STDK_EHIP after
 *    its scan was enqueued leaves the counters non-zero: the library records
 *    the buffer's address, and the next call given that address clears the
 *    counter region on its stream before anything else (one small kernel).
 *    A buffer reused with a larger layout must be zeroed again by the caller
 *    over the larger counter region.
 *  - KV cache layout (stdk_layout): element (b, h_kv, row, j) lives at
 *        base + b*stride_b + h_kv*stride_h + row*head_dim + j
 *    (rows are contiguous, head_dim elements each). Keys and values share
 *    one layout. Row starts must be 16-byte aligned.
 *  - Query / output layout: q, o are [batch][n_q_heads][head_dim] fp32,
 *    lse is [batch][n_q_heads] fp32, index outputs [batch][n_q_heads][K]
 *    int32. Query head h reads KV head h / (n_q_heads / n_kv_heads).
 *  - Scores use z_i = scale * (q . k_i); the caller passes scale (the usual
 *    value is 1/sqrt(head_dim)).
 *
 * Sources (page title and section):
 *  [RA]  "RetrievalAttention: Accelerating Long-Context LLM Inference via
 *        Vector Retrieval" (review): "Approximated Attention Formulation"
 *        (Eq. 2) and "CPU-GPU Co-Execution Architecture" (Eq. 3-5).
 *  [RT]  "Recall Before You Rank: Similarity-Guided Top-K Reuse for
 *        Efficient Long-Context Attention" (review): the exact Top-K cost
 *        section and "核心方法" 1-5.
 */
#ifndef STDK_H
#define STDK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define STDK_VERSION 100 /* 1.0.0 */

#define STDK_OK 0
#define STDK_EINVAL (-1)       /* a pointer, size or parameter is invalid */
#define STDK_EUNSUPPORTED (-2) /* valid but not supported (head_dim != 128, ...) */
#define STDK_EWORKSPACE (-3)   /* workspace missing or too small */
#define STDK_EHIP (-4)         /* a HIP call or kernel launch failed */

#define STDK_F32 0  /* KV cache stored as IEEE fp32 */
#define STDK_BF16 1 /* KV cache stored as bfloat16 */

#define STDK_MAX_RANGES 16   /* index ranges per topk_attn_decode call */
#define STDK_MAX_GROUP 8     /* query heads per KV head */

typedef struct stdk_layout {
  int32_t batch;      /* B */
  int32_t n_q_heads;  /* H_q */
  int32_t n_kv_heads; /* H_kv; H_q must be a multiple, H_q / H_kv <= STDK_MAX_GROUP */
  int32_t head_dim;   /* d; only 128 is supported */
  int64_t max_len;    /* rows allocated per (b, h_kv) */
  int32_t kv_dtype;   /* STDK_F32 or STDK_BF16 */
  int32_t reserved;
  int64_t stride_b;   /* elements between sequences (>= n_kv_heads * stride_h) */
  int64_t stride_h;   /* elements between KV heads (>= max_len * head_dim) */
} stdk_layout;

/* ------------------------------------------------------------------------
 * topk_attn_decode — [RA] Eq. 2 with the index set chosen as the exact top-K
 * of the scores ([RT] exact Top-K: full QK scan, then TopK over every score).
 *
 * For every (b, h_q): z_i = scale * q[b][h_q] . k[b][h_kv][i] for every row i
 * in the union of the half-open `ranges`; S = the top_k rows of largest z
 * (ties go to the lowest row); then
 *     m = max_S z,  s = sum_S e^{z_i - m},
 *     o = sum_S e^{z_i - m} v_i / s,  lse = m + ln s.
 * When top_k >= n (n = total rows in the ranges) every row is used (dense
 * attention). n = 0 gives o = 0, lse = -inf.
 *
 *  ranges   host, 2*n_ranges int64: begin0, end0, begin1, end1, ... ; each
 *           range within [0, max_len), non-empty, ascending and disjoint.
 *           The same ranges apply to every sequence.
 *  n_ranges 0..STDK_MAX_RANGES.
 *  top_k    >= 1; when top_k < n it must be <= 65536, else
 *           STDK_EUNSUPPORTED.
 *  idx_out  [B][H_q][top_k] int32: S in ascending row order, padded with -1
 *           when n < top_k. May be NULL.
 *  o_out    [B][H_q][128] fp32;  lse_out [B][H_q] fp32 (natural log).
 *  workspace / workspace_bytes: device scratch of at least
 *           topk_attn_decode_workspace_size(lay, n, top_k) bytes, 256-byte
 *           aligned, in the state described under "Workspace state" above
 *           (zero-filled before its first use).
 * ---------------------------------------------------------------------- */
int32_t topk_attn_decode(const stdk_layout* lay, const float* q, const void* k_cache,
                         const void* v_cache, const int64_t* ranges, int32_t n_ranges,
                         int32_t top_k, float scale, int32_t* idx_out, float* o_out,
                         float* lse_out, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Bytes of workspace topk_attn_decode needs for n_scan rows per (b, h_q). */
size_t topk_attn_decode_workspace_size(const stdk_layout* lay, int64_t n_scan, int32_t top_k);

/* ------------------------------------------------------------------------
 * topk_attn_decode_static — the decode step of [RA] "CPU-GPU Co-Execution
 * Architecture": dense attention over a static row set W (static_ranges,
 * e.g. the first 128 and the last 512 rows) together with exact top-K
 * attention over the dynamic rows Omega (ranges), combined as in Eq. 3-5.
 *
 * o and lse equal attn_merge_lse of (a) topk_attn_decode over
 * `static_ranges` with top_k >= |W| and (b) topk_attn_decode over `ranges`;
 * by Eq. 4-5 that is softmax attention over W united with the chosen rows S.
 * One pass computes it: the scan scores W beside Omega (W stays out of the
 * top-K), W's rows are appended to every chosen-row list, and the softmax.V
 * partials of S and W are combined once, with the rescaling of Eq. 4-5.
 *
 *  ranges, n_ranges               Omega, as topk_attn_decode's ranges.
 *  static_ranges, n_static        W, the same rules; no static range may
 *           overlap a dynamic one, and n_ranges + n_static <= STDK_MAX_RANGES.
 *  top_k, scale, o_out, lse_out   as topk_attn_decode (top_k applies to Omega).
 *           When top_k < |Omega|, top_k + |W| must be <= 65536
 *           (STDK_EUNSUPPORTED otherwise).
 *  idx_out  [B][H_q][top_k] int32 or NULL: the chosen Omega rows S (ascending,
 *           -1 padded), as topk_attn_decode over `ranges` would give.
 *  workspace at least topk_attn_decode_static_workspace_size(lay, |Omega|,
 *           |W|, top_k) bytes, zero-filled before first use.
 * ---------------------------------------------------------------------- */
int32_t topk_attn_decode_static(const stdk_layout* lay, const float* q, const void* k_cache,
                                const void* v_cache, const int64_t* ranges, int32_t n_ranges,
                                const int64_t* static_ranges, int32_t n_static, int32_t top_k,
                                float scale, int32_t* idx_out, float* o_out, float* lse_out,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace topk_attn_decode_static needs for n_scan dynamic and
 * n_static static rows per (b, h_q). */
size_t topk_attn_decode_static_workspace_size(const stdk_layout* lay, int64_t n_scan,
                                              int64_t n_static, int32_t top_k);

/* ------------------------------------------------------------------------
 * topk_attn_decode_static_noalloc — topk_attn_decode_static for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation. Same arguments, results and
 * errors, without the workspace: the scratch is one array of
 * STDK_NOALLOC_SCRATCH_BYTES that the library holds per GPU until the
 * process ends. The call allocates nothing (no hipMalloc, no allocating
 * library routine).
 *  - Calls whose workspace need (topk_attn_decode_static_workspace_size)
 *    exceeds the array return STDK_EWORKSPACE before any launch. The
 *    Llama-3-8B-shaped layer at 131,072 rows (32 query heads, K = 2048, 640
 *    static rows) needs about 85 MB.
 *  - Every call on one GPU uses that GPU's one array, which keeps the last
 *    call's contents; each call clears the counters it needs first (a fill
 *    kernel on `stream`). Calls that overlap on one GPU (other streams or
 *    host threads) race on the array: the caller serialises them.
 * ---------------------------------------------------------------------- */
#define STDK_NOALLOC_SCRATCH_BYTES (96u << 20)

int32_t topk_attn_decode_static_noalloc(const stdk_layout* lay, const float* q, const void* k_cache,
                                        const void* v_cache, const int64_t* ranges, int32_t n_ranges,
                                        const int64_t* static_ranges, int32_t n_static, int32_t top_k,
                                        float scale, int32_t* idx_out, float* o_out, float* lse_out,
                                        void* stream);

/* ------------------------------------------------------------------------
 * topk_multi_query — the exact Top-K of [RT] ("Exact Top-K 的隐藏成本": TopK
 * over every score) for a block of queries per head at once: the supports
 * of the last prefill queries that start the ReTopK cache ([RT] 核心方法 1),
 * and the exact nearest keys of each prefill query that [RA] "Attention-Aware
 * ANNS Index Construction" starts from. No attention output.
 *
 * For every (b, h_q, m): z_i = scale * q[b][h_q][m] . k[b][h_kv][i] over the
 * rows i of `ranges`; S = the top_k rows of largest z (ties go to the lowest
 * row); all rows when top_k >= n.
 *
 *  q          [B][H_q][n_queries][128] fp32, 16-byte aligned, finite.
 *  n_queries  M >= 1 queries per query head; H_q / H_kv * M <= 8,388,480.
 *  ranges, n_ranges   as topk_attn_decode.
 *  top_k      1..65536 (STDK_EUNSUPPORTED above).
 *  idx_out    [B][H_q][M][top_k] int32, required: S ascending, -1 padded
 *             when n < top_k.
 *  z_out      [B][H_q][M][top_k] fp32 or NULL: the scores of the rows in
 *             idx_out, -inf in the padding.
 *  workspace  at least topk_multi_query_workspace_size(lay, M, n, top_k)
 *             bytes, 256-byte aligned, any contents (this call keeps no
 *             counters in it, and leaves the first B * H_q * 16448 bytes,
 *             the decode calls' counters, untouched). Not used when n = 0.
 *  Limits: B * n_kv_heads <= 65535.
 * The scores are computed on the bf16 matrix cores with every fp32 query
 * element split into a bf16 value and a bf16 remainder (and every fp32 key
 * likewise); they differ from an fp32 dot product by about
 * 2^-16 * scale * sum_j |q_j k_j| plus the accumulation rounding, so rows
 * whose scores lie that close to the K-th score may be exchanged.
 * ---------------------------------------------------------------------- */
int32_t topk_multi_query(const stdk_layout* lay, const float* q, int32_t n_queries,
                         const void* k_cache, const int64_t* ranges, int32_t n_ranges,
                         int32_t top_k, float scale, int32_t* idx_out, float* z_out,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace topk_multi_query needs for n_queries queries per head
 * and n_scan rows. */
size_t topk_multi_query_workspace_size(const stdk_layout* lay, int32_t n_queries, int64_t n_scan,
                                       int32_t top_k);

/* ------------------------------------------------------------------------
 * int8 keys as a recall stage. [RA] "CPU memory minimization (Appendix C)"
 * proposes 8-bit scalar quantization of the key vectors without fixing a
 * scheme, and the review asks whether quantized keys shift the nearest-key
 * rankings; here the int8 codes only choose a superset and the exact keys
 * decide inside it.
 *
 * quantize_keys_int8: per-row symmetric codes of the rows in `ranges`:
 *   s = max_j |k_j| / 127,  c_j = k_j / s rounded to nearest (halves to even),
 *   each a correctly rounded fp32 operation, clamped to [-127, 127]; a zero
 *   row gives s = 0 and codes 0.
 *  codes    [B][H_kv][max_len][128] int8 (16-byte aligned), packed whatever
 *           the cache strides are; only the rows in `ranges` are written.
 *  scales   [B][H_kv][max_len] fp32.
 *  Limits: B * n_kv_heads <= 65535.
 * ---------------------------------------------------------------------- */
int32_t quantize_keys_int8(const stdk_layout* lay, const void* k_cache, const int64_t* ranges,
                           int32_t n_ranges, int8_t* codes, float* scales, void* stream);

/* topk_attn_decode_int8: for every (b, h_q), S' = the recall_k rows of the
 * ranges with the largest z'_i = scale * s_i * (q . c_i) (ties to the lowest
 * row), S = the top_k rows of S' with the largest exact z_i (ties to the
 * lowest row), then o and lse over S as topk_attn_decode ([RA] Eq. 2). With
 * recall_k >= n, S' is every row and the result is topk_attn_decode's.
 *  codes, scales  as quantize_keys_int8 wrote them for every row of `ranges`.
 *  top_k >= 1, recall_k >= top_k; recall_k <= 65536 when below n.
 *  idx_out  [B][H_q][top_k] int32 or NULL: S, ascending, -1 padded.
 *  sup_out  [B][H_q][recall_k] int32 or NULL: S', ascending, -1 padded.
 *  o_out, lse_out as topk_attn_decode.
 *  workspace at least topk_attn_decode_int8_workspace_size(lay, n, top_k,
 *           recall_k) bytes, in the "Workspace state" above.
 * Not exact: a row outside S' cannot be chosen. */
int32_t topk_attn_decode_int8(const stdk_layout* lay, const float* q, const void* k_cache,
                              const void* v_cache, const int8_t* codes, const float* scales,
                              const int64_t* ranges, int32_t n_ranges, int32_t top_k,
                              int32_t recall_k, float scale, int32_t* idx_out, int32_t* sup_out,
                              float* o_out, float* lse_out, void* workspace,
                              size_t workspace_bytes, void* stream);

size_t topk_attn_decode_int8_workspace_size(const stdk_layout* lay, int64_t n_scan, int32_t top_k,
                                            int32_t recall_k);

/* topk_attn_decode_int8_static: the decode step of [RA] "CPU-GPU
 * Co-Execution Architecture" with the int8 recall stage on the dynamic rows:
 * o and lse equal attn_merge_lse of (a) topk_attn_decode over
 * `static_ranges` with top_k >= |W| and (b) topk_attn_decode_int8 over
 * `ranges` (Eq. 4-5). One pass: the exact scoring of the superset also
 * scores W, and the softmax.V partials of S and W are combined once.
 *  ranges, static_ranges  as topk_attn_decode_static (codes and scales need
 *           only cover `ranges`).
 *  top_k, recall_k, idx_out, sup_out  as topk_attn_decode_int8 over
 *           `ranges`; when top_k < |Omega|, top_k + |W| <= 65536.
 *           With recall_k >= |Omega| the result is topk_attn_decode_static's
 *           and sup_out lists every dynamic row.
 *  workspace at least topk_attn_decode_int8_static_workspace_size(lay,
 *           |Omega|, |W|, top_k, recall_k) bytes, in the "Workspace state"
 *           above. */
int32_t topk_attn_decode_int8_static(const stdk_layout* lay, const float* q, const void* k_cache,
                                     const void* v_cache, const int8_t* codes, const float* scales,
                                     const int64_t* ranges, int32_t n_ranges,
                                     const int64_t* static_ranges, int32_t n_static, int32_t top_k,
                                     int32_t recall_k, float scale, int32_t* idx_out, int32_t* sup_out,
                                     float* o_out, float* lse_out, void* workspace,
                                     size_t workspace_bytes, void* stream);

size_t topk_attn_decode_int8_static_workspace_size(const stdk_layout* lay, int64_t n_scan,
                                                   int64_t n_static, int32_t top_k, int32_t recall_k);

/* ------------------------------------------------------------------------
 * attn_merge_lse — [RA] Eq. 4-5: combination of two partial attention
 * outputs over disjoint row sets a and b:
 *     M = max(lse_a, lse_b),  lse = M + ln(e^{lse_a - M} + e^{lse_b - M}),
 *     o = e^{lse_a - lse} o_a + e^{lse_b - lse} o_b.
 * e^{lse_j - lse} equals the pages' gamma_j. An operand with lse = -inf
 * contributes nothing; both -inf gives o = 0, lse = -inf.
 *  rows     number of (o, lse) pairs (e.g. B * H_q); d = elements per o row
 *           (1..1024). o_* are [rows][d] fp32, lse_* are [rows] fp32.
 *  o_out / lse_out may alias o_a/lse_a or o_b/lse_b exactly.
 * ---------------------------------------------------------------------- */
int32_t attn_merge_lse(int64_t rows, int32_t d, const float* o_a, const float* lse_a,
                       const float* o_b, const float* lse_b, float* o_out, float* lse_out,
                       void* stream);

/* ------------------------------------------------------------------------
 * ReTopK ([RT] 核心方法 1-5).
 * ---------------------------------------------------------------------- */
typedef struct retopk_params {
  int32_t top_k;     /* K, rows attended per step (1..65536) */
  int32_t cache_cap; /* C, FIFO entries per query head (1..64) */
  int32_t top_r;     /* R, cache entries recalled (1..C) */
  int32_t recent;    /* W, newest rows always added to the candidates (>= 0) */
  float tau;         /* similarity threshold: max cosine < tau -> exact path */
  int32_t refresh;   /* T_r: step t with t % T_r == 0 -> exact path; 0 = never */
  float scale;       /* score scale (1/sqrt(d)) */
  int32_t budget;    /* candidate budget of the reuse path (>= 0; 0 = the whole union); see below */
} retopk_params;

/* Caller-owned per-query-head state (device memory):
 *  q_hat   [B][H_q][C][128] fp32  unit-norm cached queries
 *  support [B][H_q][C][K]   int32 their supports, ascending rows, -1 padded
 *  head    [B][H_q]         int32 slot of the newest entry
 *  count   [B][H_q]         int32 valid entries (0..C)
 * Entry of age a (0 = newest) lives in slot (head - a) mod C, for a < count. */
typedef struct retopk_state {
  float* q_hat;
  int32_t* support;
  int32_t* head;
  int32_t* count;
} retopk_state;

#define RETOPK_PATH_REUSE 0    /* recall + union + exact rerank */
#define RETOPK_PATH_FALLBACK 1 /* max cosine < tau, or empty cache: exact top-K */
#define RETOPK_PATH_REFRESH 2  /* t % T_r == 0: exact top-K */

/* Fill the FIFO of every (b, h_q) with the last min(n_hist, C) (query,
 * support) pairs of q_hist [B][H_q][n_hist][128] fp32 and sup_hist
 * [B][H_q][n_hist][K] int32, oldest first ([RT] 核心方法 1: the cache starts
 * from the last C prefill queries). Queries are stored normalised. n_hist = 0
 * gives an empty cache. */
int32_t retopk_state_init(const stdk_layout* lay, const retopk_params* p, const retopk_state* st,
                          const float* q_hist, const int32_t* sup_hist, int32_t n_hist,
                          void* stream);

/* One decode step for every (b, h_q) ([RT] 核心方法 1-5):
 *   q_bar = q / ||q||;  rho_c = q_bar . q_hat_c over the valid entries;
 *   exact path if t % T_r == 0 (refresh), or count = 0, or max rho < tau;
 *   else: recall the R entries of largest rho (ties: newest first), take the
 *   union of their supports and rows [L_t - W, L_t) (rows outside [0, L_t)
 *   are dropped), score those rows exactly and keep the top K;
 *   exact path: top K over rows [0, L_t);
 *   then o, lse = renormalised softmax . V over the K rows, and push
 *   (q_bar, support) into slot (head + 1) mod C (count = min(count + 1, C)).
 * The cosine, the comparison with tau and the top-R order are evaluated in
 * fp32; scores in fp32.
 *  L_t          rows visible this step, 1..max_len (includes the row the
 *               caller appended for this step).
 *  t            0-based decode step counter (for the refresh).
 *  support_out  [B][H_q][K] int32 (ascending, -1 padded). Required.
 *  o_out, lse_out as topk_attn_decode. Required.
 *  path_out     [B][H_q] int32 RETOPK_PATH_*; may be NULL.
 *  n_cand_out   [B][H_q] int32: candidate count M_t on the reuse path, L_t on
 *               the exact path; may be NULL.
 *  cand_out     [B][H_q][R*K + W] int32: the ascending candidate rows of the
 *               reuse path (-1 padded; all -1 on the exact path); may be NULL.
 *  workspace    at least retopk_workspace_size(lay, p, L_t) bytes,
 *               zero-filled before its first use ("Workspace state" above).
 * Candidate budget ([RT] "启发 4-5": confidence votes over the recalled
 * supports, high-confidence rows first under a budget). With budget > 0 the
 * reuse path keeps the recent rows and, of the other rows of the union, the
 * `budget` rows of largest f(i) = sum of rho_c over the recalled entries c
 * whose support holds row i (rho_c added in fp32 in recall order; ties go to
 * the lowest row); the exact rerank then runs on that set. budget > 0 needs
 * top_r <= 8 and R*K + W <= 16384 (STDK_EUNSUPPORTED otherwise).
 * Limits: L_t <= 1,048,576 (the candidate bitmap lives in LDS). */
int32_t retopk_step(const stdk_layout* lay, const retopk_params* p, const retopk_state* st,
                    const float* q, const void* k_cache, const void* v_cache, int64_t L_t,
                    int64_t t, int32_t* support_out, float* o_out, float* lse_out,
                    int32_t* path_out, int32_t* n_cand_out, int32_t* cand_out, void* workspace,
                    size_t workspace_bytes, void* stream);

/* retopk_step for serving loops that replay a captured step (a HIP graph):
 * the same step, with L_t and t read on the device from `step` and advanced
 * there at the end of the step, so that every call enqueues the same
 * launches with the same arguments ([RT] "GPU Kernel": a resident,
 * pre-allocated workspace; "局限性": serving workloads).
 *  step         device memory, two int64 words [L_t, t] (8-byte aligned).
 *               The step reads them as retopk_step takes its arguments (L_t
 *               clamped to 1..max_len, t below 0 taken as 0) and, after its
 *               last launch, has added 1 to both on `stream`.
 *  workspace    at least retopk_workspace_size(lay, p, lay->max_len) bytes
 *               (every launch is sized for L_t = max_len; rows at or past the
 *               device L_t are not read).
 * Everything else, results included, is as for retopk_step with the same
 * L_t and t. The library enqueues no memory set or copy; the caller may
 * capture the call in a graph and replay it for successive steps, writing
 * the new query into `q` (and the new key and value rows into the caches)
 * between replays. STDK_EINVAL if `step` is NULL. */
int32_t retopk_step_device(const stdk_layout* lay, const retopk_params* p, const retopk_state* st,
                           const float* q, const void* k_cache, const void* v_cache, int64_t* step,
                           int32_t* support_out, float* o_out, float* lse_out, int32_t* path_out,
                           int32_t* n_cand_out, int32_t* cand_out, void* workspace, size_t workspace_bytes,
                           void* stream);

size_t retopk_workspace_size(const stdk_layout* lay, const retopk_params* p, int64_t max_L_t);

/* Bytes of one allocation that holds the four state arrays of `lay` and
 * `p`, placed at 256-byte aligned offsets in this order (S = B * H_q,
 * C = cache_cap, K = top_k, al(x) = x rounded up to a multiple of 256):
 *   q_hat   at 0                                  (S*C*128 fp32)
 *   support at al(S*C*512)                        (S*C*K int32)
 *   head    at al(S*C*512) + al(S*C*K*4)          (S int32)
 *   count   at that + al(S*4)                     (S int32)
 * The state is plain data: copying the four arrays out and back (e.g. to
 * host memory and into a fresh buffer) checkpoints and resumes a decode.
 * 0 for invalid arguments. */
size_t retopk_state_size(const stdk_layout* lay, const retopk_params* p);

/* ------------------------------------------------------------------------
 * Helpers
 * ---------------------------------------------------------------------- */
const char* stdk_last_error(void); /* host string, valid until the next call on this thread */
int32_t stdk_version(void);        /* STDK_VERSION */

/* Testing aid for the error path: the library launch numbered
 * `after_launches` (0-based, counted over all threads from this call on) is
 * not enqueued; the call that reaches it returns STDK_EHIP as if the launch
 * had failed, with the work before it already enqueued. Fires once; -1
 * disarms. STDK_EINVAL below -1. */
int32_t stdk_inject_launch_failure(int32_t after_launches);

/* Measurement aid: the plain HBM read rate of the key scan's partition.
 * Reads every byte of n_groups regions once: region g is group_bytes bytes
 * from base + g * group_stride_bytes, streamed by wg_per_group workgroups
 * of 512 threads that each take an equal contiguous share (16-byte
 * non-temporal loads, as the scan issues its key loads,
 * two sets of four in flight), the way k_scan splits a KV head's rows over
 * its workgroups. Nothing is written except, in a case that does not occur
 * for real data (an XOR of all words equal to a fixed constant), one word
 * of `sink` (4 bytes of device memory). Its duration (kernel family
 * "hbm_read") is the ceiling the scan's HBM rate is compared against.
 * base 16-byte aligned, group_bytes a positive multiple of 16, n_groups and
 * wg_per_group >= 1 with n_groups * wg_per_group <= 2^31 - 1: else
 * STDK_EINVAL. */
int32_t stdk_hbm_read(const void* base, int64_t group_stride_bytes, int32_t n_groups, int64_t group_bytes,
                      int32_t wg_per_group, uint32_t* sink, void* stream);

/* Kernel timing: while enabled, every kernel the library enqueues (or only
 * the kernel family `only`, if not NULL) is launched with a pair of
 * hipEvents attached to its dispatch (hipExtLaunchKernelGGL start/stop
 * events, on the launch stream), so the pair times the kernel itself.
 * `capacity` bounds the number of launches recorded (events are created when
 * enabling, not on the hot path). stdk_profile_read waits for the recorded
 * events and returns, for the kernel family `name`, the summed duration in
 * milliseconds and the launch count. Families: "k_scan",
 * "topk_filter_select", "sparse_sv", "dense_attn", "combine",
 * "attn_merge", "fill_empty", "retopk_select", "retopk_rerank",
 * "retopk_rerank_select", "retopk_init", "retopk_vote",
 * "mq_blockmax", "mq_threshold", "mq_collect", "mq_select", "mq_fill",
 * "k_quantize", "hbm_read", "retopk_attend", "retopk_reuse",
 * "topk_filter_select_sv", "topk_select_lds", "topk_select_lds_sv",
 * "topk_filter_lds_sv".
 * Unknown names return STDK_EINVAL. */
int32_t stdk_profile_enable(int32_t capacity, const char* only);
int32_t stdk_profile_disable(void);
int32_t stdk_profile_reset(void);
int32_t stdk_profile_read(const char* name, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* STDK_H */
