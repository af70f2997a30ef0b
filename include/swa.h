/*
 * swa.h -- C ABI of libswa.so: exact causal sliding-window attention with
 * attention sinks on AMD Instinct MI355X (gfx950).
 *
 * The operation (from the pages this library implements):
 *  - "Sliding Window and Sparse Attention, from Longformer to CSA2",
 *    s1: Attention(Q, K, V) = softmax(Q K^T / sqrt(d)) V, causal (j <= i);
 *    s2: sliding window -- query i reads keys i-w+1 .. i (w keys including
 *        itself); attention sinks -- the first g tokens stay readable forever;
 *        rolling-buffer cache -- position i overwrites slot i mod w;
 *    s10 glossary, LSE: the log-sum-exp normaliser returned so that partial
 *        results over disjoint key sets can be merged.
 *  - "Local and Sparse Attention: Reading Fewer Token Positions", Figures 1,
 *    2 and 4 and their text: a window of 3 counts the current token; an
 *    excluded score is -inf before the softmax (never 0); a position that is
 *    in the window and in the anchor (sink) set is read once; no future
 *    position is read; a window-only cache overwrites the oldest slot.
 *
 * For query position i the attended key set is
 *     A_i = { j : max(0, i-w+1) <= j <= i }  U  { j : 0 <= j < min(g, i+1) }
 * and, with s_ij = scale * q_i . k_j + sink_bias * [j < g] for j in A_i,
 *     o_i   = sum_{j in A_i} exp(s_ij - m_i) v_j / sum_{j in A_i} exp(s_ij - m_i),
 *     lse_i = m_i + ln sum_{j in A_i} exp(s_ij - m_i),   m_i = max_j s_ij.
 * sink_bias is an additive offset on the scaled score of every attended key
 * at a position below g (0 gives plain sinks).
 *
 * Conventions for every entry point
 *  - Tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates nothing and keeps no state between calls, except the fixed
 *    decode scratch of swa_decode_fwd_gqa_noalloc below.  Every tensor is
 *    contiguous with the innermost dimension last, as written below, and
 *    every pointer must be 16-byte aligned.
 *  - Work is enqueued asynchronously on `stream` (0 = the null stream); the
 *    library never synchronises.  Device-side faults surface at the caller's
 *    next synchronisation, as usual in HIP.
 *  - Arguments are validated before anything is enqueued.  On an invalid
 *    argument the call returns a negative status and launches nothing.
 *    SWA_EHIP means a launch was rejected by the HIP runtime.
 *  - Supported: dtype SWA_BF16 (bf16 storage, fp32 accumulation and softmax,
 *    probabilities rounded to bf16 before the value product, bf16 output) and
 *    SWA_F32 (fp32 throughout); head dimension d in {64, 128}.
 *  - Calls on one stream are ordered; calls that write the same memory from
 *    different streams race, as with any HIP kernel.
 */
#ifndef SWA_H
#define SWA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SWA_F32 = 0, SWA_BF16 = 1 } swa_dtype_t;

enum {
    SWA_OK = 0,
    SWA_EINVAL = -1,        /* a size, a count or a required pointer is invalid */
    SWA_EUNSUPPORTED = -2,  /* head dimension or dtype not supported            */
    SWA_EALIGN = -3,        /* a pointer is not 16-byte aligned                 */
    SWA_EHIP = -4,          /* the HIP runtime rejected a launch                */
    SWA_EWORKSPACE = -5,    /* decode workspace missing or too small            */
    SWA_ESCRATCH = -6       /* shape needs more than the fixed decode scratch   */
};

/*
 * Prefill: attention of all n queries of each (batch, head) over the same
 * sequence's keys, restricted to A_i.
 *   q, k, v, o : [batch][heads][n][d]   (dtype)
 *   lse        : [batch][heads][n] fp32, natural log; may be NULL
 *   scale      : finite, > 0 (1/sqrt(d) is the usual value)
 *   sink_bias  : finite
 *   n >= 1, w >= 1, g >= 0 (g > n is read as g = n: every position is a
 *   sink either way), batch >= 1, heads >= 1,
 *   n * d * element size < 2^32 (one (batch, head)'s rows are addressed
 *   with 32-bit byte offsets; SWA_EINVAL otherwise).
 * Only the key tiles that hold attended pairs are visited (the diagonal band
 * plus the sink tiles below it); nothing n x n is ever formed.  K and V rows
 * at positions >= n are never read.
 * Inputs must be finite at every position < n.  A key that one query of a
 * visited tile attends and another does not still enters the second query's
 * value product, with a probability of exactly 0; an Inf or NaN in that key's
 * V row would turn 0 into NaN there (0 * Inf), so non-finite K or V rows can
 * reach output rows that do not attend them.
 */
int swa_prefill_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                    int batch, int heads, int n, int d, int w, int g,
                    float scale, float sink_bias, swa_dtype_t dtype, hipStream_t stream);

/*
 * Rolling-buffer cache append.  Cache layout, per (batch, head), g + w rows:
 *   rows 0 .. g-1      : sinks, position t < g lives in row t (never overwritten)
 *   rows g .. g+w-1    : ring, position t lives in row g + (t mod w)
 *   k_cache, v_cache   : [batch][heads][g + w][d]   (dtype)
 *   k_new, v_new       : [batch][heads][t_new][d]   (dtype)
 *   pos                : [batch] int64, device; position of token 0 of each
 *                        batch entry (token j is at pos[b] + j); must be >= 0
 *                        (a negative entry, or one with pos[b] + t_new past
 *                        INT64_MAX, makes that batch entry a no-op)
 * A token at position P goes to ring row g + P mod w, and also to sink row P
 * when P < g.  When t_new > w only the last w tokens reach the ring (the
 * earlier ones would be overwritten anyway); sink rows are still written.
 */
int swa_kv_append(void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                  const int64_t *pos, int batch, int heads, int t_new, int d, int w, int g,
                  swa_dtype_t dtype, hipStream_t stream);

/*
 * Decode: one query per (batch, head) at position pos[b] against the cache
 * above.  Append-then-attend: the query's own key/value must already be in
 * the cache, and every position 0 .. pos[b] must have been appended in order.
 *   q, o      : [batch][heads][d]   (dtype)
 *   lse       : [batch][heads] fp32 or NULL
 *   pos       : [batch] int64, device, >= 0 (a negative entry yields NaN output)
 *   workspace : device scratch of at least swa_decode_workspace_bytes(...)
 *               bytes, 16-byte aligned, or NULL when that size is 0.
 *   (g + w) * d * 4 < 2^32 (one head's cache rows, 32-bit byte offsets).
 * Ring slot s is read only when it holds a position of the window; sink row t
 * is read only when position t has left the window (otherwise the ring copy
 * is the one read, so each position is read once).
 */
int swa_decode_fwd(const void *q, const void *k_cache, const void *v_cache, const int64_t *pos,
                   void *o, float *lse, int batch, int heads, int d, int w, int g,
                   float scale, float sink_bias, swa_dtype_t dtype,
                   void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes swa_decode_fwd needs for this shape (0 when the launch
 * does not split the cache rows of one (batch, head) across workgroups). */
size_t swa_decode_workspace_bytes(int batch, int heads, int d, int w, int g);

/*
 * Grouped-query attention ("Sliding Window and Sparse Attention, from
 * Longformer to CSA2", s10 glossary, GQA: several query heads share one
 * key/value head, which shrinks the KV cache by the group size): kv_heads
 * key/value heads serve heads query heads, heads % kv_heads == 0, and query
 * head h reads key/value head h / (heads / kv_heads).  kv_heads == heads is the plain calls above (which
 * forward here); kv_heads == 1 is multi-query attention.  Shapes:
 *   prefill: q, o [batch][heads][n][d]; k, v [batch][kv_heads][n][d];
 *            lse [batch][heads][n]
 *   decode:  q, o [batch][heads][d]; caches [batch][kv_heads][g + w][d]
 *            (written by swa_kv_append with its `heads` = kv_heads);
 *            lse [batch][heads]
 * Everything else (validation, layout, ownership, errors) is as for the
 * plain calls; an invalid kv_heads is SWA_EINVAL.  Decode reads each cache
 * row once for up to 8 query heads of its group (one workgroup serves them).
 */
int swa_prefill_fwd_gqa(const void *q, const void *k, const void *v, void *o, float *lse,
                        int batch, int heads, int kv_heads, int n, int d, int w, int g,
                        float scale, float sink_bias, swa_dtype_t dtype, hipStream_t stream);
int swa_decode_fwd_gqa(const void *q, const void *k_cache, const void *v_cache, const int64_t *pos,
                       void *o, float *lse, int batch, int heads, int kv_heads, int d, int w, int g,
                       float scale, float sink_bias, swa_dtype_t dtype,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);
/* Workspace bytes of swa_decode_fwd_gqa (0 also for an invalid shape). */
size_t swa_decode_workspace_bytes_gqa(int batch, int heads, int kv_heads, int d, int w, int g);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation, kernels and results as swa_decode_fwd_gqa, with no workspace
 * argument.  When the launch splits the cache rows of one (batch, head)
 * across workgroups, the partial (m, l, o) records go to a fixed scratch
 * array of swa_decode_scratch_bytes() bytes (16 MiB) that the library keeps
 * in device memory, one copy per device, from the first call on that device
 * until the process ends.  The call itself allocates nothing: its first call
 * on a device only looks up that device's copy (hipGetSymbolAddress).
 * Calls that overlap in time on one device (different streams, or host
 * threads) share the array and race; calls ordered on one stream do not.
 * Every record a call reads was written by that call's own first kernel, so
 * nothing needs clearing between calls.  Arguments, layout, ownership and
 * errors as swa_decode_fwd_gqa, plus SWA_ESCRATCH when the shape's partial
 * records (swa_decode_workspace_bytes_gqa) would exceed the array; by the
 * split rule in use no shape reaches 13 MiB, so this is a guard, not a
 * limit callers meet.
 */
int swa_decode_fwd_gqa_noalloc(const void *q, const void *k_cache, const void *v_cache, const int64_t *pos,
                               void *o, float *lse, int batch, int heads, int kv_heads, int d, int w, int g,
                               float scale, float sink_bias, swa_dtype_t dtype, hipStream_t stream);
size_t swa_decode_scratch_bytes(void);

/*
 * Chunked prefill against the rolling cache: t new tokens of each batch entry
 * b, at positions pos[b] .. pos[b]+t-1, attend the window and sinks of
 * "Sliding Window and Sparse Attention, from Longformer to CSA2", s2 (the
 * same set as swa_prefill_fwd would give those rows over the whole
 * sequence).  Keys at positions >= pos[b] come from the chunk itself; keys
 * at positions < pos[b] from the cache, which must hold positions
 * 0 .. pos[b]-1 as written by swa_kv_append (ring row g + s mod w while the
 * ring still holds s, else sink row s; "Local and Sparse Attention: Reading
 * Fewer Token Positions", Figure 4 and the multi-token buffers it mentions).
 * Call it before appending the chunk: the append overwrites ring rows that
 * the chunk's first queries read.
 *   q, o        : [batch][heads][t][d]   (dtype)
 *   k_new, v_new: [batch][kv_heads][t][d]
 *   k_cache, v_cache: [batch][kv_heads][g + w][d]
 *   pos         : [batch] int64, device; a negative entry (or one with
 *                 pos + t beyond INT_MAX - 1024) yields NaN rows for that
 *                 entry
 *   lse         : [batch][heads][t] fp32 or NULL
 *   keys        : SWA_KEYS_ALL, or a partial attention over the cache keys
 *                 only (SWA_KEYS_CACHE) or the chunk keys only
 *                 (SWA_KEYS_CHUNK); a row with no key in its part gets
 *                 o = 0 and lse = -inf, ready for swa_lse_merge.
 * Grouping as in the _gqa calls (kv_heads == heads: multi-head attention).
 * Errors: SWA_EINVAL (null pointer, sizes, keys, scale), SWA_EUNSUPPORTED
 * (d or dtype), SWA_EALIGN (16-byte tensors, 8-byte pos, 4-byte lse).
 */
enum { SWA_KEYS_ALL = 0, SWA_KEYS_CACHE = 1, SWA_KEYS_CHUNK = 2 };
int swa_chunk_prefill_fwd(const void *q, const void *k_new, const void *v_new,
                          const void *k_cache, const void *v_cache, const int64_t *pos,
                          void *o, float *lse, int batch, int heads, int kv_heads, int t, int d,
                          int w, int g, float scale, float sink_bias, int keys,
                          swa_dtype_t dtype, hipStream_t stream);

/*
 * Log-sum-exp merge of two partial attentions of the same query rows over
 * disjoint key sets (s10 glossary of the first page above, LSE: the
 * normaliser that lets partial results over disjoint key sets combine
 * exactly): with M = max(lse_a, lse_b),
 *   o   = (e^(lse_a-M) o_a + e^(lse_b-M) o_b) / (e^(lse_a-M) + e^(lse_b-M)),
 *   lse = M + ln(e^(lse_a-M) + e^(lse_b-M)).
 * A part with lse = -inf weighs 0; two empty parts give o = 0, lse = -inf.
 *   o_a, o_b, o : [rows][d] (dtype; o may alias o_a or o_b)
 *   (lse must not alias lse_a or lse_b: rows are merged by many threads)
 *   lse_a, lse_b: [rows] fp32 (required); lse: [rows] fp32 or NULL
 */
int swa_lse_merge(const void *o_a, const float *lse_a, const void *o_b, const float *lse_b,
                  void *o, float *lse, long long rows, int d, swa_dtype_t dtype, hipStream_t stream);

/*
 * FP8 window KV cache ("Sliding Window and Sparse Attention, from Longformer
 * to CSA2": s7 keeps the window KV in FP8; s10 glossary, E4M3: 1 sign, 4
 * exponent, 3 mantissa bits).  Codes are OCP E4M3 (exponent bias 7, no
 * infinities, S.1111.111 = NaN, largest finite 448), one byte per element,
 * in the cache layout above: [batch][heads][g + w][d] bytes.  Each (batch,
 * key/value head) has one fp32 scale for K and one for V (device arrays
 * [batch][heads], positive and finite; the pages give no scale convention):
 * a stored code c stands for scale * E4M3(c).
 *
 * swa_kv_append_fp8: as swa_kv_append, with every element x of k_new/v_new
 * (dtype bf16 or fp32) stored as the code of x / scale (fp32 division,
 * correctly rounded), rounded to the nearest code, ties to even, |x/scale|
 * >= 448 saturated to 448, NaN kept NaN.
 *
 * swa_decode_fwd_fp8: as swa_decode_fwd_gqa over fp8 caches; q and o have
 * the given dtype; scores use scale * k_scale * (q . code values), outputs
 * v_scale * (weighted sum of code values); fp32 arithmetic.  Workspace size
 * as swa_decode_workspace_bytes_gqa.  Errors as the bf16 calls (scales null
 * or misaligned: SWA_EINVAL / SWA_EALIGN).
 */
int swa_kv_append_fp8(void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                      const int64_t *pos, const float *k_scale, const float *v_scale,
                      int batch, int heads, int t_new, int d, int w, int g,
                      swa_dtype_t dtype, hipStream_t stream);
int swa_decode_fwd_fp8(const void *q, const void *k_cache, const void *v_cache,
                       const float *k_scale, const float *v_scale, const int64_t *pos,
                       void *o, float *lse, int batch, int heads, int kv_heads, int d, int w, int g,
                       float scale, float sink_bias, swa_dtype_t dtype,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Fixed sparse patterns on the same block-sparse tiles ("Sliding Window and
 * Sparse Attention, from Longformer to CSA2", s2 dilated windows, s4
 * block-sparse attention as a kernel primitive; "Local and Sparse
 * Attention: Reading Fewer Token Positions", Figure 2).  Shapes, grouping,
 * dtypes, alignment and errors as swa_prefill_fwd_gqa; r >= 1.
 *
 * swa_dilated_prefill_fwd: query i reads the w keys i, i-r, ..., i-(w-1)r
 * (those >= 0): the cost of a window of w over a span of (w-1)r+1.  No sinks.
 * r = 1 is the plain window.
 *
 * swa_landmark_prefill_fwd: query i reads its window i-w+1 .. i, the sinks
 * 0 .. g-1 and the landmarks, every position j <= i with j mod r == 0, each
 * position once; sink_bias on positions < g.  bf16: one launch, in which
 * each query block streams the tiles of its landmarks below the window (and
 * not below g; K/V rows strided by r) and then its window-and-sink tiles
 * through one online softmax; no workspace (0 bytes: workspace may be null).
 * fp32: the window-and-sinks part into o, the landmark part into the
 * workspace, merged into o by LSE (the arithmetic of swa_lse_merge).
 * workspace: at least swa_landmark_workspace_bytes(...) bytes, 16-byte
 * aligned, when that size is not 0 (SWA_EWORKSPACE, SWA_EALIGN otherwise).
 */
int swa_dilated_prefill_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                            int batch, int heads, int kv_heads, int n, int d, int w, int r,
                            float scale, swa_dtype_t dtype, hipStream_t stream);
int swa_landmark_prefill_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                             int batch, int heads, int kv_heads, int n, int d, int w, int g, int r,
                             float scale, float sink_bias, swa_dtype_t dtype,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);
size_t swa_landmark_workspace_bytes(int batch, int heads, int n, int d, swa_dtype_t dtype);

/* Static description of a status code. */
const char *swa_strerror(int status);

/*
 * Test hook (host only, launches nothing): the prefill tile schedule.
 * Writes triples (query_block, key_block, is_full) for every tile the
 * prefill kernel visits when queries are grouped bq at a time and keys bk at
 * a time, in visiting order, query block by query block.  is_full = 1 means
 * every pair of the tile with query < n is attended and carries no sink bias,
 * so masking can be skipped there.  The kernel visits the tiles of its
 * workgroup's query block (bq from swa_prefill_tile_shape) and applies the
 * is_full test to each wave's own 32 query rows.  Returns the number of
 * triples (writing at most `cap`), or a negative status (SWA_EINVAL also
 * when n + bq or n + bk exceeds INT_MAX).
 */
long swa_band_tiles(int n, int w, int g, int bq, int bk, int *out, long cap);

/* Test hook: the tile shape the prefill kernel uses for (dtype, d). */
int swa_prefill_tile_shape(swa_dtype_t dtype, int d, int *bq, int *bk);

/*
 * Test hook (host only): the workgroup -> (batch*head, query block) order of
 * a prefill launch with `units` (batch, head) pairs, `nqb` query blocks and
 * `group` query heads per key/value head (heads / kv_heads; 1 for
 * multi-head attention and for the strided patterns).  Writes pairs for
 * workgroup ids 0 .. units*nqb-1.  Returns the count or a negative status
 * (SWA_EINVAL when group does not divide units).
 */
long swa_prefill_order(int units, int nqb, int group, int *out, long cap);

#ifdef __cplusplus
}
#endif

#endif /* SWA_H */
