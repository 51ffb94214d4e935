/*
 * hisa.h - C ABI of libhisa: hierarchical (block-then-token) sparse
 * retrieval and sparse attention on AMD Instinct MI355X (gfx950).
 *
 * The method: keys are cut into fixed blocks of B tokens and each block is
 * summarised by the mean of its indexer keys; each query scores the block
 * summaries with the indexer's dot product, keeps m blocks (the first block
 * and the query's own block always among them), scores every token of the
 * kept blocks, keeps the best k tokens, and attends over those k tokens
 * only. Sources: "PKU HISA sparse attention mechanism: 3x long-text
 * efficiency" (intelliparadigm.com), sections 1.1, 1.2.1, 1.2.2, 1.3; the
 * QbitAI news article on HISA (m.digipub.cc), parts "block-level coarse
 * filter", "fine token selection" and "complexity". The two-level decode
 * follows "Tencent Hunyuan HiLS-Attention" (ai-engineering pages, Ch01.911),
 * section "hierarchical softmax decomposition".
 *
 * Conventions shared by every entry point
 *  - Every tensor pointer is a device pointer owned by the caller. The
 *    library never allocates, frees or synchronises; scratch memory comes
 *    in through a caller-provided workspace whose size a *_workspace_bytes
 *    query returns.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL means the
 *    default stream). Device faults surface at the caller's next
 *    synchronisation.
 *  - Arguments are validated on the host before anything is launched. A
 *    non-OK status means nothing was launched and no output was written;
 *    hisa_last_error() then returns a thread-local description.
 *  - bf16 tensors have a contiguous last dimension; the other dimensions are
 *    addressed through hisa_strides_t (in elements). Base pointers must be
 *    16-byte aligned and the strides multiples of 8 elements.
 *  - Token and block indices are relative to their own sequence. Index
 *    outputs are int32, ascending, and padded with -1 when fewer than the
 *    requested number of candidates exist.
 *  - Ties between equal scores go to the lowest index; -0.0 equals +0.0.
 *    Scores must be finite (NaN or infinite inputs give an unspecified but
 *    memory-safe selection).
 *  - Supported sizes: indexer dim d in {64, 128}; block size B in
 *    {64, 128, 256}; m >= 2; m*B <= 16384; 1 <= k <= 16384; attention
 *    (Dk, Dv) in {(64, 64), (128, 128), (576, 512)}; Hq % Hkv == 0 with
 *    Hq / Hkv <= 64. Anything else returns HISA_ERR_UNSUPPORTED.
 */
#ifndef HISA_H
#define HISA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HISA_OK = 0,
  HISA_ERR_NULL = 1,        /* a required pointer is NULL                     */
  HISA_ERR_SHAPE = 2,       /* inconsistent sizes, strides or alignment       */
  HISA_ERR_UNSUPPORTED = 3, /* valid but unsupported size                     */
  HISA_ERR_HIP = 4,         /* the HIP runtime reported a launch error        */
  HISA_ERR_WORKSPACE = 5    /* workspace missing or smaller than required     */
} hisa_status_t;

typedef void* hisa_stream_t; /* hipStream_t */

/* Strides in elements. Element (b, t, h, i) of a tensor lives at
 * base + b*batch + t*token + h*head + i. Unused members are ignored. */
typedef struct {
  int64_t batch;
  int64_t token;
  int64_t head;
} hisa_strides_t;

/* Thread-local text describing the last non-OK status (empty if none). */
const char* hisa_last_error(void);

/* ABI version of this header (incremented on incompatible changes). */
int hisa_abi_version(void);

/* Step 1: block summaries (HISA explainer 1.2.1: fixed blocks, mean pooling;
 * HISA news article: one feature vector per block).
 *   kidx     bf16 [batch][L][d], element (b, j, i) at b*ks.batch + j*ks.token + i.
 *   proj     optional bf16 [d][d] row-major; when given, every row becomes
 *            proj @ row (the two-level decode's chunk key, HiLS chapter,
 *            "learnable chunk-mass proxy", stood in by a fixed projection).
 *   summary  optional fp32 [batch][n_rows][d], n_rows = ceil(L / B): row c is
 *            the mean of tokens c*B .. min(L, (c+1)*B) - 1 (projected if proj).
 *   split    optional bf16 [batch][n_rows][3][d]: three bf16 terms hi, mid, lo
 *            whose exact sum is the fp32 row SUM (projected if proj), the
 *            operand of hisa_block_score's bf16 matrix-core product.
 * At least one of summary and split must be non-NULL. */
hisa_status_t hisa_block_summary(const void* kidx, hisa_strides_t ks, int batch, int L, int d,
                                 int B, const void* proj, float* summary, void* split,
                                 hisa_stream_t stream);

/* Step 1 for a growing cache (decode). A block's summary depends on its own
 * tokens only (HISA explainer 1.2.1, mean pooling over fixed blocks), and the
 * KV cache itself is left as it is (HISA news article, drop-in replacement),
 * so after the cache of every sequence has grown to L tokens only the rows
 * of the blocks that changed need recomputing. Recomputes rows
 * first_row .. ceil(L/B) - 1 of tables laid out with n_rows_cap rows per
 * sequence (summary fp32 [batch][n_rows_cap][d], split bf16
 * [batch][n_rows_cap][3][d]); other rows are left untouched.
 *   first_row = (L - 1) / B: the block holding the newest token (one decode
 *                step: the block it starts, extends or completes);
 *   first_row = 0: the whole table, built in this layout.
 * hisa_block_score and hisa_select_blocks then take n_rows = n_rows_cap;
 * rows past ceil(L/B) - 1 are never read. Other arguments and errors as
 * hisa_block_summary; HISA_ERR_SHAPE if n_rows_cap < ceil(L/B) or first_row
 * is outside [0, ceil(L/B)). */
hisa_status_t hisa_block_summary_update(const void* kidx, hisa_strides_t ks, int batch, int L,
                                        int d, int B, const void* proj, float* summary,
                                        void* split, int n_rows_cap, int first_row,
                                        hisa_stream_t stream);

/* Step 2: block scores (HISA explainer 1.2.1 item 2; HISA news article,
 * block-level coarse filter: the indexer's own dot product against the
 * block features only).
 *   qidx         bf16 [batch][nq][d], element (b, i, :) at b*qs.batch + i*qs.token.
 *   q_pos        int32 [batch][nq]: absolute position t of each query, 0 <= t < n_rows*B.
 *   split        the split output of hisa_block_summary for the same batch.
 *   block_scores fp32 [batch][nq][n_rows]: entry c is qidx . summary[c] for
 *                complete blocks c < t / B, and -inf for c >= t / B. */
hisa_status_t hisa_block_score(const void* qidx, hisa_strides_t qs, const int32_t* q_pos,
                               int batch, int nq, const void* split, int n_rows, int d, int B,
                               float* block_scores, hisa_stream_t stream);

/* Step 3: top-m blocks (HISA explainer 1.2.1 item 3; HISA news article: keep
 * m blocks, the first and the last always kept). With b = t / B the kept set
 * is {0, b} plus the best m - 2 of blocks 1 .. b-1 by score (ties to the
 * lowest id); when those candidates all fit, blocks 0 .. b are kept.
 *   block_scores fp32 [batch][nq][n_rows] as written by hisa_block_score.
 *   block_idx    int32 [batch][nq][m], ascending, -1 padded. */
hisa_status_t hisa_select_blocks(const float* block_scores, const int32_t* q_pos, int batch,
                                 int nq, int n_rows, int B, int m, int32_t* block_idx,
                                 hisa_stream_t stream);

/* Steps 2 and 3 in one call: the same block_idx as hisa_block_score followed
 * by hisa_select_blocks (bit for bit: the same exact products and
 * selection), without writing the block scores to memory. For m <= 130 and
 * n_rows <= 65537 the scores of 16 or 32 consecutive queries are streamed
 * through per-query candidate buffers on chip; otherwise all of their scores
 * are held on chip, which needs n_rows <= 1026 (HISA_ERR_UNSUPPORTED beyond
 * both: use the two calls). Arguments as for those two, plus:
 *   workspace  optional device scratch (NULL allowed), 256-byte aligned, of
 *              hisa_route_blocks_workspace_bytes() bytes; its contents on
 *              entry are ignored. When that size is non-zero (fewer than 1024
 *              queries, m - 2 <= 64, at most 2048 survivors per query) the
 *              candidate blocks of each query are scored and reduced to their
 *              best m - 2 in parts of 256 over several workgroups and merged,
 *              which keeps the chip busy for the few queries of a decode step;
 *              with NULL the same result comes from one workgroup per query
 *              group. A non-NULL workspace smaller than needed is
 *              HISA_ERR_WORKSPACE; for shapes that need none it is ignored. */
size_t hisa_route_blocks_workspace_bytes(int batch, int nq, int n_rows, int m);
hisa_status_t hisa_route_blocks(const void* qidx, hisa_strides_t qs, const int32_t* q_pos,
                                int batch, int nq, const void* split, int n_rows, int d, int B,
                                int m, int32_t* block_idx, void* workspace,
                                size_t workspace_bytes, hisa_stream_t stream);

/* Step 4: token top-k inside the kept blocks (HISA explainer 1.2.2; HISA news
 * article, fine token selection). Candidates are the tokens j <= t of the
 * blocks in block_idx; each scores qidx . kidx[j]; the best min(k, #cand)
 * are kept (ties to the lowest j).
 *   token_idx     int32 [batch][nq][k], ascending, -1 padded.
 *   token_scores  optional fp32 [batch][nq][k], the score of each kept token
 *                 (NaN in padded slots).
 *   workspace     device scratch of at least hisa_token_select_workspace_bytes()
 *                 bytes, 256-byte aligned; contents on entry are ignored. */
hisa_status_t hisa_token_select(const void* qidx, hisa_strides_t qs, const void* kidx,
                                hisa_strides_t ks, const int32_t* q_pos, const int32_t* block_idx,
                                int batch, int nq, int L, int d, int B, int m, int k,
                                int32_t* token_idx, float* token_scores, void* workspace,
                                size_t workspace_bytes, hisa_stream_t stream);
size_t hisa_token_select_workspace_bytes(int batch, int nq, int L, int B, int m, int k);

/* hisa_token_select without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation. Same arguments (less the workspace), checks and
 * results as hisa_token_select. Its scratch is one fixed array of
 * HISA_NOALLOC_SCRATCH_BYTES in device memory that the library holds on every
 * GPU it runs on until the process ends; the array of the current device is
 * used (the stream must belong to that device). Shapes whose
 * hisa_token_select_workspace_bytes() exceed HISA_NOALLOC_SCRATCH_BYTES (the
 * decode and small-prefill shapes fit; a 16K-query prefill does not) return
 * HISA_ERR_UNSUPPORTED. Every call on a GPU shares that GPU's array: calls that
 * overlap in time on one GPU (different streams, or threads without ordering)
 * race and their results are undefined; calls in stream order are safe (each
 * clears what it needs). Calls no allocating routine; the first call on a
 * device looks up the array's device address (HISA_ERR_HIP if that fails). */
#define HISA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
hisa_status_t hisa_token_select_noalloc(const void* qidx, hisa_strides_t qs, const void* kidx,
                                        hisa_strides_t ks, const int32_t* q_pos,
                                        const int32_t* block_idx, int batch, int nq, int L, int d,
                                        int B, int m, int k, int32_t* token_idx,
                                        float* token_scores, hisa_stream_t stream);

/* Runtime policy (HISA explainer 1.3 item 3, the adaptive mechanism, and
 * 3.2 item 2, the dynamic number of kept blocks; HISA news article: short
 * texts fall back to the original indexer). For a sequence of L keys and
 * block size B:
 *   *hierarchical  0 when L < 8192 (the caller runs flat_indexer_topk), else
 *                  1 (hisa_block_score .. hisa_token_select); the pages leave
 *                  8192 <= L <= 16384 open and this takes the hierarchical
 *                  path there.
 *   *m             max(64, L / 2000), clamped to 16384 / B (the largest
 *                  supported m*B).
 * Host-only: launches nothing. HISA_ERR_NULL for null outputs, HISA_ERR_SHAPE
 * for L < 1, HISA_ERR_UNSUPPORTED for an unsupported B. */
hisa_status_t hisa_auto_plan(int L, int B, int* hierarchical, int* m);

/* Flat comparison indexer (HISA explainer 1.1 item 1; HISA news article: the
 * original indexer scores every earlier token). Candidates are all j <= t;
 * output format as hisa_token_select. */
hisa_status_t flat_indexer_topk(const void* qidx, hisa_strides_t qs, const void* kidx,
                                hisa_strides_t ks, const int32_t* q_pos, int batch, int nq, int L,
                                int d, int k, int32_t* token_idx, float* token_scores,
                                void* workspace, size_t workspace_bytes, hisa_stream_t stream);
size_t flat_indexer_topk_workspace_bytes(int batch, int nq, int L, int k);

/* Step 5: softmax attention over the selected tokens only (HISA explainer
 * 1.1; HISA news article: the downstream sparse attention is unchanged).
 *   q    bf16 [batch][nq][Hq][Dk]   strides qs (batch, token, head).
 *   k    bf16 [batch][L][Hkv][Dk]   strides ks.
 *   v    bf16 [batch][L][Hkv][Dv]   strides vs; may alias k (the first Dv
 *        columns of a latent row, as in multi-head latent attention).
 *   token_idx int32 [batch][nq][topk]; entries outside [0, L) (the -1
 *        padding, or any other out-of-range id) are skipped: they take no
 *        part in the softmax and read no memory beyond the cache.
 *   out  bf16 [batch][nq][Hq][Dv]   strides os; like q, k and v it must be
 *        16-byte aligned with strides in multiples of 8 elements (the kernels
 *        store whole 16-byte pieces), else HISA_ERR_SHAPE.
 *   lse  optional fp32 [batch][nq][Hq]: natural-log sum of exp(scale*q.k)
 *        over the kept tokens (-inf for an empty set, whose output is 0).
 *   workspace  optional device scratch of sparse_attn_fwd_workspace_bytes()
 *        bytes, 256-byte aligned, contents on entry ignored. With it, few
 *        (query, kv head) pairs with long token lists (decode) split each list
 *        over several waves and merge the parts; NULL runs unsplit (same
 *        result up to fp32 rounding, slower for such shapes). A non-NULL
 *        workspace that is too small is HISA_ERR_WORKSPACE. The size is 0 when
 *        the shape never splits.
 * Query head h reads kv head h / (Hq / Hkv). */
hisa_status_t sparse_attn_fwd(const void* q, hisa_strides_t qs, const void* k, hisa_strides_t ks,
                              const void* v, hisa_strides_t vs, int batch, int nq, int L, int Hq,
                              int Hkv, int Dk, int Dv, const int32_t* token_idx, int topk,
                              float scale, void* out, hisa_strides_t os, float* lse,
                              void* workspace, size_t workspace_bytes, hisa_stream_t stream);
size_t sparse_attn_fwd_workspace_bytes(int batch, int nq, int Hq, int Hkv, int Dk, int Dv,
                                       int topk);

/* Two-level (chunk x token) softmax decode at position t = L - 1 (HiLS
 * chapter, "hierarchical softmax decomposition"; HiLS-7B write-up, "what is
 * HiLS-Attention"). For each (sequence, head) the output is
 *   sum over chosen chunks c of softmax_c(scale_chunk * q . khat_c)
 *       * sum over tokens j of chunk c, j <= t, of softmax_j(scale_token * q . k_j) v_j.
 *   q         bf16 [batch][H][D], strides qs (batch, head).
 *   k, v      bf16 [batch][L][H][D], strides (batch, token, head).
 *   khat      fp32 [batch*H][n_rows][D]: chunk keys from hisa_block_summary
 *             run with batch*H sequences (row b*H + h).
 *   chunk_idx int32 [batch*H][m]: chosen chunks (from hisa_select_blocks),
 *             ascending, -1 padded.
 *   out       bf16 [batch][H][D], strides os (batch, head).
 *   workspace optional device scratch of hils_two_level_attn_fwd_workspace_bytes()
 *             bytes, 256-byte aligned, contents on entry ignored. With it, few
 *             (sequence, head) pairs spread their chosen chunks over many
 *             workgroups and merge the chunk results in a second kernel; NULL
 *             runs one workgroup per pair (same result up to fp32 rounding).
 *             A non-NULL workspace that is too small is HISA_ERR_WORKSPACE;
 *             the size is 0 when the shape never splits. */
hisa_status_t hils_two_level_attn_fwd(const void* q, hisa_strides_t qs, const void* k,
                                      hisa_strides_t ks, const void* v, hisa_strides_t vs,
                                      const float* khat, const int32_t* chunk_idx, int batch,
                                      int L, int H, int D, int C, int n_rows, int m,
                                      float scale_chunk, float scale_token, void* out,
                                      hisa_strides_t os, void* workspace, size_t workspace_bytes,
                                      hisa_stream_t stream);
size_t hils_two_level_attn_fwd_workspace_bytes(int batch, int H, int D, int m);

/* Causal two-level prefill (HiLS chapter, "hierarchical softmax
 * decomposition" applied at every position, as the decode of the tokens up to
 * the query). The query of sequence b at position t = q_pos[b][i] gets, per
 * head, the two-level output of the decode over tokens 0 .. t: complete chunks
 * c < t / C keep their keys khat_c, the local chunk t / C is keyed by
 *   proj @ (mean of its tokens t/C*C .. t)
 * (formed in the kernel), and its token softmax stops at t.
 *   q         bf16 [batch][nq][H][D], strides qs (batch, token, head).
 *   k, v      bf16 [batch][L][H][D], strides (batch, token, head).
 *   khat      fp32 [batch*H][n_rows][D]: chunk keys of the whole cache from
 *             hisa_block_summary with the same proj, batch*H sequences (row
 *             b*H + h); the local chunk's row is not read.
 *   chunk_idx int32 [batch*H][nq][m]: chosen chunks of each query (from
 *             hisa_block_score / hisa_select_blocks over sequence b*H + h
 *             with q_pos[b]), ascending, -1 padded; ids above t / C are
 *             ignored.
 *   proj      bf16 [D][D] row-major, the projection khat was made with, or
 *             NULL when khat is the plain mean.
 *   q_pos     int32 [batch][nq]: each query's position, clamped to [0, L-1].
 *   out       bf16 [batch][nq][H][D], strides os (batch, token, head).
 *   workspace optional device scratch of hils_two_level_prefill_fwd_workspace_bytes()
 *             bytes, 256-byte aligned, contents on entry ignored. With it, the
 *             (query, slot) entries are bucketed by chunk and each chunk's K
 *             and V rows are read once per 64 entries (matrix cores), with a
 *             per-entry partial result (fp16, scaled per row by a power of
 *             two: 11 significant bits relative to the row's largest value)
 *             merged per query; NULL runs one workgroup per (query, head)
 *             gathering its own chunks in fp32 (for few queries; the two
 *             differ by that rounding). Too small is
 *             HISA_ERR_WORKSPACE. Its size is about batch*H*(nq*m*(2D + 13)
 *             + L*D*4) bytes (fp16 per-entry partials, the local keys).
 * q, k, v and out 16-byte aligned with strides in multiples of 8 elements;
 * khat and proj 16-byte aligned. batch*H <= 65535, batch*H*nq*m < 2^32; sizes must be
 * >= 1. */
hisa_status_t hils_two_level_prefill_fwd(const void* q, hisa_strides_t qs, const void* k,
                                         hisa_strides_t ks, const void* v, hisa_strides_t vs,
                                         const float* khat, const int32_t* chunk_idx,
                                         const void* proj, const int32_t* q_pos, int batch,
                                         int nq, int L, int H, int D, int C, int n_rows, int m,
                                         float scale_chunk, float scale_token, void* out,
                                         hisa_strides_t os, void* workspace,
                                         size_t workspace_bytes, hisa_stream_t stream);
size_t hils_two_level_prefill_fwd_workspace_bytes(int batch, int nq, int L, int H, int D, int C,
                                                  int m);

/* Gather-rate probe: the memory side of sparse attention alone. For each of
 * nq queries it streams the rows named by ids[q][0 .. topk) of a resident
 * table into on-chip memory the way the attention kernels do (16-byte direct
 * loads, 8 lanes per 128-byte line, one workgroup per query, queries dealt
 * to the XCDs in contiguous ranges, `depth` tiles of 32 rows in flight per
 * wave) and discards them. Its rate is the ceiling that gathering alone
 * allows for those id lists; the attention over the selected tokens (HISA
 * explainer 1.1) and the memory-bound token selection (explainer 1.3) are
 * measured against it. Writes no memory.
 *   table      device rows of row_stride_bytes (a multiple of 16, >= row_bytes),
 *              n_rows of them, 16-byte aligned.
 *   row_bytes  256 or 1152 (a 128-wide bf16 K row, or a 576-wide latent row).
 *   ids        int32 [nq][topk], 1 <= topk <= 4096; ids outside [0, n_rows)
 *              read row 0.
 *   waves      4 or 8 waves per workgroup; depth 1 .. 4.
 *   rot_ticks  0: every query reads its rows in list order. > 0: each query
 *              starts at tile (t / rot_ticks) mod tiles, t the GPU's
 *              constant-rate real-time counter when its workgroup starts, and
 *              wraps around (the order of the rows read changes, not the set).
 * HISA_ERR_NULL / _SHAPE / _UNSUPPORTED on bad arguments, HISA_ERR_HIP on a
 * launch error. */
hisa_status_t hisa_gather_probe(const void* table, int64_t row_stride_bytes, int row_bytes,
                                int n_rows, const int32_t* ids, int nq, int topk, int waves,
                                int depth, int rot_ticks, hisa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* HISA_H */
