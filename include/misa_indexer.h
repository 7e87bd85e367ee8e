/*
 * misa_indexer.h -- C ABI of the MI355X (gfx950) token-level sparse-attention
 * indexer: the dense DSA indexer, its MISA form (block-pooled head router,
 * routed-head token scoring, top-k) and the MISA-dagger rerank.
 *
 * What the calls compute follows "MISA: Mixture of Indexer Sparse Attention
 * for Long-Context LLM Inference" (gist.science explainer), Technical Summary
 * -- Problem Statement (the DSA indexer scores every prefix token with all
 * H_I heads and keeps a per-query top-k), Methodology: MISA (router over
 * M = ceil(L/B) mean-pooled blocks keeps h heads; only those heads score the
 * prefix; top-k of the reduced score), Hierarchical Variant (MISA-dagger: the
 * routed pass keeps k' candidates, the all-head indexer rescores them and
 * keeps k) -- and the MISA abstract (heads share one selected token set; a
 * query-dependent subset of heads).
 *
 * Where the pages are silent this library takes these readings:
 *   - the prefix of a query at position p is tokens 0..p (inclusive);
 *   - the indexer score of token i is I(i) = sum_j w_j * max(0, q_j . k_i)
 *     over the scoring heads j (no extra scale: fold it into w);
 *   - blocks start at token 0; a block's pooled key is the mean of the keys
 *     present in it; the query's own last block is the mean of its prefix
 *     tokens in that block;
 *   - router importance g_j = w'_j * sum_b max(0, q_j . Kbar_b) over the
 *     query's blocks, w' = w (mode 0) or |w| (mode 1); the top-h heads by
 *     (g desc, head id asc) are routed;
 *   - token ranking is (score desc, token id asc); -0.0 ranks as +0.0.
 *
 * Conventions for every call
 *   - Tensor pointers are DEVICE pointers (hipMalloc'd or from a framework
 *     allocator).  The caller owns every buffer; the library keeps no pointer
 *     after returning and allocates nothing.  Its one global object is the
 *     static scratch array of misa_indexer_noalloc (see there).
 *   - keys, q, pooled keys, workspaces and misa_score's output are moved in
 *     16-byte vectors: their base addresses must be 16-byte aligned (any
 *     allocator's are; a view into one may not be), else the call returns
 *     MISA_ERR_UNSUPPORTED.  Every other pointer needs only its element's
 *     natural alignment (misa_topk's score rows included).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues kernels on it: no host synchronisation, no
 *     allocation, no memset node (graph capture is safe).
 *   - Workspaces are caller-provided device buffers of at least the size
 *     misa_workspace_bytes() reports for the same arguments; their contents
 *     on entry do not matter and are overwritten.  Calls that share a
 *     workspace must be ordered on one stream.
 *   - Selected-token outputs idx[T][k] are SETS: the order of the k entries of
 *     a row is unspecified.  A slot with no token holds idx = -1 and
 *     score = -inf (a prefix, or a candidate list, shorter than k).
 *   - Only host-visible arguments are validated, all before any HIP call; a
 *     failed check returns a negative status and enqueues nothing.  Values
 *     that live on the device (q_pos < seq_lens[q_seq], head and candidate
 *     ids in range and distinct) are NOT checked: out-of-range values are
 *     undefined behaviour.  A launch error returns MISA_ERR_HIP.  No C++
 *     exception crosses the boundary.
 */
#ifndef MISA_INDEXER_H
#define MISA_INDEXER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MISA_OK 0
#define MISA_ERR_NULL (-1)        /* a required pointer is NULL                 */
#define MISA_ERR_SHAPE (-2)       /* a size or count is out of range            */
#define MISA_ERR_UNSUPPORTED (-3) /* a valid request the library does not handle */
#define MISA_ERR_WORKSPACE (-4)   /* workspace smaller than required            */
#define MISA_ERR_HIP (-5)         /* a HIP launch or runtime call failed        */
#define MISA_ERR_TOO_LARGE (-6)   /* more scratch than misa_indexer_noalloc's
                                     static buffer holds                        */

/* The key dimension the library supports. */
#define MISA_D 128
/* Largest number of indexer heads H (and routed heads h). */
#define MISA_MAX_HEADS 128

/*
 * One batch of indexer inputs.  All pointers are device pointers.
 *   keys     bf16 bits [S][Lmax][d], row-major: one indexing key per token,
 *            shared by all heads (MISA abstract).
 *   seq_lens int32 [S]: keys present in each sequence (read by misa_pool).
 *   q        bf16 bits [T][H][d]: H indexer-head queries per query row.
 *   w        fp32 [T][H]: per-query head weights.
 *   q_seq    int32 [T]: the sequence of each query row.
 *   q_pos    int32 [T]: the position p_t of each query; its prefix is 0..p_t.
 * d must equal MISA_D; 1 <= H <= MISA_MAX_HEADS; S, T, Lmax >= 1.
 * Calls that take query rows accept T <= 65535 (rows go on a grid dimension
 * of that size); misa_pool and misa_pool_append accept S <= 65535, and
 * misa_topk rows <= 65535.  Larger values return MISA_ERR_UNSUPPORTED.
 */
typedef struct misa_batch {
  const uint16_t *keys;
  const int32_t *seq_lens;
  const uint16_t *q;
  const float *w;
  const int32_t *q_seq;
  const int32_t *q_pos;
  int32_t S, Lmax, d, T, H;
} misa_batch;

/* Operation selector for misa_workspace_bytes. */
#define MISA_OP_DENSE 0       /* indexer_dense                        */
#define MISA_OP_ROUTE 1       /* misa_route                           */
#define MISA_OP_SCORE_TOPK 2  /* misa_score_topk                      */
#define MISA_OP_RERANK 3      /* misa_rerank                          */
#define MISA_OP_TOPK 4        /* misa_topk (b->T rows of b->Lmax)     */
#define MISA_OP_INDEXER 5     /* misa_indexer                         */
#define MISA_OP_HISA 6        /* hisa_indexer, hisa_blocks (kc = m)   */

/*
 * misa_workspace_bytes: device workspace needed by operation `op` for this
 * batch shape.  B is the block size (MISA_OP_ROUTE), h the routed head count
 * (MISA_OP_ROUTE / MISA_OP_SCORE_TOPK), k the selection size, kc the
 * candidate count (MISA_OP_RERANK).  Only the shape fields of `b` are read.
 * Writes the size to *bytes; returns a status.
 */
int misa_workspace_bytes(const misa_batch *b, int32_t op, int32_t B, int32_t h,
                         int32_t k, int32_t kc, size_t *bytes);

/*
 * misa_pool -- mean-pooled indexing keys (Methodology: MISA, Lightweight
 * Block-Pooled Router: the prefix is cut into M = ceil(L/B) blocks
 * summarised by mean-pooled indexing keys).
 *   pooled  fp32 [S][ceil(Lmax/B)][d] (output): pooled[s][b] = mean of
 *           keys[s][i] over i in [bB, min(bB+B, seq_lens[s])); a block with
 *           no key present is written as zeros.
 * Run once per key cache (and again after keys are appended); misa_route
 * reads it.  Uses keys, seq_lens, S, Lmax, d.  1 <= B <= Lmax.
 */
int misa_pool(const misa_batch *b, int32_t B, float *pooled, void *stream);

/*
 * misa_pool_append -- bring misa_pool's output up to date after keys were
 * appended to the sequences (streaming decode), recomputing only the blocks
 * that hold an appended key.  The router's block summaries are a cache
 * computed once (Methodology: MISA, Lightweight Block-Pooled Router, whose
 * cost is per-head affinities over the M pooled blocks); appending a token
 * changes only block floor(L / B), so each decode step costs O(B d) here.
 *   seq_lens  (in the batch) the lengths after the append.
 *   old_lens  int32 [S] (device): the lengths pooled last reflects.
 *   max_new   host: an upper bound of seq_lens[s] - old_lens[s] over s;
 *             0 <= max_new <= Lmax.
 *   pooled    fp32 [S][ceil(Lmax/B)][d], updated in place: blocks
 *             floor(old_lens[s]/B) .. ceil(seq_lens[s]/B)-1 are rewritten
 *             exactly as misa_pool writes them; the others are not touched.
 * Device-resident values are not checked: 0 <= old_lens[s] <= seq_lens[s]
 * <= Lmax and seq_lens[s] - old_lens[s] <= max_new are the caller's to
 * keep (otherwise some appended blocks are left stale).
 */
int misa_pool_append(const misa_batch *b, int32_t B, const int32_t *old_lens, int32_t max_new,
                     float *pooled, void *stream);

/*
 * misa_route -- the block-pooled head router (Methodology: MISA,
 * Lightweight Block-Pooled Router; the MISA abstract's query-dependent
 * subset of heads).  For query t with b_t = floor(p_t / B):
 *   g[t][j] = w'_j * ( sum_{b < b_t} max(0, q_j . pooled[s][b])
 *                      + max(0, q_j . mean(keys[s][b_t*B .. p_t])) ),
 * w' = w (mode 0) or |w| (mode 1); heads[t][0..h) = the top-h heads by
 * (g desc, head id asc), in that rank order.
 *   pooled      misa_pool's output for the same keys and the same B; only
 *               complete blocks b < b_t are read, the query's own last block
 *               is pooled from the keys.
 *   heads       int32 [T][h] (output).
 *   head_score  fp32 [T][H] (output, may be NULL): g.
 *   ws/ws_bytes workspace (MISA_OP_ROUTE).
 * 1 <= h <= H; mode in {0, 1}; 1 <= B <= Lmax.
 */
int misa_route(const misa_batch *b, const float *pooled, int32_t B, int32_t h,
               int32_t mode, int32_t *heads, float *head_score, void *ws,
               size_t ws_bytes, void *stream);

/*
 * misa_score -- indexer score rows (Methodology: MISA, Sparse Token Scoring;
 * with heads == NULL, the dense DSA indexer of the Problem Statement).
 *   heads   int32 [T][h] routed head ids, or NULL for all H heads.
 *   scores  fp32 [T][Lmax] (output): I(i) for i <= p_t, -inf for i > p_t.
 * bf16 products, fp32 accumulation.  1 <= h <= H when heads != NULL.  One
 * sequence with at least 64 rows takes the MFMA tiling of misa_score_topk;
 * several sequences are scored row by row (this call has no workspace for
 * the tile table).
 */
int misa_score(const misa_batch *b, const int32_t *heads, int32_t h,
               float *scores, void *stream);

/*
 * misa_topk -- per-row top-k of fp32 score rows by (score desc, index asc).
 *   scores   fp32 [rows][ld]; row r's candidates are columns [0, row_len[r]).
 *   row_len  int32 [rows] (device), each in [0, ld].
 *   idx      int32 [rows][k] (output), val fp32 [rows][k] (output, may be
 *            NULL): the selected columns and their scores (a set).
 * Scores must not be NaN.  ws: MISA_OP_TOPK with the batch {T=rows, Lmax=ld}.
 */
int misa_topk(const float *scores, int32_t rows, int32_t ld,
              const int32_t *row_len, int32_t k, int32_t *idx, float *val,
              void *ws, size_t ws_bytes, void *stream);

/*
 * misa_score_topk -- routed token scoring and per-query top-k (Methodology:
 * MISA, Sparse Token Scoring).  With k = k' this is MISA-dagger's Coarse
 * Stage (Hierarchical Variant).
 *   heads   int32 [T][h] (misa_route's output), or NULL for all H heads.
 *   idx     int32 [T][k] (output) selected token ids, val fp32 [T][k]
 *           (output, may be NULL) their scores.
 * 1 <= k <= Lmax.  ws: MISA_OP_SCORE_TOPK.
 * How it runs (results are the same up to fp32 summation order):
 *   - one sequence (S = 1), at least 64 rows, at most 64 head slots a query:
 *     a 32x32 MFMA tiling that reads each key once per tile of queries; with
 *     5..16 routed heads and at least 256 rows longer than 16384 keys the
 *     top-k comes from threshold lists the tiling writes instead of score
 *     rows, and rows those lists cannot settle are rescored one by one;
 *   - several sequences with at least two rows per sequence on average: the
 *     same tiling over a table of runs of equal q_seq built on the device,
 *     so a sequence's rows share one pass over its keys.  Keep the rows of
 *     a sequence contiguous; otherwise every row is scored on its own
 *     (still correct);
 *   - otherwise each row streams its prefix.
 */
int misa_score_topk(const misa_batch *b, const int32_t *heads, int32_t h,
                    int32_t k, int32_t *idx, float *val, void *ws,
                    size_t ws_bytes, void *stream);

/*
 * misa_score_topk_ev -- misa_score_topk with a measurement hook: ev_start and
 * ev_stop (hipEvent_t passed as void*, created by the caller; either may be
 * NULL) are attached to the token-scoring kernel launches on `stream`
 * (hipExtLaunchKernelGGL), which stamp them with the begin of the first and
 * the end of the last of those kernels, so hipEventElapsedTime(ev_start,
 * ev_stop) is the scoring kernels' own duration.  Everything else is exactly
 * misa_score_topk.
 */
int misa_score_topk_ev(const misa_batch *b, const int32_t *heads, int32_t h,
                       int32_t k, int32_t *idx, float *val, void *ws,
                       size_t ws_bytes, void *stream, void *ev_start,
                       void *ev_stop);

/*
 * indexer_dense -- the DSA lightning indexer: all H heads score every
 * prefix key, then the per-query top-k (Problem Statement).  Same outputs as
 * misa_score_topk with heads == NULL.  ws: MISA_OP_DENSE.
 */
int indexer_dense(const misa_batch *b, int32_t k, int32_t *idx, float *val,
                  void *ws, size_t ws_bytes, void *stream);

/*
 * misa_rerank -- MISA-dagger's Fine Stage (Hierarchical Variant): the
 * all-head indexer rescores only the candidates and keeps the top-k.
 *   cand    int32 [T][kc]: distinct token ids of query t's prefix, -1 for an
 *           empty slot (misa_score_topk's idx with k = kc).
 *   idx     int32 [T][k] (output) token ids, val fp32 [T][k] (output, may be
 *           NULL) their all-head scores, ranked (score desc, token id asc).
 * 1 <= k <= kc.  ws: MISA_OP_RERANK.
 */
int misa_rerank(const misa_batch *b, const int32_t *cand, int32_t kc, int32_t k,
                int32_t *idx, float *val, void *ws, size_t ws_bytes,
                void *stream);

/*
 * misa_indexer -- the whole MISA indexer step in one call: the router
 * (exactly misa_route), then routed token scoring and the per-query top-k
 * (exactly misa_score_topk with those heads) -- Methodology: MISA, both
 * stages.  Outputs as the two calls: heads [T][h] (rank order), head_score
 * [T][H] (may be NULL), idx/val [T][k].  One workspace (MISA_OP_INDEXER with
 * B, h and k) holds both steps' scratch.
 */
int misa_indexer(const misa_batch *b, const float *pooled, int32_t B, int32_t h,
                 int32_t mode, int32_t k, int32_t *heads, float *head_score,
                 int32_t *idx, float *val, void *ws, size_t ws_bytes,
                 void *stream);

/*
 * misa_indexer_ev -- misa_indexer with the measurement hook of
 * misa_score_topk_ev (events around the token-scoring kernel).
 */
int misa_indexer_ev(const misa_batch *b, const float *pooled, int32_t B,
                    int32_t h, int32_t mode, int32_t k, int32_t *heads,
                    float *head_score, int32_t *idx, float *val, void *ws,
                    size_t ws_bytes, void *stream, void *ev_start,
                    void *ev_stop);

/*
 * misa_indexer_noalloc -- misa_indexer for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, outputs
 * and kernels as misa_indexer, without ws / ws_bytes: the scratch is a
 * static device array of MISA_NOALLOC_SCRATCH_BYTES inside the library, one
 * copy per GPU (on the device current at the call, which must be the
 * stream's device), reserved when the library is loaded on that GPU and held
 * until the process ends.  The first call on a device looks up that copy's
 * address (hipGetSymbolAddress); no call allocates or frees memory.
 *   Limit: a batch whose MISA_OP_INDEXER workspace (misa_workspace_bytes with
 *   the same B, h, k) exceeds MISA_NOALLOC_SCRATCH_BYTES is rejected with
 *   MISA_ERR_TOO_LARGE before anything is enqueued -- for example 16
 *   sequences of 131072 keys with k = 2048 need about 25 MiB, 32 such
 *   sequences do not fit.
 *   Every call on one GPU uses the same scratch, and a call leaves its
 *   contents behind: calls on one GPU must be ordered (one stream, or events
 *   between streams); calls that overlap race and give undefined results.
 */
#define MISA_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)
int misa_indexer_noalloc(const misa_batch *b, const float *pooled, int32_t B,
                         int32_t h, int32_t mode, int32_t k, int32_t *heads,
                         float *head_score, int32_t *idx, float *val,
                         void *stream);

/*
 * hisa_indexer -- the hierarchical block-to-token indexer ("HISA: Efficient
 * Hierarchical Indexing for Fine-Grained Sparse Attention", abstract: first
 * whole blocks are ranked by a score on their pooled summaries and the
 * low-ranked ones dropped, then the unchanged token-level indexer scores only
 * the tokens of the blocks that survive and returns its usual top-k set).
 * Readings, the pages giving no formula: a block's representation is its
 * mean key (misa_pool's cache; the query's own last block is the mean over
 * [floor(p/B)*B, p]); its score is the indexer's form on that mean,
 *   s_b = sum_{j in heads} w_j * max(0, q_j . Kbar_b);
 * the m blocks with the largest s_b are kept (ties: lower block id); every
 * prefix token of the kept blocks is scored with the same heads and the
 * top-k by (score desc, token id asc) is written, padded with -1 / -inf.
 *   pooled  misa_pool's output for the same keys and B.
 *   m       kept blocks, 1 <= m <= ceil(Lmax/B) (not on the pages).
 *   heads   NULL: all H heads (HISA; h must be 0).  int32 [T][h] (device):
 *           these heads in both stages -- the routed heads of misa_route,
 *           giving MISA composed with HISA (head axis, then token axis).
 *   idx/val [T][k] (val may be NULL).  Workspace: misa_workspace_bytes with
 *           MISA_OP_HISA, kc = m.  1 <= k <= Lmax.
 */
int hisa_indexer(const misa_batch *b, const float *pooled, int32_t B, int32_t m,
                 const int32_t *heads, int32_t h, int32_t k, int32_t *idx, float *val, void *ws,
                 size_t ws_bytes, void *stream);

/* hisa_indexer with the measurement hook of misa_score_topk_ev: the
 * hipEvent_t handles (either may be NULL) mark the begin and end of the
 * token-level scoring kernel. */
int hisa_indexer_ev(const misa_batch *b, const float *pooled, int32_t B, int32_t m,
                    const int32_t *heads, int32_t h, int32_t k, int32_t *idx, float *val, void *ws,
                    size_t ws_bytes, void *stream, void *ev_start, void *ev_stop);

/*
 * hisa_blocks -- hisa_indexer's coarse stage alone: block scores
 * fp32 [T][ceil(Lmax/B)] (-inf past the query's floor(p/B)+1 blocks; may be
 * NULL) and the m kept block ids int32 [T][m] (a set, -1 padded; may be
 * NULL).  Same arguments and workspace as hisa_indexer (k unused).
 */
int hisa_blocks(const misa_batch *b, const float *pooled, int32_t B, int32_t m,
                const int32_t *heads, int32_t h, float *block_scores, int32_t *blocks, void *ws,
                size_t ws_bytes, void *stream);

/*
 * misa_stream_read -- a plain streaming read of `bytes` of device memory at
 * `buf`, the bandwidth ceiling the decode roofline is measured against: the
 * buffer is cut into `wgs` contiguous slices, one workgroup each, read with
 * the 16-byte non-temporal loads the token-scoring kernel streams keys with.
 * sink (uint32 [wgs], device) receives one folded word per workgroup (its
 * value is meaningless).  ev_start / ev_stop: as misa_score_topk_ev (either
 * may be NULL).  buf and bytes must be 16-byte multiples; 1 <= wgs <= 65535.
 */
int misa_stream_read(const void *buf, size_t bytes, int32_t wgs, uint32_t *sink,
                     void *stream, void *ev_start, void *ev_stop);

/* misa_status_str -- a static English description of a status code. */
const char *misa_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* MISA_INDEXER_H */
