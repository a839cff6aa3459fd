/*
 * qsa.h -- C ABI of the MI355X (gfx950) Qwen Sparse Attention layer library.
 *
 * One QSA layer has three stages:
 *   1. an MQA indexer (4 query heads, 1 shared key head, dim 128) scores the
 *      mean-pooled 4-token micro-blocks of the causal past,
 *   2. each query keeps its top `budget` blocks (512 blocks = 2048 tokens),
 *   3. GQA attention (24 query heads, 2 KV heads, dim 256, RoPE on the first 64
 *      dims) runs over the selected blocks plus the query's own block.
 *
 * Sources (web pages on the Qwen3.8-Flash-Next release):
 *   [PKR] discuss.pytorch.kr, "Qwen3.8-Flash-Next, 1/9의 학습 비용으로
 *         Qwen3.7-Plus(397B-A17B) 수준에 도달한 125B-A6B 모델":
 *         spec table (rows Qwen Sparse Attention, QSA 인덱서, QSA 예산);
 *         section "QSA: 인덱서 자체의 비용을 줄이는 희소 어텐션" (pooling,
 *         compression before RoPE, score I_ib, block-causal rule, budget,
 *         always-included tail); section "100만 토큰까지 늘리기" (rope_parameters).
 *   [LMF] llmfeed.kr, "Qwen 팀, 새 구조를 적용한 Qwen3.8-Flash-Next 공개 가중치로
 *         출시", section "규모와 구조" (QSA bullet: shapes and budget).
 *   [YaRN] Peng et al. 2023, NTK-by-parts frequency ramp and temperature.
 *
 * Conventions for every entry point below
 *   - Pointers named q, k, v, q_idx, k_idx, *_cache, kpend, scores, block_idx,
 *     out, ws are DEVICE pointers to caller-owned memory; the library never
 *     allocates or frees them.  Every device pointer must be 16-byte aligned.
 *   - bf16 means IEEE bfloat16 stored as uint16_t.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and is asynchronous: the call returns before the GPU finishes.  Nothing
 *     synchronises the host.
 *   - All arguments are checked on the host before anything is enqueued.  A
 *     status other than QSA_OK means no kernel was launched and no buffer was
 *     touched, except QSA_ERR_HIP, which reports a failed launch (the HIP code
 *     is then available from qsa_last_hip_error()).  Faults inside kernels
 *     surface at the caller's next synchronisation.
 *   - A call with L = 0 is a no-op that returns QSA_OK after the shape checks
 *     (its pointers may then be NULL).
 *   - The batch B is 1 .. 65535 (QSA_ERR_SHAPE otherwise).
 *   - Inputs must be finite; non-finite values are not detected.
 *   - Calls that share a cache must be ordered (same stream or explicit
 *     events); the handle itself is immutable and may be shared by threads.
 *
 * Token-major input layouts (per call, positions q_offset .. q_offset+L-1):
 *   q      bf16 [B][L][24][256]     query heads
 *   k, v   bf16 [B][L][2][256]      key / value heads
 *   q_idx  bf16 [B][L][4][128]      indexer query heads
 *   k_idx  bf16 [B][L][128]         indexer key (one shared head)
 *   out    bf16 [B][L][24][256]     attention output (RNE from fp32)
 *
 * Caches (capacity max_ctx tokens per sequence; max_ctx is a multiple of 4):
 *   k_cache    bf16 [B][2][max_ctx/4][8][4][32]  rotated keys; micro-block
 *              `blk` of head g is 2 KiB at [b][g][blk]; inside it element
 *              (token 4*blk+t, dim d) sits at [d/32][t][d%32].
 *   v_cache    bf16 [B][2][max_ctx/4][256][4]    values; inside block `blk`
 *              element (token 4*blk+t, dim d) sits at [d][t].
 *   kbar_cache bf16 [B][max_ctx/4][128]          pooled, rotated indexer key
 *              of every complete block.
 *   kpend      bf16 [B][4][128]                  raw indexer keys of the
 *              current incomplete block (slot = position % 4).
 *
 * Scores (qsa_index output) are fp32 [B][L][ncol], ncol = ceil((q_offset+L)/4):
 *   entry (p, blk) = I_p,blk for blk < floor(p/4) (the candidates), else -1.
 * Selections are int32 [B][L][budget]: the selected candidate blocks of each
 *   query in ascending order, padded with -1.  The query's own block
 *   floor(p/4) is never listed; it is always attended over 4*floor(p/4)..p.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QSA_OK = 0,
    QSA_ERR_NULL = 1,         /* a required pointer is NULL */
    QSA_ERR_SHAPE = 2,        /* a size or count is out of range */
    QSA_ERR_UNSUPPORTED = 3,  /* head counts/dims other than the built ones */
    QSA_ERR_ALIGN = 4,        /* pointer not 16-byte aligned, or q_offset % 4 != 0 */
    QSA_ERR_CAPACITY = 5,     /* positions would reach beyond max_ctx */
    QSA_ERR_WORKSPACE = 6,    /* ws_bytes smaller than qsa_workspace_size() */
    QSA_ERR_HIP = 7           /* a HIP runtime call failed */
} qsa_status;

/* Layer parameters, fixed at handle creation.  The library is built for the
 * shapes of [PKR] spec table / [LMF] "규모와 구조": 24 query heads, 2 KV heads,
 * head dim 256, rotary dim 64; indexer 4 heads x 128 with rotary dim 64; micro-
 * block 4.  Other values return QSA_ERR_UNSUPPORTED.  budget_blocks is 1..512
 * ([PKR] spec table row QSA 예산).  The rotary frequencies are
 * rope_theta^(-2j/64), j = 0..31 ([PKR] "100만 토큰까지 늘리기": theta 1e7,
 * partial factor 0.25); yarn_factor > 1 applies the [YaRN] NTK-by-parts ramp
 * (alpha 1, beta 32) over yarn_orig_ctx and multiplies the attention logits by
 * (0.1 ln(yarn_factor) + 1)^2. */
typedef struct qsa_params {
    int32_t n_q_heads;      /* 24 */
    int32_t n_kv_heads;     /* 2 */
    int32_t head_dim;       /* 256 */
    int32_t rope_dim;       /* 64 */
    int32_t n_idx_heads;    /* 4 */
    int32_t idx_dim;        /* 128 */
    int32_t idx_rope_dim;   /* 64 */
    int32_t block;          /* 4 */
    int32_t budget_blocks;  /* 1..512 */
    int32_t topk_cap;       /* candidate list per query of the fused index + select
                               stage: 0 = 8192, else 64..8192 (smaller lists save
                               workspace; a list that overflows is recomputed exactly) */
    int64_t max_ctx;        /* cache capacity in tokens, multiple of 4, >= 4 */
    double  rope_theta;     /* 1e7 */
    double  yarn_factor;    /* 1.0 = off, else > 1 */
    int64_t yarn_orig_ctx;  /* 262144 */
} qsa_params;

typedef struct qsa_handle qsa_handle;

/* Operation codes for qsa_workspace_size. */
enum { QSA_OP_APPEND = 0, QSA_OP_INDEX = 1, QSA_OP_SELECT = 2, QSA_OP_ATTEND = 3,
       QSA_OP_FORWARD = 4, QSA_OP_DECODE = 5, QSA_OP_INDEX_SELECT = 6, QSA_OP_INDEX_DECODE = 7,
       QSA_OP_TOKEN_INDEX_SELECT = 8, QSA_OP_TOKEN_INDEX_DECODE = 9, QSA_OP_TRAIN_FORWARD = 10,
       QSA_OP_TRAIN_BACKWARD = 11 };

/* Fill *p with the layer's published shapes, budget 512, max_ctx 262144,
 * theta 1e7, no YaRN (factor 1), yarn_orig_ctx 262144.  Host only. */
void qsa_default_params(qsa_params *p);

/* Validate *params, build the fp32 cos/sin tables of positions 0..max_ctx-1 on
 * the host (fp64 libm cos/sin of position * frequency, rounded once to fp32)
 * and upload them to `device`.  The handle owns that device memory (2 x
 * max_ctx x 32 x 4 bytes) until qsa_destroy.  Returns QSA_ERR_NULL,
 * QSA_ERR_UNSUPPORTED, QSA_ERR_SHAPE or QSA_ERR_HIP on failure (*out = NULL). */
qsa_status qsa_create(const qsa_params *params, int device, qsa_handle **out);

/* Release the handle and its tables.  NULL is a no-op.  Not stream-ordered:
 * the caller must make sure no enqueued call still uses the handle. */
void qsa_destroy(qsa_handle *h);

/* Copy the handle's parameters to *out.  Host only. */
qsa_status qsa_get_params(const qsa_handle *h, qsa_params *out);

/* Workspace bytes `op` needs for `batch` sequences and `len` new tokens at
 * `q_offset` (for QSA_OP_DECODE: len = 1 and q_offset = ctx_bound, the host
 * upper bound of cache_len).  0 for invalid arguments.  Host only. */
size_t qsa_workspace_size(const qsa_handle *h, int op, int32_t batch, int64_t len, int64_t q_offset);

/* Cache fill (the keys' half of the prologue): for positions
 * t = q_offset .. q_offset+L-1 of each sequence, rotate k at t into k_cache,
 * copy v into v_cache, and push raw k_idx into the micro-block pool: every
 * block that becomes complete gets k̄ = bf16(rotate(mean of its 4 raw keys,
 * 4*blk)) in kbar_cache ([PKR] "QSA: ..." -- mean pooling, compression before
 * the positional encoding, block-start position); raw keys of a trailing
 * incomplete block are left in kpend.  Blocks that were incomplete before the
 * call take their earlier tokens from kpend.  Rotations are fp32 with every
 * product and sum rounded separately, then bf16 RNE.
 * Requires q_offset + L <= max_ctx; q_offset need not be a multiple of 4.
 * ws may be NULL (needs none). */
qsa_status qsa_append(const qsa_handle *h, void *stream, int32_t B, int64_t L, int64_t q_offset,
                      const uint16_t *k, const uint16_t *v, const uint16_t *k_idx,
                      uint16_t *k_cache, uint16_t *v_cache, uint16_t *kbar_cache, uint16_t *kpend);

/* Indexer ([PKR] "QSA: ...", equation I_ib = sum_h ReLU(<q_i^h, k̄_b>)):
 * rotates q_idx at positions q_offset .. q_offset+L-1 and writes the score
 * matrix `scores` (layout above) of those queries against every complete block
 * before each query's own block (block-causal: only fully observed blocks are
 * scored; non-candidates get -1).  kbar_cache must already hold those blocks
 * (qsa_append).  Scores accumulate in fp32 from bf16 operands (matrix cores).
 * q_offset % 4 == 0.  ws: qsa_workspace_size(QSA_OP_INDEX) bytes. */
qsa_status qsa_index(const qsa_handle *h, void *stream, int32_t B, int64_t L, int64_t q_offset,
                     const uint16_t *q_idx, const uint16_t *kbar_cache, float *scores,
                     void *ws, size_t ws_bytes);

/* Selection ([PKR] "QSA: ...": K = 2048 tokens, r = 4, up to 512 blocks per
 * query): for each query p, the min(budget, floor(p/4)) candidates with the
 * largest scores, ties broken toward the larger block index, written ascending
 * and padded with -1 into block_idx [B][L][budget].  Reads `scores` as written
 * by qsa_index for the same (B, L, q_offset).  q_offset % 4 == 0.  Needs no
 * workspace. */
qsa_status qsa_select(const qsa_handle *h, void *stream, int32_t B, int64_t L, int64_t q_offset,
                      const float *scores, int32_t *block_idx);

/* qsa_index followed by qsa_select without materialising the score matrix:
 * one fused kernel computes the same scores tile by tile and keeps, per query,
 * only the (score, block) pairs at or above a running threshold that provably
 * lies at or below the query's budget-th largest score; the exact selection is
 * then taken from that short list.  A list longer than topk_cap is recomputed
 * exactly for its row.  Same results as qsa_index + qsa_select.  The
 * workspace holds the rotated queries and the lists of at most 16 GiB of
 * query rows at a time (8 topk_cap bytes per row and sequence).  ws: qsa_workspace_size(QSA_OP_INDEX_SELECT) bytes. */
qsa_status qsa_index_select(const qsa_handle *h, void *stream, int32_t B, int64_t L, int64_t q_offset,
                            const uint16_t *q_idx, const uint16_t *kbar_cache, int32_t *block_idx,
                            void *ws, size_t ws_bytes);

/* Sparse core attention ([PKR] "QSA: ...", sparse core attention over the
 * selected blocks; the tail of the last incomplete block is always included):
 * for each query p = q_offset + i and head h (KV head h / 12) computes
 * softmax(sigma * q~_h . K~^T) V over the tokens of the blocks in block_idx[p]
 * plus tokens 4*floor(p/4) .. p, read from the caches, with q~ = q rotated at p
 * and sigma = 1/16 (times the YaRN temperature).  The caches must already hold
 * positions 0..p (qsa_append).  Entries of block_idx outside [0, floor(p/4))
 * are skipped.  Logits and softmax in fp32, P rounded to bf16 for the PV
 * product, output bf16.  q_offset % 4 == 0.  Needs no workspace. */
qsa_status qsa_attend(const qsa_handle *h, void *stream, int32_t B, int64_t L, int64_t q_offset,
                      const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                      const int32_t *block_idx, uint16_t *out);

/* Dense causal GQA attention over the same caches: the dense baseline of the
 * pages' module speed-ups ([PKR] "QSA: ...", kernel-latency figure: indexer +
 * sparse core attention against a dense paged GQA kernel).  For each query
 * p = q_offset + i and head h (KV head h / 12): softmax(sigma * q~_h . K~^T) V
 * over every token 0..p, with the rotation, scale and precision of
 * qsa_attend (bf16 operands, fp32 logits and softmax, P rounded to bf16 for the
 * PV product, bf16 output); this equals qsa_attend with every block before the
 * query's own selected.  The caches must hold positions 0..p.
 * q_offset % 4 == 0.  Needs no workspace. */
qsa_status qsa_dense_attend(const qsa_handle *h, void *stream, int32_t B, int64_t L, int64_t q_offset,
                            const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache, uint16_t *out);

/* Prefill (or one prefill chunk): qsa_append, qsa_index_select and qsa_attend
 * for positions q_offset .. q_offset+L-1.  block_idx may be NULL; when given
 * it receives the selection ([B][L][budget]).  Earlier chunks must already be
 * in the caches.  q_offset % 4 == 0.
 * ws: qsa_workspace_size(QSA_OP_FORWARD) bytes. */
qsa_status qsa_forward(const qsa_handle *h, void *stream, int32_t B, int64_t L, int64_t q_offset,
                       const uint16_t *q, const uint16_t *k, const uint16_t *v,
                       const uint16_t *q_idx, const uint16_t *k_idx,
                       uint16_t *k_cache, uint16_t *v_cache, uint16_t *kbar_cache, uint16_t *kpend,
                       uint16_t *out, int32_t *block_idx, void *ws, size_t ws_bytes);

/* Decode one new token per sequence.  cache_len is a DEVICE int32 [B]: sequence
 * b holds positions 0..cache_len[b]-1 in its caches and the new token sits at
 * p = cache_len[b].  The call appends the new token (k, v, k_idx of shape
 * [B][1][...]), scores its query against every complete block before its own,
 * selects the top budget blocks and attends (same rules as qsa_forward).
 * ctx_bound is a host-side bound: cache_len[b] <= ctx_bound < max_ctx for all b
 * (grids are sized by it).  cache_len is not modified; the caller advances it.
 * ws: qsa_workspace_size(QSA_OP_DECODE, B, 1, ctx_bound) bytes. */
qsa_status qsa_decode(const qsa_handle *h, void *stream, int32_t B, const int32_t *cache_len,
                      int64_t ctx_bound,
                      const uint16_t *q, const uint16_t *k, const uint16_t *v,
                      const uint16_t *q_idx, const uint16_t *k_idx,
                      uint16_t *k_cache, uint16_t *v_cache, uint16_t *kbar_cache, uint16_t *kpend,
                      uint16_t *out, int32_t *block_idx, void *ws, size_t ws_bytes);

/* qsa_decode for callers that cannot allocate device memory -- code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc: the same
 * kernels and results as qsa_decode, with no workspace argument.  The step's
 * scratch (score rows, histogram summaries, selection lists, split partials)
 * lives in a fixed device array of QSA_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends; its address is
 * resolved once per device by qsa_create.  The caller still passes every input,
 * cache and output.  Returns QSA_ERR_WORKSPACE, before anything is enqueued,
 * when qsa_workspace_size(QSA_OP_DECODE, B, 1, ctx_bound) exceeds
 * QSA_NOALLOC_SCRATCH_BYTES (it covers, for instance, B = 64 at ctx_bound =
 * 131,072 and B = 8 at 1,048,576).  Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (other streams, other threads, other
 * handles) race and must be serialised by the caller.  The array keeps the last
 * call's contents; a call reads no word of it that the same call has not
 * written first, so nothing needs clearing between calls.  Calls no hipMalloc,
 * hipFree or other allocating routine. */
#define QSA_NOALLOC_SCRATCH_BYTES (32u << 20)
qsa_status qsa_decode_noalloc(const qsa_handle *h, void *stream, int32_t B, const int32_t *cache_len,
                              int64_t ctx_bound,
                              const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const uint16_t *q_idx, const uint16_t *k_idx,
                              uint16_t *k_cache, uint16_t *v_cache, uint16_t *kbar_cache, uint16_t *kpend,
                              uint16_t *out, int32_t *block_idx);

/* Decode one new token per sequence reusing a block selection made at an
 * earlier position instead of scoring and selecting again ([PKR] section on the
 * MTP module for speculative decoding: the top-k block indices are reused
 * between speculative steps).  Sequence b's new token sits at p = cache_len[b]
 * (appended as in qsa_decode, including its indexer key); block_idx [B][budget]
 * is the selection qsa_decode returned for position p0 = sel_pos[b] (DEVICE
 * int32 [B], clamped to [0, p]).  The token attends over the selected blocks
 * below p0's own block plus every token from the start of p0's own block up to
 * p; with p0 = p this is exactly qsa_decode's attention.  No indexer query is
 * read.  ctx_bound as for qsa_decode.
 * ws: qsa_workspace_size(QSA_OP_DECODE, B, 1, ctx_bound) bytes. */
qsa_status qsa_decode_reuse(const qsa_handle *h, void *stream, int32_t B, const int32_t *cache_len,
                            const int32_t *sel_pos, int64_t ctx_bound,
                            const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *k_idx,
                            uint16_t *k_cache, uint16_t *v_cache, uint16_t *kbar_cache, uint16_t *kpend,
                            const int32_t *block_idx, uint16_t *out, void *ws, size_t ws_bytes);

/* The selection half of qsa_decode alone: append the new token's indexer key
 * (pending slot; pooling when its block completes), rotate its indexer query at
 * p = cache_len[b], score the complete blocks before its own block and write the
 * top budget blocks to block_idx [B][budget] (ascending, -1 padded), exactly as
 * qsa_decode selects them.  No K/V cache is touched and nothing is attended
 * (for instance to select once for several speculative steps that then call
 * qsa_decode_reuse).  Sizes, ctx_bound and errors as for qsa_decode.
 * ws: qsa_workspace_size(QSA_OP_INDEX_DECODE, B, 1, ctx_bound) bytes. */
qsa_status qsa_index_decode(const qsa_handle *h, void *stream, int32_t B, const int32_t *cache_len,
                            int64_t ctx_bound, const uint16_t *q_idx, const uint16_t *k_idx,
                            uint16_t *kbar_cache, uint16_t *kpend, int32_t *block_idx, void *ws, size_t ws_bytes);

/* Token-level indexer, compression ratio r = 1: the indexer QSA's pooled one is
 * measured against ([PKR] section "QSA: 인덱서 자체의 비용을 줄이는 희소 어텐션":
 * a per-token indexer as in DeepSeek-V3.2's DSA costs O(n^2); pooling r tokens per
 * key brings it to O(n^2/r); the figure after the table of results there gives
 * the indexer's speed-up at r = 4).  Every key is its own block: the indexer
 * key of position t, rotated at t on its first 64 dims (no pooling), is stored
 * in ktok_cache [B][max_ctx][128] bf16; query p scores every t < p with
 * I[p][t] = sum_h ReLU(<q~_h(p), k~_t>) and keeps the top min(budget, p)
 * tokens under (score desc, t desc), written ascending and -1 padded to
 * token_idx [B][L][budget] (budget = the handle's budget_blocks, counted in
 * tokens here).  Same kernels as qsa_index_select.
 * qsa_token_index_select: the L tokens at q_offset .. q_offset+L-1 (any offset;
 * keys of earlier positions must already be in ktok_cache), q_idx [B][L][4][128],
 * k_idx [B][L][128].  ws: qsa_workspace_size(QSA_OP_TOKEN_INDEX_SELECT, B, L,
 * q_offset) bytes.
 * qsa_token_index_decode: one new token per sequence at p = cache_len[b] (DEVICE
 * int32 [B]); q_idx [B][1][4][128], k_idx [B][1][128]; token_idx [B][budget].
 * ctx_bound as for qsa_decode.  ws: qsa_workspace_size(QSA_OP_TOKEN_INDEX_DECODE,
 * B, 1, ctx_bound) bytes.
 * Errors as for qsa_index_select / qsa_decode (no alignment rule on q_offset). */
qsa_status qsa_token_index_select(const qsa_handle *h, void *stream, int32_t B, int64_t L, int64_t q_offset,
                                  const uint16_t *q_idx, const uint16_t *k_idx, uint16_t *ktok_cache,
                                  int32_t *token_idx, void *ws, size_t ws_bytes);
qsa_status qsa_token_index_decode(const qsa_handle *h, void *stream, int32_t B, const int32_t *cache_len,
                                  int64_t ctx_bound, const uint16_t *q_idx, const uint16_t *k_idx,
                                  uint16_t *ktok_cache, int32_t *token_idx, void *ws, size_t ws_bytes);

/* Training path ([PKR] "QSA: ..." section: the indexer learns the attention
 * distribution matched per micro-block with max pooling, and a fused kernel
 * computes the sparse attention output and the indexer's KL-divergence loss
 * without materialising intermediates).  Whole sequences: positions 0..L-1 of
 * each of B sequences, whose caches qsa_append has filled (k_cache, v_cache,
 * kbar_cache as in qsa_forward), with a selection block_idx [B][L][budget] (for
 * instance from qsa_index_select; the top-k itself is not differentiated).
 *
 * qsa_train_forward: out [B][L][24][256] bf16 = qsa_attend's output; stats
 * [B][L][32] fp32 per query: [0..23] each query head's natural-log log-sum-exp
 * of its scaled logits over the token set T(p), [24] ln Z, [25] the log-sum-exp
 * of the indexer scores over S(p), [26..31] 0; kl [B][L] fp32 = KL(pi || s),
 * where for the valid selected blocks b of S(p) (the own block takes no part)
 * A_b = max over the block's 4 tokens of the 24 heads' mean attention
 * probability, Z = sum A, pi_b = A_b / Z, s_b = softmax over S(p) of the
 * indexer scores I_b; kl = 0 when S(p) has fewer than 2 blocks.  With a budget
 * covering every block the teacher is the dense one (the distillation stage).
 * ws: qsa_workspace_size(QSA_OP_TRAIN_FORWARD, B, L, 0) bytes.
 *
 * qsa_train_backward_indexer: gradients of sum_p dkl[p] * kl[p] (dkl [B][L]
 * fp32) with respect to the raw indexer queries, dq_idx [B][L][4][128] fp32,
 * and raw indexer keys, dk_idx [B][L][128] fp32 (0 for the tokens of a
 * trailing partial block), holding the teacher constant: dkl/dI_b = s_b - pi_b,
 * ReLU' = [logit > 0], transposed rotations, 1/4 per pooled key.  stats: the
 * forward's.  The gradient of the attention output with respect to q, k, v
 * comes from qsa_train_backward_attention.
 * ws: qsa_workspace_size(QSA_OP_TRAIN_BACKWARD, B, L, 0) bytes.  Both: q_idx [B][L][4][128], q [B][L][24][256] raw bf16; errors as for
 * qsa_forward with q_offset = 0. */
qsa_status qsa_train_forward(const qsa_handle *h, void *stream, int32_t B, int64_t L, const uint16_t *q,
                             const uint16_t *q_idx, const uint16_t *k_cache, const uint16_t *v_cache,
                             const uint16_t *kbar_cache, const int32_t *block_idx, uint16_t *out, float *stats,
                             float *kl, void *ws, size_t ws_bytes);
qsa_status qsa_train_backward_indexer(const qsa_handle *h, void *stream, int32_t B, int64_t L, const uint16_t *q,
                                      const uint16_t *q_idx, const uint16_t *k_cache, const uint16_t *kbar_cache,
                                      const int32_t *block_idx, const float *stats, const float *dkl,
                                      float *dq_idx, float *dk_idx, void *ws, size_t ws_bytes);

/* Backward of the sparse attention (the backbone's gradient in the training
 * path): with P = softmax over T(p) of the scaled logits (from the per-head
 * log-sum-exp in stats, as qsa_train_forward wrote it) and D_h = <dout_h, out_h>,
 * dS = P (dout V^T - D); dq [B][L][24][256] fp32 = gradient with respect to the
 * raw q (sigma dS K~ rotated back at p); dk, dv [B][L][2][256] fp32 = gradients
 * with respect to the raw k (rotated back at each token's position) and v,
 * summed over every query that attends the token.  out [B][L][24][256] bf16 is
 * qsa_train_forward's output, dout the same shape (the upstream gradient);
 * block_idx and the caches as for qsa_train_forward.  dk and dv are cleared and
 * accumulated with atomics (the summation order, and so the last bits, can vary
 * between runs).  No workspace.  Errors as for qsa_train_forward. */
qsa_status qsa_train_backward_attention(const qsa_handle *h, void *stream, int32_t B, int64_t L, const uint16_t *q,
                                        const uint16_t *k_cache, const uint16_t *v_cache, const int32_t *block_idx,
                                        const uint16_t *out, const uint16_t *dout, const float *stats, float *dq,
                                        float *dk, float *dv);

/* Gated DeltaNet chunked prefill: the hybrid's other token mixer ([PKR]
 * section "어텐션: GDN이 기억하고 QSA가 찾아낸다": per V head the state S
 * [128][128] follows S_t = (alpha_t I - beta_t k_t k_t^T) S_{t-1} + beta_t
 * k_t v_t^T; spec table: 48 V heads, 16 QK heads, head dim 128; section
 * "FlashQLA": the chunked-prefill interface).  Independent of any qsa_handle;
 * runs on the calling thread's current HIP device.
 *
 * nseq sequences packed back to back: cu_seqlens (device, int32 [nseq + 1],
 * non-decreasing, cu_seqlens[0] = 0) gives sequence s the tokens
 * cu_seqlens[s] .. cu_seqlens[s+1]-1 of the n_tokens packed ones, and no
 * sequence may be longer than max_len (offsets outside [0, n_tokens] are
 * clamped and longer sequences are cut at max_len, so a bad table cannot make
 * the kernels touch memory outside the buffers).  q, k [n_tokens][hq_heads][128]
 * bf16 (already normalised, as the layer's short convolution and L2 norm leave
 * them), v [n_tokens][hv_heads][128] bf16, g [n_tokens][hv_heads] fp32 = ln
 * alpha_t (<= 0), beta [n_tokens][hv_heads] fp32 in [0, 1]; V head h reads QK
 * head h / (hv_heads / hq_heads).  initial_state [nseq][hv_heads][128][128]
 * fp32 (S[k_dim][v_dim], NULL = zeros).  Outputs: o [n_tokens][hv_heads][128]
 * bf16 with o_t = scale * S_t^T q_t (the state after token t); final_state
 * (same layout as initial_state, may be NULL, may alias initial_state) the
 * state after each sequence's last token.  ws: qsa_gdn_workspace_size(nseq,
 * max_len, hq_heads, hv_heads) bytes.  Errors: QSA_ERR_NULL (q, k, v, g, beta, o,
 * cu_seqlens or a needed ws missing), QSA_ERR_SHAPE (nseq outside 1..65535,
 * n_tokens or max_len negative or max_len above 2^30, hq_heads outside 1..65535,
 * hv_heads not a positive multiple of hq_heads, or nseq * ceil(max_len / 64) *
 * hv_heads above 2^32 - 1), QSA_ERR_ALIGN (q, k or ws not
 * 16-byte aligned), QSA_ERR_WORKSPACE, QSA_ERR_HIP. */
size_t qsa_gdn_workspace_size(int32_t nseq, int64_t max_len, int32_t hq_heads, int32_t hv_heads);
qsa_status qsa_gdn_chunk_prefill(void *stream, int32_t nseq, const int32_t *cu_seqlens, int64_t n_tokens,
                                 int64_t max_len, int32_t hq_heads, int32_t hv_heads, float scale, const uint16_t *q,
                                 const uint16_t *k, const uint16_t *v, const float *g, const float *beta,
                                 const float *initial_state, uint16_t *o, float *final_state, void *ws,
                                 size_t ws_bytes);

/* The two stages of qsa_gdn_chunk_prefill, for callers that time or schedule
 * them apart (same arguments and errors; run qsa_gdn_prep, then qsa_gdn_scan
 * on the same ws and stream).  qsa_gdn_prep writes, for every chunk of 64
 * tokens and V head, the two 64 x 64 bf16 matrices that do not depend on the
 * state (the inverse of the chunk's unit lower-triangular delta-rule system
 * times diag(beta), and the decayed, scaled causal q.k products) into ws;
 * qsa_gdn_scan walks the chunks in order, carrying the state, and writes o and
 * final_state. */
qsa_status qsa_gdn_prep(void *stream, int32_t nseq, const int32_t *cu_seqlens, int64_t n_tokens, int64_t max_len,
                        int32_t hq_heads, int32_t hv_heads, float scale, const uint16_t *q, const uint16_t *k,
                        const float *g, const float *beta, void *ws, size_t ws_bytes);
qsa_status qsa_gdn_scan(void *stream, int32_t nseq, const int32_t *cu_seqlens, int64_t n_tokens, int64_t max_len,
                        int32_t hq_heads, int32_t hv_heads, float scale, const uint16_t *q, const uint16_t *k,
                        const uint16_t *v, const float *g, const float *initial_state, uint16_t *o,
                        float *final_state, const void *ws, size_t ws_bytes);

/* Static string for a status code. */
const char *qsa_status_string(qsa_status s);

/* HIP error code of the last QSA_ERR_HIP returned on this thread (0 if none). */
int qsa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
