/*
 * qsa.h -- C ABI of libqsa: indexer-selected sparse attention over pooled
 * block keys, hand-written HIP for gfx950 (one GPU).
 *
 * The method (described in prose on the pages cited below; no formulas are
 * printed there):
 *   - every history block of `block` tokens has one pooled indexer key;
 *   - each query scores every complete block with its indexer query, keeps
 *     the `topk` best blocks plus the trailing tokens of the incomplete last
 *     block (all tokens when there are at most `topk` complete blocks);
 *   - it gathers only those K/V rows and runs softmax attention over them;
 *   - prefill walks history tiles in the outer loop and merges the partial
 *     softmax results by log-sum-exp.
 * Sources: "3090x3で 314 万コンテキスト" (sections "なぜ", "カーネルを書き換え
 * ずに済む", "VRAM に残す必要があるもの", "ちなみにこの欠点"); "GLM-5.3 最適化
 * 第2部：16基のH200上でのPCP、DCP、およびHybrid HiSparse" (sections "PCP",
 * "DCP", footnote 1); "125B MoE を 3090 3 枚で運用する vLLM 最適化編"
 * (section 3.3, ties in top-k go to the smaller id; section 5, the K/V row
 * cache in device memory).
 *
 * Conventions for every entry point:
 *   - Pointers marked (device) are device memory owned by the caller; the
 *     library never allocates, frees or keeps them. Pointers marked (host)
 *     are read before the call returns.
 *   - Each call validates its arguments on the host, then enqueues its
 *     kernels on `stream` (a hipStream_t; NULL = the null stream) and returns
 *     without synchronising. Nothing is launched when validation fails.
 *   - bf16 arrays are raw bit patterns (uint16) and must be 16-byte aligned;
 *     fp32 / int32 arrays must be 16-byte aligned as well.
 *   - Per-query context lengths `q_ctx` live in device memory (so a captured
 *     graph can be replayed as positions advance); `max_ctx` is a host-side
 *     upper bound used to size launches and validate buffers. A q_ctx entry
 *     outside [0, max_ctx] is a caller error: kernels clamp it into range
 *     (so no access leaves the buffers) and the results for that query are
 *     unspecified. Setting QSA_VALIDATE=1 in the environment makes each call
 *     copy q_ctx / q_seq back and return QSA_ERR_ARG instead (synchronising).
 *   - Setting QSA_SYNC_CHECK=1 makes each call synchronise its stream and
 *     return QSA_ERR_LAUNCH if a kernel failed.
 *   - Results are bit-identical from run to run (no floating-point atomics).
 *   - Calls keep no global mutable state and may be issued from several
 *     threads on different streams.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t qsa_bf16;      /* bf16 bit pattern */
typedef void*    qsa_stream_t;  /* hipStream_t */

typedef enum {
  QSA_OK = 0,
  QSA_ERR_ARG = 1,          /* null or misaligned pointer, negative size, short stride */
  QSA_ERR_UNSUPPORTED = 2,  /* well-formed but outside the compiled shapes */
  QSA_ERR_WORKSPACE = 3,    /* workspace smaller than the matching *_workspace_bytes() */
  QSA_ERR_LAUNCH = 4,       /* a kernel launch (or, with QSA_SYNC_CHECK=1, a kernel) failed */
  QSA_ERR_DEVICE = 5        /* no usable gfx950 device */
} qsa_status;

/* Storage of indexer keys.
 *   QSA_KEYS_BF16: key b of a sequence is idx_dim bf16 values at
 *     keys + seq * keys_seq_stride + b * idx_dim (strides in elements).
 *   QSA_KEYS_FP8: each key is idx_dim OCP E4M3 codes plus one fp32 scale
 *     and stands for code * scale ("GLM-5.3 ...", footnote 3: 128 FP8
 *     values and a 4-byte scale, 132 bytes per key). Keys are stored in
 *     pages of 64: page p holds the codes of keys 64p .. 64p+63 (idx_dim
 *     bytes each, key-major) followed by their 64 scales, so key b's codes
 *     start at byte (b/64) * 64*(idx_dim+4) + (b%64) * idx_dim and its scale
 *     at (b/64) * 64*(idx_dim+4) + 64*idx_dim + 4*(b%64) of its sequence;
 *     sequence strides are in bytes (multiples of 16).
 *     qsa_fp8_keys_bytes gives the bytes n keys need; qsa_quantize_keys and
 *     qsa_kv_append write this layout. Supported for both indexers (132
 *     bytes per pooled 128-d key, 68 bytes per 64-d token key). */
typedef enum { QSA_KEYS_BF16 = 0, QSA_KEYS_FP8 = 1 } qsa_key_format;

/* Indexer / selection parameters.
 *   variant A (pooled block keys):   block 4, topk 512,  idx_dim 128, idx_heads 1
 *   variant B (token keys, MLA-like): block 1, topk 2048, idx_dim 64,  idx_heads 4
 * Supported: block in {1, 4}; 1 <= topk <= 2048; (idx_dim, idx_heads) in
 * {(128, 1), (64, 4)}; key_format a qsa_key_format. */
typedef struct {
  int32_t block;
  int32_t topk;
  int32_t idx_dim;
  int32_t idx_heads;
  int32_t key_format;
} qsa_sel_cfg;

/* Attention shape. Query head h reads kv head h / (hq / hkv).
 * Supported: (hq, hkv, dk, dv) = (16, 2, 256, 256) [variant A] and
 * (64, 1, 576, 512) [variant B, V = first dv columns of the K row]. */
typedef struct {
  int32_t hq;
  int32_t hkv;
  int32_t dk;
  int32_t dv;
  float scale;   /* softmax scale applied to q.k (1/16 for dk = 256) */
} qsa_attn_cfg;

/* K/V cache of one layer for several sequences (device).
 * Element d of the K row of (sequence s, token t, kv head g) is
 *   k[s * seq_stride + t * tok_stride + g * head_stride + d]
 * and likewise for v (v may equal k: the MLA latent row serves as both).
 * Strides are in elements and must be multiples of 8; `capacity` is the
 * number of token rows each sequence holds (every query needs
 * q_ctx <= capacity). The pages' gather kernel uses
 * [token][kv_head][head_dim] ("カーネルを書き換えずに済む"): tok_stride =
 * hkv * dk, head_stride = dk. */
typedef enum { QSA_KV_BF16 = 0, QSA_KV_FP8_MLA = 1 } qsa_kv_format;

/* format QSA_KV_FP8_MLA (the shared-latent shape only, v == k): each token
 * holds one 656-byte FP8 sparse-MLA row ("GLM-5.3 ...", footnote 1): bytes
 * [0, 512) the first 512 latent values as OCP E4M3 codes, [512, 528) four
 * fp32 scales (one per 128 codes; value = code * scale), [528, 656) the 64
 * rotary values as bf16. k points at the rows; the row of (sequence s,
 * token t) starts at byte s * seq_stride + t * tok_stride (strides in
 * bytes, multiples of 16, tok_stride >= 656; head_stride unused).
 * qsa_quantize_latent and qsa_kv_append write these rows. */
typedef struct {
  const qsa_bf16* k;
  const qsa_bf16* v;
  int64_t seq_stride;
  int64_t tok_stride;
  int64_t head_stride;
  int64_t capacity;
  int32_t format;   /* qsa_kv_format */
} qsa_kv;

/* ---------------------------------------------------------------- A1 ----
 * qsa_pool_keys: pooled indexer keys for the complete blocks of tokens
 * [tok_begin, tok_end) of n_seq sequences.
 *   pooled[s][b][d] = bf16_rne( mean_{j < block} raw[s][block*b + j][d] )
 * i.e. the exact mean rounded once to bf16 (nearest, ties to even); exact
 * whenever the block's nonzero values lie within a factor 2^44 of each
 * other. ("3090x3で 314 万コンテキスト", "VRAM に残す必要があるもの": one
 * pooled key of 128 bf16 per block; the mean is the workload's definition.)
 *   raw    (device) bf16 [n_seq][raw_seq_stride]: token t of sequence s at
 *          raw + s*raw_seq_stride + t*dim.
 *   pooled (device) bf16 [n_seq][pooled_seq_stride]: block b at
 *          pooled + s*pooled_seq_stride + b*dim.
 *   tok_begin must be a multiple of block; blocks b in
 *   [tok_begin/block, tok_end/block) are written, nothing else.
 *   dim must be a multiple of 8, at most 1024. */
qsa_status qsa_pool_keys(const qsa_bf16* raw, int64_t raw_seq_stride,
                         qsa_bf16* pooled, int64_t pooled_seq_stride,
                         int32_t n_seq, int64_t tok_begin, int64_t tok_end,
                         int32_t dim, int32_t block, qsa_stream_t stream);

/* -------------------------------------------------------- A1, FP8 ----
 * qsa_quantize_keys: FP8 indexer keys (QSA_KEYS_FP8 layout) from bf16 keys
 * [key_begin, key_end) of n_seq sequences, for instance pooled keys written
 * by qsa_pool_keys. Per key: scale = amax / 448 (amax the largest |value|;
 * fp32 division, correctly rounded) and code[d] = the E4M3 value nearest to
 * the fp32 quotient key[d] / scale (ties to even, magnitudes past 448 set
 * to 448); an all-zero key gets scale 0 and zero codes. ("GLM-5.3 ...",
 * footnote 3: FP8 values with one 4-byte scale per key.)
 *   keys (device) bf16: key b of sequence s at keys + s*keys_seq_stride + b*dim.
 *   out  (device) FP8 pages of sequence s at out + s*out_seq_stride (bytes,
 *        a multiple of 16); only the codes and scales of the keys in range
 *        are written.
 *   dim in {64, 128}. */
qsa_status qsa_quantize_keys(const qsa_bf16* keys, int64_t keys_seq_stride, void* out,
                             int64_t out_seq_stride, int32_t n_seq, int64_t key_begin,
                             int64_t key_end, int32_t dim, qsa_stream_t stream);

/* Bytes that hold FP8 keys 0 .. n_keys-1 of one sequence (whole pages). */
int64_t qsa_fp8_keys_bytes(int64_t n_keys, int32_t dim);

/* qsa_quantize_latent: FP8 sparse-MLA rows (QSA_KV_FP8_MLA) of tokens
 * [tok_begin, tok_end) of n_seq sequences from 576-wide bf16 latent rows:
 * values 128g .. 128g+127 (g < 4) quantized as qsa_quantize_keys does with
 * one scale per group, the 64 rotary values copied. ("GLM-5.3 ...",
 * footnote 1: the 656-byte FP8 row.)
 *   latent (device) bf16: row (s, t) at latent + s*seq_stride + t*tok_stride
 *          (elements, multiples of 8, tok_stride >= 576).
 *   out    (device): row (s, t) at byte s*out_seq_stride + t*out_tok_stride
 *          (multiples of 16, out_tok_stride >= 656). */
qsa_status qsa_quantize_latent(const qsa_bf16* latent, int64_t seq_stride, int64_t tok_stride, void* out,
                               int64_t out_seq_stride, int64_t out_tok_stride, int32_t n_seq,
                               int64_t tok_begin, int64_t tok_end, qsa_stream_t stream);

/* ------------------------------------------------- A1 at decode time ----
 * qsa_kv_append: the decode step's write of one new token per query into
 * the cache, before the layer reads it. Query i writes, at position
 * q_pos[i] of sequence q_seq[i] (sequence i if q_seq is NULL):
 *   - its K row for every kv head (k_new[i], hkv x dk) and, unless the
 *     cache's v is its k (a shared latent row), its V row (v_new[i],
 *     hkv x dv), addressed as in qsa_kv; a QSA_KV_FP8_MLA cache gets the
 *     row quantized as qsa_quantize_latent does;
 *   - its raw indexer key (raw_new[i], idx_dim values) at raw_keys +
 *     seq * raw_seq_stride + pos * idx_dim, when raw_new is given; with
 *     block 1 (the raw key is the indexer key) and QSA_KEYS_FP8, quantized
 *     as qsa_quantize_keys does into raw_keys as FP8 pages (stride in bytes);
 *   - when pos + 1 is a multiple of block and pooled is given, the pooled
 *     key of the block it completes, bit-identical to qsa_pool_keys over the
 *     same raw keys (the block's earlier tokens are read from raw_keys);
 *     with sel_cfg->key_format QSA_KEYS_FP8, that key quantized as
 *     qsa_quantize_keys does, into FP8 pages (pooled_seq_stride in bytes).
 * ("3090x3で 314 万コンテキスト", "VRAM に残す必要があるもの": pooled keys stay
 * device-resident and the raw keys are kept so that blocks can be pooled;
 * "カーネルを書き換えずに済む": per (token, kv head) addressing.)
 *   q_seq (device) int32 [nq] or NULL; q_pos (device) int32 [nq], positions
 *          in [0, kv->capacity): a query with another position writes
 *          nothing. At most one query per sequence per call (a block's
 *          pooling reads the sequence's earlier tokens).
 *   k_new, v_new, raw_new (device) bf16 rows as above; v_new must be NULL
 *          exactly when kv->v == kv->k. raw_new, raw_keys: both or neither;
 *          pooled needs them, and block 4 (NULL for block 1, where the raw
 *          key is the indexer key).
 * Graph-capturable: positions are read on the device at replay. */
qsa_status qsa_kv_append(const qsa_sel_cfg* sel_cfg, const qsa_attn_cfg* attn_cfg, int32_t nq,
                         const int32_t* q_seq, const int32_t* q_pos, const qsa_bf16* k_new,
                         const qsa_bf16* v_new, const qsa_bf16* raw_new, const qsa_kv* kv,
                         qsa_bf16* raw_keys, int64_t raw_seq_stride, void* pooled,
                         int64_t pooled_seq_stride, qsa_stream_t stream);

/* ---------------------------------------------------------------- A2 ----
 * qsa_index_scores: indexer scores of every candidate block for nq queries.
 * Query i reads the keys of sequence q_seq[i] and has n_i = q_ctx[i] / block
 * candidates; for b < n_i:
 *   variant A (idx_heads 1): scores[i][b] = q_idx[i] . keys[b]
 *   variant B (idx_heads H): scores[i][b] = sum_h w_idx[i][h] * max(0, q_idx[i][h] . keys[b])
 * accumulated in fp32. Entries b >= n_i are not written.
 * ("VRAM に残す必要があるもの": every pooled key is scored at every step;
 * "GLM-5.3 ...", "PCP": a token-level indexer scores all earlier tokens.)
 *   q_seq  (device) int32 [nq], or NULL: every query reads sequence 0
 *          (a prefill chunk; enables the MFMA query-tile path).
 *   q_ctx  (device) int32 [nq] visible tokens per query (its own included).
 *   q_idx  (device) bf16 [nq][idx_heads][idx_dim].
 *   w_idx  (device) fp32 [nq][idx_heads]; NULL when idx_heads == 1.
 *   keys   (device) in cfg->key_format: bf16 key b of sequence s at
 *          keys + s*keys_seq_stride + b*idx_dim, or FP8 pages (then the
 *          score uses code * scale for each key value); pooled block keys
 *          for block 4, per-token keys for block 1.
 *   scores (device) fp32 [nq][ld_scores], ld_scores >= max_ctx / block. */
qsa_status qsa_index_scores(const qsa_sel_cfg* cfg, int32_t nq,
                            const int32_t* q_seq, const int32_t* q_ctx, int32_t max_ctx,
                            const qsa_bf16* q_idx, const float* w_idx,
                            const void* keys, int64_t keys_seq_stride,
                            float* scores, int64_t ld_scores, qsa_stream_t stream);

/* ---------------------------------------------------------------- A3 ----
 * qsa_topk_blocks: the blocks each query attends.
 * With n_i = q_ctx[i] / block candidates: if n_i <= topk every block is
 * selected; otherwise the topk blocks ranked first by (score descending,
 * block index ascending), -0.0 ranking equal to +0.0. Scores must be finite.
 * ("3090x3で 314 万コンテキスト", "なぜ": fixed budget, full history below
 * 4*topk + 3 tokens; "125B MoE ...", 3.3: equal values go to the smaller id.)
 *   sel   (device) int32 [nq][topk]: row i holds n_sel[i] ascending block
 *         indices, then -1 up to topk.
 *   n_sel (device) int32 [nq] = min(n_i, topk).
 *   ws    (device) workspace of at least qsa_topk_workspace_bytes(cfg, nq,
 *         max_ctx) bytes, contents ignored on entry (may be NULL if that is 0). */
qsa_status qsa_topk_blocks(const qsa_sel_cfg* cfg, int32_t nq,
                           const int32_t* q_ctx, int32_t max_ctx,
                           const float* scores, int64_t ld_scores,
                           int32_t* sel, int32_t* n_sel,
                           void* ws, size_t ws_bytes, qsa_stream_t stream);

size_t qsa_topk_workspace_bytes(const qsa_sel_cfg* cfg, int32_t nq, int32_t max_ctx);

/* ----------------------------------------------------------- A2 + A3 ----
 * qsa_index_topk: qsa_index_scores followed by qsa_topk_blocks, in one
 * launch (decode: each query scores the pooled keys of its own sequence).
 * Writes exactly what the two calls write: scores[i][b] for b < n_i and the
 * selection sel / n_sel, bit-identical to them. Each work-group scores one
 * chunk of blocks and keeps the chunk's best candidates; the last
 * work-group of a query to finish selects the exact top-k from them.
 * ("3090x3で 314 万コンテキスト", "VRAM に残す必要があるもの" and "なぜ".)
 * Variant A only (block 4, idx_dim 128, idx_heads 1; bf16 or FP8 keys);
 * other configurations return QSA_ERR_UNSUPPORTED.
 *   q_seq, q_ctx, q_idx, keys, scores, ld_scores: as qsa_index_scores.
 *   sel, n_sel: as qsa_topk_blocks.
 *   ws (device) workspace of at least qsa_index_topk_workspace_bytes(cfg,
 *      nq, max_ctx) bytes. Its first bytes are per-query arrival counters:
 *      the whole workspace must be zero before the first call, and every
 *      completed call leaves the counters zero again (so one zero-fill at
 *      allocation suffices). Calls that share a workspace must not run
 *      concurrently. */
qsa_status qsa_index_topk(const qsa_sel_cfg* cfg, int32_t nq, const int32_t* q_seq,
                          const int32_t* q_ctx, int32_t max_ctx, const qsa_bf16* q_idx,
                          const void* keys, int64_t keys_seq_stride,
                          float* scores, int64_t ld_scores, int32_t* sel, int32_t* n_sel,
                          void* ws, size_t ws_bytes, qsa_stream_t stream);

size_t qsa_index_topk_workspace_bytes(const qsa_sel_cfg* cfg, int32_t nq, int32_t max_ctx);

/* --------------------------------------- A2 + A3 for a prefill chunk ----
 * qsa_index_topk_prefill: the selections of qsa_index_scores followed by
 * qsa_topk_blocks for a prefill chunk of the token-level indexer ("GLM-5.3
 * 最適化 第2部", section "PCP": 4 heads x 64 dims, every earlier token scored,
 * the top-2048 attended), bit for bit, without writing every score: a score
 * pass over every s-th key sets a per-query threshold, the full pass keeps
 * only the scores ranked at or above it, and the top-k is taken from those.
 * A query for which that leaves fewer than topk candidates (or more than
 * the workspace holds) gets its full scores in `scores` and an exact
 * select over them; for every other query `scores` is not written.
 * One sequence (keys as in qsa_index_scores with q_seq NULL), cfg with
 * block 1, idx_heads 4, idx_dim 64 (bf16 or FP8 keys), 16 <= nq <= 65535,
 * max_ctx <= 262144. Other arguments as in qsa_index_scores and
 * qsa_topk_blocks.
 *   ws (device) workspace of at least qsa_index_topk_prefill_workspace_bytes
 *      (cfg, nq, max_ctx) bytes (0: not supported), contents ignored on
 *      entry. Calls that share a workspace must not run concurrently. */
qsa_status qsa_index_topk_prefill(const qsa_sel_cfg* cfg, int32_t nq, const int32_t* q_ctx,
                                  int32_t max_ctx, const qsa_bf16* q_idx, const float* w_idx,
                                  const void* keys, float* scores, int64_t ld_scores,
                                  int32_t* sel, int32_t* n_sel, void* ws, size_t ws_bytes,
                                  qsa_stream_t stream);
size_t qsa_index_topk_prefill_workspace_bytes(const qsa_sel_cfg* cfg, int32_t nq, int32_t max_ctx);

/* --------------------------------------------- A2 + chunk lists of A3 ----
 * qsa_index_lists: the pooled-key scan that qsa_decode_layer issues first,
 * on its own: writes scores[i][b] for b < n_i (as qsa_index_scores) and, in
 * the workspace, each chunk's best candidate blocks with a bound (the best
 * block it left out); it selects nothing (sel / n_sel are not written).
 * qsa_decode_layer continues from such lists inside its own workspace;
 * calling this entry point separately lets a caller time or schedule the
 * scan on its own. ("3090x3で 314 万コンテキスト", "VRAM に残す必要があるもの":
 * every pooled key is scored at every step.)
 * Variant A only (block 4, idx_dim 128, idx_heads 1; bf16 or FP8 keys).
 *   q_seq, q_ctx, q_idx, keys, scores, ld_scores: as qsa_index_scores;
 *          scores may be NULL (no scores written, ld_scores ignored).
 *   ws (device) workspace of at least qsa_index_topk_workspace_bytes(cfg,
 *      nq, max_ctx) bytes; contents ignored on entry, list layout internal.
 *      Calls that share a workspace must not run concurrently. */
qsa_status qsa_index_lists(const qsa_sel_cfg* cfg, int32_t nq, const int32_t* q_seq,
                           const int32_t* q_ctx, int32_t max_ctx, const qsa_bf16* q_idx,
                           const void* keys, int64_t keys_seq_stride,
                           float* scores, int64_t ld_scores,
                           void* ws, size_t ws_bytes, qsa_stream_t stream);

/* ---------------------------------------------------------------- A4 ----
 * qsa_sparse_decode: softmax attention of each query over its selected
 * tokens, split into n_split partial results.
 * The token list of query i is, in ascending order: the `block` tokens of
 * each selected block sel[i][0..n_sel[i]), then the trailing tokens
 * [block * (q_ctx[i]/block), q_ctx[i]). Split j covers list positions
 * [j*L/n_split, (j+1)*L/n_split) with L the list length. For head h, kv
 * head g = h / (hq/hkv):
 *   z_t = scale * q[i][h] . k[t][g],  lse = ln sum_t exp(z_t),
 *   O   = sum_t exp(z_t - lse) v[t][g][0..dv)
 * An empty split gives O = 0, lse = -inf. ("なぜ": only the selected K/V
 * rows are read; "カーネルを書き換えずに済む": rows addressed per token and
 * kv head.)
 *   q        (device) bf16 [nq][hq][dk].
 *   kv       bf16 rows, or (shared-latent shape) FP8 sparse-MLA rows, each
 *            standing for its dequantized values in both K and V.
 *   o_part   (device) fp32 [n_split][nq][hq][dv];
 *   lse_part (device) fp32 [n_split][nq][hq] (natural log).
 *   1 <= n_split <= 256. Combine the splits with qsa_lse_merge. */
qsa_status qsa_sparse_decode(const qsa_sel_cfg* sel_cfg, const qsa_attn_cfg* attn_cfg,
                             int32_t nq, const int32_t* q_seq, const int32_t* q_ctx,
                             int32_t max_ctx, const qsa_bf16* q, const qsa_kv* kv,
                             const int32_t* sel, const int32_t* n_sel, int32_t n_split,
                             float* o_part, float* lse_part, qsa_stream_t stream);

/* ------------------------------------------------- A2 + A3 + A4 + A5 ----
 * qsa_decode_layer: one decode layer: exactly what qsa_index_topk, then
 * qsa_sparse_decode with n_split parts, then qsa_lse_merge of those parts
 * compute, with the parts held in the workspace. Two launches: the scan
 * (qsa_index_lists), then one work-group per (query, kv head, split) that
 * selects the query's blocks from the chunk lists itself, attends its part
 * and merges with the other parts in the same launch (a third launch merges
 * when the parts cannot all be resident at once).
 * ("3090x3で 314 万コンテキスト", "VRAM に残す必要があるもの" and "なぜ";
 * "GLM-5.3 ...", "DCP".)
 * Variant A only (block 4, idx_dim 128, idx_heads 1, bf16 or FP8 keys; hq
 * 16, hkv 2, dk = dv = 256; bf16 K/V rows); other configurations return
 * QSA_ERR_UNSUPPORTED. nq <= 4096.
 *   q_seq, q_ctx, q_idx, keys, scores, ld_scores, sel, n_sel: as
 *          qsa_index_topk (scores, sel and n_sel are written as there).
 *          scores may be NULL (ld_scores is then ignored): the scan writes
 *          no scores (4 bytes per block less traffic), and a query whose
 *          selection cannot come from the chunk lists (at most 4096 blocks,
 *          too few or too many chunks, or a chunk's bound ranking above
 *          the 512th) recomputes its scores from the keys inside the exact
 *          streamed select, bit for bit the scan's: same selection, much
 *          slower for such queries (every pass reads the query's keys).
 *   q, kv, n_split: as qsa_sparse_decode (1 <= n_split <= 256).
 *   o_out      (device) fp32 [nq][hq][dv], or NULL;
 *   o_out_bf16 (device) bf16 [nq][hq][dv] (nearest-even of o_out), or NULL;
 *   lse_out    (device) fp32 [nq][hq] (natural log), or NULL; at least one
 *              of the three must be given.
 *   ws (device) workspace of at least qsa_decode_layer_workspace_bytes(...)
 *      bytes, zero before the first call; every completed call leaves its
 *      counters zero again. Calls sharing a workspace must not overlap.
 *      The parts of a (query, kv head) wait for each other before they
 *      merge; the wait is bounded: if it runs out (which only a corrupted
 *      workspace or a device shared with other work can cause) a sticky
 *      error word in the workspace is set and results are unspecified. The
 *      error word is the workspace's first 4 bytes (uint32, device memory):
 *      once the stream has completed the call, a nonzero value means a wait
 *      ran out (callers that run layers concurrently on several streams
 *      read it after their step). With QSA_SYNC_CHECK=1 the call itself
 *      returns QSA_ERR_LAUNCH. Zero the workspace to clear it. */
qsa_status qsa_decode_layer(const qsa_sel_cfg* sel_cfg, const qsa_attn_cfg* attn_cfg, int32_t nq,
                            const int32_t* q_seq, const int32_t* q_ctx, int32_t max_ctx,
                            const qsa_bf16* q_idx, const void* keys, int64_t keys_seq_stride,
                            const qsa_bf16* q, const qsa_kv* kv,
                            float* scores, int64_t ld_scores, int32_t* sel, int32_t* n_sel,
                            int32_t n_split, float* o_out, qsa_bf16* o_out_bf16, float* lse_out,
                            void* ws, size_t ws_bytes, qsa_stream_t stream);

size_t qsa_decode_layer_workspace_bytes(const qsa_sel_cfg* sel_cfg, const qsa_attn_cfg* attn_cfg,
                                        int32_t nq, int32_t max_ctx, int32_t n_split);

/* ------------------------------------- A2-A5, no caller workspace ----
 * qsa_decode_layer_noalloc: for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). Computes exactly what qsa_decode_layer computes, bit for bit,
 * with the same kernels, but its workspace is a static array in the
 * library's device code (16 MiB = 16,777,216 bytes, one per device, held
 * until the process ends) instead of a caller buffer; it allocates and frees
 * nothing. Arguments as qsa_decode_layer, without ws / ws_bytes.
 *   - A call needs qsa_decode_layer_workspace_bytes(sel_cfg, attn_cfg, nq,
 *     max_ctx, n_split) bytes of it (e.g. 1.15 MiB for 4 queries at
 *     1,048,320 tokens with 16 splits); a larger call returns
 *     QSA_ERR_UNSUPPORTED and launches nothing.
 *   - Each call clears the control words it relies on (the error word and
 *     the merge counters) in its first launch, so the contents left by an
 *     earlier call do not matter.
 *   - Every call on one device shares that device's array: calls that
 *     overlap on one device (different streams or threads without ordering)
 *     race and their results are unspecified. Serialize them.
 *   - A timed-out merge wait is reported with QSA_SYNC_CHECK=1 as for
 *     qsa_decode_layer; the error word is not otherwise readable. */
qsa_status qsa_decode_layer_noalloc(const qsa_sel_cfg* sel_cfg, const qsa_attn_cfg* attn_cfg, int32_t nq,
                                    const int32_t* q_seq, const int32_t* q_ctx, int32_t max_ctx,
                                    const qsa_bf16* q_idx, const void* keys, int64_t keys_seq_stride,
                                    const qsa_bf16* q, const qsa_kv* kv, float* scores, int64_t ld_scores,
                                    int32_t* sel, int32_t* n_sel, int32_t n_split, float* o_out,
                                    qsa_bf16* o_out_bf16, float* lse_out, qsa_stream_t stream);

/* ------------------------------------ A2 + A3 + A4 + A5, shared latent ----
 * qsa_decode_layer_latent: one decode layer of the token-level indexer over
 * the shared 576-wide latent: exactly what qsa_index_scores, then
 * qsa_topk_blocks, then qsa_sparse_decode with n_split parts, then
 * qsa_lse_merge of those parts compute ("GLM-5.3 最適化 第2部", section
 * "PCP": every earlier token is scored by the 4-head ReLU-weighted indexer
 * and the best topk tokens feed the sparse MLA; section "DCP": the parts
 * are merged by log-sum-exp). Three launches: the scan, which also keeps
 * each 512-token chunk's 32 best tokens and the best one it left out; one
 * work-group per (query, split) that selects the query's exact top-k itself
 * (from the chunk lists, or from the scores when the lists cannot show it
 * exact) and attends its part; the merge.
 * Block 1, idx_dim 64, idx_heads 4 (bf16 or FP8 token keys), topk <= 2048;
 * hq 64, hkv 1, dk 576, dv 512 with bf16 latent rows; other configurations
 * return QSA_ERR_UNSUPPORTED. nq <= 65535.
 *   q_seq, q_ctx, q_idx, w_idx, keys, keys_seq_stride: as qsa_index_scores
 *          (w_idx required).
 *   scores, ld_scores (>= max_ctx): written as qsa_index_scores writes them.
 *   sel, n_sel: written as qsa_topk_blocks writes them.
 *   q, kv, n_split: as qsa_sparse_decode (1 <= n_split <= 256).
 *   o_out, o_out_bf16, lse_out: as qsa_decode_layer (at least one given).
 *   ws (device) at least qsa_decode_layer_latent_workspace_bytes(...) bytes,
 *      16-byte aligned, any contents (the call keeps no state in it between
 *      calls); calls sharing a workspace must not overlap. */
qsa_status qsa_decode_layer_latent(const qsa_sel_cfg* sel_cfg, const qsa_attn_cfg* attn_cfg, int32_t nq,
                                   const int32_t* q_seq, const int32_t* q_ctx, int32_t max_ctx,
                                   const qsa_bf16* q_idx, const float* w_idx, const void* keys,
                                   int64_t keys_seq_stride, const qsa_bf16* q, const qsa_kv* kv,
                                   float* scores, int64_t ld_scores, int32_t* sel, int32_t* n_sel,
                                   int32_t n_split, float* o_out, qsa_bf16* o_out_bf16, float* lse_out,
                                   void* ws, size_t ws_bytes, qsa_stream_t stream);

size_t qsa_decode_layer_latent_workspace_bytes(const qsa_sel_cfg* sel_cfg, const qsa_attn_cfg* attn_cfg,
                                               int32_t nq, int32_t max_ctx, int32_t n_split);

/* ------------------------------------------- A4 with an HBM row cache ----
 * For K/V rows kept in host memory (pinned, read zero-copy): a direct-mapped
 * cache of rows in device memory that later decode steps read instead of
 * crossing the host link again ("125B MoE を 3090 3 枚で運用する vLLM 最適化編", section 5:
 * consecutive selections overlap by 0.72 on average; one slot holds a
 * token's K and V for every kv head, keyed by the row's position; the slots
 * of stored rows are invalidated; per step an epoch, hit marks and claimed
 * fill rights keep reads and fills consistent inside one launch).
 * The pooled-block attention shape only (hq 16, hkv 2, dk = dv = 256).
 *
 * qsa_row_cache_bytes: bytes of a cache of n_slots rows (0 if unsupported).
 *   The caller allocates it in device memory, zero-filled once, one per layer
 *   (it may be shared by the sequences of one kv: keys are seq * capacity +
 *   token).
 * qsa_row_cache_step: once per step and layer, before that layer's
 *   qsa_sparse_decode_cached: advances the cache's epoch and drops the rows
 *   at (row_seq[j], row_pos[j]), j < n_rows: every row of kv stored since
 *   the cache last saw it (e.g. by qsa_kv_append) must be listed, else a
 *   later hit returns its old bytes; row_seq NULL: sequence j. Positions
 *   outside [0, capacity) are ignored. To drop every row (e.g. after a
 *   prefill rewrote many), zero-fill the cache again instead.
 * qsa_sparse_decode_cached: exactly what qsa_sparse_decode computes, bit for
 *   bit, reading each selected row from the cache when it holds it and from
 *   kv otherwise, and leaving rows read from kv in the cache (a slot keeps
 *   one row; of several rows that want one slot in a step, one is kept).
 *   plan_ws: device workspace of qsa_decode_cached_plan_bytes(sel_cfg, nq)
 *   bytes (contents ignored). Calls sharing a cache must not overlap. */
size_t qsa_row_cache_bytes(const qsa_attn_cfg* attn_cfg, int64_t n_slots);
size_t qsa_decode_cached_plan_bytes(const qsa_sel_cfg* sel_cfg, int32_t nq);
qsa_status qsa_row_cache_step(const qsa_attn_cfg* attn_cfg, void* cache, size_t cache_bytes, int64_t n_slots,
                              int32_t n_rows, const int32_t* row_seq, const int32_t* row_pos,
                              const qsa_kv* kv, qsa_stream_t stream);
qsa_status qsa_sparse_decode_cached(const qsa_sel_cfg* sel_cfg, const qsa_attn_cfg* attn_cfg, int32_t nq,
                                    const int32_t* q_seq, const int32_t* q_ctx, int32_t max_ctx,
                                    const qsa_bf16* q, const qsa_kv* kv, const int32_t* sel,
                                    const int32_t* n_sel, int32_t n_split, float* o_part, float* lse_part,
                                    void* cache, size_t cache_bytes, int64_t n_slots, void* plan_ws,
                                    size_t plan_ws_bytes, qsa_stream_t stream);

/* ---------------------------------------------------------------- A6 ----
 * qsa_sparse_prefill: the same attention restricted to one history tile:
 * query i attends the tokens of its list that lie in [tile_begin, tile_end)
 * and writes one partial (O, lse); a query with no token in the tile gets
 * O = 0, lse = -inf. Partials of consecutive tiles merged with
 * qsa_lse_merge equal the untiled result (up to rounding).
 * ("3090x3で 314 万コンテキスト", "ちなみにこの欠点": history in fixed tiles in
 * the outer loop, all queries computed per tile, partial softmax results
 * merged across tiles.)
 *   q_seq may be NULL (all queries in sequence 0).
 *   tile_begin must be a multiple of block and 0 <= tile_begin <= tile_end.
 *   o_part (device) fp32 [nq][hq][dv]; lse_part (device) fp32 [nq][hq]. */
qsa_status qsa_sparse_prefill(const qsa_sel_cfg* sel_cfg, const qsa_attn_cfg* attn_cfg,
                              int32_t nq, const int32_t* q_seq, const int32_t* q_ctx,
                              int32_t max_ctx, const qsa_bf16* q, const qsa_kv* kv,
                              const int32_t* sel, const int32_t* n_sel,
                              int64_t tile_begin, int64_t tile_end,
                              float* o_part, float* lse_part, qsa_stream_t stream);

/* qsa_sparse_prefill_merge: qsa_sparse_prefill for one history tile, merged
 * at once into the running result of the tiles before it (the same
 * log-sum-exp combination as qsa_lse_merge, one tile at a time), so that no
 * per-tile partials are kept and no final merge is needed (same sources as
 * qsa_sparse_prefill; "GLM-5.3 最適化 第2部", section "DCP", for the merge).
 *   o_run (device) fp32 [nq][hq][dv] and lse_run (device) fp32 [nq][hq]:
 *     with first == 0, the merge of the earlier tiles (as this call left
 *     it); with first != 0 their contents are ignored. On return they hold
 *     the merge including this tile; a query with no token in any tile so
 *     far has O = 0, lse = -inf.
 *   last != 0 and o_out_bf16 (device, 16-byte aligned, [nq][hq][dv]) non-NULL:
 *     the merged output is also written as bf16.
 *   Tiles merge in call order: issue them on one stream. Equal to
 *   qsa_sparse_prefill per tile followed by qsa_lse_merge up to rounding.
 *   Pooled-block variant (16 / 2 heads, head dim 256, bf16 K/V rows); and
 *   the shared latent (64 heads, dk 576, dv 512, block 1, bf16 rows) for a
 *   call that is both first and last (the whole history in one tile: the
 *   attention's result is final, written with its bf16 copy in the same
 *   launch, identical to qsa_sparse_prefill followed by a one-partial
 *   qsa_lse_merge); otherwise QSA_ERR_UNSUPPORTED. Other arguments and
 *   errors as qsa_sparse_prefill. */
qsa_status qsa_sparse_prefill_merge(const qsa_sel_cfg* sel_cfg, const qsa_attn_cfg* attn_cfg,
                                    int32_t nq, const int32_t* q_seq, const int32_t* q_ctx,
                                    int32_t max_ctx, const qsa_bf16* q, const qsa_kv* kv,
                                    const int32_t* sel, const int32_t* n_sel,
                                    int64_t tile_begin, int64_t tile_end, int32_t first, int32_t last,
                                    float* o_run, float* lse_run, qsa_bf16* o_out_bf16,
                                    qsa_stream_t stream);

/* ---------------------------------------------------------------- A5 ----
 * qsa_lse_merge: combine n_part partial softmax results per row.
 *   lse = M + ln sum_p exp(lse_p - M), M = max_p lse_p;
 *   O   = sum_p exp(lse_p - lse) O_p; partials with lse_p = -inf add nothing;
 *   rows whose partials are all empty get O = 0, lse = -inf.
 * ("GLM-5.3 ...", "DCP": partial attention combined by log-sum-exp.)
 *   o_parts   (device) fp32: partial p, row r at o_parts + p*o_part_stride + r*dv.
 *   lse_parts (device) fp32: lse_parts + p*lse_part_stride + r.
 *   o_out (device, fp32 [rows][dv]), o_out_bf16 (device, bf16 [rows][dv],
 *   nearest-even of the fp32 value) and lse_out (device, fp32 [rows]) may
 *   each be NULL. 1 <= n_part <= 4096; dv a multiple of 4, at most 1024. */
qsa_status qsa_lse_merge(int32_t n_part, int64_t rows, int32_t dv,
                         const float* o_parts, int64_t o_part_stride,
                         const float* lse_parts, int64_t lse_part_stride,
                         float* o_out, qsa_bf16* o_out_bf16, float* lse_out,
                         qsa_stream_t stream);

/* ------------------------------------------------------------- misc ---- */
const char* qsa_status_string(qsa_status s);
/* Message of the last failed call on this thread ("" if none). */
const char* qsa_last_error(void);
/* Library version: major * 10000 + minor * 100 + patch. */
int32_t qsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
