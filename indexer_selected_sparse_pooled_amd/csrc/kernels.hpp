// Host-side launchers of the libqsa kernels. Arguments are validated by the
// C-ABI layer (api.hip) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qsa {

hipError_t launch_pool(const uint16_t* raw, int64_t raw_ss, uint16_t* pooled, int64_t pooled_ss,
                       int n_seq, int64_t b0, int64_t nb, int dim, int block, hipStream_t s);
// FP8 indexer keys (pages of 64: codes, then fp32 scales) of keys [k0, k0 + nk)
// of n_seq sequences; out_ss in bytes.
hipError_t launch_quantize(const uint16_t* keys, int64_t keys_ss, uint8_t* out, int64_t out_ss, int n_seq,
                           int64_t k0, int64_t nk, int dim, hipStream_t s);
// FP8 sparse-MLA rows (656 bytes) of tokens [t0, t0 + nt) of n_seq sequences
// from 576-wide bf16 latent rows; ss, ts in elements, oss, ots in bytes.
hipError_t launch_quantize_latent(const uint16_t* lat, int64_t ss, int64_t ts, uint8_t* out, int64_t oss, int64_t ots,
                                  int n_seq, int64_t t0, int64_t nt, hipStream_t s);

// Decode-step append (one new token per query).
struct AppendArgs {
  int nq;
  const int* q_seq;  // nullable: query i appends to sequence i
  const int* q_pos;  // [nq] position of the new token
  int capacity;      // token rows per sequence
  const uint16_t* k_new;    // [nq][k_row]
  const uint16_t* v_new;    // [nq][v_row] or nullptr
  const uint16_t* raw_new;  // [nq][dim] or nullptr
  uint16_t* k;
  uint16_t* v;
  int64_t seq_stride, tok_stride, head_stride;  // elements; bytes for FP8 rows
  int kv_fp8;               // the cache holds FP8 sparse-MLA rows (k_new is then quantized)
  int k_row, v_row;         // elements per token row: hkv * head_dim, hkv * v_dim
  int head_dim, v_dim;
  uint16_t* raw;            // raw indexer keys, or nullptr
  int64_t raw_ss;           // elements; bytes for FP8 pages
  int raw_fp8;              // one-token blocks with FP8 keys: raw points to FP8 pages (the key is quantized)
  void* pooled;             // pooled keys (bf16 rows, or FP8 pages), or nullptr (no pooling)
  int64_t pooled_ss;        // elements for bf16 rows, bytes for FP8 pages
  int pooled_fp8;
  int dim, block;
};
hipError_t launch_append(const AppendArgs& a, hipStream_t s);

// list-mode counters, one per 128-byte line: every work-group of a query
// row adds to its queries' counters
constexpr int kCountStride = 32;
struct ScoreArgs {
  const int* q_seq;   // nullable
  const int* q_ctx;
  int max_ctx;
  int nq;
  int block;
  int idx_dim;
  int idx_heads;
  const uint16_t* q_idx;
  const float* w_idx;  // nullable when idx_heads == 1
  const void* keys;    // bf16 rows, or FP8 pages (key_fp8; keys_ss then in bytes)
  int64_t keys_ss;
  int key_fp8;
  float* scores;
  int64_t ld;
  // prefill chunk of variant B only (scores_gemm_b):
  int64_t tok_step;        // column t scores key t * tok_step (0 or 1: every key)
  const uint32_t* only;    // nullable: score only the queries flagged here
  const uint64_t* theta;   // list mode: per query, the rank64-style threshold (key << 32 | index)
  uint64_t* lists;         // list mode: [nq][list_cap] entries (score bits << 32) | index, unordered
  uint32_t* counts;        // list mode: entries reserved for query q at counts[q * kCountStride] (may exceed list_cap)
  int list_cap;
};
hipError_t launch_scores(const ScoreArgs& a, hipStream_t s);
// the variant B chunk GEMM over n_cols columns (keys t * tok_step): scores, or lists
hipError_t launch_scores_gemm_b(const ScoreArgs& a, int64_t n_cols, bool lists, hipStream_t s);

struct TopkArgs {
  const int* q_ctx;
  int max_ctx;
  int nq;
  int block;
  int topk;
  const float* scores;
  int64_t ld;
  int* sel;
  int* n_sel;
  void* ws;
  const uint32_t* only;  // nullable: select only for the queries flagged here
};
// Workspace layout of the chunked (large-context) path.
struct TopkPlan {
  bool chunked;      // false: every query is selected directly (or all taken)
  bool filter;       // chunk lists keep every score above a sampled threshold (else the best list_len)
  int chunk;         // scores per chunk
  int n_chunks;      // chunks per query at max_ctx
  int list_len;      // candidates kept per chunk (capacity in filter mode)
  int final_threads; // work-group size of the per-query selection (256 or 1024)
  int direct_max;    // queries with at most this many candidates skip the chunk lists
  bool stream_only;  // one launch: an exact select over all scores for each flagged query (needs a.only,
                     // queries with more than 8192 candidates; no workspace)
  size_t ws_bytes;
};
TopkPlan plan_topk(int nq, int max_ctx, int block, int topk);
hipError_t launch_topk(const TopkArgs& a, const TopkPlan& p, hipStream_t s);

// A2 + A3 of a variant B prefill chunk without materialised scores
// (prefill_select.hip); the scores buffer is used only by flagged queries.
struct PrefillSelectPlan {
  bool supported;  // keys per query within the list select's bitmap, topk within half the list
  int64_t step;    // sample stride
  int n_samp;      // sample columns per query
  int cap;         // list capacity per query
  TopkPlan tp;     // the regular top-k for flagged queries
  size_t off_samp, off_theta, off_counts, off_fail, off_lists, ws_bytes;
};
PrefillSelectPlan plan_prefill_select(int nq, int max_ctx, int block, int topk);
hipError_t launch_prefill_select(const ScoreArgs& sa, const TopkArgs& ta, const PrefillSelectPlan& p, void* ws,
                                 hipStream_t s);

struct AttendArgs {
  const int* q_seq;  // nullable
  const int* q_ctx;
  int max_ctx;
  int nq;
  int hq, hkv, dk, dv;
  float scale;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t seq_stride, tok_stride, head_stride;  // elements; bytes for FP8 rows
  int kv_fp8;                                    // FP8 sparse-MLA rows (656 bytes) instead of bf16
  const int* sel;
  const int* n_sel;
  int topk;
  int block;
  int n_split;
  int64_t tile_begin, tile_end;
  float* o_part;    // [n_split][nq][hq][dv]
  float* lse_part;  // [n_split][nq][hq]
  // merge inside the launch (decode layer); counter == nullptr: none
  uint32_t* counter;  // [nq][hkv] pairs of lines (kCounterStride words each), zero before the first call, left zero
  uint32_t* error;    // sticky error word (bit 1: a merge wait ran out), or nullptr
  float* o_out;       // [nq][hq][dv] or nullptr
  uint16_t* o_bf16;   // [nq][hq][dv] or nullptr
  float* lse_out;     // [nq][hq] or nullptr
  // running merge over history tiles (n_split 1, pooled-block variant):
  // o_part / lse_part hold the merge of the earlier tiles and receive the
  // merge with this one. 0: off; else bit 2 set, bit 0: first tile (no
  // earlier result), bit 1: last tile (the merged output also goes to
  // o_bf16 when given)
  int acc;
  // HBM row cache (qsa_sparse_decode_cached); src == nullptr: none
  const int* src;           // [nq][src_ld] per list position: -(slot + 1) for a hit, else the token
  int src_ld;
  unsigned char* c_rows;    // [n_slots][row_bytes]: per slot, kv head g's K then V (bf16)
  uint64_t* c_tag;          // [n_slots] key + 1 of the held row (0: empty)
  const uint32_t* c_hit;    // [n_slots] epoch of the last step with a hit on the slot
  const uint64_t* c_claim;  // [n_slots] epoch << 32 | claimer id, the step's fill right
  const uint32_t* c_epoch;
  int64_t n_slots, row_bytes, key_stride;  // key of (seq, tok) = seq * key_stride + tok
};
hipError_t launch_attend(const AttendArgs& a, hipStream_t s);

// Row cache: layout of the caller's buffer, the per-step invalidation and
// epoch advance, and the plan of one decode launch.
struct RowCacheLayout {
  int64_t n_slots, row_bytes;
  size_t off_tag, off_hit, off_claim, off_rows, bytes;
};
RowCacheLayout row_cache_layout(int64_t n_slots, int64_t row_bytes);
hipError_t launch_row_cache_step(unsigned char* cache, const RowCacheLayout& L, int n_rows, const int* row_seq,
                                 const int* row_pos, int64_t key_stride, hipStream_t s);
hipError_t launch_row_cache_plan(const AttendArgs& a, unsigned char* cache, const RowCacheLayout& L, int* src,
                                 int src_ld, hipStream_t s);

// Decode scan + exact top-k in one launch (variant A: 128-d pooled keys).
struct IndexTopkArgs {
  const int* q_seq;  // nullable
  const int* q_ctx;
  int max_ctx;
  int nq;
  const uint16_t* q_idx;
  const void* keys;  // bf16 rows, or FP8 pages (key_fp8; keys_ss then in bytes)
  int64_t keys_ss;
  int key_fp8;
  float* scores;
  int64_t ld;
  int topk;
  int* sel;
  int* n_sel;
  // workspace views and list sizes (filled by launch_index_topk)
  uint32_t* counter;     // [nq] lines of kCounterStride words: chunks finished
  uint64_t* list;        // [nq][n_chunks][keep] (key << 32 | block), 0 = empty
  uint64_t* list_bound;  // [nq][n_chunks]
  int n_chunks;
  int chunk_blocks;      // blocks per chunk
  int keep;              // candidates kept per chunk
  int wkeep;             // candidates kept per wave
  // words the first work-group of index_lists_a zeroes before it scans
  // (control words a later launch of the same call relies on), or NULL
  uint32_t* clear;
  int n_clear;
};
struct IndexTopkPlan {
  int tpw;        // 64-key tiles per wave (chunk = 256 * tpw keys)
  int n_chunks;   // chunks per query at max_ctx
  int keep, wkeep;
  size_t off_list, off_bound, ws_bytes;
};
IndexTopkPlan plan_index_topk(int nq, int max_ctx, int topk);
hipError_t launch_index_topk(IndexTopkArgs a, const IndexTopkPlan& p, void* ws, hipStream_t s);
// The scan and chunk lists alone (no selection), into an index_topk workspace.
hipError_t launch_index_lists(IndexTopkArgs a, const IndexTopkPlan& p, void* ws, hipStream_t s);


// One decode layer (variant A): scan with chunk lists, then attention whose
// work-groups select their query's blocks themselves and merge in-launch
// (a third launch merges when the parts cannot be resident together).
struct DecodeLayerPlan {
  IndexTopkPlan itk;
  size_t off_merge_cnt, off_itk, off_o, off_lse, ws_bytes;
};
DecodeLayerPlan plan_decode_layer(int nq, int max_ctx, int topk, int hq, int hkv, int dv, int n_split);
// itk / att: everything but the workspace views (filled in from ws).
// clear_control: the scan launch zeroes the workspace's control words (the
// error word and the merge counters, bytes [0, p.off_itk)) first, so their
// contents on entry do not matter.
hipError_t launch_decode_layer(IndexTopkArgs itk, AttendArgs att, const DecodeLayerPlan& p, void* ws,
                               hipStream_t s, bool clear_control = false);

// One decode layer of the shared-latent variant (token-level indexer, top-k
// of single tokens, 64 heads over one latent row): scan with chunk lists,
// then attention whose work-groups select their query's tokens themselves,
// then the merge (three launches).
struct DecodeLayerBPlan {
  int n_chunks;  // 512-key chunks per query at max_ctx
  size_t off_list, off_bound, off_o, off_lse, ws_bytes;
};
constexpr int kDecodeBChunk = 512;     // keys per chunk
constexpr int kDecodeBKeep = 32;       // candidates kept per chunk
constexpr int kDecodeBMaxChunks = 256;  // most chunks per query whose lists the select holds (one per thread)
DecodeLayerBPlan plan_decode_layer_b(int nq, int max_ctx, int hq, int dv, int n_split);
// sa: the scan's arguments (scores, q_idx, w_idx, keys ...); att: the
// attention's (sel, n_sel, the outputs) without the workspace views.
hipError_t launch_decode_layer_b(ScoreArgs sa, AttendArgs att, const DecodeLayerBPlan& p, void* ws, hipStream_t s);

hipError_t launch_merge(int n_part, int64_t rows, int dv, const float* o_parts, int64_t o_ps,
                        const float* lse_parts, int64_t l_ps, float* o_out, uint16_t* o_bf16,
                        float* lse_out, hipStream_t s);

}  // namespace qsa
