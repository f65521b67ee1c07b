// C ABI of libqsa (declared in include/qsa.h): argument validation on the
// host, then kernel launches on the caller's stream. No entry point
// allocates memory or synchronises unless QSA_VALIDATE / QSA_SYNC_CHECK ask.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/qsa.h"
#include "fp8.hpp"
#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

qsa_status fail(qsa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

bool env_on(const char* name) {
  const char* v = std::getenv(name);
  return v && v[0] && std::strcmp(v, "0") != 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Per-device record of the architecture check: 0 unknown, 1 gfx950, 2 other.
std::atomic<int> g_arch_ok[64];

qsa_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(QSA_ERR_DEVICE, "no HIP device");
  if (dev < 0 || dev >= 64) return fail(QSA_ERR_DEVICE, "device index %d out of range", dev);
  int st = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(QSA_ERR_DEVICE, "hipGetDeviceProperties failed");
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(st, std::memory_order_relaxed);
  }
  if (st != 1) return fail(QSA_ERR_DEVICE, "device %d is not gfx950", dev);
  return QSA_OK;
}

qsa_status finish(hipError_t e, hipStream_t s, const char* what) {
  if (e != hipSuccess) return fail(QSA_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  if (env_on("QSA_SYNC_CHECK")) {
    hipError_t e2 = hipStreamSynchronize(s);
    if (e2 == hipSuccess) e2 = hipGetLastError();
    if (e2 != hipSuccess) return fail(QSA_ERR_LAUNCH, "%s: kernel failed: %s", what, hipGetErrorString(e2));
  }
  g_err[0] = 0;
  return QSA_OK;
}

// Optional synchronous check of the device-side per-query arrays.
qsa_status validate_queries(int nq, const int32_t* q_seq, const int32_t* q_ctx, int max_ctx, hipStream_t s) {
  if (!env_on("QSA_VALIDATE") || nq <= 0) return QSA_OK;
  std::vector<int32_t> h(nq);
  if (hipMemcpyAsync(h.data(), q_ctx, sizeof(int32_t) * nq, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return fail(QSA_ERR_ARG, "QSA_VALIDATE: cannot read q_ctx");
  for (int i = 0; i < nq; i++)
    if (h[i] < 0 || h[i] > max_ctx) return fail(QSA_ERR_ARG, "q_ctx[%d] = %d outside [0, max_ctx = %d]", i, h[i], max_ctx);
  if (q_seq) {
    if (hipMemcpyAsync(h.data(), q_seq, sizeof(int32_t) * nq, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return fail(QSA_ERR_ARG, "QSA_VALIDATE: cannot read q_seq");
    for (int i = 0; i < nq; i++)
      if (h[i] < 0) return fail(QSA_ERR_ARG, "q_seq[%d] = %d is negative", i, h[i]);
  }
  return QSA_OK;
}

qsa_status check_sel_cfg(const qsa_sel_cfg* c) {
  if (!c) return fail(QSA_ERR_ARG, "sel_cfg is NULL");
  if (c->block != 1 && c->block != 4) return fail(QSA_ERR_UNSUPPORTED, "block %d not in {1, 4}", c->block);
  if (c->topk < 1 || c->topk > 2048) return fail(QSA_ERR_UNSUPPORTED, "topk %d not in [1, 2048]", c->topk);
  const bool a = c->idx_dim == 128 && c->idx_heads == 1;
  const bool b = c->idx_dim == 64 && c->idx_heads == 4;
  if (!a && !b) return fail(QSA_ERR_UNSUPPORTED, "(idx_dim, idx_heads) = (%d, %d) not supported", c->idx_dim, c->idx_heads);
  if (c->key_format != QSA_KEYS_BF16 && c->key_format != QSA_KEYS_FP8)
    return fail(QSA_ERR_UNSUPPORTED, "key_format %d not supported", c->key_format);
  return QSA_OK;
}

// Indexer keys: bf16 rows (stride in elements, a multiple of 8) or FP8 pages
// (stride in bytes, a multiple of 16).
// per_seq: queries read their own sequences, so the stride must hold nmax keys.
qsa_status check_keys(const qsa_sel_cfg* c, const void* keys, int64_t ss, int64_t nmax, bool per_seq) {
  if (!keys || !aligned16(keys)) return fail(QSA_ERR_ARG, "keys must be a non-NULL 16-byte aligned pointer");
  if (c->key_format == QSA_KEYS_FP8) {
    if (ss % 16 || ss < 0) return fail(QSA_ERR_ARG, "FP8 keys_seq_stride must be a non-negative multiple of 16 bytes");
    if (per_seq && ss < qsa::fp8_keys_bytes(nmax, c->idx_dim))
      return fail(QSA_ERR_ARG, "keys_seq_stride smaller than the pages of max_ctx / block keys");
  } else {
    if (ss % 8 || ss < 0) return fail(QSA_ERR_ARG, "keys_seq_stride must be a non-negative multiple of 8");
    if (per_seq && ss < nmax * c->idx_dim) return fail(QSA_ERR_ARG, "keys_seq_stride smaller than max_ctx / block keys");
  }
  return QSA_OK;
}

// The cache format: bf16 rows, or FP8 sparse-MLA rows (656 bytes, strides in
// bytes, multiples of 16; the shared-latent shape with v == k only).
qsa_status check_kv_format(const qsa_attn_cfg* ac, const qsa_kv* kv) {
  if (kv->format == QSA_KV_BF16) return QSA_OK;
  if (kv->format != QSA_KV_FP8_MLA) return fail(QSA_ERR_UNSUPPORTED, "kv format %d not supported", kv->format);
  if (!(ac->hq == 64 && ac->hkv == 1 && ac->dk == 576 && ac->dv == 512))
    return fail(QSA_ERR_UNSUPPORTED, "FP8 rows: only the 576-wide shared latent (hq 64, hkv 1, dk 576, dv 512)");
  if (kv->v != kv->k) return fail(QSA_ERR_ARG, "FP8 rows: v must equal k (one latent row per token)");
  if (kv->tok_stride < 656 || kv->tok_stride % 16 || kv->seq_stride % 16 || kv->seq_stride < 0)
    return fail(QSA_ERR_ARG, "FP8 rows: tok_stride >= 656 and strides multiples of 16 bytes");
  return QSA_OK;
}

// Attention inputs (everything but the output buffers).
qsa_status check_attn_inputs(const qsa_sel_cfg* sc, const qsa_attn_cfg* ac, int nq, const int32_t* q_ctx,
                             int max_ctx, const qsa_bf16* q, const qsa_kv* kv, const int32_t* sel,
                             const int32_t* n_sel) {
  qsa_status st = check_sel_cfg(sc);
  if (st != QSA_OK) return st;
  if (!ac) return fail(QSA_ERR_ARG, "attn_cfg is NULL");
  if (!kv) return fail(QSA_ERR_ARG, "kv is NULL");
  if (nq < 0 || max_ctx < 0) return fail(QSA_ERR_ARG, "negative nq or max_ctx");
  if (ac->hq <= 0 || ac->hkv <= 0 || ac->hq % ac->hkv != 0) return fail(QSA_ERR_ARG, "hq %% hkv != 0");
  if (!(ac->hq == 16 && ac->hkv == 2 && ac->dk == 256 && ac->dv == 256) &&
      !(ac->hq == 64 && ac->hkv == 1 && ac->dk == 576 && ac->dv == 512))
    return fail(QSA_ERR_UNSUPPORTED, "attention shape (hq %d, hkv %d, dk %d, dv %d) not compiled", ac->hq, ac->hkv,
                ac->dk, ac->dv);
  if (!(ac->scale > 0.f) || !(ac->scale < 1e30f)) return fail(QSA_ERR_ARG, "scale must be positive and finite");
  if (nq == 0) return QSA_OK;
  if (!q_ctx || !q || !kv->k || !kv->v || !sel || !n_sel) return fail(QSA_ERR_ARG, "NULL pointer argument");
  if (!aligned16(q) || !aligned16(kv->k) || !aligned16(kv->v) || !aligned16(sel))
    return fail(QSA_ERR_ARG, "q, k, v and sel must be 16-byte aligned");
  st = check_kv_format(ac, kv);
  if (st != QSA_OK) return st;
  if (kv->format == QSA_KV_BF16) {
    if (kv->tok_stride % 8 || kv->head_stride % 8 || kv->seq_stride % 8 || kv->tok_stride <= 0 ||
        kv->head_stride < 0 || kv->seq_stride < 0)
      return fail(QSA_ERR_ARG, "kv strides must be non-negative multiples of 8");
    if (int64_t(ac->hkv - 1) * kv->head_stride + ac->dk > kv->tok_stride)
      return fail(QSA_ERR_ARG, "tok_stride too small for hkv heads of dk");
  }
  if (kv->capacity < max_ctx) return fail(QSA_ERR_ARG, "kv capacity %lld < max_ctx %d", (long long)kv->capacity, max_ctx);
  return QSA_OK;
}

// Attention inputs and the partial-result buffers.
qsa_status check_attn(const qsa_sel_cfg* sc, const qsa_attn_cfg* ac, int nq, const int32_t* q_ctx, int max_ctx,
                      const qsa_bf16* q, const qsa_kv* kv, const int32_t* sel, const int32_t* n_sel,
                      const float* o_part, const float* lse_part) {
  const qsa_status st = check_attn_inputs(sc, ac, nq, q_ctx, max_ctx, q, kv, sel, n_sel);
  if (st != QSA_OK || nq == 0) return st;
  if (!o_part || !lse_part) return fail(QSA_ERR_ARG, "NULL pointer argument");
  if (!aligned16(o_part)) return fail(QSA_ERR_ARG, "o_part must be 16-byte aligned");
  return QSA_OK;
}

qsa::AttendArgs attend_args(const qsa_sel_cfg* sc, const qsa_attn_cfg* ac, int nq, const int32_t* q_seq,
                            const int32_t* q_ctx, int max_ctx, const qsa_bf16* q, const qsa_kv* kv,
                            const int32_t* sel, const int32_t* n_sel, int n_split, int64_t t0, int64_t t1,
                            float* o_part, float* lse_part) {
  qsa::AttendArgs a{};
  a.q_seq = q_seq;
  a.q_ctx = q_ctx;
  a.max_ctx = max_ctx;
  a.nq = nq;
  a.hq = ac->hq;
  a.hkv = ac->hkv;
  a.dk = ac->dk;
  a.dv = ac->dv;
  a.scale = ac->scale;
  a.q = q;
  a.k = kv->k;
  a.v = kv->v;
  a.seq_stride = kv->seq_stride;
  a.tok_stride = kv->tok_stride;
  a.head_stride = kv->head_stride;
  a.kv_fp8 = kv->format == QSA_KV_FP8_MLA;
  a.sel = sel;
  a.n_sel = n_sel;
  a.topk = sc->topk;
  a.block = sc->block;
  a.n_split = n_split;
  a.tile_begin = t0;
  a.tile_end = t1;
  a.o_part = o_part;
  a.lse_part = lse_part;
  return a;
}

}  // namespace

extern "C" {

qsa_status qsa_pool_keys(const qsa_bf16* raw, int64_t raw_seq_stride, qsa_bf16* pooled, int64_t pooled_seq_stride,
                         int32_t n_seq, int64_t tok_begin, int64_t tok_end, int32_t dim, int32_t block,
                         qsa_stream_t stream) {
  if (block != 1 && block != 4) return fail(QSA_ERR_UNSUPPORTED, "block %d not in {1, 4}", block);
  if (dim < 8 || dim > 1024 || dim % 8) return fail(QSA_ERR_UNSUPPORTED, "dim %d must be a multiple of 8 in [8, 1024]", dim);
  if (n_seq < 0 || tok_begin < 0 || tok_end < tok_begin) return fail(QSA_ERR_ARG, "bad n_seq or token range");
  if (tok_begin % block) return fail(QSA_ERR_ARG, "tok_begin must be a multiple of block");
  const int64_t b0 = tok_begin / block, b1 = tok_end / block;
  if (n_seq == 0 || b1 <= b0) return QSA_OK;
  if (!raw || !pooled) return fail(QSA_ERR_ARG, "NULL pointer argument");
  if (!aligned16(raw) || !aligned16(pooled)) return fail(QSA_ERR_ARG, "raw and pooled must be 16-byte aligned");
  if (raw_seq_stride % 8 || pooled_seq_stride % 8) return fail(QSA_ERR_ARG, "strides must be multiples of 8");
  if (n_seq > 1 && (raw_seq_stride < b1 * block * dim || pooled_seq_stride < b1 * dim))
    return fail(QSA_ERR_ARG, "sequence strides too small");
  if (n_seq > 65535) return fail(QSA_ERR_UNSUPPORTED, "n_seq > 65535");
  qsa_status st = check_device();
  if (st != QSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(qsa::launch_pool(raw, raw_seq_stride, pooled, pooled_seq_stride, n_seq, b0, b1 - b0, dim, block, s), s,
                "qsa_pool_keys");
}

qsa_status qsa_quantize_latent(const qsa_bf16* latent, int64_t seq_stride, int64_t tok_stride, void* out,
                               int64_t out_seq_stride, int64_t out_tok_stride, int32_t n_seq, int64_t tok_begin,
                               int64_t tok_end, qsa_stream_t stream) {
  if (n_seq < 0 || tok_begin < 0 || tok_end < tok_begin) return fail(QSA_ERR_ARG, "bad n_seq or token range");
  if (n_seq == 0 || tok_end == tok_begin) return QSA_OK;
  if (!latent || !out) return fail(QSA_ERR_ARG, "NULL pointer argument");
  if (!aligned16(latent) || !aligned16(out)) return fail(QSA_ERR_ARG, "latent and out must be 16-byte aligned");
  if (seq_stride % 8 || tok_stride % 8 || seq_stride < 0 || tok_stride < 576)
    return fail(QSA_ERR_ARG, "latent strides: multiples of 8 elements, tok_stride >= 576");
  if (out_seq_stride % 16 || out_tok_stride % 16 || out_seq_stride < 0 || out_tok_stride < 656)
    return fail(QSA_ERR_ARG, "out strides: multiples of 16 bytes, out_tok_stride >= 656");
  if (n_seq > 65535 || tok_end - tok_begin > 0x7FFFFFFF) return fail(QSA_ERR_UNSUPPORTED, "too many rows");
  qsa_status st = check_device();
  if (st != QSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(qsa::launch_quantize_latent(latent, seq_stride, tok_stride, static_cast<uint8_t*>(out), out_seq_stride,
                                            out_tok_stride, n_seq, tok_begin, tok_end - tok_begin, s),
                s, "qsa_quantize_latent");
}

int64_t qsa_fp8_keys_bytes(int64_t n_keys, int32_t dim) {
  if (n_keys < 0 || dim <= 0) return 0;
  return qsa::fp8_keys_bytes(n_keys, dim);
}

qsa_status qsa_quantize_keys(const qsa_bf16* keys, int64_t keys_seq_stride, void* out, int64_t out_seq_stride,
                             int32_t n_seq, int64_t key_begin, int64_t key_end, int32_t dim, qsa_stream_t stream) {
  if (dim != 64 && dim != 128) return fail(QSA_ERR_UNSUPPORTED, "dim %d not in {64, 128}", dim);
  if (n_seq < 0 || key_begin < 0 || key_end < key_begin) return fail(QSA_ERR_ARG, "bad n_seq or key range");
  if (n_seq == 0 || key_end == key_begin) return QSA_OK;
  if (!keys || !out) return fail(QSA_ERR_ARG, "NULL pointer argument");
  if (!aligned16(keys) || !aligned16(out)) return fail(QSA_ERR_ARG, "keys and out must be 16-byte aligned");
  if (keys_seq_stride % 8 || keys_seq_stride < 0) return fail(QSA_ERR_ARG, "keys_seq_stride must be a multiple of 8");
  if (out_seq_stride % 16 || out_seq_stride < 0) return fail(QSA_ERR_ARG, "out_seq_stride must be a multiple of 16");
  if (n_seq > 1 && (keys_seq_stride < key_end * dim || out_seq_stride < qsa::fp8_keys_bytes(key_end, dim)))
    return fail(QSA_ERR_ARG, "sequence strides too small");
  if (n_seq > 65535) return fail(QSA_ERR_UNSUPPORTED, "n_seq > 65535");
  if ((key_end - key_begin + 3) / 4 > 0x7FFFFFFF) return fail(QSA_ERR_UNSUPPORTED, "too many keys");
  qsa_status st = check_device();
  if (st != QSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(qsa::launch_quantize(keys, keys_seq_stride, static_cast<uint8_t*>(out), out_seq_stride, n_seq,
                                     key_begin, key_end - key_begin, dim, s),
                s, "qsa_quantize_keys");
}

qsa_status qsa_kv_append(const qsa_sel_cfg* sel_cfg, const qsa_attn_cfg* attn_cfg, int32_t nq,
                         const int32_t* q_seq, const int32_t* q_pos, const qsa_bf16* k_new,
                         const qsa_bf16* v_new, const qsa_bf16* raw_new, const qsa_kv* kv,
                         qsa_bf16* raw_keys, int64_t raw_seq_stride, void* pooled,
                         int64_t pooled_seq_stride, qsa_stream_t stream) {
  qsa_status st = check_sel_cfg(sel_cfg);
  if (st != QSA_OK) return st;
  if (!attn_cfg || !kv) return fail(QSA_ERR_ARG, "attn_cfg or kv is NULL");
  if (nq < 0) return fail(QSA_ERR_ARG, "negative nq");
  if (nq == 0) return QSA_OK;
  if (nq > 65535) return fail(QSA_ERR_UNSUPPORTED, "nq > 65535");
  const int hkv = attn_cfg->hkv, dk = attn_cfg->dk, dv = attn_cfg->dv;
  if (hkv <= 0 || dk <= 0 || dv <= 0 || dk % 8 || dv % 8 || dv > dk)
    return fail(QSA_ERR_ARG, "hkv, dk, dv must be positive multiples of 8 with dv <= dk");
  if (!q_pos || !k_new || !kv->k) return fail(QSA_ERR_ARG, "NULL pointer argument");
  st = check_kv_format(attn_cfg, kv);
  if (st != QSA_OK) return st;
  const bool fp8_rows = kv->format == QSA_KV_FP8_MLA;
  const bool shared = kv->v == kv->k;  // a latent row serves as K and (its first dv columns) V
  if (!shared && (!v_new || !kv->v)) return fail(QSA_ERR_ARG, "v_new and kv->v are required when v != k");
  if (shared && v_new) return fail(QSA_ERR_ARG, "v_new must be NULL when kv->v == kv->k");
  if (!aligned16(k_new) || (v_new && !aligned16(v_new)) || !aligned16(kv->k) || !aligned16(kv->v))
    return fail(QSA_ERR_ARG, "k_new, v_new, k and v must be 16-byte aligned");
  if (!fp8_rows && (kv->tok_stride % 8 || kv->head_stride % 8 || kv->seq_stride % 8 || kv->tok_stride <= 0 ||
                    kv->head_stride < 0 || kv->seq_stride < 0))
    return fail(QSA_ERR_ARG, "kv strides must be non-negative multiples of 8");
  if (!fp8_rows && int64_t(hkv - 1) * kv->head_stride + dk > kv->tok_stride)
    return fail(QSA_ERR_ARG, "tok_stride too small");
  if (kv->capacity <= 0 || kv->capacity > 0x7FFFFFFF) return fail(QSA_ERR_ARG, "bad kv capacity");
  const int dim = sel_cfg->idx_dim;
  // with one-token blocks the raw key is the indexer key: FP8 keys are then
  // written to raw_keys as FP8 pages
  const bool raw_fp8 = sel_cfg->block == 1 && sel_cfg->key_format == QSA_KEYS_FP8;
  if (raw_new || raw_keys) {
    if (!raw_new || !raw_keys) return fail(QSA_ERR_ARG, "raw_new and raw_keys go together");
    if (!aligned16(raw_new) || !aligned16(raw_keys)) return fail(QSA_ERR_ARG, "raw_new and raw_keys must be 16-byte aligned");
    if (raw_fp8 && (raw_seq_stride % 16 || raw_seq_stride < 0))
      return fail(QSA_ERR_ARG, "FP8 raw_seq_stride must be a non-negative multiple of 16 bytes");
    if (!raw_fp8 && (raw_seq_stride % 8 || raw_seq_stride < 0))
      return fail(QSA_ERR_ARG, "raw_seq_stride must be a multiple of 8");
    if (pooled) {
      if (sel_cfg->block == 1) return fail(QSA_ERR_ARG, "pooled must be NULL when block == 1");
      if (!aligned16(pooled)) return fail(QSA_ERR_ARG, "pooled must be 16-byte aligned");
      if (sel_cfg->key_format == QSA_KEYS_FP8) {
        if (pooled_seq_stride % 16 || pooled_seq_stride < 0)
          return fail(QSA_ERR_ARG, "FP8 pooled_seq_stride must be a non-negative multiple of 16 bytes");
      } else if (pooled_seq_stride % 8 || pooled_seq_stride < 0) {
        return fail(QSA_ERR_ARG, "pooled_seq_stride must be a multiple of 8");
      }
    }
  } else if (pooled) {
    return fail(QSA_ERR_ARG, "pooling needs raw_new and raw_keys");
  }
  st = check_device();
  if (st != QSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  qsa::AppendArgs a{};
  a.nq = nq;
  a.q_seq = q_seq;
  a.q_pos = q_pos;
  a.capacity = int(kv->capacity);
  a.k_new = k_new;
  a.v_new = shared ? nullptr : v_new;
  a.raw_new = raw_new;
  a.k = const_cast<qsa_bf16*>(kv->k);
  a.v = const_cast<qsa_bf16*>(kv->v);
  a.seq_stride = kv->seq_stride;
  a.tok_stride = kv->tok_stride;
  a.head_stride = kv->head_stride;
  a.kv_fp8 = fp8_rows;
  a.k_row = hkv * dk;
  a.v_row = hkv * dv;
  a.head_dim = dk;
  a.v_dim = dv;
  a.raw = raw_keys;
  a.raw_ss = raw_seq_stride;
  a.raw_fp8 = raw_fp8;
  a.pooled = pooled;
  a.pooled_ss = pooled_seq_stride;
  a.pooled_fp8 = sel_cfg->key_format == QSA_KEYS_FP8;
  a.dim = dim;
  a.block = sel_cfg->block;
  return finish(qsa::launch_append(a, s), s, "qsa_kv_append");
}

qsa_status qsa_index_scores(const qsa_sel_cfg* cfg, int32_t nq, const int32_t* q_seq, const int32_t* q_ctx,
                            int32_t max_ctx, const qsa_bf16* q_idx, const float* w_idx, const void* keys,
                            int64_t keys_seq_stride, float* scores, int64_t ld_scores, qsa_stream_t stream) {
  qsa_status st = check_sel_cfg(cfg);
  if (st != QSA_OK) return st;
  if (nq < 0 || max_ctx < 0) return fail(QSA_ERR_ARG, "negative nq or max_ctx");
  if (nq == 0) return QSA_OK;
  if (nq > 65535) return fail(QSA_ERR_UNSUPPORTED, "nq > 65535");
  if (!q_ctx || !q_idx || !scores) return fail(QSA_ERR_ARG, "NULL pointer argument");
  if (cfg->idx_heads > 1 && !w_idx) return fail(QSA_ERR_ARG, "w_idx required when idx_heads > 1");
  if (!aligned16(q_idx) || !aligned16(scores)) return fail(QSA_ERR_ARG, "q_idx and scores must be 16-byte aligned");
  const int64_t nmax = int64_t(max_ctx) / cfg->block;
  if (ld_scores < nmax) return fail(QSA_ERR_ARG, "ld_scores %lld < max_ctx / block = %lld", (long long)ld_scores, (long long)nmax);
  st = check_keys(cfg, keys, keys_seq_stride, nmax, q_seq != nullptr);
  if (st != QSA_OK) return st;
  st = check_device();
  if (st != QSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = validate_queries(nq, q_seq, q_ctx, max_ctx, s);
  if (st != QSA_OK) return st;
  qsa::ScoreArgs a{};
  a.q_seq = q_seq;
  a.q_ctx = q_ctx;
  a.max_ctx = max_ctx;
  a.nq = nq;
  a.block = cfg->block;
  a.idx_dim = cfg->idx_dim;
  a.idx_heads = cfg->idx_heads;
  a.q_idx = q_idx;
  a.w_idx = w_idx;
  a.keys = keys;
  a.keys_ss = keys_seq_stride;
  a.key_fp8 = cfg->key_format == QSA_KEYS_FP8;
  a.scores = scores;
  a.ld = ld_scores;
  return finish(qsa::launch_scores(a, s), s, "qsa_index_scores");
}

size_t qsa_topk_workspace_bytes(const qsa_sel_cfg* cfg, int32_t nq, int32_t max_ctx) {
  if (!cfg || cfg->block <= 0 || cfg->topk <= 0 || nq <= 0 || max_ctx <= 0) return 0;
  return qsa::plan_topk(nq, max_ctx, cfg->block, cfg->topk).ws_bytes;
}

qsa_status qsa_topk_blocks(const qsa_sel_cfg* cfg, int32_t nq, const int32_t* q_ctx, int32_t max_ctx,
                           const float* scores, int64_t ld_scores, int32_t* sel, int32_t* n_sel, void* ws,
                           size_t ws_bytes, qsa_stream_t stream) {
  qsa_status st = check_sel_cfg(cfg);
  if (st != QSA_OK) return st;
  if (nq < 0 || max_ctx < 0) return fail(QSA_ERR_ARG, "negative nq or max_ctx");
  if (nq == 0) return QSA_OK;
  if (nq > 1000000) return fail(QSA_ERR_UNSUPPORTED, "nq too large");
  if (!q_ctx || !scores || !sel || !n_sel) return fail(QSA_ERR_ARG, "NULL pointer argument");
  if (!aligned16(scores) || !aligned16(sel)) return fail(QSA_ERR_ARG, "scores and sel must be 16-byte aligned");
  const int64_t nmax = int64_t(max_ctx) / cfg->block;
  if (ld_scores < nmax) return fail(QSA_ERR_ARG, "ld_scores < max_ctx / block");
  if (nmax > 8388608) return fail(QSA_ERR_UNSUPPORTED, "more than 8388608 candidates per query");
  const qsa::TopkPlan plan = qsa::plan_topk(nq, max_ctx, cfg->block, cfg->topk);
  if (plan.chunked && nq > 65535) return fail(QSA_ERR_UNSUPPORTED, "nq > 65535 with more than 8192 candidates");
  if (ws_bytes < plan.ws_bytes || (plan.ws_bytes && !ws))
    return fail(QSA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, plan.ws_bytes);
  if (ws && !aligned16(ws)) return fail(QSA_ERR_ARG, "workspace must be 16-byte aligned");
  st = check_device();
  if (st != QSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = validate_queries(nq, nullptr, q_ctx, max_ctx, s);
  if (st != QSA_OK) return st;
  qsa::TopkArgs a{};
  a.q_ctx = q_ctx;
  a.max_ctx = max_ctx;
  a.nq = nq;
  a.block = cfg->block;
  a.topk = cfg->topk;
  a.scores = scores;
  a.ld = ld_scores;
  a.sel = sel;
  a.n_sel = n_sel;
  a.ws = ws;
  return finish(qsa::launch_topk(a, plan, s), s, "qsa_topk_blocks");
}

size_t qsa_index_topk_prefill_workspace_bytes(const qsa_sel_cfg* cfg, int32_t nq, int32_t max_ctx) {
  if (!cfg || cfg->block <= 0 || cfg->topk <= 0 || nq <= 0 || max_ctx < 0) return 0;
  const qsa::PrefillSelectPlan p = qsa::plan_prefill_select(nq, max_ctx, cfg->block, cfg->topk);
  return p.supported ? p.ws_bytes : 0;
}

qsa_status qsa_index_topk_prefill(const qsa_sel_cfg* cfg, int32_t nq, const int32_t* q_ctx, int32_t max_ctx,
                                  const qsa_bf16* q_idx, const float* w_idx, const void* keys, float* scores,
                                  int64_t ld_scores, int32_t* sel, int32_t* n_sel, void* ws, size_t ws_bytes,
                                  qsa_stream_t stream) {
  qsa_status st = check_sel_cfg(cfg);
  if (st != QSA_OK) return st;
  if (cfg->block != 1 || cfg->idx_dim != 64 || cfg->idx_heads != 4)
    return fail(QSA_ERR_UNSUPPORTED, "qsa_index_topk_prefill: only the 4-head, 64-d token-level indexer");
  if (nq < 0 || max_ctx < 0) return fail(QSA_ERR_ARG, "negative nq or max_ctx");
  if (nq == 0) return QSA_OK;
  if (nq < 16 || nq > 65535) return fail(QSA_ERR_UNSUPPORTED, "qsa_index_topk_prefill: nq %d not in [16, 65535]", nq);
  if (!q_ctx || !q_idx || !w_idx || !scores || !sel || !n_sel) return fail(QSA_ERR_ARG, "NULL pointer argument");
  if (!aligned16(q_idx) || !aligned16(scores) || !aligned16(sel))
    return fail(QSA_ERR_ARG, "q_idx, scores and sel must be 16-byte aligned");
  const int64_t nmax = int64_t(max_ctx) / cfg->block;
  if (ld_scores < nmax) return fail(QSA_ERR_ARG, "ld_scores %lld < max_ctx = %lld", (long long)ld_scores, (long long)nmax);
  st = check_keys(cfg, keys, 0, nmax, false);
  if (st != QSA_OK) return st;
  const qsa::PrefillSelectPlan plan = qsa::plan_prefill_select(nq, max_ctx, cfg->block, cfg->topk);
  if (!plan.supported) return fail(QSA_ERR_UNSUPPORTED, "qsa_index_topk_prefill: more than 262144 keys per query");
  if (!ws || ws_bytes < plan.ws_bytes)
    return fail(QSA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, plan.ws_bytes);
  if (!aligned16(ws)) return fail(QSA_ERR_ARG, "workspace must be 16-byte aligned");
  st = check_device();
  if (st != QSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = validate_queries(nq, nullptr, q_ctx, max_ctx, s);
  if (st != QSA_OK) return st;
  qsa::ScoreArgs a{};
  a.q_ctx = q_ctx;
  a.max_ctx = max_ctx;
  a.nq = nq;
  a.block = cfg->block;
  a.idx_dim = cfg->idx_dim;
  a.idx_heads = cfg->idx_heads;
  a.q_idx = q_idx;
  a.w_idx = w_idx;
  a.keys = keys;
  a.key_fp8 = cfg->key_format == QSA_KEYS_FP8;
  a.scores = scores;
  a.ld = ld_scores;
  qsa::TopkArgs t{};
  t.q_ctx = q_ctx;
  t.max_ctx = max_ctx;
  t.nq = nq;
  t.block = cfg->block;
  t.topk = cfg->topk;
  t.scores = scores;
  t.ld = ld_scores;
  t.sel = sel;
  t.n_sel = n_sel;
  return finish(qsa::launch_prefill_select(a, t, plan, ws, s), s, "qsa_index_topk_prefill");
}

size_t qsa_index_topk_workspace_bytes(const qsa_sel_cfg* cfg, int32_t nq, int32_t max_ctx) {
  if (!cfg || nq <= 0 || max_ctx < 0) return 0;
  return qsa::plan_index_topk(nq, max_ctx, cfg->topk).ws_bytes;
}

qsa_status qsa_index_topk(const qsa_sel_cfg* cfg, int32_t nq, const int32_t* q_seq, const int32_t* q_ctx,
                          int32_t max_ctx, const qsa_bf16* q_idx, const void* keys, int64_t keys_seq_stride,
                          float* scores, int64_t ld_scores, int32_t* sel, int32_t* n_sel, void* ws,
                          size_t ws_bytes, qsa_stream_t stream) {
  qsa_status st = check_sel_cfg(cfg);
  if (st != QSA_OK) return st;
  if (cfg->block != 4 || cfg->idx_dim != 128 || cfg->idx_heads != 1)
    return fail(QSA_ERR_UNSUPPORTED, "qsa_index_topk: only pooled 4-token blocks with a 128-d single-head indexer");
  if (nq < 0 || max_ctx < 0) return fail(QSA_ERR_ARG, "negative nq or max_ctx");
  if (nq == 0) return QSA_OK;
  if (nq > 65535) return fail(QSA_ERR_UNSUPPORTED, "nq > 65535");
  if (!q_ctx || !q_idx || !scores || !sel || !n_sel) return fail(QSA_ERR_ARG, "NULL pointer argument");
  if (!aligned16(q_idx) || !aligned16(scores) || !aligned16(sel))
    return fail(QSA_ERR_ARG, "q_idx, scores and sel must be 16-byte aligned");
  const int64_t nmax = int64_t(max_ctx) / 4;
  if (ld_scores < nmax) return fail(QSA_ERR_ARG, "ld_scores %lld < max_ctx / 4 = %lld", (long long)ld_scores, (long long)nmax);
  st = check_keys(cfg, keys, keys_seq_stride, nmax, q_seq != nullptr);
  if (st != QSA_OK) return st;
  const qsa::IndexTopkPlan plan = qsa::plan_index_topk(nq, max_ctx, cfg->topk);
  if (plan.n_chunks > 65535) return fail(QSA_ERR_UNSUPPORTED, "context too long");
  if (!ws || ws_bytes < plan.ws_bytes)
    return fail(QSA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, plan.ws_bytes);
  if (!aligned16(ws)) return fail(QSA_ERR_ARG, "workspace must be 16-byte aligned");
  st = check_device();
  if (st != QSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = validate_queries(nq, q_seq, q_ctx, max_ctx, s);
  if (st != QSA_OK) return st;
  qsa::IndexTopkArgs a{};
  a.q_seq = q_seq;
  a.q_ctx = q_ctx;
  a.max_ctx = max_ctx;
  a.nq = nq;
  a.q_idx = q_idx;
  a.keys = keys;
  a.keys_ss = keys_seq_stride;
  a.key_fp8 = cfg->key_format == QSA_KEYS_FP8;
  a.scores = scores;
  a.ld = ld_scores;
  a.topk = cfg->topk;
  a.sel = sel;
  a.n_sel = n_sel;
  return finish(qsa::launch_index_topk(a, plan, ws, s), s, "qsa_index_topk");
}

qsa_status qsa_index_lists(const qsa_sel_cfg* cfg, int32_t nq, const int32_t* q_seq, const int32_t* q_ctx,
                           int32_t max_ctx, const qsa_bf16* q_idx, const void* keys, int64_t keys_seq_stride,
                           float* scores, int64_t ld_scores, void* ws, size_t ws_bytes, qsa_stream_t stream) {
  qsa_status st = check_sel_cfg(cfg);
  if (st != QSA_OK) return st;
  if (cfg->block != 4 || cfg->idx_dim != 128 || cfg->idx_heads != 1)
    return fail(QSA_ERR_UNSUPPORTED, "qsa_index_lists: only pooled 4-token blocks with a 128-d single-head indexer");
  if (nq < 0 || max_ctx < 0) return fail(QSA_ERR_ARG, "negative nq or max_ctx");
  if (nq == 0) return QSA_OK;
  if (nq > 65535) return fail(QSA_ERR_UNSUPPORTED, "nq > 65535");
  if (!q_ctx || !q_idx) return fail(QSA_ERR_ARG, "NULL pointer argument");
  if (!aligned16(q_idx) || (scores && !aligned16(scores)))
    return fail(QSA_ERR_ARG, "q_idx and scores must be 16-byte aligned");
  const int64_t nmax = int64_t(max_ctx) / 4;
  if (scores && ld_scores < nmax)
    return fail(QSA_ERR_ARG, "ld_scores %lld < max_ctx / 4 = %lld", (long long)ld_scores, (long long)nmax);
  st = check_keys(cfg, keys, keys_seq_stride, nmax, q_seq != nullptr);
  if (st != QSA_OK) return st;
  const qsa::IndexTopkPlan plan = qsa::plan_index_topk(nq, max_ctx, cfg->topk);
  if (plan.n_chunks > 65535) return fail(QSA_ERR_UNSUPPORTED, "context too long");
  if (!ws || ws_bytes < plan.ws_bytes)
    return fail(QSA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, plan.ws_bytes);
  if (!aligned16(ws)) return fail(QSA_ERR_ARG, "workspace must be 16-byte aligned");
  st = check_device();
  if (st != QSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = validate_queries(nq, q_seq, q_ctx, max_ctx, s);
  if (st != QSA_OK) return st;
  qsa::IndexTopkArgs a{};
  a.q_seq = q_seq;
  a.q_ctx = q_ctx;
  a.max_ctx = max_ctx;
  a.nq = nq;
  a.q_idx = q_idx;
  a.keys = keys;
  a.keys_ss = keys_seq_stride;
  a.key_fp8 = cfg->key_format == QSA_KEYS_FP8;
  a.scores = scores;
  a.ld = ld_scores;
  a.topk = cfg->topk;
  return finish(qsa::launch_index_lists(a, plan, ws, s), s, "qsa_index_lists");
}

size_t qsa_decode_layer_workspace_bytes(const qsa_sel_cfg* sel_cfg, const qsa_attn_cfg* attn_cfg, int32_t nq,
                                        int32_t max_ctx, int32_t n_split) {
  if (!sel_cfg || !attn_cfg || nq <= 0 || max_ctx < 0 || n_split < 1 || attn_cfg->hq <= 0 || attn_cfg->hkv <= 0 ||
      attn_cfg->dv <= 0)
    return 0;
  return qsa::plan_decode_layer(nq, max_ctx, sel_cfg->topk, attn_cfg->hq, attn_cfg->hkv, attn_cfg->dv, n_split)
      .ws_bytes;
}

namespace {

// Scratch of qsa_decode_layer_noalloc: one array per device, kept until the
// process ends. In host code `scratch` names a host-side stand-in, not the
// device array: its device address comes from hipGetSymbolAddress, looked up
// once per device (scratch_on_device) and used everywhere host code needs it.
constexpr size_t kNoallocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

// The current device's address of `scratch` (looked up on the first call on
// that device, with that device current).
qsa_status scratch_on_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(QSA_ERR_DEVICE, "no HIP device");
  if (dev < 0 || dev >= 64) return fail(QSA_ERR_DEVICE, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(QSA_ERR_DEVICE, "cannot find the device address of the static scratch: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return QSA_OK;
}

// qsa_decode_layer with the workspace given (noalloc false) or the static
// scratch (noalloc true: ws / ws_bytes are ignored, the call's control words
// are cleared by its first launch).
qsa_status decode_layer_call(const char* fn, const qsa_sel_cfg* sel_cfg, const qsa_attn_cfg* attn_cfg, int32_t nq,
                             const int32_t* q_seq, const int32_t* q_ctx, int32_t max_ctx, const qsa_bf16* q_idx,
                             const void* keys, int64_t keys_seq_stride, const qsa_bf16* q, const qsa_kv* kv,
                             float* scores, int64_t ld_scores, int32_t* sel, int32_t* n_sel, int32_t n_split,
                             float* o_out, qsa_bf16* o_out_bf16, float* lse_out, void* ws, size_t ws_bytes,
                             bool noalloc, qsa_stream_t stream) {
  qsa_status st = check_sel_cfg(sel_cfg);
  if (st != QSA_OK) return st;
  if (sel_cfg->block != 4 || sel_cfg->idx_dim != 128 || sel_cfg->idx_heads != 1)
    return fail(QSA_ERR_UNSUPPORTED, "%s: only pooled 4-token blocks with a 128-d single-head indexer", fn);
  st = check_attn_inputs(sel_cfg, attn_cfg, nq, q_ctx, max_ctx, q, kv, sel, n_sel);
  if (st != QSA_OK) return st;
  if (n_split < 1 || n_split > 256) return fail(QSA_ERR_ARG, "n_split %d not in [1, 256]", n_split);
  if (nq == 0) return QSA_OK;
  if (nq > 4096) return fail(QSA_ERR_UNSUPPORTED, "nq > 4096");
  if (kv->format != QSA_KV_BF16) return fail(QSA_ERR_UNSUPPORTED, "%s: bf16 K/V rows only", fn);
  if (!q_idx) return fail(QSA_ERR_ARG, "NULL pointer argument");
  if (!o_out && !o_out_bf16 && !lse_out) return fail(QSA_ERR_ARG, "no output requested");
  if (!aligned16(q_idx) || (scores && !aligned16(scores)))
    return fail(QSA_ERR_ARG, "q_idx and scores must be 16-byte aligned");
  if ((o_out && !aligned16(o_out)) || (o_out_bf16 && !aligned16(o_out_bf16)))
    return fail(QSA_ERR_ARG, "o_out and o_out_bf16 must be 16-byte aligned");
  const int64_t nmax = int64_t(max_ctx) / 4;
  if (scores && ld_scores < nmax)
    return fail(QSA_ERR_ARG, "ld_scores %lld < max_ctx / 4 = %lld", (long long)ld_scores, (long long)nmax);
  st = check_keys(sel_cfg, keys, keys_seq_stride, nmax, q_seq != nullptr);
  if (st != QSA_OK) return st;
  const qsa::DecodeLayerPlan plan = qsa::plan_decode_layer(nq, max_ctx, sel_cfg->topk, attn_cfg->hq, attn_cfg->hkv,
                                                           attn_cfg->dv, n_split);
  if (int64_t(nq) * (plan.itk.n_chunks + attn_cfg->hkv * n_split) > 0x7FFFFFFF)
    return fail(QSA_ERR_UNSUPPORTED, "too many work items");
  if (noalloc) {
    if (plan.ws_bytes > kNoallocScratchBytes)
      return fail(QSA_ERR_UNSUPPORTED,
                  "%s: this call needs %zu bytes of scratch; the static scratch holds %zu (use qsa_decode_layer "
                  "with a workspace of qsa_decode_layer_workspace_bytes)",
                  fn, plan.ws_bytes, kNoallocScratchBytes);
  } else {
    if (!ws || ws_bytes < plan.ws_bytes)
      return fail(QSA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, plan.ws_bytes);
    if (!aligned16(ws)) return fail(QSA_ERR_ARG, "workspace must be 16-byte aligned");
  }
  st = check_device();
  if (st != QSA_OK) return st;
  if (noalloc) {
    st = scratch_on_device(&ws);
    if (st != QSA_OK) return st;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = validate_queries(nq, q_seq, q_ctx, max_ctx, s);
  if (st != QSA_OK) return st;
  qsa::IndexTopkArgs it{};
  it.q_seq = q_seq;
  it.q_ctx = q_ctx;
  it.max_ctx = max_ctx;
  it.nq = nq;
  it.q_idx = q_idx;
  it.keys = keys;
  it.keys_ss = keys_seq_stride;
  it.key_fp8 = sel_cfg->key_format == QSA_KEYS_FP8;
  it.scores = scores;
  it.ld = ld_scores;
  it.topk = sel_cfg->topk;
  it.sel = sel;
  it.n_sel = n_sel;
  qsa::AttendArgs at = attend_args(sel_cfg, attn_cfg, nq, q_seq, q_ctx, max_ctx, q, kv, sel, n_sel, n_split, 0,
                                   int64_t(max_ctx), nullptr, nullptr);
  at.o_out = o_out;
  at.o_bf16 = o_out_bf16;
  at.lse_out = lse_out;
  const qsa_status fs = finish(qsa::launch_decode_layer(it, at, plan, ws, s, noalloc), s, fn);
  if (fs != QSA_OK || !env_on("QSA_SYNC_CHECK")) return fs;
  uint32_t err = 0;
  if (hipMemcpy(&err, ws, 4, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(QSA_ERR_LAUNCH, "%s: cannot read the error word", fn);
  if (err) return fail(QSA_ERR_LAUNCH, "%s: a merge wait ran out (error word %u)", fn, err);
  return QSA_OK;
}

}  // namespace

qsa_status qsa_decode_layer(const qsa_sel_cfg* sel_cfg, const qsa_attn_cfg* attn_cfg, int32_t nq,
                            const int32_t* q_seq, const int32_t* q_ctx, int32_t max_ctx, const qsa_bf16* q_idx,
                            const void* keys, int64_t keys_seq_stride, const qsa_bf16* q, const qsa_kv* kv,
                            float* scores, int64_t ld_scores, int32_t* sel, int32_t* n_sel, int32_t n_split,
                            float* o_out, qsa_bf16* o_out_bf16, float* lse_out, void* ws, size_t ws_bytes,
                            qsa_stream_t stream) {
  return decode_layer_call("qsa_decode_layer", sel_cfg, attn_cfg, nq, q_seq, q_ctx, max_ctx, q_idx, keys,
                           keys_seq_stride, q, kv, scores, ld_scores, sel, n_sel, n_split, o_out, o_out_bf16, lse_out,
                           ws, ws_bytes, false, stream);
}

qsa_status qsa_decode_layer_noalloc(const qsa_sel_cfg* sel_cfg, const qsa_attn_cfg* attn_cfg, int32_t nq,
                                    const int32_t* q_seq, const int32_t* q_ctx, int32_t max_ctx,
                                    const qsa_bf16* q_idx, const void* keys, int64_t keys_seq_stride,
                                    const qsa_bf16* q, const qsa_kv* kv, float* scores, int64_t ld_scores,
                                    int32_t* sel, int32_t* n_sel, int32_t n_split, float* o_out,
                                    qsa_bf16* o_out_bf16, float* lse_out, qsa_stream_t stream) {
  return decode_layer_call("qsa_decode_layer_noalloc", sel_cfg, attn_cfg, nq, q_seq, q_ctx, max_ctx, q_idx, keys,
                           keys_seq_stride, q, kv, scores, ld_scores, sel, n_sel, n_split, o_out, o_out_bf16, lse_out,
                           nullptr, 0, true, stream);
}

size_t qsa_decode_layer_latent_workspace_bytes(const qsa_sel_cfg* sel_cfg, const qsa_attn_cfg* attn_cfg,
                                               int32_t nq, int32_t max_ctx, int32_t n_split) {
  if (!sel_cfg || !attn_cfg || nq <= 0 || max_ctx < 0 || n_split < 1 || attn_cfg->hq <= 0 || attn_cfg->dv <= 0)
    return 0;
  return qsa::plan_decode_layer_b(nq, max_ctx, attn_cfg->hq, attn_cfg->dv, n_split).ws_bytes;
}

qsa_status qsa_decode_layer_latent(const qsa_sel_cfg* sel_cfg, const qsa_attn_cfg* attn_cfg, int32_t nq,
                                   const int32_t* q_seq, const int32_t* q_ctx, int32_t max_ctx,
                                   const qsa_bf16* q_idx, const float* w_idx, const void* keys,
                                   int64_t keys_seq_stride, const qsa_bf16* q, const qsa_kv* kv, float* scores,
                                   int64_t ld_scores, int32_t* sel, int32_t* n_sel, int32_t n_split, float* o_out,
                                   qsa_bf16* o_out_bf16, float* lse_out, void* ws, size_t ws_bytes,
                                   qsa_stream_t stream) {
  const char* fn = "qsa_decode_layer_latent";
  qsa_status st = check_sel_cfg(sel_cfg);
  if (st != QSA_OK) return st;
  if (sel_cfg->block != 1 || sel_cfg->idx_dim != 64 || sel_cfg->idx_heads != 4)
    return fail(QSA_ERR_UNSUPPORTED, "%s: only the token-level indexer (block 1, 4 heads of 64 dims)", fn);
  if (sel_cfg->topk > 2048) return fail(QSA_ERR_UNSUPPORTED, "%s: topk %d > 2048", fn, sel_cfg->topk);
  st = check_attn_inputs(sel_cfg, attn_cfg, nq, q_ctx, max_ctx, q, kv, sel, n_sel);
  if (st != QSA_OK) return st;
  if (!(attn_cfg->hq == 64 && attn_cfg->hkv == 1 && attn_cfg->dk == 576 && attn_cfg->dv == 512))
    return fail(QSA_ERR_UNSUPPORTED, "%s: only the 576-wide shared latent (hq 64, hkv 1, dk 576, dv 512)", fn);
  if (kv->format != QSA_KV_BF16) return fail(QSA_ERR_UNSUPPORTED, "%s: bf16 latent rows only", fn);
  if (n_split < 1 || n_split > 256) return fail(QSA_ERR_ARG, "n_split %d not in [1, 256]", n_split);
  if (nq == 0) return QSA_OK;
  if (nq > 65535) return fail(QSA_ERR_UNSUPPORTED, "nq > 65535");
  if (!q_idx || !w_idx || !scores) return fail(QSA_ERR_ARG, "NULL pointer argument");
  if (!o_out && !o_out_bf16 && !lse_out) return fail(QSA_ERR_ARG, "no output requested");
  if (!aligned16(q_idx) || !aligned16(scores)) return fail(QSA_ERR_ARG, "q_idx and scores must be 16-byte aligned");
  if ((o_out && !aligned16(o_out)) || (o_out_bf16 && !aligned16(o_out_bf16)))
    return fail(QSA_ERR_ARG, "o_out and o_out_bf16 must be 16-byte aligned");
  const int64_t nmax = int64_t(max_ctx);
  if (ld_scores < nmax) return fail(QSA_ERR_ARG, "ld_scores %lld < max_ctx = %lld", (long long)ld_scores, (long long)nmax);
  st = check_keys(sel_cfg, keys, keys_seq_stride, nmax, q_seq != nullptr);
  if (st != QSA_OK) return st;
  const qsa::DecodeLayerBPlan plan = qsa::plan_decode_layer_b(nq, max_ctx, attn_cfg->hq, attn_cfg->dv, n_split);
  if (int64_t(nq) * n_split > 0x7FFFFFFF) return fail(QSA_ERR_UNSUPPORTED, "nq * n_split too large");
  if (!ws || ws_bytes < plan.ws_bytes)
    return fail(QSA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, plan.ws_bytes);
  if (!aligned16(ws)) return fail(QSA_ERR_ARG, "workspace must be 16-byte aligned");
  st = check_device();
  if (st != QSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = validate_queries(nq, q_seq, q_ctx, max_ctx, s);
  if (st != QSA_OK) return st;
  qsa::ScoreArgs sa{};
  sa.q_seq = q_seq;
  sa.q_ctx = q_ctx;
  sa.max_ctx = max_ctx;
  sa.nq = nq;
  sa.block = 1;
  sa.idx_dim = 64;
  sa.idx_heads = 4;
  sa.q_idx = q_idx;
  sa.w_idx = w_idx;
  sa.keys = keys;
  sa.keys_ss = keys_seq_stride;
  sa.key_fp8 = sel_cfg->key_format == QSA_KEYS_FP8;
  sa.scores = scores;
  sa.ld = ld_scores;
  qsa::AttendArgs at = attend_args(sel_cfg, attn_cfg, nq, q_seq, q_ctx, max_ctx, q, kv, sel, n_sel, n_split, 0,
                                   int64_t(max_ctx), nullptr, nullptr);
  at.o_out = o_out;
  at.o_bf16 = o_out_bf16;
  at.lse_out = lse_out;
  return finish(qsa::launch_decode_layer_b(sa, at, plan, ws, s), s, fn);
}

qsa_status qsa_sparse_decode(const qsa_sel_cfg* sel_cfg, const qsa_attn_cfg* attn_cfg, int32_t nq,
                             const int32_t* q_seq, const int32_t* q_ctx, int32_t max_ctx, const qsa_bf16* q,
                             const qsa_kv* kv, const int32_t* sel, const int32_t* n_sel, int32_t n_split,
                             float* o_part, float* lse_part, qsa_stream_t stream) {
  qsa_status st = check_attn(sel_cfg, attn_cfg, nq, q_ctx, max_ctx, q, kv, sel, n_sel, o_part, lse_part);
  if (st != QSA_OK) return st;
  if (n_split < 1 || n_split > 256) return fail(QSA_ERR_ARG, "n_split %d not in [1, 256]", n_split);
  if (nq == 0) return QSA_OK;
  if (int64_t(nq) * n_split > 0x7FFFFFFF) return fail(QSA_ERR_UNSUPPORTED, "nq * n_split too large");
  st = check_device();
  if (st != QSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = validate_queries(nq, q_seq, q_ctx, max_ctx, s);
  if (st != QSA_OK) return st;
  const qsa::AttendArgs a = attend_args(sel_cfg, attn_cfg, nq, q_seq, q_ctx, max_ctx, q, kv, sel, n_sel, n_split, 0,
                                        int64_t(max_ctx), o_part, lse_part);
  return finish(qsa::launch_attend(a, s), s, "qsa_sparse_decode");
}

size_t qsa_row_cache_bytes(const qsa_attn_cfg* attn_cfg, int64_t n_slots) {
  if (!attn_cfg || n_slots <= 0) return 0;
  if (!(attn_cfg->hq == 16 && attn_cfg->hkv == 2 && attn_cfg->dk == 256 && attn_cfg->dv == 256)) return 0;
  return qsa::row_cache_layout(n_slots, int64_t(attn_cfg->hkv) * (attn_cfg->dk + attn_cfg->dv) * 2).bytes;
}

size_t qsa_decode_cached_plan_bytes(const qsa_sel_cfg* sel_cfg, int32_t nq) {
  if (!sel_cfg || nq <= 0 || sel_cfg->block <= 0 || sel_cfg->topk <= 0) return 0;
  return size_t(nq) * size_t(sel_cfg->topk * sel_cfg->block + sel_cfg->block - 1) * 4;
}

namespace {
qsa_status check_row_cache(const qsa_attn_cfg* ac, const void* cache, size_t cache_bytes, int64_t n_slots) {
  if (!ac || !cache) return fail(QSA_ERR_ARG, "NULL pointer argument");
  if (!(ac->hq == 16 && ac->hkv == 2 && ac->dk == 256 && ac->dv == 256))
    return fail(QSA_ERR_UNSUPPORTED, "row cache: the pooled-block attention shape only (hq 16, hkv 2, dk = dv = 256)");
  if (n_slots < 1 || n_slots > 0x7FFFFFFF) return fail(QSA_ERR_ARG, "n_slots %lld not in [1, 2^31)", (long long)n_slots);
  if (!aligned16(cache)) return fail(QSA_ERR_ARG, "cache must be 16-byte aligned");
  const size_t need = qsa_row_cache_bytes(ac, n_slots);
  if (cache_bytes < need) return fail(QSA_ERR_WORKSPACE, "row cache %zu bytes < %zu required", cache_bytes, need);
  return QSA_OK;
}
}  // namespace

qsa_status qsa_row_cache_step(const qsa_attn_cfg* attn_cfg, void* cache, size_t cache_bytes, int64_t n_slots,
                              int32_t n_rows, const int32_t* row_seq, const int32_t* row_pos, const qsa_kv* kv,
                              qsa_stream_t stream) {
  qsa_status st = check_row_cache(attn_cfg, cache, cache_bytes, n_slots);
  if (st != QSA_OK) return st;
  if (!kv || kv->capacity <= 0) return fail(QSA_ERR_ARG, "kv with a positive capacity is required");
  if (n_rows < 0) return fail(QSA_ERR_ARG, "negative n_rows");
  if (n_rows > 0 && !row_pos) return fail(QSA_ERR_ARG, "NULL pointer argument");
  st = check_device();
  if (st != QSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const qsa::RowCacheLayout L = qsa::row_cache_layout(n_slots, int64_t(attn_cfg->hkv) * (attn_cfg->dk + attn_cfg->dv) * 2);
  return finish(qsa::launch_row_cache_step(static_cast<unsigned char*>(cache), L, n_rows, row_seq, row_pos, kv->capacity, s), s,
                "qsa_row_cache_step");
}

qsa_status qsa_sparse_decode_cached(const qsa_sel_cfg* sel_cfg, const qsa_attn_cfg* attn_cfg, int32_t nq,
                                    const int32_t* q_seq, const int32_t* q_ctx, int32_t max_ctx, const qsa_bf16* q,
                                    const qsa_kv* kv, const int32_t* sel, const int32_t* n_sel, int32_t n_split,
                                    float* o_part, float* lse_part, void* cache, size_t cache_bytes, int64_t n_slots,
                                    void* plan_ws, size_t plan_ws_bytes, qsa_stream_t stream) {
  qsa_status st = check_attn(sel_cfg, attn_cfg, nq, q_ctx, max_ctx, q, kv, sel, n_sel, o_part, lse_part);
  if (st != QSA_OK) return st;
  if (n_split < 1 || n_split > 256) return fail(QSA_ERR_ARG, "n_split %d not in [1, 256]", n_split);
  st = check_row_cache(attn_cfg, cache, cache_bytes, n_slots);
  if (st != QSA_OK) return st;
  if (kv->format != QSA_KV_BF16) return fail(QSA_ERR_UNSUPPORTED, "row cache: bf16 K/V rows only");
  if (nq == 0) return QSA_OK;
  if (int64_t(nq) * n_split > 0x7FFFFFFF || nq > 65535) return fail(QSA_ERR_UNSUPPORTED, "too many work-groups");
  const size_t need = qsa_decode_cached_plan_bytes(sel_cfg, nq);
  if (!plan_ws || plan_ws_bytes < need) return fail(QSA_ERR_WORKSPACE, "plan workspace %zu bytes < %zu", plan_ws_bytes, need);
  if (!aligned16(plan_ws)) return fail(QSA_ERR_ARG, "plan workspace must be 16-byte aligned");
  if (need / 4 >= 0xFFFFFFFFull) return fail(QSA_ERR_UNSUPPORTED, "too many list positions");
  st = check_device();
  if (st != QSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = validate_queries(nq, q_seq, q_ctx, max_ctx, s);
  if (st != QSA_OK) return st;
  qsa::AttendArgs a = attend_args(sel_cfg, attn_cfg, nq, q_seq, q_ctx, max_ctx, q, kv, sel, n_sel, n_split, 0,
                                  int64_t(max_ctx), o_part, lse_part);
  const qsa::RowCacheLayout L = qsa::row_cache_layout(n_slots, int64_t(attn_cfg->hkv) * (attn_cfg->dk + attn_cfg->dv) * 2);
  unsigned char* c = static_cast<unsigned char*>(cache);
  const int src_ld = sel_cfg->topk * sel_cfg->block + sel_cfg->block - 1;
  a.src_ld = src_ld;
  a.c_rows = c + L.off_rows;
  a.c_tag = reinterpret_cast<uint64_t*>(c + L.off_tag);
  a.c_hit = reinterpret_cast<const uint32_t*>(c + L.off_hit);
  a.c_claim = reinterpret_cast<const uint64_t*>(c + L.off_claim);
  a.c_epoch = reinterpret_cast<const uint32_t*>(c);
  a.n_slots = n_slots;
  a.row_bytes = L.row_bytes;
  a.key_stride = kv->capacity;
  hipError_t e = qsa::launch_row_cache_plan(a, c, L, static_cast<int*>(plan_ws), src_ld, s);
  if (e != hipSuccess) return finish(e, s, "qsa_sparse_decode_cached");
  a.src = static_cast<const int*>(plan_ws);
  return finish(qsa::launch_attend(a, s), s, "qsa_sparse_decode_cached");
}

qsa_status qsa_sparse_prefill(const qsa_sel_cfg* sel_cfg, const qsa_attn_cfg* attn_cfg, int32_t nq,
                              const int32_t* q_seq, const int32_t* q_ctx, int32_t max_ctx, const qsa_bf16* q,
                              const qsa_kv* kv, const int32_t* sel, const int32_t* n_sel, int64_t tile_begin,
                              int64_t tile_end, float* o_part, float* lse_part, qsa_stream_t stream) {
  qsa_status st = check_attn(sel_cfg, attn_cfg, nq, q_ctx, max_ctx, q, kv, sel, n_sel, o_part, lse_part);
  if (st != QSA_OK) return st;
  if (tile_begin < 0 || tile_end < tile_begin) return fail(QSA_ERR_ARG, "bad tile range");
  if (tile_begin % sel_cfg->block) return fail(QSA_ERR_ARG, "tile_begin must be a multiple of block");
  if (tile_end % sel_cfg->block && tile_end < max_ctx)
    return fail(QSA_ERR_ARG, "tile_end must be a multiple of block (or >= max_ctx)");
  if (nq == 0) return QSA_OK;
  st = check_device();
  if (st != QSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = validate_queries(nq, q_seq, q_ctx, max_ctx, s);
  if (st != QSA_OK) return st;
  const qsa::AttendArgs a = attend_args(sel_cfg, attn_cfg, nq, q_seq, q_ctx, max_ctx, q, kv, sel, n_sel, 1,
                                        tile_begin, tile_end, o_part, lse_part);
  return finish(qsa::launch_attend(a, s), s, "qsa_sparse_prefill");
}

qsa_status qsa_sparse_prefill_merge(const qsa_sel_cfg* sel_cfg, const qsa_attn_cfg* attn_cfg, int32_t nq,
                                    const int32_t* q_seq, const int32_t* q_ctx, int32_t max_ctx, const qsa_bf16* q,
                                    const qsa_kv* kv, const int32_t* sel, const int32_t* n_sel, int64_t tile_begin,
                                    int64_t tile_end, int32_t first, int32_t last, float* o_run, float* lse_run,
                                    qsa_bf16* o_out_bf16, qsa_stream_t stream) {
  qsa_status st = check_attn(sel_cfg, attn_cfg, nq, q_ctx, max_ctx, q, kv, sel, n_sel, o_run, lse_run);
  if (st != QSA_OK) return st;
  const bool pooled = attn_cfg->hq == 16 && attn_cfg->hkv == 2 && attn_cfg->dk == 256 && attn_cfg->dv == 256;
  // the shared latent (token-level selection, bf16 rows): a single tile only
  const bool latent_single = attn_cfg->hq == 64 && attn_cfg->hkv == 1 && attn_cfg->dk == 576 &&
                             attn_cfg->dv == 512 && sel_cfg->block == 1 && first && last;
  if (!(pooled || latent_single) || kv->format != QSA_KV_BF16)
    return fail(QSA_ERR_UNSUPPORTED, "the running tile merge covers the pooled-block variant (16 / 2 heads, "
                                     "head dim 256) and a single-tile call of the shared latent (64 heads, "
                                     "576 / 512, token-level selection), with bf16 rows");
  if (tile_begin < 0 || tile_end < tile_begin) return fail(QSA_ERR_ARG, "bad tile range");
  if (tile_begin % sel_cfg->block) return fail(QSA_ERR_ARG, "tile_begin must be a multiple of block");
  if (tile_end % sel_cfg->block && tile_end < max_ctx)
    return fail(QSA_ERR_ARG, "tile_end must be a multiple of block (or >= max_ctx)");
  if (o_out_bf16 && !aligned16(o_out_bf16)) return fail(QSA_ERR_ARG, "o_out_bf16 must be 16-byte aligned");
  if (nq == 0) return QSA_OK;
  st = check_device();
  if (st != QSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = validate_queries(nq, q_seq, q_ctx, max_ctx, s);
  if (st != QSA_OK) return st;
  qsa::AttendArgs a = attend_args(sel_cfg, attn_cfg, nq, q_seq, q_ctx, max_ctx, q, kv, sel, n_sel, 1, tile_begin,
                                  tile_end, o_run, lse_run);
  a.acc = 4 | (first ? 1 : 0) | (last ? 2 : 0);
  a.o_bf16 = last ? reinterpret_cast<uint16_t*>(o_out_bf16) : nullptr;
  return finish(qsa::launch_attend(a, s), s, "qsa_sparse_prefill_merge");
}

qsa_status qsa_lse_merge(int32_t n_part, int64_t rows, int32_t dv, const float* o_parts, int64_t o_part_stride,
                         const float* lse_parts, int64_t lse_part_stride, float* o_out, qsa_bf16* o_out_bf16,
                         float* lse_out, qsa_stream_t stream) {
  if (n_part < 1 || n_part > 4096) return fail(QSA_ERR_ARG, "n_part %d not in [1, 4096]", n_part);
  if (rows < 0) return fail(QSA_ERR_ARG, "negative rows");
  if (dv < 4 || dv > 1024 || dv % 4) return fail(QSA_ERR_UNSUPPORTED, "dv %d must be a multiple of 4 in [4, 1024]", dv);
  if (rows == 0) return QSA_OK;
  if (!o_parts || !lse_parts) return fail(QSA_ERR_ARG, "NULL pointer argument");
  if (!aligned16(o_parts) || (o_out && !aligned16(o_out)) || (o_out_bf16 && !aligned16(o_out_bf16)))
    return fail(QSA_ERR_ARG, "o_parts, o_out and o_out_bf16 must be 16-byte aligned");
  if (n_part > 1 && (o_part_stride < rows * dv || lse_part_stride < rows || o_part_stride % 4))
    return fail(QSA_ERR_ARG, "partial strides too small");
  if (rows > int64_t(0x7FFFFFFF) * 4) return fail(QSA_ERR_UNSUPPORTED, "too many rows");
  qsa_status st = check_device();
  if (st != QSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(qsa::launch_merge(n_part, rows, dv, o_parts, o_part_stride, lse_parts, lse_part_stride, o_out,
                                  o_out_bf16, lse_out, s),
                s, "qsa_lse_merge");
}

const char* qsa_status_string(qsa_status s) {
  switch (s) {
    case QSA_OK: return "ok";
    case QSA_ERR_ARG: return "invalid argument";
    case QSA_ERR_UNSUPPORTED: return "unsupported shape";
    case QSA_ERR_WORKSPACE: return "workspace too small";
    case QSA_ERR_LAUNCH: return "launch failed";
    case QSA_ERR_DEVICE: return "no usable gfx950 device";
  }
  return "unknown status";
}

const char* qsa_last_error(void) { return g_err; }

int32_t qsa_version(void) { return 100; }

}  // extern "C"
