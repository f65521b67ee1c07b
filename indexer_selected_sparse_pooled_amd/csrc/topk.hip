// A3: the blocks each query attends.
// "3090x3で 314 万コンテキスト", section "なぜ": the indexer keeps a fixed
// budget of topk blocks; with at most topk complete blocks the whole history
// is read. "125B MoE を 3090 3 枚で運用する vLLM 最適化編", section 3.3: the
// top-k there packs an order-preserving integer image of the value with the
// id so that equal values go to the smaller id. Here every score becomes an
// order-preserving 32-bit key; ranking is (key descending, index ascending).
//
// Exact selection, three paths:
//  * n <= topk: every block.
//  * n <= kLdsMax: one work-group per query holds all keys in LDS, finds the
//    topk-th largest key with four 8-bit radix passes, then writes the
//    selection in ascending index order with a ballot-based ordered
//    compaction (the first `need` keys equal to the threshold win).
//  * larger n: (1) one work-group per chunk of C scores keeps its local top-L
//    (same LDS select, L = 64); (2) one work-group per query takes the
//    union U of the lists (ascending index order by construction), finds
//    tau = the topk-th largest of U, and checks every chunk whose list might
//    be incomplete above tau (its smallest listed element ranks >= tau). If
//    none is, the global top-k is exactly {x in U : x ranks >= tau}.
//    Otherwise it falls back to the radix select over all n scores read
//    from global memory. Both give the same, exact answer.
#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace qsa {
namespace {

constexpr int kLdsMax = 32768;  // scores a single work-group keeps in LDS
constexpr int kListLen = 64;    // candidates per chunk
constexpr int kUnionCap = 16384;

struct Scratch {
  StreamLds st;
  int flag;
  int tau_idx;
};

__device__ __forceinline__ int query_n(const TopkArgs& a, int i) {
  return clamp_ctx(a.q_ctx[i], a.max_ctx) / a.block;
}

struct Ws {
  int* list_idx;       // [nq][n_chunks][L]
  uint32_t* list_key;  // [nq][n_chunks][L]
};
__device__ __forceinline__ Ws ws_of(const TopkArgs& a, const TopkPlan& p) {
  Ws w;
  w.list_idx = reinterpret_cast<int*>(a.ws);
  w.list_key = reinterpret_cast<uint32_t*>(w.list_idx + size_t(a.nq) * p.n_chunks * p.list_len);
  return w;
}

// Per-chunk local top-L for queries with n > kLdsMax. grid = (n_chunks, nq).
__global__ __launch_bounds__(256) void topk_local(TopkArgs a, TopkPlan p) {
  extern __shared__ uint32_t lkeys[];
  __shared__ Scratch sh;
  const int i = blockIdx.y, w = blockIdx.x;
  const int n = query_n(a, i);
  if (n <= kLdsMax) return;
  const int lo = w * p.chunk;
  if (lo >= n) return;
  const int m = min(n - lo, p.chunk);
  const float* sc = a.scores + int64_t(i) * a.ld + lo;
  for (int j = threadIdx.x; j < m; j += 256) lkeys[j] = order_key(sc[j]);
  __syncthreads();
  Ws ws = ws_of(a, p);
  const size_t base = (size_t(i) * p.n_chunks + w) * p.list_len;
  auto key_at = [&](int j) { return lkeys[j]; };
  if (m <= p.list_len) {
    for (int j = threadIdx.x; j < m; j += 256) {
      ws.list_idx[base + j] = lo + j;
      ws.list_key[base + j] = lkeys[j];
    }
    return;
  }
  uint32_t kstar;
  int need;
  stream_select<256>(key_at, m, p.list_len, sh.st, kstar, need);
  stream_compact<256>(key_at, m, kstar, need, sh.st, [&](int pos, int j) {
    ws.list_idx[base + pos] = lo + j;
    ws.list_key[base + pos] = lkeys[j];
  });
}

// Selection per query. grid = nq, block = 1024.
__global__ __launch_bounds__(1024) void topk_final(TopkArgs a, TopkPlan p) {
  extern __shared__ uint32_t dyn[];
  __shared__ Scratch sh;
  const int i = blockIdx.x;
  const int n = query_n(a, i);
  const int topk = a.topk;
  int* sel = a.sel + int64_t(i) * topk;
  if (n <= topk) {
    for (int j = threadIdx.x; j < topk; j += 1024) sel[j] = j < n ? j : -1;
    if (threadIdx.x == 0) a.n_sel[i] = n;
    return;
  }
  if (threadIdx.x == 0) a.n_sel[i] = topk;
  const float* sc = a.scores + int64_t(i) * a.ld;
  if (n <= kLdsMax) {
    for (int j = threadIdx.x; j < n; j += 1024) dyn[j] = order_key(sc[j]);
    __syncthreads();
    auto key_at = [&](int j) { return dyn[j]; };
    uint32_t kstar;
    int need;
    stream_select<1024>(key_at, n, topk, sh.st, kstar, need);
    stream_compact<1024>(key_at, n, kstar, need, sh.st, [&](int pos, int j) { sel[pos] = j; });
    return;
  }
  // union of the chunk lists, ascending index order
  const int nch = (n + p.chunk - 1) / p.chunk;
  const int last_m = n - (nch - 1) * p.chunk;
  const int u = (nch - 1) * p.list_len + min(last_m, p.list_len);
  uint32_t* ukey = dyn;
  int* uidx = reinterpret_cast<int*>(dyn + kUnionCap);
  Ws ws = ws_of(a, p);
  const size_t base = size_t(i) * p.n_chunks * p.list_len;
  for (int j = threadIdx.x; j < u; j += 1024) {
    ukey[j] = ws.list_key[base + j];
    uidx[j] = ws.list_idx[base + j];
  }
  if (threadIdx.x == 0) sh.flag = 0;
  __syncthreads();
  uint32_t kstar;
  int need;
  auto gkey_at = [&](int j) { return order_key(sc[j]); };
  if (u < topk) {
    // too few listed candidates to bound the threshold: select over everything
    stream_select<1024>(gkey_at, n, topk, sh.st, kstar, need);
    stream_compact<1024>(gkey_at, n, kstar, need, sh.st, [&](int pos, int j) { sel[pos] = j; });
    return;
  }
  auto ukey_at = [&](int j) { return ukey[j]; };
  stream_select<1024>(ukey_at, u, topk, sh.st, kstar, need);
  const int tau_idx = stream_nth_equal<1024>(ukey_at, u, kstar, need, sh.st, &sh.tau_idx);
  // a full list whose smallest element (lowest key, then highest index)
  // ranks at or above tau may have left out elements that also do
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int c = wave; c < nch; c += 16) {
    const int m = c == nch - 1 ? last_m : p.chunk;
    if (m <= p.list_len) continue;
    const int e = c * p.list_len + lane;  // list_len == 64 == wave size
    const uint64_t k64 = (uint64_t(ukey[e]) << 32) | uint32_t(~uint32_t(uidx[e]));
    uint64_t mn = k64;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const uint64_t o = __shfl_xor(mn, d);
      mn = o < mn ? o : mn;
    }
    const uint32_t mkey = uint32_t(mn >> 32);
    const int midx = int(~uint32_t(mn));
    if (lane == 0 && (mkey > kstar || (mkey == kstar && midx <= tau_idx))) sh.flag = 1;
  }
  __syncthreads();
  if (!sh.flag) {
    stream_compact<1024>(ukey_at, u, kstar, need, sh.st, [&](int pos, int j) { sel[pos] = uidx[j]; });
    return;
  }
  // fallback: exact select over every score, read from global memory
  stream_select<1024>(gkey_at, n, topk, sh.st, kstar, need);
  stream_compact<1024>(gkey_at, n, kstar, need, sh.st, [&](int pos, int j) { sel[pos] = j; });
}

}  // namespace

TopkPlan plan_topk(int nq, int max_ctx, int block, int topk) {
  TopkPlan p{};
  const int64_t nmax = int64_t(max_ctx) / block;
  p.list_len = kListLen;
  if (nmax <= kLdsMax) {
    p.chunked = false;
    p.chunk = 0;
    p.n_chunks = 0;
    p.ws_bytes = 0;
    return p;
  }
  // Chunk size: at most a quarter of a list expected above the global
  // threshold per chunk (chunk <= 16 * n / topk), the union of all lists
  // within kUnionCap, and the chunk within one work-group's LDS.
  int64_t c = 256;
  while (c * 2 <= 16 * nmax / topk && c < 4096) c *= 2;
  while ((nmax + c - 1) / c * kListLen > kUnionCap) c *= 2;
  p.chunked = true;
  p.chunk = int(c);
  p.n_chunks = int((nmax + c - 1) / c);
  p.ws_bytes = size_t(nq) * p.n_chunks * p.list_len * 8;
  return p;
}

hipError_t launch_topk(const TopkArgs& a, const TopkPlan& p, hipStream_t s) {
  if (a.nq <= 0) return hipSuccess;
  const int64_t nmax = int64_t(a.max_ctx) / a.block;
  if (p.chunked) {
    if (size_t(p.chunk) * 4 > 65536) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_local),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, p.chunk * 4);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(topk_local, dim3(unsigned(p.n_chunks), unsigned(a.nq)), dim3(256),
                       size_t(p.chunk) * 4, s, a, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  size_t lds = 0;
  if (p.chunked)
    lds = size_t(kUnionCap) * 8;
  else
    lds = size_t(nmax > 0 ? nmax : 1) * 4;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_final),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(topk_final, dim3(unsigned(a.nq)), dim3(1024), lds, s, a, p);
  return hipGetLastError();
}

}  // namespace qsa
