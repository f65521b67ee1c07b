// A3: the blocks (or tokens) each query attends.
// "3090x3で 314 万コンテキスト", section "なぜ": the indexer keeps a fixed
// budget of topk blocks; with at most topk candidates the whole history is
// read. "125B MoE を 3090 3 枚で運用する vLLM 最適化編", section 3.3: the
// top-k there packs an order-preserving integer image of the value with the
// id so that equal values go to the smaller id. Here every score becomes an
// order-preserving 32-bit key; ranking is (key descending, index ascending),
// so the selection is unique.
//
// Paths (chosen per query from its candidate count n):
//  * n <= topk: every candidate.
//  * n <= 8192 (2048 when the lists of the larger queries are short): one
//    work-group holds all keys in registers (8 per thread) and selects directly (radix threshold over LDS histograms that
//    start below the keys' common prefix, then ordered positions).
//  * larger n: (1) one work-group per chunk of 4096 scores (256 threads x 16
//    registers) keeps the chunk's best L as a list in ascending index order,
//    with a bound: the best element it left out; L is about twice a chunk's
//    expected share of the top-k plus a margin. (2) One work-group per query
//    selects the top-k of the union of the lists (at most 8192 entries, in
//    registers; 256 threads when it holds at most 2048). With tau the topk-th best of the union, a chunk can hide a
//    better element only if its bound ranks above tau; if none does, the
//    union's top-k is the exact top-k. If the chunks only left out keys equal
//    to the union's topk-th key (ties, e.g. many scores of exactly zero), one
//    ordered pass over all n scores picks the smallest indices among them.
//    Otherwise (rare: a chunk holding far more than its share) the query
//    falls back to an exact radix select over all n scores read from memory.
// Every path writes the same, exact answer in ascending index order.
#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace qsa {
namespace {

constexpr int kNTc = 256, kRc = 16, kChunk = kNTc * kRc;  // chunk phase: 4096 scores
constexpr int kRf = 8;                                   // final phase: 8 entries per thread
constexpr int kUnionMax = 1024 * kRf;                    // ... of at most 1024 threads
constexpr int kSmallMax = 256 * kRf;                     // 256 threads suffice up to here

struct ChunkLds {
  RegSelLds<kNTc> rs;
  uint64_t wb[kNTc / 64];
};
template <int NT>
struct FinalLds {
  RegSelLds<NT> rs;
  StreamLds st;
};

__device__ __forceinline__ int query_n(const TopkArgs& a, int i) {
  return clamp_ctx(a.q_ctx[i], a.max_ctx) / a.block;
}

// list of (query i, chunk c): p.list_len entries (key << 32 | index), 0 = empty
__device__ __forceinline__ uint64_t* list_of(const TopkArgs& a, const TopkPlan& p, int i, int c) {
  return reinterpret_cast<uint64_t*>(a.ws) + (size_t(i) * p.n_chunks + c) * p.list_len;
}
__device__ __forceinline__ uint64_t* bound_of(const TopkArgs& a, const TopkPlan& p, int i) {
  return reinterpret_cast<uint64_t*>(a.ws) + size_t(a.nq) * p.n_chunks * p.list_len + size_t(i) * p.n_chunks;
}

// Chunk lists. grid = (n_chunks, nq), 256 threads.
__global__ __launch_bounds__(256) void topk_chunks(TopkArgs a, TopkPlan p) {
  __shared__ ChunkLds sh;
  const int i = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const int n = query_n(a, i);
  if (n <= a.topk || n <= p.direct_max) return;  // the final kernel handles these alone
  const int lo = c * kChunk;
  if (lo >= n) return;
  const int m = n - lo < kChunk ? n - lo : kChunk;
  const float* sc = a.scores + int64_t(i) * a.ld + lo;
  uint64_t* lst = list_of(a, p, i, c);
  const int L = p.list_len;
  // thread t holds chunk elements 16t .. 16t+15: element order is index order
  uint32_t key[kRc];
  int idx[kRc];
#pragma unroll
  for (int r = 0; r < kRc; r++) {
    const int j = kRc * tid + r;
    key[r] = j < m ? order_key(sc[j]) : 0u;
    idx[r] = lo + j;
  }
  if (m <= L) {  // the whole chunk is its list
#pragma unroll
    for (int r = 0; r < kRc; r++) {
      const int j = kRc * tid + r;
      if (j < L) lst[j] = j < m ? (uint64_t(key[r]) << 32) | uint32_t(idx[r]) : 0ull;
    }
    if (tid == 0) bound_of(a, p, i)[c] = 0ull;
    return;
  }
  uint32_t kstar;
  int need;
  regsel_threshold<kNTc, kRc>(key, L, sh.rs, kstar, need);
  int pos[kRc];
  regsel_positions<kNTc, kRc>(key, idx, kstar, need, sh.rs, pos);
  uint64_t b = 0ull;  // best element left out
#pragma unroll
  for (int r = 0; r < kRc; r++) {
    if (pos[r] >= 0)
      lst[pos[r]] = (uint64_t(key[r]) << 32) | uint32_t(idx[r]);
    else if (key[r] != 0u) {
      const uint64_t k64 = rank64(key[r], idx[r]);
      b = k64 > b ? k64 : b;
    }
  }
  b = wave_max_u64(b);
  if ((tid & 63) == 0) sh.wb[tid >> 6] = b;
  __syncthreads();
  if (tid == 0) {
    uint64_t bb = 0ull;
#pragma unroll
    for (int w = 0; w < kNTc / 64; w++) bb = sh.wb[w] > bb ? sh.wb[w] : bb;
    bound_of(a, p, i)[c] = bb;
  }
}

// Selection per query. grid = nq, NT threads; NT * kRf covers the union (or
// every candidate of a directly selected query).
template <int NT>
__global__ __launch_bounds__(NT) void topk_final(TopkArgs a, TopkPlan p) {
  constexpr int kNTf = NT;
  constexpr int kCap = NT * kRf;
  __shared__ FinalLds<NT> sh;
  const int i = blockIdx.x, tid = threadIdx.x;
  const int n = query_n(a, i);
  const int topk = a.topk;
  int* sel = a.sel + int64_t(i) * topk;
  if (n <= topk) {
    for (int j = tid; j < topk; j += kNTf) sel[j] = j < n ? j : -1;
    if (tid == 0) a.n_sel[i] = n;
    return;
  }
  if (tid == 0) a.n_sel[i] = topk;
  const float* sc = a.scores + int64_t(i) * a.ld;
  const bool direct = n <= kCap;
  bool usable = true;
  uint32_t key[kRf];
  int idx[kRf];
  uint64_t my_bound = 0ull;
  if (direct) {
#pragma unroll
    for (int r = 0; r < kRf; r++) {
      const int j = kRf * tid + r;
      key[r] = j < n ? order_key(sc[j]) : 0u;
      idx[r] = j;
    }
  } else {
    // union of the chunk lists: entry e = chunk e / L, slot e % L (ascending index order)
    const int L = p.list_len;
    const int nch = (n + kChunk - 1) / kChunk;
    const int m_last = n - (nch - 1) * kChunk;
    const int filled = (nch - 1) * (kChunk < L ? kChunk : L) + (m_last < L ? m_last : L);
    usable = p.chunked && nch <= p.n_chunks && int64_t(nch) * L <= kCap && filled >= topk;
    const uint64_t* lists = list_of(a, p, i, 0);
#pragma unroll
    for (int r = 0; r < kRf; r++) {
      const int e = kRf * tid + r;
      const uint64_t v = usable && e < nch * L ? lists[e] : 0ull;
      key[r] = uint32_t(v >> 32);
      idx[r] = int(uint32_t(v));
    }
    if (usable && tid < nch) my_bound = bound_of(a, p, i)[tid];
  }
  if (usable) {
    uint32_t kstar;
    int need;
    regsel_threshold<kNTf, kRf>(key, topk, sh.rs, kstar, need);
    int pos[kRf];
    regsel_positions<kNTf, kRf>(key, idx, kstar, need, sh.rs, pos);
    bool ok = true, ties_only = false;
    if (!direct) {
      const uint64_t tau = rank64(kstar, sh.rs.tau_val);
      ok = !__syncthreads_or(my_bound > tau);
      // if no chunk left out a key above kstar, the lists hold every key
      // above it, kstar is also the global topk-th key, and only the choice
      // among keys equal to kstar (the smallest indices) needs every score
      if (!ok) ties_only = !__syncthreads_or(uint32_t(my_bound >> 32) > kstar);
    }
    if (ok) {
#pragma unroll
      for (int r = 0; r < kRf; r++)
        if (pos[r] >= 0) sel[pos[r]] = idx[r];
      return;
    }
    if (ties_only) {
      auto gkey_at = [&](int j) { return order_key(sc[j]); };
      stream_compact<kNTf>(gkey_at, n, kstar, need, sh.st, [&](int pos, int j) { sel[pos] = j; });
      return;
    }
  }
  // exact select over every score, read from memory
  auto gkey_at = [&](int j) { return order_key(sc[j]); };
  uint32_t kstar;
  int need;
  stream_select<kNTf>(gkey_at, n, topk, sh.st, kstar, need);
  stream_compact<kNTf>(gkey_at, n, kstar, need, sh.st, [&](int pos, int j) { sel[pos] = j; });
}

}  // namespace

TopkPlan plan_topk(int nq, int max_ctx, int block, int topk) {
  TopkPlan p{};
  const int64_t nmax = int64_t(max_ctx) / block;
  p.final_threads = 1024;
  p.direct_max = kUnionMax;
  if (nmax <= kUnionMax || nmax <= topk) {
    p.chunked = false;
    if (nmax <= kSmallMax) {
      p.final_threads = 256;
      p.direct_max = kSmallMax;
    }
    return p;
  }
  // list length: twice a chunk's expected share of the top-k plus a margin,
  // rounded up to 16, within the chunk and within the final union
  const int64_t nch = (nmax + kChunk - 1) / kChunk;
  const double mu = double(kChunk) * double(topk) / double(nmax);
  int64_t L = (int64_t(2.0 * mu) + 48 + 15) / 16 * 16;
  if (L > kChunk) L = kChunk;
  if (nch * L > kUnionMax) L = kUnionMax / nch;
  p.chunked = L >= 1;
  if (nch * L <= kSmallMax) {
    p.final_threads = 256;
    p.direct_max = kSmallMax;
  }
  p.chunk = kChunk;
  p.n_chunks = int(nch);
  p.list_len = int(L < 1 ? 1 : L);
  p.ws_bytes = p.chunked ? size_t(nq) * size_t(nch) * (size_t(p.list_len) + 1) * 8 : 0;
  return p;
}

hipError_t launch_topk(const TopkArgs& a, const TopkPlan& p, hipStream_t s) {
  if (a.nq <= 0) return hipSuccess;
  if (p.chunked) {
    hipLaunchKernelGGL(topk_chunks, dim3(unsigned(p.n_chunks), unsigned(a.nq)), dim3(kNTc), 0, s, a, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.final_threads == 256)
    hipLaunchKernelGGL(topk_final<256>, dim3(unsigned(a.nq)), dim3(256), 0, s, a, p);
  else
    hipLaunchKernelGGL(topk_final<1024>, dim3(unsigned(a.nq)), dim3(1024), 0, s, a, p);
  return hipGetLastError();
}

}  // namespace qsa
