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
//  * larger n, threshold lists (when a chunk's list can hold twice its
//    expected share): (0) one work-group per query reads 4096 of its scores
//    (256 evenly spread runs of 16) and takes as threshold theta the sample
//    key that about 1.75 x topk of all scores exceed; (1) one work-group per
//    chunk of 4096 scores lists every score above theta, in index order (one
//    prefix sum, no select), and counts the scores above and equal to theta;
//    (2) one work-group per query selects the top-k of the union. Every score
//    left out is at most theta, below every listed one, so when no list
//    overflowed and the union holds at least topk scores its top-k is the
//    exact top-k. If fewer scores exceed theta but enough equal it (ties,
//    e.g. exact zeros after a ReLU), one ordered pass over all n scores takes
//    the smallest indices among those equal to theta.
//  * larger n otherwise: (1) one work-group per chunk of 4096 scores
//    (256 threads x 16 registers) keeps the chunk's best L as a list in
//    ascending index order, with a bound: the best element it left out; L is
//    about twice a chunk's expected share of the top-k plus a margin. (2) One
//    work-group per query selects the top-k of the union of the lists (at
//    most 8192 entries, in registers; 256 threads when it holds at most
//    2048). With tau the topk-th best of the union, a chunk can hide a better
//    element only if its bound ranks above tau; if none does, the union's
//    top-k is the exact top-k. If the chunks only left out keys equal to the
//    union's topk-th key (ties), one ordered pass over all n scores picks the
//    smallest indices among them.
//  * Otherwise (rare: a chunk holding far more than its share, or a
//    threshold above too many scores) the query falls back to an exact
//    radix select over all n scores read from memory.
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

// Sum of x over the work-group (every thread gets it); uses rs.wg.
template <int NT>
__device__ __forceinline__ int block_sum(int x, RegSelLds<NT>& rs) {
  const int w = wave_incl_sum(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 63) rs.wg[threadIdx.x >> 6] = w;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int k = 0; k < NT / 64; k++) t += rs.wg[k];
  return t;
}

__device__ __forceinline__ int query_n(const TopkArgs& a, int i) {
  return clamp_ctx(a.q_ctx[i], a.max_ctx) / a.block;
}

// list of (query i, chunk c): p.list_len entries (key << 32 | index), 0 = empty
__device__ __forceinline__ uint64_t* list_of(const TopkArgs& a, const TopkPlan& p, int i, int c) {
  return reinterpret_cast<uint64_t*>(a.ws) + (size_t(i) * p.n_chunks + c) * p.list_len;
}
// per-chunk word: the bound (best element left out), or in filter mode the
// counts of scores above (low 32 bits) and equal to (high 32 bits) theta
__device__ __forceinline__ uint64_t* bound_of(const TopkArgs& a, const TopkPlan& p, int i) {
  return reinterpret_cast<uint64_t*>(a.ws) + size_t(a.nq) * p.n_chunks * p.list_len + size_t(i) * p.n_chunks;
}
// filter mode: the threshold key of query i
__device__ __forceinline__ uint32_t* theta_of(const TopkArgs& a, const TopkPlan& p, int i) {
  return reinterpret_cast<uint32_t*>(reinterpret_cast<uint64_t*>(a.ws) + size_t(a.nq) * p.n_chunks * (p.list_len + 1)) +
         i;
}
// filter mode: how many scores equal to theta query i takes (0: none, its
// selection is complete without them)
__device__ __forceinline__ int* ties_of(const TopkArgs& a, const TopkPlan& p, int i) {
  return reinterpret_cast<int*>(theta_of(a, p, 0) + a.nq) + i;
}

// Filter mode, step 0: the threshold of each chunked query. grid = nq, 256
// threads; thread t reads the 16 consecutive scores of run t, runs spread
// evenly over [0, n).
__global__ __launch_bounds__(256) void topk_sample(TopkArgs a, TopkPlan p) {
  __shared__ RegSelLds<kNTc> sh;
  const int i = blockIdx.x, tid = threadIdx.x;
  if (a.only && !a.only[i]) return;  // another path selected this query
  const int n = query_n(a, i);
  if (n <= a.topk || n <= p.direct_max) return;
  const float* sc = a.scores + int64_t(i) * a.ld;
  const int64_t start = int64_t(tid) * (n - kRc) / (kNTc - 1);
  uint32_t key[kRc];
#pragma unroll
  for (int r = 0; r < kRc; r++) key[r] = order_key(sc[start + r]);
  // rank of the sample that about 1.75 x topk of the n scores exceed
  int rank = int((7.0 * double(a.topk) * double(kChunk) + 4.0 * double(n) - 1.0) / (4.0 * double(n)));
  rank = rank < 1 ? 1 : (rank > kChunk ? kChunk : rank);
  uint32_t kstar;
  int need;
  regsel_threshold<kNTc, kRc>(key, rank, sh, kstar, need);
  if (tid == 0) *theta_of(a, p, i) = kstar;
}

// Chunk lists. grid = (n_chunks, nq), 256 threads.
__global__ __launch_bounds__(256) void topk_chunks(TopkArgs a, TopkPlan p) {
  __shared__ ChunkLds sh;
  const int i = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  if (a.only && !a.only[i]) return;  // another path selected this query
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

// Filter mode, step 1: the threshold lists. grid = (ceil(n_chunks / kCpw),
// nq), 256 threads; each work-group takes kCpw consecutive chunks of one
// query, all their scores loaded before any is used (thread t holds
// elements 16t .. 16t+15 of each chunk). A chunk's list holds every score
// above theta in index order (one prefix sum); its word counts the scores
// above (low half) and equal to (high half) theta.
constexpr int kCpw = 4;

__device__ __forceinline__ void load16(const float* p, bool vec, float (&v)[kRc]) {
  if (vec) {
#pragma unroll
    for (int q = 0; q < kRc / 4; q++) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(p + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; e++) v[4 * q + e] = x[e];
    }
  } else {
#pragma unroll
    for (int r = 0; r < kRc; r++) v[r] = p[r];
  }
}

__global__ __launch_bounds__(256) void topk_chunks_threshold(TopkArgs a, TopkPlan p) {
  __shared__ int wsum[kCpw][kNTc / 64];
  const int i = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (a.only && !a.only[i]) return;  // another path selected this query
  const int n = query_n(a, i);
  if (n <= a.topk || n <= p.direct_max) return;
  const int c0 = blockIdx.x * kCpw;
  if (int64_t(c0) * kChunk >= n) return;
  const float* row = a.scores + int64_t(i) * a.ld;
  // 16-byte loads when every thread's 16 scores are 16-byte aligned
  const bool vec = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
  float v[kCpw][kRc];
#pragma unroll
  for (int k = 0; k < kCpw; k++) {
    const int lo = (c0 + k) * kChunk + kRc * tid;
    if (lo + kRc <= n) {
      load16(row + lo, vec, v[k]);
    } else {
#pragma unroll
      for (int r = 0; r < kRc; r++) v[k][r] = lo + r < n ? row[lo + r] : 0.f;
    }
  }
  const uint32_t th = *theta_of(a, p, i);
  const int L = p.list_len;
#pragma unroll
  for (int k = 0; k < kCpw; k++) {
    const int c = c0 + k;
    const int lo = c * kChunk;
    if (lo >= n) break;  // uniform
    const int j0 = lo + kRc * tid;
    uint32_t key[kRc];
    int cg = 0, ce = 0;
#pragma unroll
    for (int r = 0; r < kRc; r++) {
      key[r] = j0 + r < n ? order_key(v[k][r]) : 0u;
      cg += key[r] > th ? 1 : 0;
      ce += key[r] == th ? 1 : 0;
    }
    const int pk = cg + (ce << 16);  // at most 4096 each
    const int ic = wave_incl_sum(pk);
    if (lane == 63) wsum[k][wave] = ic;
    __syncthreads();
    int off = ic - pk, tot = 0;
#pragma unroll
    for (int w = 0; w < kNTc / 64; w++) {
      const int x = wsum[k][w];
      if (w < wave) off += x;
      tot += x;
    }
    uint64_t* lst = list_of(a, p, i, c);
    int slot = off & 0xFFFF;
#pragma unroll
    for (int r = 0; r < kRc; r++) {
      if (key[r] > th) {
        if (slot < L) lst[slot] = (uint64_t(key[r]) << 32) | uint32_t(j0 + r);
        slot++;
      }
    }
    if (tid == 0) bound_of(a, p, i)[c] = uint64_t(uint32_t(tot & 0xFFFF)) | (uint64_t(uint32_t(tot >> 16)) << 32);
  }
}

// Filter mode, ties (after topk_final_threshold): for a query whose top-k
// holds every score above theta and the `need` smallest-index scores equal
// to it, chunk c writes its share in index order at its offset: the chunks
// before it contribute all their scores above theta and, in chunk order, the
// equal ones until `need` are taken. grid = (n_chunks, nq), 256 threads.
__global__ __launch_bounds__(kNTc) void topk_ties(TopkArgs a, TopkPlan p) {
  __shared__ int wsum[kNTc / 64];
  __shared__ int hdr[2];
  const int i = blockIdx.y, c = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (a.only && !a.only[i]) return;  // another path selected this query
  const int n = query_n(a, i);
  if (n <= a.topk || n <= p.final_threads * kRf) return;  // not a filter-path query
  const int need = *ties_of(a, p, i);
  if (need <= 0) return;
  const int lo = c * kChunk;
  if (lo >= n) return;
  const uint64_t* cnts = bound_of(a, p, i);
  if (tid == 0) {
    int off = 0, eq_before = 0;
    for (int j = 0; j < c; j++) {
      const int g = int(uint32_t(cnts[j]) & 0xFFFFu), e = int(uint32_t(cnts[j] >> 32));
      const int take = need - eq_before < e ? (need - eq_before > 0 ? need - eq_before : 0) : e;
      off += g + take;
      eq_before += e;
    }
    const int e_c = int(uint32_t(cnts[c] >> 32));
    const int quota = need - eq_before < e_c ? (need - eq_before > 0 ? need - eq_before : 0) : e_c;
    hdr[0] = off;
    hdr[1] = quota;
  }
  __syncthreads();
  const int off = hdr[0], quota = hdr[1];
  const uint32_t th = *theta_of(a, p, i);
  const float* row = a.scores + int64_t(i) * a.ld;
  const int j0 = lo + kRc * tid;
  uint32_t key[kRc];
  int ne = 0;
#pragma unroll
  for (int r = 0; r < kRc; r++) {
    key[r] = j0 + r < n ? order_key(row[j0 + r]) : 0u;
    ne += key[r] == th ? 1 : 0;
  }
  // rank of the lane's first equal score among the chunk's equal scores
  const int ie = wave_incl_sum(ne);
  if (lane == 63) wsum[wave] = ie;
  __syncthreads();
  int e_rank = ie - ne;
#pragma unroll
  for (int w = 0; w < kNTc / 64; w++) e_rank += w < wave ? wsum[w] : 0;
  __syncthreads();
  bool take[kRc];
  int ns = 0;
#pragma unroll
  for (int r = 0; r < kRc; r++) {
    const bool eqk = key[r] == th;
    take[r] = key[r] > th || (eqk && e_rank < quota);
    e_rank += eqk ? 1 : 0;
    ns += take[r] ? 1 : 0;
  }
  const int is = wave_incl_sum(ns);
  if (lane == 63) wsum[wave] = is;
  __syncthreads();
  int pos = off + is - ns;
#pragma unroll
  for (int w = 0; w < kNTc / 64; w++) pos += w < wave ? wsum[w] : 0;
  int* sel = a.sel + int64_t(i) * a.topk;
#pragma unroll
  for (int r = 0; r < kRc; r++)
    if (take[r]) {
      if (pos < a.topk) sel[pos] = j0 + r;
      pos++;
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
  if (a.only && !a.only[i]) return;  // another path selected this query
  const int n = query_n(a, i);
  const int topk = a.topk;
  int* sel = a.sel + int64_t(i) * topk;
  if (n <= topk) {
    for (int j = tid; j < topk; j += kNTf) sel[j] = j < n ? j : -1;
    if (tid == 0) a.n_sel[i] = n;
    return;
  }
  const bool direct = n <= kCap;
  if (p.filter && !direct) return;  // topk_final_threshold selects these
  if (tid == 0) a.n_sel[i] = topk;
  const float* sc = a.scores + int64_t(i) * a.ld;
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

// Filter mode, step 2: selection per chunked query from the threshold lists
// (see the file comment). grid = nq, NT threads; NT * kRf covers the union.
template <int NT>
__global__ __launch_bounds__(NT) void topk_final_threshold(TopkArgs a, TopkPlan p) {
  constexpr int kNTf = NT;
  constexpr int kCap = NT * kRf;
  __shared__ FinalLds<NT> sh;
  const int i = blockIdx.x, tid = threadIdx.x;
  if (a.only && !a.only[i]) return;  // another path selected this query
  const int n = query_n(a, i);
  const int topk = a.topk;
  if (n <= topk || n <= kCap) return;  // topk_final selects these
  int* sel = a.sel + int64_t(i) * topk;
  if (tid == 0) a.n_sel[i] = topk;
  const float* sc = a.scores + int64_t(i) * a.ld;
  if (p.stream_only) {  // exact select over every score, read from memory
    auto gk = [sc](int j) { return order_key(sc[j]); };
    uint32_t kstar;
    int need;
    stream_select<kNTf>(gk, n, topk, sh.st, kstar, need);
    stream_compact<kNTf>(gk, n, kstar, need, sh.st, [&](int pos, int j) { sel[pos] = j; });
    return;
  }
  const int L = p.list_len;
  const int nch = (n + kChunk - 1) / kChunk;
  const uint32_t th = *theta_of(a, p, i);
  const uint64_t* lists = list_of(a, p, i, 0);
  const uint64_t* cnts = bound_of(a, p, i);
  if (tid == 0) *ties_of(a, p, i) = 0;
  // counts above / equal to theta: thread t < nch holds chunk t's
  const uint64_t cw = tid < nch ? cnts[tid] : 0ull;
  const int gt = int(uint32_t(cw)), eq = int(uint32_t(cw >> 32));
  const bool overflow = __syncthreads_or(gt > L);
  const int n_gt = block_sum<kNTf>(gt, sh.rs);
  if (!overflow && nch <= p.n_chunks && int64_t(nch) * L <= kCap && n_gt >= topk) {
    // union entry e = chunk e / L, slot e % L (ascending index order); slots
    // past a chunk's count are empty
    uint32_t key[kRf];
    int idx[kRf];
#pragma unroll
    for (int r = 0; r < kRf; r++) {
      const int e = kRf * tid + r;
      const int ch = e / L, slot = e % L;
      const bool in = ch < nch && slot < int(uint32_t(cnts[ch]));
      const uint64_t v = in ? lists[e] : 0ull;
      key[r] = uint32_t(v >> 32);
      idx[r] = int(uint32_t(v));
    }
    uint32_t kstar;
    int need;
    regsel_threshold<kNTf, kRf>(key, topk, sh.rs, kstar, need);
    int pos[kRf];
    regsel_positions<kNTf, kRf>(key, idx, kstar, need, sh.rs, pos);
#pragma unroll
    for (int r = 0; r < kRf; r++)
      if (pos[r] >= 0) sel[pos[r]] = idx[r];
    return;
  }
  auto gkey_at = [sc](int j) { return order_key(sc[j]); };
  int* const out = sel;
  auto emit = [out](int pos, int j) { out[pos] = j; };
  const int n_eq = block_sum<kNTf>(eq, sh.rs);
  if (n_gt < topk && topk <= n_gt + n_eq) {
    // every score above theta, then the smallest indices among those equal
    // to it: written chunk by chunk by topk_ties (the counts fix each
    // chunk's share and offset)
    if (tid == 0) *ties_of(a, p, i) = topk - n_gt;
    return;
  }
  // exact select over every score, read from memory
  uint32_t kstar;
  int need;
  stream_select<kNTf>(gkey_at, n, topk, sh.st, kstar, need);
  stream_compact<kNTf>(gkey_at, n, kstar, need, sh.st, emit);
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
  const int64_t nch = (nmax + kChunk - 1) / kChunk;
  // threshold lists: a chunk's list holds twice its expected count above
  // the sampled threshold (1.75 x its share of the top-k) plus a margin,
  // within the chunk and the final union
  {
    const double expect = 1.75 * double(kChunk) * double(topk) / double(nmax);
    const int64_t cap = (int64_t(2.0 * expect) + 32 + 15) / 16 * 16;
    if (cap <= kChunk && nch * cap <= kUnionMax) {
      p.chunked = true;
      p.filter = true;
      p.chunk = kChunk;
      p.n_chunks = int(nch);
      p.list_len = int(cap);
      if (nch * cap <= kSmallMax) {
        p.final_threads = 256;
        p.direct_max = kSmallMax;
      }
      // lists, one word per chunk, one threshold per query
      p.ws_bytes = size_t(nq) * size_t(nch) * (size_t(cap) + 1) * 8 + size_t(nq) * 8;  // + theta, ties
      return p;
    }
  }
  // list length: twice a chunk's expected share of the top-k plus a margin,
  // rounded up to 16, within the chunk and within the final union
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
  if (p.stream_only) {
    if (!a.only) return hipErrorInvalidValue;
    hipLaunchKernelGGL(topk_final_threshold<1024>, dim3(unsigned(a.nq)), dim3(1024), 0, s, a, p);
    return hipGetLastError();
  }
  if (p.filter) {
    hipLaunchKernelGGL(topk_sample, dim3(unsigned(a.nq)), dim3(kNTc), 0, s, a, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.filter) {
    hipLaunchKernelGGL(topk_chunks_threshold, dim3(unsigned((p.n_chunks + kCpw - 1) / kCpw), unsigned(a.nq)),
                       dim3(kNTc), 0, s, a, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else if (p.chunked) {
    hipLaunchKernelGGL(topk_chunks, dim3(unsigned(p.n_chunks), unsigned(a.nq)), dim3(kNTc), 0, s, a, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.filter) {
    if (p.final_threads == 256)
      hipLaunchKernelGGL(topk_final_threshold<256>, dim3(unsigned(a.nq)), dim3(256), 0, s, a, p);
    else
      hipLaunchKernelGGL(topk_final_threshold<1024>, dim3(unsigned(a.nq)), dim3(1024), 0, s, a, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_ties, dim3(unsigned(p.n_chunks), unsigned(a.nq)), dim3(kNTc), 0, s, a, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // direct queries (and, outside filter mode, every query)
  if (p.final_threads == 256)
    hipLaunchKernelGGL(topk_final<256>, dim3(unsigned(a.nq)), dim3(256), 0, s, a, p);
  else
    hipLaunchKernelGGL(topk_final<1024>, dim3(unsigned(a.nq)), dim3(1024), 0, s, a, p);
  return hipGetLastError();
}

}  // namespace qsa
