// A2 + A3 for a prefill chunk of the token-level indexer, without
// materialising the scores.
// "GLM-5.3 最適化 第2部", section "PCP": the indexer scores every earlier token
// of every chunk query (its cost grows with the square of the context); its
// top-2048 feed the sparse MLA. Writing every score (4 bytes each) and
// reading them back to select would move 2 x 1 GiB at the 2048-query,
// 131,072-token chunk, more than the MFMA work of the scores themselves, so
// the selection is folded into the score pass:
//   1. sample: the score GEMM over every s-th key (s = ceil(keys / 4096));
//   2. threshold: per query, the sample element ranked about 1.75 x topk /
//      (keys / s) in (key descending, index ascending) order, as a 64-bit
//      (order key, index) pair;
//   3. lists: the full score GEMM keeps, per query, every score ranked at
//      least as high as the threshold (unordered: a query row's lane group
//      stages its entries in LDS and reserves list slots with one atomic per
//      1024-key span);
//   4. select: per query the top-k of its list, written in ascending index
//      order through an LDS bitmap of the candidates.
// Every score left out ranks below the threshold and every listed one at or
// above it, so when a list holds at least topk entries and did not overflow,
// its top-k is the exact top-k (ties included: the threshold carries an
// index). A query whose list came up short or overflowed is flagged; the
// regular path (full scores for the flagged queries only, then an exact
// select over them) then selects it, so every query gets the exact answer.
#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace qsa {
namespace {

constexpr int kSampleMax = 4096;  // sample scores per query
constexpr int kCap = 8192;        // list capacity per query
constexpr int kFinalNT = 1024, kFinalR = kCap / kFinalNT;
constexpr int kMaxKeys = 262144;  // keys per query this path handles (bitmap of 32 KiB)
constexpr int kSampleNT = 256, kSampleR = kSampleMax / kSampleNT;

__device__ __forceinline__ int keys_of(const ScoreArgs& a, int i) {
  return clamp_ctx(a.q_ctx[i], a.max_ctx) / a.block;
}

// Step 2, one work-group per query: its threshold (or keep-all / keep-none),
// and its list counter and flag cleared.
__global__ __launch_bounds__(kSampleNT) void select_threshold(ScoreArgs a, const float* samp, int64_t samp_ld,
                                                              int64_t step, int topk, uint32_t* fail) {
  __shared__ RegSelLds<kSampleNT> sh;
  const int i = blockIdx.x, tid = threadIdx.x;
  const int n = keys_of(a, i);
  uint64_t* theta = const_cast<uint64_t*>(a.theta);
  if (tid == 0) {
    a.counts[int64_t(i) * kCountStride] = 0u;
    fail[i] = 0u;
  }
  if (n <= topk) {  // every key is selected; no list
    if (tid == 0) theta[i] = ~0ull;
    return;
  }
  if (n <= kCap) {  // the list can hold every key
    if (tid == 0) theta[i] = 0ull;
    return;
  }
  const int m = int((int64_t(n) + step - 1) / step);  // sample elements of this query
  uint32_t key[kSampleR];
  int val[kSampleR];
#pragma unroll
  for (int r = 0; r < kSampleR; r++) {
    const int j = tid * kSampleR + r;
    key[r] = j < m ? order_key(samp[int64_t(i) * samp_ld + j]) : 0u;
    val[r] = j;
  }
  int rank = int((7.0 * double(topk) * double(m) + 4.0 * double(n) - 1.0) / (4.0 * double(n)));
  rank = rank < 1 ? 1 : (rank > m ? m : rank);
  uint32_t kstar;
  int need;
  regsel_threshold<kSampleNT, kSampleR>(key, rank, sh, kstar, need);
  int pos[kSampleR];
  regsel_positions<kSampleNT, kSampleR>(key, val, kstar, need, sh, pos);
  if (tid == 0) theta[i] = (uint64_t(kstar) << 32) | uint64_t(int64_t(sh.tau_val) * step);
}

struct FinalLds {
  RegSelLds<kFinalNT> rs;
  uint32_t bits[kMaxKeys / 32];
  int wsum[kFinalNT / 64];
};

// Exclusive prefix sum of x over the work-group, and the total.
__device__ __forceinline__ int block_excl_sum(int x, int* wsum, int& total) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int inc = wave_incl_sum(x);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kFinalNT / 64; w++) {
    before += w < wave ? wsum[w] : 0;
    total += wsum[w];
  }
  return before + inc - x;
}

// Step 4, one work-group per query.
__global__ __launch_bounds__(kFinalNT) void select_lists(ScoreArgs a, int topk, int* sel, int* n_sel,
                                                         uint32_t* fail) {
  __shared__ FinalLds sh;
  const int i = blockIdx.x, tid = threadIdx.x;
  const int n = keys_of(a, i);
  int* out = sel + int64_t(i) * topk;
  if (n <= topk) {
    for (int j = tid; j < topk; j += kFinalNT) out[j] = j < n ? j : -1;
    if (tid == 0) n_sel[i] = n > 0 ? n : 0;
    return;
  }
  const uint32_t c = a.counts[int64_t(i) * kCountStride];
  if (c < uint32_t(topk) || c > uint32_t(kCap)) {
    if (tid == 0) fail[i] = 1u;
    return;
  }
  const uint64_t* lst = a.lists + int64_t(i) * a.list_cap;
  uint32_t key[kFinalR];
  int idx[kFinalR];
#pragma unroll
  for (int r = 0; r < kFinalR; r++) {
    const uint32_t j = uint32_t(r * kFinalNT + tid);
    const uint64_t e = j < c ? lst[j] : 0ull;  // score bits << 32 | index
    key[r] = j < c ? order_key(__uint_as_float(uint32_t(e >> 32))) : 0u;
    idx[r] = int(uint32_t(e));
  }
  uint32_t kstar;
  int need;
  regsel_threshold<kFinalNT, kFinalR>(key, topk, sh.rs, kstar, need);
  int eq = 0;
#pragma unroll
  for (int r = 0; r < kFinalR; r++) eq += (key[r] == kstar && key[r] != 0u) ? 1 : 0;
  int eq_total;
  block_excl_sum(eq, sh.wsum, eq_total);
  // ties at kstar: the `need` smallest indices among them
  uint32_t istar = 0u;
  if (eq_total > need) {
    uint32_t key2[kFinalR];
#pragma unroll
    for (int r = 0; r < kFinalR; r++) key2[r] = (key[r] == kstar && key[r] != 0u) ? ~uint32_t(idx[r]) : 0u;
    int need2;
    __syncthreads();
    regsel_threshold<kFinalNT, kFinalR>(key2, need, sh.rs, istar, need2);
  }
  const int nw = (n + 31) / 32;
  for (int w = tid; w < nw; w += kFinalNT) sh.bits[w] = 0u;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kFinalR; r++) {
    const bool take = key[r] != 0u && (key[r] > kstar || (key[r] == kstar && ~uint32_t(idx[r]) >= istar));
    if (take) atomicOr(&sh.bits[idx[r] >> 5], 1u << (idx[r] & 31));
  }
  __syncthreads();
  // ascending compaction: thread t owns words [t * per, (t + 1) * per)
  const int per = (nw + kFinalNT - 1) / kFinalNT;
  const int w0 = tid * per, w1 = w0 + per < nw ? w0 + per : nw;
  int cnt = 0;
  for (int w = w0; w < w1; w++) cnt += __popc(sh.bits[w]);
  int total;
  int p = block_excl_sum(cnt, sh.wsum, total);
  for (int w = w0; w < w1; w++) {
    uint32_t b = sh.bits[w];
    while (b) {
      const int bit = __ffs(int(b)) - 1;
      b &= b - 1u;
      if (p < topk) out[p] = 32 * w + bit;
      p++;
    }
  }
  if (tid == 0) n_sel[i] = topk;
}

}  // namespace

PrefillSelectPlan plan_prefill_select(int nq, int max_ctx, int block, int topk) {
  PrefillSelectPlan p{};
  const int64_t nmax = int64_t(max_ctx) / block;
  p.supported = nmax <= kMaxKeys && topk <= kCap / 2;
  p.step = nmax <= kSampleMax ? 1 : (nmax + kSampleMax - 1) / kSampleMax;
  p.n_samp = int((nmax + p.step - 1) / p.step);
  if (p.n_samp < 1) p.n_samp = 1;
  p.cap = kCap;
  p.tp = plan_topk(nq, max_ctx, block, topk);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t off = 0;
  p.off_samp = off;
  off = up(off + size_t(nq) * size_t(p.n_samp) * 4);
  p.off_theta = off;
  off = up(off + size_t(nq) * 8);
  p.off_counts = off;
  off = up(off + size_t(nq) * kCountStride * 4);
  p.off_fail = off;
  off = up(off + size_t(nq) * 4);
  p.off_lists = off;
  off = up(off + size_t(nq) * size_t(kCap) * 8);
  p.ws_bytes = off;
  return p;
}

hipError_t launch_prefill_select(const ScoreArgs& sa, const TopkArgs& ta, const PrefillSelectPlan& p, void* ws,
                                 hipStream_t s) {
  if (sa.nq <= 0) return hipSuccess;
  const int64_t nmax = int64_t(sa.max_ctx) / sa.block;
  unsigned char* w = static_cast<unsigned char*>(ws);
  float* samp = reinterpret_cast<float*>(w + p.off_samp);
  uint64_t* theta = reinterpret_cast<uint64_t*>(w + p.off_theta);
  uint32_t* counts = reinterpret_cast<uint32_t*>(w + p.off_counts);
  uint32_t* fail = reinterpret_cast<uint32_t*>(w + p.off_fail);
  uint64_t* lists = reinterpret_cast<uint64_t*>(w + p.off_lists);
  // 1. sample scores
  ScoreArgs a1 = sa;
  a1.tok_step = p.step;
  a1.scores = samp;
  a1.ld = p.n_samp;
  a1.only = nullptr;
  a1.lists = nullptr;
  hipError_t e = launch_scores_gemm_b(a1, p.n_samp, false, s);
  if (e != hipSuccess) return e;
  // 2. thresholds (also clear the counters and flags)
  ScoreArgs a2 = sa;
  a2.theta = theta;
  a2.counts = counts;
  hipLaunchKernelGGL(select_threshold, dim3(unsigned(sa.nq)), dim3(kSampleNT), 0, s, a2, samp, int64_t(p.n_samp),
                     int64_t(p.step), ta.topk, fail);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 3. lists
  ScoreArgs a3 = sa;
  a3.tok_step = 1;
  a3.theta = theta;
  a3.lists = lists;
  a3.counts = counts;
  a3.list_cap = p.cap;
  a3.only = nullptr;
  e = launch_scores_gemm_b(a3, nmax, true, s);
  if (e != hipSuccess) return e;
  // 4. per-query selection from the lists
  hipLaunchKernelGGL(select_lists, dim3(unsigned(sa.nq)), dim3(kFinalNT), 0, s, a3, ta.topk, ta.sel, ta.n_sel, fail);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 5. flagged queries: their full scores, then an exact select over them (one launch)
  ScoreArgs a5 = sa;
  a5.tok_step = 1;
  a5.only = fail;
  a5.lists = nullptr;
  e = launch_scores(a5, s);
  if (e != hipSuccess) return e;
  TopkArgs t5 = ta;
  t5.only = fail;
  t5.ws = nullptr;
  TopkPlan tp5 = p.tp;
  tp5.stream_only = true;  // flagged queries all have more than kCap keys
  return launch_topk(t5, tp5, s);
}

}  // namespace qsa
