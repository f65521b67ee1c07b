// HBM row cache for K/V rows kept in host memory.
// "125B MoE を 3090 3 枚で運用する vLLM 最適化編", section 5 (decode, third part): selections
// at consecutive steps overlap (0.72 on average), so rows read over the host
// link are kept in a direct-mapped cache in device memory, one slot per token
// (its K and V for every kv head), keyed by the row's physical position. Per
// layer and step:
//   1. invalidate the slots of rows stored since (their host bytes changed)
//      and advance the epoch (launch_row_cache_step);
//   2. plan: a hit marks its slot with the epoch; a miss takes the slot's
//      fill right by an atomic maximum of (epoch, claimer) (launch_row_cache_plan);
//   3. attention reads hits from the cache and misses from host memory, and a
//      miss that holds its slot's fill right, on a slot no hit marked this
//      step, writes the row and its tag (attend.hpp, cached variant).
// A slot with a hit this step is never written in it, and attention never
// reads a tag (the plan did), so the cache stays consistent without any
// synchronisation inside the attention launch; epochs in the marks and claims
// make per-step clearing unnecessary.
//
// Buffer layout (zero-filled by the caller once): [0, 256) the epoch (uint32);
// then tag (uint64 per slot: key + 1, 0 = empty), hitmark (uint32), claim
// (uint64) and the rows (row_bytes per slot), each 256-byte aligned.
#include "attend.hpp"

namespace qsa {
namespace {

__global__ __launch_bounds__(256) void row_cache_step_kernel(unsigned char* cache, RowCacheLayout L, int n,
                                                             const int* row_seq, const int* row_pos, int64_t ks) {
  uint32_t* epoch = reinterpret_cast<uint32_t*>(cache);
  uint64_t* tag = reinterpret_cast<uint64_t*>(cache + L.off_tag);
  if (threadIdx.x == 0) *epoch = *epoch + 1u;
  for (int j = threadIdx.x; j < n; j += 256) {
    const int seq = row_seq ? row_seq[j] : j;
    const int pos = row_pos[j];
    if (pos < 0 || pos >= ks) continue;  // a caller error: nothing to invalidate
    const uint64_t key = uint64_t(int64_t(seq) * ks + pos) + 1u;
    const int64_t c = int64_t((key - 1u) % uint64_t(L.n_slots));
    if (tag[c] == key) tag[c] = 0u;
  }
}

// Work-group (i, y): list positions 256y .. 256y + 255 of query i, one per
// thread (a single round of dependent loads per position).
__global__ __launch_bounds__(256) void row_cache_plan_kernel(AttendArgs a, unsigned char* cache, RowCacheLayout L,
                                                             int* src, int src_ld) {
  const int i = blockIdx.x;
  const int p = int(blockIdx.y) * 256 + int(threadIdx.x);
  const int seq = a.q_seq ? a.q_seq[i] : 0;
  const int ctx = clamp_ctx(a.q_ctx[i], a.max_ctx);
  att::List<false> lv;
  lv.sel = a.sel + int64_t(i) * a.topk;
  lv.block = a.block;
  lv.nblk = ctx / a.block;
  const int ns_max = lv.nblk < a.topk ? lv.nblk : a.topk;
  const int ns = a.n_sel[i];
  lv.ns = ns < 0 ? 0 : (ns > ns_max ? ns_max : ns);
  lv.L = lv.ns * a.block + (ctx - lv.nblk * a.block);
  const int Lq = lv.L < src_ld ? lv.L : src_ld;
  if (p >= Lq) return;
  const uint32_t epoch = *reinterpret_cast<const uint32_t*>(cache);
  const uint64_t* tag = reinterpret_cast<const uint64_t*>(cache + L.off_tag);
  uint32_t* hit = reinterpret_cast<uint32_t*>(cache + L.off_hit);
  unsigned long long* claim = reinterpret_cast<unsigned long long*>(cache + L.off_claim);
  const int tok = lv.tok(p);
  const uint64_t key = uint64_t(int64_t(seq) * a.key_stride + tok) + 1u;
  const int64_t c = int64_t((key - 1u) % uint64_t(L.n_slots));
  if (tag[c] == key) {
    hit[c] = epoch;
    src[int64_t(i) * src_ld + p] = -int(c) - 1;
  } else {
    const uint32_t id = uint32_t(int64_t(i) * src_ld + p) + 1u;
    atomicMax(claim + c, (static_cast<unsigned long long>(epoch) << 32) | id);
    src[int64_t(i) * src_ld + p] = tok;
  }
}

}  // namespace

RowCacheLayout row_cache_layout(int64_t n_slots, int64_t row_bytes) {
  RowCacheLayout L{};
  L.n_slots = n_slots;
  L.row_bytes = row_bytes;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t off = 256;
  L.off_tag = off;
  off = up(off + size_t(n_slots) * 8);
  L.off_hit = off;
  off = up(off + size_t(n_slots) * 4);
  L.off_claim = off;
  off = up(off + size_t(n_slots) * 8);
  L.off_rows = off;
  L.bytes = off + size_t(n_slots) * size_t(row_bytes);
  return L;
}

hipError_t launch_row_cache_step(unsigned char* cache, const RowCacheLayout& L, int n_rows, const int* row_seq,
                                 const int* row_pos, int64_t key_stride, hipStream_t s) {
  hipLaunchKernelGGL(row_cache_step_kernel, dim3(1), dim3(256), 0, s, cache, L, n_rows, row_seq, row_pos, key_stride);
  return hipGetLastError();
}

hipError_t launch_row_cache_plan(const AttendArgs& a, unsigned char* cache, const RowCacheLayout& L, int* src,
                                 int src_ld, hipStream_t s) {
  if (a.nq <= 0) return hipSuccess;
  const unsigned gy = unsigned((src_ld + 255) / 256);
  hipLaunchKernelGGL(row_cache_plan_kernel, dim3(unsigned(a.nq), gy), dim3(256), 0, s, a, cache, L, src, src_ld);
  return hipGetLastError();
}

}  // namespace qsa
