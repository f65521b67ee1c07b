// One decode layer (pooled-block variant) in two launches: A2 + A3 + A4 + A5.
// "3090x3で 314 万コンテキスト": every pooled key is scored at every step
// (section "VRAM に残す必要があるもの"), a fixed budget of blocks is kept and
// only their K/V rows are read (section "なぜ"); "GLM-5.3 最適化 第2部",
// section "DCP": the partial attention results are merged by log-sum-exp.
//
// Launch 1 (index_lists_a, also qsa_index_lists on its own): each
// work-group scores one chunk of one query's pooled keys and writes the
// chunk's best candidates and a bound (index_topk.hpp, without the
// selection).
//
// Launch 2 (attend_select_a): one work-group per (query, kv head, split).
// Every work-group selects its query's exact top-k itself, from the chunk
// lists, into LDS (final_select, the same code the last chunk of
// qsa_index_topk runs): the parts of a query repeat the same register
// select side by side instead of waiting for one of them to publish it.
// Part (kv head 0, split 0) also copies it to sel and n_sel. Each part then
// attends its split of the token list (attend.hpp) and stores its partial
// result; the parts of a (query, kv head) wait for each other and merge,
// each part one slice of the output dims. That wait needs every part
// resident at once: the host checks it with the occupancy API, and
// otherwise the parts only write their partials and a third launch merges.
//
// Counters live in the caller's workspace; each call leaves them zero.
// Every wait is bounded: past the bound the kernel sets a sticky error word
// and carries on (every access stays inside the buffers).
#include "attend.hpp"
#include "index_topk.hpp"

namespace qsa {
namespace {

constexpr int kMaxTopk = 2048;
// tiles of 64 tokens an attention part loads at once (a decode part of the
// 1M-context batch-4 layer holds two)
constexpr int kLayerGT = 2;

struct SelAttnLds {
  int sel[kMaxTopk + 64];  // the query's selected blocks, ascending (then one dummy slot per lane)
  union {
    itk::FinalLds f;
    att::Lds<kLayerGT> a;
  } u;
};

template <int TPW, bool kFp8>
__global__ __launch_bounds__(256) void index_lists_a(IndexTopkArgs a) {
  __shared__ itk::FinalLds sh;
  if (a.clear && blockIdx.x == 0 && blockIdx.y == 0)
    for (int j = threadIdx.x; j < a.n_clear; j += 256) a.clear[j] = 0u;
  itk::chunk_step<TPW, false, kFp8>(a, blockIdx.y, blockIdx.x, sh);
}

template <bool kFp8>
void launch_lists_tpw(const IndexTopkArgs& a, int tpw, dim3 grid, hipStream_t s) {
  switch (tpw) {
    case 1: hipLaunchKernelGGL((index_lists_a<1, kFp8>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((index_lists_a<2, kFp8>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((index_lists_a<4, kFp8>), grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((index_lists_a<8, kFp8>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((index_lists_a<16, kFp8>), grid, dim3(256), 0, s, a); break;
  }
}

// kKeys: the call gave no score buffer, so a query whose selection cannot
// come from the chunk lists recomputes its scores from the keys (a separate
// instance, so that the code of that fallback does not weigh on the
// register allocation of the instance that reads stored scores).
template <bool kKeys>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void attend_select_a(IndexTopkArgs it,
                                                                                       AttendArgs at) {
  __shared__ SelAttnLds sh;
  const int tid = threadIdx.x;
  const int n_att = at.hkv * at.n_split;
  const int i = int(blockIdx.x) / n_att, r = int(blockIdx.x) % n_att;
  const int g = r / at.n_split, split = r % at.n_split;
  // the lists and bounds are loaded at the plan's full size before the
  // query's context arrives (one round trip instead of two); entries past
  // the query's own lists are dropped below
  // (written by the first launch: plain loads)
  uint64_t ent[itk::kRegR];
  itk::load_union<false>(it, i, it.n_chunks * it.keep, ent);
  const uint64_t* bq = it.list_bound + size_t(i) * it.n_chunks;
  const uint64_t b0 = tid < it.n_chunks ? bq[tid] : 0ull;
  const uint64_t b1 = tid + itk::kNT < it.n_chunks ? bq[tid + itk::kNT] : 0ull;
  const int n = clamp_ctx(it.q_ctx[i], it.max_ctx) / 4;
  // the attention's own view of the query (loaded now, used after the select)
  const int actx = clamp_ctx(at.q_ctx[i], at.max_ctx);
  const int aseq = at.q_seq ? at.q_seq[i] : 0;
  const int topk = it.topk;
  const int ns = n < topk ? n : topk;
  const bool writer = g == 0 && split == 0;
  int* gsel = it.sel + int64_t(i) * topk;
  int* const lsel = sh.sel;
  // selectors call emit(-1, block) for keys they leave out: those go to the
  // lane's dummy slot
  const int dummy = kMaxTopk + (tid & 63);
  auto emit = [lsel, dummy](int pos, int blk) { lsel[pos >= 0 ? pos : dummy] = blk; };
  if (n <= topk) {  // every complete block
    for (int j = tid; j < ns; j += 256) sh.sel[j] = j;
  } else if (itk::use_union(it, n) && it.n_chunks <= 2 * itk::kNT) {
    const int nch = (n + it.chunk_blocks - 1) / it.chunk_blocks;
    const int u = nch * it.keep;
    uint32_t ukey[itk::kRegR];
    int uidx[itk::kRegR];
#pragma unroll
    for (int rr = 0; rr < itk::kRegR; rr++) {
      const bool in = tid * itk::kRegR + rr < u;
      ukey[rr] = in ? uint32_t(ent[rr] >> 32) : 0u;
      uidx[rr] = int(uint32_t(ent[rr]));
    }
    uint64_t my_bound = tid < nch ? b0 : 0ull;
    if (tid + itk::kNT < nch) my_bound = b1 > my_bound ? b1 : my_bound;
    if (!itk::select_registers(it, true, ukey, uidx, my_bound, sh.u.f, emit)) {
      if constexpr (kKeys)
        itk::select_streamed_keys(it, i, n, sh.u.f, emit);
      else
        itk::select_streamed(it.scores + int64_t(i) * it.ld, n, topk, sh.u.f, emit);
    }
  } else if constexpr (kKeys) {  // no score buffer: the scores are recomputed from the keys
    itk::select_streamed_keys(it, i, n, sh.u.f, emit);
  } else {
    itk::final_select(it, i, n, sh.u.f, emit);
  }
  __syncthreads();
  if (writer) {  // the query's selection, padded with -1
    for (int j = tid; j < topk; j += 256) gsel[j] = j < ns ? sh.sel[j] : -1;
    if (tid == 0) it.n_sel[i] = ns;
  }
  att::attend_part<false, kLayerGT>(at, split, g, i, sh.u.a, (att::LdsIntPtr)(sh.sel), ns, actx, aseq);
}

template __global__ void attend_select_a<false>(IndexTopkArgs, AttendArgs);
template __global__ void attend_select_a<true>(IndexTopkArgs, AttendArgs);

// Work-groups of attend_select_a (either instance) the current device holds
// at once.
int resident_groups() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int per_cu = 0, per_cu_keys = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attend_select_a<false>, 256, 0) != hipSuccess) per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_keys, attend_select_a<true>, 256, 0) != hipSuccess)
      per_cu_keys = 0;
    if (per_cu_keys < per_cu) per_cu = per_cu_keys;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
    cache[dev] = per_cu * cus > 0 ? per_cu * cus : -1;
  }
  return cache[dev];
}

}  // namespace

hipError_t launch_index_lists(IndexTopkArgs a, const IndexTopkPlan& p, void* ws, hipStream_t s) {
  if (a.nq <= 0) return hipSuccess;
  char* w = static_cast<char*>(ws);
  a.counter = reinterpret_cast<uint32_t*>(w);
  a.list = reinterpret_cast<uint64_t*>(w + p.off_list);
  a.list_bound = reinterpret_cast<uint64_t*>(w + p.off_bound);
  a.n_chunks = p.n_chunks;
  a.chunk_blocks = 256 * p.tpw;
  a.keep = p.keep;
  a.wkeep = p.wkeep;
  dim3 grid(unsigned(p.n_chunks), unsigned(a.nq));
  if (a.key_fp8)
    launch_lists_tpw<true>(a, p.tpw, grid, s);
  else
    launch_lists_tpw<false>(a, p.tpw, grid, s);
  return hipGetLastError();
}

DecodeLayerPlan plan_decode_layer(int nq, int max_ctx, int topk, int hq, int hkv, int dv, int n_split) {
  DecodeLayerPlan p{};
  p.itk = plan_index_topk(nq, max_ctx, topk);
  // the error word, the merge counters (two lines per (query, kv head)),
  // the scan's workspace, the parts
  size_t off = 256;
  p.off_merge_cnt = off;
  off += size_t(nq) * hkv * 2 * kCounterStride * 4;
  off = (off + 255) / 256 * 256;
  p.off_itk = off;
  off += (p.itk.ws_bytes + 255) / 256 * 256;
  p.off_o = off;
  off += size_t(n_split) * nq * hq * dv * 4;
  p.off_lse = off;
  off += (size_t(n_split) * nq * hq * 4 + 255) / 256 * 256;
  p.ws_bytes = off;
  return p;
}

hipError_t launch_decode_layer(IndexTopkArgs itk, AttendArgs att, const DecodeLayerPlan& p, void* ws,
                               hipStream_t s, bool clear_control) {
  if (itk.nq <= 0) return hipSuccess;
  char* w = static_cast<char*>(ws);
  itk.clear = clear_control ? reinterpret_cast<uint32_t*>(w) : nullptr;
  itk.n_clear = clear_control ? int(p.off_itk / 4) : 0;
  char* wi = w + p.off_itk;
  att.o_part = reinterpret_cast<float*>(w + p.off_o);
  att.lse_part = reinterpret_cast<float*>(w + p.off_lse);
  att.error = reinterpret_cast<uint32_t*>(w);
  const int n_att_all = itk.nq * att.hkv * att.n_split;
  const bool merge_in = n_att_all <= resident_groups();
  att.counter = merge_in ? reinterpret_cast<uint32_t*>(w + p.off_merge_cnt) : nullptr;

  hipError_t e = launch_index_lists(itk, p.itk, wi, s);
  if (e != hipSuccess) return e;
  itk.clear = nullptr;
  itk.n_clear = 0;
  itk.counter = reinterpret_cast<uint32_t*>(wi);
  itk.list = reinterpret_cast<uint64_t*>(wi + p.itk.off_list);
  itk.list_bound = reinterpret_cast<uint64_t*>(wi + p.itk.off_bound);
  itk.n_chunks = p.itk.n_chunks;
  itk.chunk_blocks = 256 * p.itk.tpw;
  itk.keep = p.itk.keep;
  itk.wkeep = p.itk.wkeep;
  if (itk.scores)
    hipLaunchKernelGGL(attend_select_a<false>, dim3(unsigned(n_att_all)), dim3(256), 0, s, itk, att);
  else
    hipLaunchKernelGGL(attend_select_a<true>, dim3(unsigned(n_att_all)), dim3(256), 0, s, itk, att);
  e = hipGetLastError();
  if (e != hipSuccess || merge_in) return e;
  // too many parts to be resident together: merge in a third launch
  const int64_t rows = int64_t(att.nq) * att.hq;
  return launch_merge(att.n_split, rows, att.dv, att.o_part, rows * att.dv, att.lse_part, rows, att.o_out, att.o_bf16,
                      att.lse_out, s);
}

}  // namespace qsa
