// One decode layer in one launch (pooled-block variant): A2 + A3 + A4 + A5.
// "3090x3で 314 万コンテキスト": every pooled key is scored at every step
// (section "VRAM に残す必要があるもの"), a fixed budget of blocks is kept and
// only their K/V rows are read (section "なぜ"); "GLM-5.3 最適化 第2部",
// section "DCP": the partial attention results are merged by log-sum-exp.
//
// One work item per work-group, in block order: first the scan chunks of
// every query (index_topk.hpp: score a chunk, keep its best candidates; the
// last chunk of a query to finish selects its top-k), then the attention
// parts (attend.hpp: one (kv head, split) part each; the last part of a kv
// head merges). An attention item waits until the selection of its query
// is published, so a query's attention overlaps the scans still running for
// later queries, and the whole layer costs one launch.
//
// Why this cannot deadlock: a scan item never waits, and the attention
// items are fewer than the work-groups the chip holds at once (the host
// checks this before it launches, and otherwise issues the scan, the
// attention and the merge as three launches). So however the hardware
// orders the dispatch, waiting attention items can never take every slot:
// the scans always progress and publish every selection. Every wait is
// also bounded: past the bound the kernel raises a sticky error word and
// carries on (selections are clamped into range, so every access stays
// inside the buffers).
//
// Counters and flags live in the caller's workspace; each call leaves them
// zero. No counter is shared by all work-groups (a single device-scope
// atomic per work-group on one address serialises at the memory side), and
// each has a line of its own.
#include "attend.hpp"
#include "index_topk.hpp"

namespace qsa {
namespace {

constexpr unsigned kSpinLimit = 1u << 22;  // polls of a selection flag (seconds)
// Each selection flag has kFlagCopies copies kFlagStride bytes apart, and
// the attention parts of a query poll different copies with a growing
// pause: hundreds of pollers on one line would tie up the memory channel
// that serves it, and with it the scans still running.
constexpr int kFlagCopies = 8;
constexpr int kFlagStride = 4096;

struct LayerArgs {
  IndexTopkArgs itk;
  AttendArgs att;
  uint32_t* error;     // [1] sticky: 1 = a wait ran out
  char* flag;          // copy c of query q's flag at flag + (q * kFlagCopies + c) * kFlagStride
  uint32_t* att_cnt;   // [nq] lines: attention items of query q finished
  int nq, n_chunks, n_att;
};

union LayerLds {
  itk::FinalLds scan;
  att::Lds attn;
};

__device__ __forceinline__ uint32_t* flag_at(const LayerArgs& L, int q, int c) {
  return reinterpret_cast<uint32_t*>(L.flag + (size_t(q) * kFlagCopies + c) * kFlagStride);
}

template <int TPW>
__global__ __launch_bounds__(256) void decode_layer_a(LayerArgs L) {
  __shared__ LayerLds sh;
  const int tid = threadIdx.x;
  const int n_scan = L.nq * L.n_chunks;
  const int t = int(blockIdx.x);
  const bool scan = t < n_scan;
  const int q = scan ? t / L.n_chunks : (t - n_scan) / L.n_att;
  const int idx = scan ? t % L.n_chunks : (t - n_scan) % L.n_att;
  if (scan) {
    if (itk::chunk_step<TPW>(L.itk, q, idx, sh.scan) && tid < kFlagCopies)
      st_coherent(flag_at(L, q, tid), 1u);
  } else {
    if (tid == 0) {
      const uint32_t* f = flag_at(L, q, idx % kFlagCopies);
      unsigned polls = 0, pause = 1;
      while (ld_coherent(f) == 0u) {
        if (++polls > kSpinLimit) {
          atomicOr(L.error, 1u);
          break;
        }
        for (unsigned k = 0; k < pause; k++) __builtin_amdgcn_s_sleep(8);  // 512 cycles each
        pause = pause < 4 ? 2 * pause : 4;
      }
    }
    __syncthreads();
    const int n_split = L.att.n_split;
    att::attend_part<true>(L.att, idx % n_split, idx / n_split, q, sh.attn);
    if (tid == 0) {
      // the last attention item of the query clears its flag: every other
      // item of the query has passed its wait
      uint32_t* cnt = L.att_cnt + size_t(q) * kCounterStride;
      if (atomicAdd(cnt, 1u) == unsigned(L.n_att - 1)) {
        atomicExch(cnt, 0u);
        for (int c = 0; c < kFlagCopies; c++) st_coherent(flag_at(L, q, c), 0u);
      }
    }
  }
}

// Work-groups of decode_layer_a<TPW> the current device holds at once.
template <int TPW>
int resident_groups() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_layer_a<TPW>, 256, 0) != hipSuccess) per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
    cache[dev] = per_cu * cus > 0 ? per_cu * cus : -1;
  }
  return cache[dev];
}

template <int TPW>
hipError_t launch_t(const LayerArgs& L, hipStream_t s, bool& launched) {
  const int n_att_all = L.nq * L.n_att;
  launched = n_att_all < resident_groups<TPW>();
  if (!launched) return hipSuccess;
  const unsigned grid = unsigned(L.nq * (L.n_chunks + L.n_att));
  hipLaunchKernelGGL(decode_layer_a<TPW>, dim3(grid), dim3(256), 0, s, L);
  return hipGetLastError();
}

}  // namespace

DecodeLayerPlan plan_decode_layer(int nq, int max_ctx, int topk, int hq, int hkv, int dv, int n_split) {
  DecodeLayerPlan p{};
  p.itk = plan_index_topk(nq, max_ctx, topk);
  // the error word, the per-query counters, the merge counters, the flags
  // (page aligned), the scan's own workspace, the parts
  size_t off = 64;
  p.off_att_cnt = off;
  off += size_t(nq) * kCounterStride * 4;
  p.off_merge_cnt = off;
  off += size_t(nq) * hkv * kCounterStride * 4;
  off = (off + kFlagStride - 1) / kFlagStride * kFlagStride;
  p.off_flag = off;
  off += size_t(nq) * kFlagCopies * kFlagStride;
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
                               hipStream_t s) {
  if (itk.nq <= 0) return hipSuccess;
  char* w = static_cast<char*>(ws);
  char* wi = w + p.off_itk;
  itk.counter = reinterpret_cast<uint32_t*>(wi);
  itk.list = reinterpret_cast<uint64_t*>(wi + p.itk.off_list);
  itk.list_bound = reinterpret_cast<uint64_t*>(wi + p.itk.off_bound);
  itk.n_chunks = p.itk.n_chunks;
  itk.keep = p.itk.keep;
  itk.wkeep = p.itk.wkeep;
  att.counter = reinterpret_cast<uint32_t*>(w + p.off_merge_cnt);
  att.o_part = reinterpret_cast<float*>(w + p.off_o);
  att.lse_part = reinterpret_cast<float*>(w + p.off_lse);
  LayerArgs L{};
  L.itk = itk;
  L.att = att;
  L.error = reinterpret_cast<uint32_t*>(w);
  L.flag = w + p.off_flag;
  L.att_cnt = reinterpret_cast<uint32_t*>(w + p.off_att_cnt);
  L.nq = itk.nq;
  L.n_chunks = p.itk.n_chunks;
  L.n_att = att.hkv * att.n_split;
  bool launched = false;
  hipError_t e;
  switch (p.itk.tpw) {
    case 1: e = launch_t<1>(L, s, launched); break;
    case 2: e = launch_t<2>(L, s, launched); break;
    case 4: e = launch_t<4>(L, s, launched); break;
    case 8: e = launch_t<8>(L, s, launched); break;
    default: e = launch_t<16>(L, s, launched); break;
  }
  if (e != hipSuccess || launched) return e;
  // too many attention parts to wait inside one launch: three launches
  e = launch_index_topk(itk, p.itk, wi, s);
  if (e != hipSuccess) return e;
  AttendArgs a2 = att;
  a2.counter = nullptr;
  e = launch_attend(a2, s);
  if (e != hipSuccess) return e;
  const int64_t rows = int64_t(att.nq) * att.hq;
  return launch_merge(att.n_split, rows, att.dv, att.o_part, rows * att.dv, att.lse_part, rows, att.o_out, att.o_bf16,
                      att.lse_out, s);
}

}  // namespace qsa
