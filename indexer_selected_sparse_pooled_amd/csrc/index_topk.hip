// A2 + A3 in one launch for decode (device code in index_topk.hpp): grid
// (chunks, queries), one chunk per work-group; the last work-group of a
// query to finish selects.
#include "index_topk.hpp"

namespace qsa {
namespace {

template <int TPW, bool kFp8>
__global__ __launch_bounds__(256) void index_topk_a(IndexTopkArgs a) {
  __shared__ itk::FinalLds sh;
  itk::chunk_step<TPW, true, kFp8>(a, blockIdx.y, blockIdx.x, sh);
}

template <bool kFp8>
void launch_tpw(const IndexTopkArgs& a, int tpw, dim3 grid, hipStream_t s) {
  switch (tpw) {
    case 1: hipLaunchKernelGGL((index_topk_a<1, kFp8>), grid, dim3(itk::kNT), 0, s, a); break;
    case 2: hipLaunchKernelGGL((index_topk_a<2, kFp8>), grid, dim3(itk::kNT), 0, s, a); break;
    case 4: hipLaunchKernelGGL((index_topk_a<4, kFp8>), grid, dim3(itk::kNT), 0, s, a); break;
    case 8: hipLaunchKernelGGL((index_topk_a<8, kFp8>), grid, dim3(itk::kNT), 0, s, a); break;
    default: hipLaunchKernelGGL((index_topk_a<16, kFp8>), grid, dim3(itk::kNT), 0, s, a); break;
  }
}

}  // namespace

IndexTopkPlan plan_index_topk(int nq, int max_ctx, int topk) {
  IndexTopkPlan p{};
  const int64_t nmax = int64_t(max_ctx) / 4;
  // at most 512 chunks per query (a 1M-token context: 512 blocks per chunk,
  // 2048 work-groups for 4 queries). Small chunks balance best: the chip
  // holds about 768 of these work-groups and hands out the rest as they
  // finish, so no CU is left with a long chunk at the end (2048 / 1024 /
  // 512 work-groups: 57 / 60 / 65 us for the scan and top-512)
  int tpw = 1;
  while (tpw < 16 && (nmax + 256 * tpw - 1) / (256 * tpw) > 2 * itk::kNT) tpw *= 2;
  p.tpw = tpw;
  p.n_chunks = int(nmax <= 0 ? 1 : (nmax + 256 * tpw - 1) / (256 * tpw));
  // candidates kept: 8 per wave, 16 per chunk up to 256 chunks, else 8, so
  // the union never exceeds 4096 entries
  p.keep = p.n_chunks <= itk::kNT ? itk::kChunkKeep : itk::kChunkKeep / 2;
  p.wkeep = itk::kWaveKeep;
  // counters first, one line per query (they must be zero before the first
  // call; each call leaves them zero), then the lists and bounds
  const size_t cnt = size_t(nq) * kCounterStride * 4;
  const size_t lists = size_t(nq) * p.n_chunks * p.keep;
  p.off_list = cnt;
  p.off_bound = p.off_list + lists * 8;
  p.ws_bytes = p.off_bound + size_t(nq) * p.n_chunks * 8;
  (void)topk;
  return p;
}

hipError_t launch_index_topk(IndexTopkArgs a, const IndexTopkPlan& p, void* ws, hipStream_t s) {
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
    launch_tpw<true>(a, p.tpw, grid, s);
  else
    launch_tpw<false>(a, p.tpw, grid, s);
  return hipGetLastError();
}

}  // namespace qsa
