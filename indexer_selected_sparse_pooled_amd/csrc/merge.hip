// A5: combine partial softmax results by log-sum-exp.
// "GLM-5.3 最適化 第2部", section "DCP": attention over disjoint parts of the
// context is computed separately and the partial results are combined with
// log-sum-exp; "3090x3で 314 万コンテキスト", section "ちなみにこの欠点":
// prefill merges the softmax partials of consecutive history tiles.
// One wave per 256 dims of an output row (a row of dv dims is `pieces` =
// ceil(dv / 256) waves, so a small merge still spreads over the chip); each
// lane owns 4 consecutive dims. The row's lse values are wave-uniform
// (scalar loads), so every lane computes the partials' weights itself, with
// no cross-lane step, and a batch of PB partials (O pieces and lse values)
// is loaded before any of it is used: a merge of up to PB partials costs
// one memory round trip. The first piece of a row writes its lse.
#include "common.hpp"
#include "kernels.hpp"

namespace qsa {
namespace {

template <int ND, int PB>
__global__ __launch_bounds__(256) void merge_kernel(int n_part, int64_t rows, int dv, int pieces,
                                                    const float* __restrict__ o, int64_t ops,
                                                    const float* __restrict__ l, int64_t lps,
                                                    float* __restrict__ oo, uint16_t* __restrict__ ob,
                                                    float* __restrict__ lo) {
  const int lane = threadIdx.x & 63;
  const int64_t w = int64_t(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int64_t row = w / pieces;
  const int piece = int(w - row * pieces);
  if (row >= rows) return;
  const int dbase = 256 * ND * piece;  // the wave's first dim
  bool in[ND];
#pragma unroll
  for (int c = 0; c < ND; c++) in[c] = dbase + 256 * c + 4 * lane < dv;
  const float* src0 = o + row * dv + dbase + 4 * lane;
  f32x4 acc[ND];
#pragma unroll
  for (int c = 0; c < ND; c++) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  // running maximum mx and sum tot of exp(lse_p - mx) over the partials
  float mx = -INFINITY, tot = 0.f;
  for (int p0 = 0; p0 < n_part; p0 += PB) {
    f32x4 v[PB][ND];
    float lp[PB];
#pragma unroll
    for (int q = 0; q < PB; q++) {
      const bool ok = p0 + q < n_part;
      lp[q] = ok ? l[int64_t(p0 + q) * lps + row] : -INFINITY;
#pragma unroll
      for (int c = 0; c < ND; c++)
        v[q][c] = (ok && in[c]) ? *reinterpret_cast<const f32x4*>(src0 + int64_t(p0 + q) * ops + 256 * c)
                                : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float bm = mx;
#pragma unroll
    for (int q = 0; q < PB; q++) bm = fmaxf(bm, lp[q]);
    if (bm == -INFINITY) continue;  // every partial so far is empty
    // rescale what was accumulated against the old maximum
    const float sc = expf(mx - bm);
    tot *= sc;
#pragma unroll
    for (int c = 0; c < ND; c++) acc[c] *= sc;
    mx = bm;
#pragma unroll
    for (int q = 0; q < PB; q++) {
      if (lp[q] == -INFINITY) continue;  // an empty partial adds nothing
      const float w = expf(lp[q] - mx);
      tot += w;
#pragma unroll
      for (int c = 0; c < ND; c++) acc[c] += w * v[q][c];
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
  for (int c = 0; c < ND; c++) {
    const int d0 = dbase + 256 * c + 4 * lane;
    if (!in[c]) continue;
    const f32x4 r = acc[c] * inv;
    if (oo) *reinterpret_cast<f32x4*>(oo + row * dv + d0) = r;
    if (ob) {
      u32x2 pk;
      pk[0] = uint32_t(f32_to_bf16(r[0])) | (uint32_t(f32_to_bf16(r[1])) << 16);
      pk[1] = uint32_t(f32_to_bf16(r[2])) | (uint32_t(f32_to_bf16(r[3])) << 16);
      *reinterpret_cast<u32x2*>(ob + row * dv + d0) = pk;
    }
  }
  if (lane == 0 && piece == 0 && lo) lo[row] = tot > 0.f ? mx + logf(tot) : -INFINITY;
}

}  // namespace

hipError_t launch_merge(int n_part, int64_t rows, int dv, const float* o_parts, int64_t o_ps,
                        const float* lse_parts, int64_t l_ps, float* o_out, uint16_t* o_bf16,
                        float* lse_out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int pieces = (dv + 255) / 256;
  const dim3 grid(unsigned((rows * pieces + 3) / 4));
  hipLaunchKernelGGL((merge_kernel<1, 16>), grid, dim3(256), 0, s, n_part, rows, dv, pieces, o_parts, o_ps,
                     lse_parts, l_ps, o_out, o_bf16, lse_out);
  return hipGetLastError();
}

}  // namespace qsa
