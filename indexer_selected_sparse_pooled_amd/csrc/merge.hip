// A5: combine partial softmax results by log-sum-exp.
// "GLM-5.3 最適化 第2部", section "DCP": attention over disjoint parts of the
// context is computed separately and the partial results are combined with
// log-sum-exp; "3090x3で 314 万コンテキスト", section "ちなみにこの欠点":
// prefill merges the softmax partials of consecutive history tiles.
// One wave per output row; each lane owns 4 consecutive dims per 256; the
// partials' weights are computed once (one lane each) and broadcast.
#include "common.hpp"
#include "kernels.hpp"

namespace qsa {
namespace {

// ND = ceil(dv / 256) passes of 256 dims; PB partials are loaded per batch,
// all before any is used (the loads do not depend on the weights), so a
// merge of up to PB partials costs one memory round trip.
template <int ND, int PB>
__global__ __launch_bounds__(256) void merge_kernel(int n_part, int64_t rows, int dv,
                                                    const float* __restrict__ o, int64_t ops,
                                                    const float* __restrict__ l, int64_t lps,
                                                    float* __restrict__ oo, uint16_t* __restrict__ ob,
                                                    float* __restrict__ lo) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + wave;
  if (row >= rows) return;
  bool in[ND];
#pragma unroll
  for (int c = 0; c < ND; c++) in[c] = 256 * c + 4 * lane < dv;
  const float* src0 = o + row * dv + 4 * lane;
  // first batch of partials, in flight together with the lse loads
  f32x4 v[PB][ND];
#pragma unroll
  for (int q = 0; q < PB; q++)
#pragma unroll
    for (int c = 0; c < ND; c++)
      v[q][c] = (q < n_part && in[c]) ? *reinterpret_cast<const f32x4*>(src0 + q * ops + 256 * c)
                                     : f32x4{0.f, 0.f, 0.f, 0.f};
  // lse of partial p0 + lane in this lane
  float mx = -INFINITY;
  for (int p0 = 0; p0 < n_part; p0 += 64) {
    const int p = p0 + lane;
    if (p < n_part) mx = fmaxf(mx, l[p * lps + row]);
  }
  mx = wave_max(mx);
  float tot = 0.f;
  if (mx != -INFINITY)
    for (int p0 = 0; p0 < n_part; p0 += 64) {
      const int p = p0 + lane;
      if (p < n_part) tot += expf(l[p * lps + row] - mx);
    }
  tot = wave_sum(tot);
  const float lse = mx == -INFINITY ? -INFINITY : mx + logf(tot);
  f32x4 acc[ND];
#pragma unroll
  for (int c = 0; c < ND; c++) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (mx != -INFINITY) {
    for (int p0 = 0; p0 < n_part; p0 += PB) {
      if (p0 > 0) {
#pragma unroll
        for (int q = 0; q < PB; q++)
#pragma unroll
          for (int c = 0; c < ND; c++)
            v[q][c] = (p0 + q < n_part && in[c]) ? *reinterpret_cast<const f32x4*>(src0 + (p0 + q) * ops + 256 * c)
                                                 : f32x4{0.f, 0.f, 0.f, 0.f};
      }
      // weight of partial (p0 & ~63) + lane, broadcast per partial
      const int pl = (p0 & ~63) + lane;
      const float w_lane = pl < n_part ? expf(l[pl * lps + row] - lse) : 0.f;
#pragma unroll
      for (int q = 0; q < PB; q++) {
        if (p0 + q >= n_part) break;
        const float w =
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_lane), (p0 + q) & 63));
        if (w != 0.f) {  // an empty partial (lse = -inf) adds nothing
#pragma unroll
          for (int c = 0; c < ND; c++) acc[c] += w * v[q][c];
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < ND; c++) {
    const int d0 = 256 * c + 4 * lane;
    if (!in[c]) continue;
    if (oo) *reinterpret_cast<f32x4*>(oo + row * dv + d0) = acc[c];
    if (ob) {
      u32x2 pk;
      pk[0] = uint32_t(f32_to_bf16(acc[c][0])) | (uint32_t(f32_to_bf16(acc[c][1])) << 16);
      pk[1] = uint32_t(f32_to_bf16(acc[c][2])) | (uint32_t(f32_to_bf16(acc[c][3])) << 16);
      *reinterpret_cast<u32x2*>(ob + row * dv + d0) = pk;
    }
  }
  if (lane == 0 && lo) lo[row] = lse;
}

}  // namespace

hipError_t launch_merge(int n_part, int64_t rows, int dv, const float* o_parts, int64_t o_ps,
                        const float* lse_parts, int64_t l_ps, float* o_out, uint16_t* o_bf16,
                        float* lse_out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid(unsigned((rows + 3) / 4));
  const int nd = (dv + 255) / 256;
  if (nd == 1)
    hipLaunchKernelGGL((merge_kernel<1, 16>), grid, dim3(256), 0, s, n_part, rows, dv, o_parts, o_ps, lse_parts,
                       l_ps, o_out, o_bf16, lse_out);
  else if (nd == 2)
    hipLaunchKernelGGL((merge_kernel<2, 8>), grid, dim3(256), 0, s, n_part, rows, dv, o_parts, o_ps, lse_parts,
                       l_ps, o_out, o_bf16, lse_out);
  else
    hipLaunchKernelGGL((merge_kernel<4, 4>), grid, dim3(256), 0, s, n_part, rows, dv, o_parts, o_ps, lse_parts,
                       l_ps, o_out, o_bf16, lse_out);
  return hipGetLastError();
}

}  // namespace qsa
