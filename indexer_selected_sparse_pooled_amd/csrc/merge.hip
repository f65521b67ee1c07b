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

__global__ __launch_bounds__(256) void merge_kernel(int n_part, int64_t rows, int dv,
                                                    const float* __restrict__ o, int64_t ops,
                                                    const float* __restrict__ l, int64_t lps,
                                                    float* __restrict__ oo, uint16_t* __restrict__ ob,
                                                    float* __restrict__ lo) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + wave;
  if (row >= rows) return;
  float mx = -INFINITY;
  for (int p = lane; p < n_part; p += 64) mx = fmaxf(mx, l[p * lps + row]);
  mx = wave_max(mx);
  float tot = 0.f;
  if (mx != -INFINITY)
    for (int p = lane; p < n_part; p += 64) tot += expf(l[p * lps + row] - mx);
  tot = wave_sum(tot);
  const float lse = mx == -INFINITY ? -INFINITY : mx + logf(tot);
  const int nd = (dv + 255) / 256;  // 256 dims per pass of the wave (4 per lane)
  f32x4 acc[4];
#pragma unroll
  for (int c = 0; c < 4; c++) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (mx != -INFINITY) {
    for (int p0 = 0; p0 < n_part; p0 += 64) {
      // weight of partial p0 + lane, then broadcast one partial at a time
      const int p = p0 + lane;
      const float w_lane = p < n_part ? expf(l[p * lps + row] - lse) : 0.f;
      const int cnt = min(64, n_part - p0);
#pragma unroll 8
      for (int pp = 0; pp < cnt; pp++) {
        const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_lane), pp));
        const float* src = o + (p0 + pp) * ops + row * dv + 4 * lane;
#pragma unroll
        for (int c = 0; c < 4; c++) {
          if (c < nd && 256 * c + 4 * lane < dv) {
            // loads are unconditional so that several partials are in flight;
            // an empty partial (lse = -inf, weight 0) adds nothing
            const f32x4 v = *reinterpret_cast<const f32x4*>(src + 256 * c);
            if (w != 0.f) acc[c] += w * v;
          }
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 4; c++) {
    const int d0 = 256 * c + 4 * lane;
    if (c >= nd || d0 >= dv) continue;
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
  const int64_t grid = (rows + 3) / 4;
  hipLaunchKernelGGL(merge_kernel, dim3(unsigned(grid)), dim3(256), 0, s, n_part, rows, dv, o_parts,
                     o_ps, lse_parts, l_ps, o_out, o_bf16, lse_out);
  return hipGetLastError();
}

}  // namespace qsa
