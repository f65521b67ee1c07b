// A5: combine partial softmax results by log-sum-exp.
// "GLM-5.3 最適化 第2部", section "DCP": attention over disjoint parts of the
// context is computed separately and the partial results are combined with
// log-sum-exp; "3090x3で 314 万コンテキスト", section "ちなみにこの欠点":
// prefill merges the softmax partials of consecutive history tiles.
// One wave per output row; each lane owns 4 consecutive dims per 256.
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
  for (int d0 = 4 * lane; d0 < dv; d0 += 256) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (mx != -INFINITY) {
      for (int p = 0; p < n_part; p++) {
        const float lp = l[p * lps + row];
        if (lp == -INFINITY) continue;
        const float w = expf(lp - lse);
        const f32x4 v = *reinterpret_cast<const f32x4*>(o + p * ops + row * dv + d0);
        acc += w * v;
      }
    }
    if (oo) *reinterpret_cast<f32x4*>(oo + row * dv + d0) = acc;
    if (ob) {
      u32x2 pk;
      pk[0] = uint32_t(f32_to_bf16(acc[0])) | (uint32_t(f32_to_bf16(acc[1])) << 16);
      pk[1] = uint32_t(f32_to_bf16(acc[2])) | (uint32_t(f32_to_bf16(acc[3])) << 16);
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
