// A1: pooled indexer keys, one per complete block of tokens.
// "3090x3で 314 万コンテキスト", section "VRAM に残す必要があるもの": each
// block's keys are summarised into one 128 x bf16 pooled key; here the
// summary is the exact mean rounded once to bf16 (nearest, ties to even).
#include "common.hpp"
#include "kernels.hpp"

namespace qsa {
namespace {

// Round a double to the nearest bf16 (ties to even), straight from double.
// The spacing of bf16 values near x = m * 2^e (0.5 <= |m| < 1) is 2^(e-8),
// and 2^-133 below the normal range.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  if (x == 0.0) return __double_as_longlong(x) < 0 ? 0x8000 : 0x0000;
  int e;
  (void)frexp(x, &e);
  int q = e - 8;
  if (q < -133) q = -133;
  double r = rint(ldexp(x, -q));
  float f = float(ldexp(r, q));  // exact: at most 8 significant bits (or inf)
  return uint16_t(__float_as_uint(f) >> 16);
}

// One thread per (block, 8-wide dim chunk); blockIdx.y = sequence.
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t* __restrict__ raw, int64_t raw_ss,
                                                   uint16_t* __restrict__ pooled, int64_t pooled_ss,
                                                   int64_t b0, int64_t nb, int dim, int block) {
  const int nchunk = dim >> 3;
  const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= nb * nchunk) return;
  const int64_t b = b0 + t / nchunk;
  const int c = int(t % nchunk);
  const int s = blockIdx.y;
  const uint16_t* src = raw + s * raw_ss + (b * block) * dim + 8 * c;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; e++) acc[e] = 0.0;
  for (int j = 0; j < block; j++) {
    u32x4 w = ld16(src + int64_t(j) * dim);
#pragma unroll
    for (int e = 0; e < 4; e++) {
      acc[2 * e] += double(bf16_lo(w[e]));
      acc[2 * e + 1] += double(bf16_hi(w[e]));
    }
  }
  u32x4 out;
#pragma unroll
  for (int e = 0; e < 4; e++) {
    uint32_t lo = f64_to_bf16(acc[2 * e] / block);
    uint32_t hi = f64_to_bf16(acc[2 * e + 1] / block);
    out[e] = lo | (hi << 16);
  }
  st16(pooled + s * pooled_ss + b * dim + 8 * c, out);
}

}  // namespace

hipError_t launch_pool(const uint16_t* raw, int64_t raw_ss, uint16_t* pooled, int64_t pooled_ss,
                       int n_seq, int64_t b0, int64_t nb, int dim, int block, hipStream_t s) {
  if (nb <= 0 || n_seq <= 0) return hipSuccess;
  const int64_t threads = nb * (dim / 8);
  const int64_t grid = (threads + 255) / 256;
  hipLaunchKernelGGL(pool_kernel, dim3(unsigned(grid), unsigned(n_seq)), dim3(256), 0, s, raw, raw_ss,
                     pooled, pooled_ss, b0, nb, dim, block);
  return hipGetLastError();
}

}  // namespace qsa
