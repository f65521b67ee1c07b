// A1: pooled indexer keys, one per complete block of tokens, and the decode
// step's append of a new token (its K/V rows, its raw indexer key, and the
// pooled key of the block it completes).
// "3090x3で 314 万コンテキスト", section "VRAM に残す必要があるもの": each
// block's keys are summarised into one 128 x bf16 pooled key, kept in VRAM
// and completed as tokens arrive (the raw keys are kept so a block can be
// pooled); here the summary is the exact mean rounded once to bf16
// (nearest, ties to even). Section "カーネルを書き換えずに済む": the cache is
// addressed per (token, kv head).
#include "common.hpp"
#include "fp8.hpp"
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

// FP8 indexer keys ("GLM-5.3 最適化 第2部", footnote 3: FP8 values plus a
// 4-byte scale per key): one wave per key, dim <= 128. scale = amax / 448
// and code = E4M3(x / scale), both quotients correctly rounded fp32
// divisions; an all-zero key gets scale 0 and zero codes.
__device__ __forceinline__ void quantize_key_wave(float x0, float x1, int dim, uint8_t* row, float* scale_at) {
  const int lane = threadIdx.x & 63;
  const float m = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
  const float sc = m / kE4m3Max;
  if (lane < dim) row[lane] = uint8_t(sc > 0.f ? e4m3_code(x0 / sc) : 0u);
  if (lane + 64 < dim) row[lane + 64] = uint8_t(sc > 0.f ? e4m3_code(x1 / sc) : 0u);
  if (lane == 0) *scale_at = sc;
}

__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ keys, int64_t keys_ss,
                                                       uint8_t* __restrict__ out, int64_t out_ss, int64_t k0,
                                                       int64_t nk, int dim) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t kk = int64_t(blockIdx.x) * 4 + wave;
  if (kk >= nk) return;  // wave-uniform
  const int64_t b = k0 + kk;
  const int s = blockIdx.y;
  const uint16_t* src = keys + s * keys_ss + b * dim;
  const float x0 = lane < dim ? bf16_to_f32(src[lane]) : 0.f;
  const float x1 = lane + 64 < dim ? bf16_to_f32(src[lane + 64]) : 0.f;
  uint8_t* base = out + s * out_ss;
  quantize_key_wave(x0, x1, dim, base + fp8_code_off(b, dim), reinterpret_cast<float*>(base + fp8_scale_off(b, dim)));
}

// One FP8 sparse-MLA row ("GLM-5.3 最適化 第2部", footnote 1: 656 bytes)
// from a 576-wide bf16 latent row, by a 256-thread work-group: wave g
// quantizes columns 128g .. 128g+127 with one scale (codes at bytes 128g..,
// scale at byte 512 + 4g); wave 0 also copies the 64 rotary values (bytes
// 528 .. 655) unchanged.
__device__ __forceinline__ void quantize_latent_row(const uint16_t* src, uint8_t* dst) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float x0 = bf16_to_f32(src[128 * wave + lane]);
  const float x1 = bf16_to_f32(src[128 * wave + 64 + lane]);
  quantize_key_wave(x0, x1, 128, dst + 128 * wave, reinterpret_cast<float*>(dst + 512 + 4 * wave));
  if (wave == 0 && lane < 8) st16(dst + 528 + 16 * lane, ld16(src + 512 + 8 * lane));
}

__global__ __launch_bounds__(256) void quantize_latent_kernel(const uint16_t* __restrict__ lat, int64_t ss, int64_t ts,
                                                              uint8_t* __restrict__ out, int64_t oss, int64_t ots,
                                                              int64_t t0) {
  const int64_t t = t0 + blockIdx.x;
  const int s = blockIdx.y;
  quantize_latent_row(lat + s * ss + t * ts, out + s * oss + t * ots);
}

// One work-group per appended token (query i): copies the token's K and V
// rows (every kv head) and its raw indexer key into the cache at position
// q_pos[i] of sequence q_seq[i]; when the token completes a block, also
// writes the block's pooled key with pool_kernel's arithmetic (exact fp64
// sum of the block's raw keys, mean rounded once to bf16). The block's
// earlier tokens are read from the cache and the new one from its input
// row, so the pooled key never depends on a store of this launch.
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int i = blockIdx.x, tid = threadIdx.x;
  const int seq = a.q_seq ? a.q_seq[i] : i;
  const int pos = a.q_pos[i];
  if (pos < 0 || pos >= a.capacity) return;  // a caller error: nothing is written
  int kc = a.k_row / 8;
  const int vc = a.v_row / 8, rc = a.dim / 8;
  const uint16_t* kn = a.k_new + int64_t(i) * a.k_row;
  const uint16_t* vn = a.v_new ? a.v_new + int64_t(i) * a.v_row : nullptr;
  const uint16_t* rn = a.raw_new ? a.raw_new + int64_t(i) * a.dim : nullptr;
  if (a.kv_fp8) {  // one FP8 sparse-MLA row (strides in bytes)
    quantize_latent_row(kn, reinterpret_cast<uint8_t*>(a.k) + int64_t(seq) * a.seq_stride + int64_t(pos) * a.tok_stride);
    kc = 0;  // written
  }
  // rows of one token: kv head g at k + tok * tok_stride + g * head_stride
  for (int c = tid; c < kc; c += 256) {
    const int g = (8 * c) / a.head_dim, d = (8 * c) % a.head_dim;
    st16(a.k + int64_t(seq) * a.seq_stride + int64_t(pos) * a.tok_stride + int64_t(g) * a.head_stride + d,
         ld16(kn + 8 * c));
  }
  if (vn) {
    for (int c = tid; c < vc; c += 256) {
      const int g = (8 * c) / a.v_dim, d = (8 * c) % a.v_dim;
      st16(a.v + int64_t(seq) * a.seq_stride + int64_t(pos) * a.tok_stride + int64_t(g) * a.head_stride + d,
           ld16(vn + 8 * c));
    }
  }
  if (!rn) return;
  if (a.raw_fp8) {  // the token's indexer key, quantized into FP8 pages (wave 0; dim <= 128)
    if (tid < 64) {
      const float x0 = tid < a.dim ? bf16_to_f32(rn[tid]) : 0.f;
      const float x1 = tid + 64 < a.dim ? bf16_to_f32(rn[tid + 64]) : 0.f;
      uint8_t* base = reinterpret_cast<uint8_t*>(a.raw) + int64_t(seq) * a.raw_ss;
      quantize_key_wave(x0, x1, a.dim, base + fp8_code_off(pos, a.dim),
                        reinterpret_cast<float*>(base + fp8_scale_off(pos, a.dim)));
    }
    return;
  }
  for (int c = tid; c < rc; c += 256)
    st16(a.raw + int64_t(seq) * a.raw_ss + int64_t(pos) * a.dim + 8 * c, ld16(rn + 8 * c));
  if (!a.pooled || (pos + 1) % a.block != 0) return;
  const int64_t b = pos / a.block;
  if (a.pooled_fp8) {
    // the bf16 pooled key as below, then quantized (wave 0; dim <= 128)
    if (tid >= 64) return;
    const int lane = tid;
    float x[2] = {0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const int d = lane + 64 * h;
      if (d < a.dim) {
        double acc = double(bf16_to_f32(rn[d]));
        for (int j = 0; j < a.block - 1; j++)
          acc += double(bf16_to_f32(a.raw[int64_t(seq) * a.raw_ss + (b * a.block + j) * a.dim + d]));
        x[h] = bf16_to_f32(f64_to_bf16(acc / a.block));
      }
    }
    uint8_t* base = static_cast<uint8_t*>(a.pooled) + int64_t(seq) * a.pooled_ss;
    quantize_key_wave(x[0], x[1], a.dim, base + fp8_code_off(b, a.dim),
                      reinterpret_cast<float*>(base + fp8_scale_off(b, a.dim)));
    return;
  }
  for (int c = tid; c < rc; c += 256) {
    double acc[8];
    u32x4 w = ld16(rn + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; e++) {
      acc[2 * e] = double(bf16_lo(w[e]));
      acc[2 * e + 1] = double(bf16_hi(w[e]));
    }
    for (int j = 0; j < a.block - 1; j++) {
      w = ld16(a.raw + int64_t(seq) * a.raw_ss + (b * a.block + j) * a.dim + 8 * c);
#pragma unroll
      for (int e = 0; e < 4; e++) {
        acc[2 * e] += double(bf16_lo(w[e]));
        acc[2 * e + 1] += double(bf16_hi(w[e]));
      }
    }
    u32x4 out;
#pragma unroll
    for (int e = 0; e < 4; e++)
      out[e] = uint32_t(f64_to_bf16(acc[2 * e] / a.block)) | (uint32_t(f64_to_bf16(acc[2 * e + 1] / a.block)) << 16);
    st16(static_cast<uint16_t*>(a.pooled) + int64_t(seq) * a.pooled_ss + b * a.dim + 8 * c, out);
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.nq <= 0) return hipSuccess;
  hipLaunchKernelGGL(append_kernel, dim3(unsigned(a.nq)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t* keys, int64_t keys_ss, uint8_t* out, int64_t out_ss, int n_seq,
                           int64_t k0, int64_t nk, int dim, hipStream_t s) {
  if (nk <= 0 || n_seq <= 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_kernel, dim3(unsigned((nk + 3) / 4), unsigned(n_seq)), dim3(256), 0, s, keys, keys_ss,
                     out, out_ss, k0, nk, dim);
  return hipGetLastError();
}

hipError_t launch_quantize_latent(const uint16_t* lat, int64_t ss, int64_t ts, uint8_t* out, int64_t oss, int64_t ots,
                                  int n_seq, int64_t t0, int64_t nt, hipStream_t s) {
  if (nt <= 0 || n_seq <= 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_latent_kernel, dim3(unsigned(nt), unsigned(n_seq)), dim3(256), 0, s, lat, ss, ts, out,
                     oss, ots, t0);
  return hipGetLastError();
}

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
