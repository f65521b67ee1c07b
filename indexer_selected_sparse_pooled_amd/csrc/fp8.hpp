// FP8 indexer keys: layout and device helpers.
// "GLM-5.3 最適化 第2部", footnote 3: an FP8 indexer key is its FP8 values
// plus a 4-byte scale (128 values: 132 bytes per key). Values are OCP E4M3
// (gfx950's FP8 conversions use this format); a key's fp32 scale is its
// largest magnitude / 448 and it stands for code * scale.
//
// Layout: keys are stored in pages of 64; a page holds the 64 keys' codes
// (dim bytes each, key-major) followed by their 64 fp32 scales, so every
// key costs dim + 4 bytes and every array stays 16-byte aligned. Key b of a
// sequence sits in page b / 64, slot b % 64.
#pragma once

#include "common.hpp"

namespace qsa {

constexpr int kFp8PageKeys = 64;
constexpr float kE4m3Max = 448.f;

__host__ __device__ __forceinline__ int64_t fp8_page_bytes(int dim) { return int64_t(kFp8PageKeys) * (dim + 4); }
// bytes that hold keys [0, n) (whole pages)
__host__ __device__ __forceinline__ int64_t fp8_keys_bytes(int64_t n, int dim) {
  return (n + kFp8PageKeys - 1) / kFp8PageKeys * fp8_page_bytes(dim);
}
__host__ __device__ __forceinline__ int64_t fp8_code_off(int64_t b, int dim) {
  return (b / kFp8PageKeys) * fp8_page_bytes(dim) + (b % kFp8PageKeys) * dim;
}
__host__ __device__ __forceinline__ int64_t fp8_scale_off(int64_t b, int dim) {
  return (b / kFp8PageKeys) * fp8_page_bytes(dim) + int64_t(kFp8PageKeys) * dim + (b % kFp8PageKeys) * 4;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Four E4M3 codes (bytes of w, low first) as floats, exactly.
__device__ __forceinline__ void e4m3x4(uint32_t w, float& a, float& b, float& c, float& d) {
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(w), false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(w), true);
  a = lo.x;
  b = lo.y;
  c = hi.x;
  d = hi.y;
}

// The E4M3 code nearest to x (ties to even), magnitudes past 448 saturating.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const float c = fminf(fmaxf(x, -kE4m3Max), kE4m3Max);
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false)) & 0xFFu;
}

// Eight E4M3 codes as a bf16 B operand (exact: an E4M3 value has 4
// significant bits and lies within bf16's exponent range).
__device__ __forceinline__ bf16x8 e4m3x8_bf16(u32x2 w) {
  float f[8];
  e4m3x4(w[0], f[0], f[1], f[2], f[3]);
  e4m3x4(w[1], f[4], f[5], f[6], f[7]);
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; j++) r[j] = (__float_as_uint(f[2 * j]) >> 16) | (__float_as_uint(f[2 * j + 1]) & 0xFFFF0000u);
  return __builtin_bit_cast(bf16x8, r);
}

namespace fp8 {

// A tile is 64 consecutive keys of 128 dims (one page when tile0 is a
// multiple of 64). Lane (g, c) = (lane / 8, lane % 8) reads bytes 16c ..
// 16c+15 of keys tile0 + 8k + g, k = 0..7 (each instruction covers 1 KiB of
// consecutive codes), and its own key's scale. Keys past n are clamped to
// n - 1 (read, then ignored), so the loads carry no branch.
__device__ __forceinline__ void load_tile(const uint8_t* kb, int64_t tile0, int64_t n, u32x4 (&v)[8], float& sc) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 3, c = lane & 7;
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const int64_t blk = tile0 + 8 * k + g;
    v[k] = ld16_nt(kb + fp8_code_off(blk < n ? blk : n - 1, 128) + 16 * c);
  }
  const int64_t own = tile0 + lane < n ? tile0 + lane : n - 1;
  sc = __builtin_nontemporal_load(reinterpret_cast<const float*>(kb + fp8_scale_off(own, 128)));
  __builtin_amdgcn_sched_barrier(0);
}

// The query's dims 16c .. 16c+15 (c = lane % 8) as floats.
__device__ __forceinline__ void load_query(const uint16_t* q, float (&qf)[16]) {
  const int c = threadIdx.x & 7;
  const u32x4 a = ld16(q + 16 * c), b = ld16(q + 16 * c + 8);
#pragma unroll
  for (int j = 0; j < 4; j++) {
    qf[2 * j] = bf16_lo(a[j]);
    qf[2 * j + 1] = bf16_hi(a[j]);
    qf[8 + 2 * j] = bf16_lo(b[j]);
    qf[8 + 2 * j + 1] = bf16_hi(b[j]);
  }
}

// Scores of the tile (keys past n score 0): lane l returns
// scale(key tile0 + l) * (q . codes(key tile0 + l)); the dot is accumulated
// in fp32 from exact products.
__device__ __forceinline__ float tile_scores(const u32x4 (&v)[8], float sc, int64_t tile0, int64_t n,
                                             const float (&qf)[16]) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 3, c = lane & 7;
  float p[8];
#pragma unroll
  for (int k = 0; k < 8; k++) {
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; w++) {
      float x0, x1, x2, x3;
      e4m3x4(v[k][w], x0, x1, x2, x3);
      acc = fmaf(x0, qf[4 * w], acc);
      acc = fmaf(x1, qf[4 * w + 1], acc);
      acc = fmaf(x2, qf[4 * w + 2], acc);
      acc = fmaf(x3, qf[4 * w + 3], acc);
    }
    p[k] = tile0 + 8 * k + g < n ? acc : 0.f;
  }
  // transposing butterfly over the 8 lanes of a group: afterwards lane
  // (g, c) holds the full dot product of key 8c + g
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const bool up = c & 4;
    const float keep = up ? p[j + 4] : p[j];
    const float send = up ? p[j] : p[j + 4];
    p[j] = keep + __shfl_xor(send, 4);
  }
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const bool up = c & 2;
    const float keep = up ? p[j + 2] : p[j];
    const float send = up ? p[j] : p[j + 2];
    p[j] = keep + __shfl_xor(send, 2);
  }
  {
    const bool up = c & 1;
    const float keep = up ? p[1] : p[0];
    const float send = up ? p[0] : p[1];
    p[0] = keep + __shfl_xor(send, 1);
  }
  // key l = 8c + g sits in lane 8 * (l % 8) + l / 8
  return __shfl(p[0], 8 * (lane & 7) + (lane >> 3)) * sc;
}

}  // namespace fp8
}  // namespace qsa
