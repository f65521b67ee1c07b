// The decode scan tile of the token-level indexer (variant B): 64-d token
// keys, 4 indexer heads, score = sum_h w_h ReLU(q_h . k) ("GLM-5.3 最適化
// 第2部", section "PCP", for the indexer; shared by the stand-alone scan and
// the one-call decode layer).
//
// A wave owns 128 consecutive keys (16 KiB); lane (g = lane / 8, c = lane %
// 8) loads dims [8c, 8c + 8) of keys 8k + g, k = 0 .. 15; after the
// butterfly over the 8 lanes of a group it holds the 4 head dots of keys
// 8 (2c + j) + g, j = 0, 1, and weighs them. kFp8: FP8 token keys (pages of
// 64 keys of 64 codes + scales): each lane reads its 8 codes, converts them
// to bf16 exactly, and the key's scale multiplies the final score (ReLU
// commutes with a non-negative scale).
#pragma once

#include "common.hpp"
#include "fp8.hpp"
#include "kernels.hpp"

namespace qsa {
namespace sb {

// the key of lane `lane`'s score j in the tile starting at tile0
__device__ __forceinline__ int64_t tile_token(int64_t tile0, int lane, int j) {
  return tile0 + 8 * (2 * (lane & 7) + j) + (lane >> 3);
}

__device__ __forceinline__ float dot8(u32x4 k, u32x4 q) {
  float acc = 0.f;
  acc = dot2(k[0], q[0], acc);
  acc = dot2(k[1], q[1], acc);
  acc = dot2(k[2], q[2], acc);
  acc = dot2(k[3], q[3], acc);
  return acc;
}

// s[j]: the score of key tile_token(tile0, lane, j) of query i (sequence
// seq, n keys, tile0 < n); keys past n score 0. Lanes whose key is past n
// load key n - 1 instead (no branch per load, so all 16 loads are in
// flight together) and their scores are dropped at the end.
template <bool kFp8>
__device__ __forceinline__ void tile_scores(const ScoreArgs& a, int i, int seq, int64_t n, int64_t tile0,
                                            float (&s)[2]) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 3, c = lane & 7;
  u32x4 qv[4];
  float w[4];
#pragma unroll
  for (int h = 0; h < 4; h++) {
    qv[h] = ld16(a.q_idx + (int64_t(i) * 4 + h) * 64 + 8 * c);
    w[h] = a.w_idx[int64_t(i) * 4 + h];
  }
  const uint16_t* kb = static_cast<const uint16_t*>(a.keys) + int64_t(seq) * a.keys_ss;
  const uint8_t* kb8 = static_cast<const uint8_t*>(a.keys) + int64_t(seq) * a.keys_ss;
  const int64_t last = n - 1;
  u32x4 kv[16];
  u32x2 kc[16];
#pragma unroll
  for (int k = 0; k < 16; k++) {
    const int64_t tok = tile0 + 8 * k + g;
    const int64_t tc = tok < n ? tok : last;
    if constexpr (kFp8)
      kc[k] = *reinterpret_cast<const u32x2*>(kb8 + fp8_code_off(tc, 64) + 8 * c);
    else
      kv[k] = ld16_nt(kb + tc * 64 + 8 * c);
  }
  float p[16][4];
#pragma unroll
  for (int k = 0; k < 16; k++) {
    u32x4 v;
    if constexpr (kFp8)
      v = __builtin_bit_cast(u32x4, e4m3x8_bf16(kc[k]));
    else
      v = kv[k];
#pragma unroll
    for (int h = 0; h < 4; h++) p[k][h] = dot8(v, qv[h]);
  }
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const bool up = c & 4;
#pragma unroll
    for (int h = 0; h < 4; h++) {
      const float keep = up ? p[j + 8][h] : p[j][h];
      const float send = up ? p[j][h] : p[j + 8][h];
      p[j][h] = keep + __shfl_xor(send, 4);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const bool up = c & 2;
#pragma unroll
    for (int h = 0; h < 4; h++) {
      const float keep = up ? p[j + 4][h] : p[j][h];
      const float send = up ? p[j][h] : p[j + 4][h];
      p[j][h] = keep + __shfl_xor(send, 2);
    }
  }
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const bool up = c & 1;
#pragma unroll
    for (int h = 0; h < 4; h++) {
      const float keep = up ? p[j + 2][h] : p[j][h];
      const float send = up ? p[j][h] : p[j + 2][h];
      p[j][h] = keep + __shfl_xor(send, 1);
    }
  }
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int64_t tok = tile_token(tile0, lane, j);
    float v = 0.f;
#pragma unroll
    for (int h = 0; h < 4; h++) v += w[h] * fmaxf(p[j][h], 0.f);
    if constexpr (kFp8) v *= *reinterpret_cast<const float*>(kb8 + fp8_scale_off(tok < n ? tok : last, 64));
    s[j] = tok < n ? v : 0.f;
  }
}

}  // namespace sb
}  // namespace qsa
