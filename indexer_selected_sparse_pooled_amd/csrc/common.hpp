// Device helpers shared by the libqsa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (NaN -> quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Order-preserving map fp32 -> uint32: a > b  <=>  key(a) > key(b);
// -0.0 and +0.0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Loads and stores that are coherent across the L2 caches of all XCDs
// (agent scope, "sc1"): data handed from one work-group to another inside a
// launch goes through these, so no L2 write-back or invalidate is needed.
__device__ __forceinline__ void st_coherent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_coherent(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_coherent(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory access this thread issued has completed
// (s_waitcnt vmcnt(0)); coherent stores are then visible chip-wide.
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Device-scope counters (work-group hand-off) sit kCounterStride words
// apart, one per 256-byte line, so that counters of different queries or
// heads never share a line.
constexpr int kCounterStride = 64;

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

// a.x*b.x + a.y*b.y + c (bf16 pairs, fp32 accumulate)
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a), as_bf16x2(b), c, false);
}

__device__ __forceinline__ int clamp_ctx(int c, int max_ctx) {
  return c < 0 ? 0 : (c > max_ctx ? max_ctx : c);
}

// Cross-lane moves through DPP, without an LDS round trip (gfx9 controls:
// row_shr:n = 0x110 + n, row_bcast:15 = 0x142, row_bcast:31 = 0x143).
// Lanes outside kRowMask, and lanes whose source is out of range when
// kZero is false, return `old`; with kZero they read 0 instead.
template <int kCtrl, int kRowMask = 0xf, bool kZero = false>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(int(old), int(v), kCtrl, kRowMask, 0xf, kZero));
}

// Inclusive prefix sum over the 64 lanes of a wave: a scan within each row
// of 16 lanes, then the totals of rows 0 and 2 are added to rows 1 and 3,
// and the total of rows 0-1 to rows 2-3.
__device__ __forceinline__ int wave_incl_sum(int x) {
  x += int(dpp<0x111, 0xf, true>(0u, uint32_t(x)));
  x += int(dpp<0x112, 0xf, true>(0u, uint32_t(x)));
  x += int(dpp<0x114, 0xf, true>(0u, uint32_t(x)));
  x += int(dpp<0x118, 0xf, true>(0u, uint32_t(x)));
  x += int(dpp<0x142, 0xa>(0u, uint32_t(x)));
  x += int(dpp<0x143, 0xc>(0u, uint32_t(x)));
  return x;
}

// Wave-wide maximum / minimum of unsigned values, the same steps with max or
// min in place of the sum (a lane with no source keeps its own value); lane
// 63 ends with the result, which is returned to every lane.
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
  v = op(v, dpp<0x111>(v, v));
  v = op(v, dpp<0x112>(v, v));
  v = op(v, dpp<0x114>(v, v));
  v = op(v, dpp<0x118>(v, v));
  v = op(v, dpp<0x142, 0xa>(v, v));
  v = op(v, dpp<0x143, 0xc>(v, v));
  return uint32_t(__builtin_amdgcn_readlane(int(v), 63));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  auto step = [](uint64_t x, uint32_t hi, uint32_t lo) {
    const uint64_t o = (uint64_t(hi) << 32) | lo;
    return o > x ? o : x;
  };
  v = step(v, dpp<0x111>(uint32_t(v >> 32), uint32_t(v >> 32)), dpp<0x111>(uint32_t(v), uint32_t(v)));
  v = step(v, dpp<0x112>(uint32_t(v >> 32), uint32_t(v >> 32)), dpp<0x112>(uint32_t(v), uint32_t(v)));
  v = step(v, dpp<0x114>(uint32_t(v >> 32), uint32_t(v >> 32)), dpp<0x114>(uint32_t(v), uint32_t(v)));
  v = step(v, dpp<0x118>(uint32_t(v >> 32), uint32_t(v >> 32)), dpp<0x118>(uint32_t(v), uint32_t(v)));
  v = step(v, dpp<0x142, 0xa>(uint32_t(v >> 32), uint32_t(v >> 32)), dpp<0x142, 0xa>(uint32_t(v), uint32_t(v)));
  v = step(v, dpp<0x143, 0xc>(uint32_t(v >> 32), uint32_t(v >> 32)), dpp<0x143, 0xc>(uint32_t(v), uint32_t(v)));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v >> 32)), 63));
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v)), 63));
  return (uint64_t(hi) << 32) | lo;
}

// Reductions over each row of 16 lanes, every lane getting its row's
// result, through DPP (no LDS round trip): lanes xor 1 and xor 2 by quad
// permutes, then the other quads of the row by rotations of 4 and 8.
// (gfx9 controls: quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E,
// row_ror:4 = 0x124, row_ror:8 = 0x128.)
__device__ __forceinline__ float dppf(float v, int ctrl) {
  switch (ctrl) {
    case 0xB1: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xf, 0xf, false));
    case 0x4E: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xf, 0xf, false));
    case 0x124: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xf, 0xf, false));
    default: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
  }
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dppf(v, 0xB1));
  v = fmaxf(v, dppf(v, 0x4E));
  v = fmaxf(v, dppf(v, 0x124));
  return fmaxf(v, dppf(v, 0x128));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dppf(v, 0xB1);
  v += dppf(v, 0x4E);
  v += dppf(v, 0x124);
  return v + dppf(v, 0x128);
}

// Wave-wide reductions (64 lanes).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

}  // namespace qsa
