// Device code of A4 / A6 for the shared-latent variant: 64 query heads attend
// one 576-wide bf16 latent row per selected token; the first 512 columns of
// the same row serve as V.
// "GLM-5.3 最適化 第2部：16基のH200上でのPCP、DCP、およびHybrid HiSparse",
// section "PCP" (the indexer picks 2,048 tokens per query for sparse MLA;
// the latent is shared by all 64 heads) and footnote 1 (576-d QK, 512-d PV
// per latent row); section "DCP" (partials combined by log-sum-exp).
//
// Every gathered row serves all 64 heads, so here the contractions are
// dense enough for MFMA to matter (about 120 FLOP per gathered byte). One
// work-group per (query, split); wave w owns heads 16w .. 16w+15 and keeps
// their 576-d queries in registers as MFMA A operands. The part's token list
// is walked in tiles of 32 tokens:
//   * the 32 latent rows go straight from global memory to LDS
//     (global_load_lds_dwordx4) with a row stride of 74 x 16 bytes, so rows
//     that are read together fall on different banks (the two-buffer form
//     below: 66 x 16-byte rows of the first 512 columns and a separate
//     region for the 64 rotary columns);
//   * S = Q K^T on MFMA 16x16x32 bf16, B operands read from LDS (18 k-steps
//     of 32 per 16-token half);
//   * online softmax per head on the MFMA result layout (each wave its own
//     heads, no barrier);
//   * O += P V on MFMA 16x16x32: P as bf16 hi + lo parts (two MFMAs, ~16
//     significant bits) through a per-wave LDS tile, V read transposed from
//     the same LDS rows with ds_read_tr16_b64; each wave accumulates 16
//     heads x 512 dims.
// Output: normalised partial O (fp32) and natural-log lse per head.
#pragma once

#include <cfloat>

#include "attend.hpp"
#include "fp8.hpp"

namespace qsa {
namespace mla {

constexpr int kH = 64;      // query heads
constexpr int kDK = 576;    // latent row (QK)
constexpr int kDV = 512;    // V columns (first kDV of the row)
constexpr int kTT = 32;     // tokens per tile
constexpr int kRowC = kDK / 8;          // 16-byte chunks per latent row (72)
// LDS chunks per row incl. two pad chunks (74). gfx950's LDS serves a
// 16-byte read of 32 lanes per cycle from 128 four-byte banks: the 32
// chunks must fall on distinct (chunk mod 32). The MFMA operand reads take
// rows r = 0..15 at chunks c and c + 1 in one half-wave, and 74 r mod 32
// (= 10 r) runs over 16 distinct even values, so the two columns never
// meet; the transposed V reads (rows 4kq + r/4, 32 bytes each) land on 16
// distinct multiples of 4 eight-byte units. With 73 both were 2-way
// conflicts (measured: 49.6% of LDS cycles).
constexpr int kRowL = kRowC + 2;
constexpr int kNTPART = 256;             // threads of every shared-latent attention work-group
constexpr int kTileC = kTT * kRowL;     // LDS chunks per tile (2368)
constexpr int kPStr = kTT + 8;          // LDS row of P in elements (80 bytes)
constexpr float kLazyMax = 8.f;         // log2 headroom of a head's softmax reference (bf16 and FP8 rows)

struct Lds {
  __attribute__((aligned(16))) unsigned char kv[kTileC * 16];
  __attribute__((aligned(16))) uint16_t p[4][2][16 * kPStr];  // per wave: P hi, lo [head][token]
  int cnt[kNTPART / 64];
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <bool kCoh>
__device__ void attend_part(const AttendArgs& a, int split, int i, Lds& sh) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, kq = lane >> 4;

  const int seq = a.q_seq ? a.q_seq[i] : 0;
  const int ctx = clamp_ctx(a.q_ctx[i], a.max_ctx);
  att::List<kCoh> lv;
  lv.sel = a.sel + int64_t(i) * a.topk;
  lv.block = a.block;
  lv.nblk = ctx / a.block;
  const int ns_max = lv.nblk < a.topk ? lv.nblk : a.topk;
  const int ns = kCoh ? ns_max : a.n_sel[i];
  lv.ns = ns < 0 ? 0 : (ns > ns_max ? ns_max : ns);
  lv.L = lv.ns * a.block + (ctx - lv.nblk * a.block);
  int P0_, P1_;
  att::part_range<kCoh, kNTPART>(lv, a, split, ctx, sh.cnt, P0_, P1_);
  const int P0 = P0_, P1 = P1_;

  const uint16_t* kvbase = a.k + int64_t(seq) * a.seq_stride;
  const float sl2 = a.scale * kLog2e;

  // A operands: Q[head 16*wave + r][32*ks + 8*kq .. +7]
  bf16x8 qa[kDK / 32];
  {
    const uint16_t* qrow = a.q + (int64_t(i) * kH + 16 * wave + r) * kDK + 8 * kq;
#pragma unroll
    for (int ks = 0; ks < kDK / 32; ks++) qa[ks] = as_bf16x8(ld16(qrow + 32 * ks));
  }

  float m[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; e++) {
    m[e] = -INFINITY;
    l[e] = 0.f;
  }
  f32x4 o[kDV / 16];
#pragma unroll
  for (int nt = 0; nt < kDV / 16; nt++) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint16_t* phi = sh.p[wave][0];
  uint16_t* plo = sh.p[wave][1];

  for (int pb = P0; pb < P1; pb += kTT) {
    const int cnt = (P1 - pb) < kTT ? (P1 - pb) : kTT;
    // lane l < 32 holds the token of tile row l (rows past cnt repeat row 0)
    const int tokl = lv.tok(pb + ((lane & 31) < cnt ? (lane & 31) : 0));
    // latent rows -> LDS: wave instruction slot s covers LDS chunks 64s .. 64s+63
    for (int s = wave; s * 64 < kTileC; s += 4) {
      const int c = 64 * s + lane;
      const int row = c / kRowL, col = c % kRowL;
      const int rt = __shfl(tokl, row < kTT ? row : 0);
      if (c < kTileC) {
        const int cc = col < kRowC ? col : 0;  // the pad chunk takes a copy of chunk 0
        __builtin_amdgcn_global_load_lds(kvbase + int64_t(rt) * a.tok_stride + 8 * cc,
                                         (__attribute__((address_space(3))) void*)(sh.kv + 1024 * s), 16, 0, 0);
      }
    }
    wait_memory();
    __syncthreads();
    // S = Q K^T for the two 16-token halves: lane (kq, r) holds S[head 4kq+e][token 16h + r]
    f32x4 acc[2];
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
      acc[hf] = f32x4{0.f, 0.f, 0.f, 0.f};
      const unsigned char* krow = sh.kv + ((16 * hf + r) * kRowL + kq) * 16;
#pragma unroll
      for (int ks = 0; ks < kDK / 32; ks++) {
        const bf16x8 kb = as_bf16x8(*reinterpret_cast<const u32x4*>(krow + 64 * ks));
        acc[hf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kb, acc[hf], 0, 0, 0);
      }
    }
    // online softmax per head over the tile's 32 tokens (16 lanes x 2 halves)
    float alpha[4];
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const float s0 = r < cnt ? acc[0][e] * sl2 : -INFINITY;
      const float s1 = 16 + r < cnt ? acc[1][e] * sl2 : -INFINITY;
      const float tm = row16_max(fmaxf(s0, s1));
      const float mn = fmaxf(m[e], tm);
      float p0 = 0.f, p1 = 0.f;
      alpha[e] = 1.f;
      if (mn != -INFINITY) {
        p0 = exp2f(s0 - mn);
        p1 = exp2f(s1 - mn);
        alpha[e] = exp2f(m[e] - mn);
      }
      const float ps = row16_sum(p0 + p1);
      l[e] = l[e] * alpha[e] + ps;
      m[e] = mn;
      const int row = 4 * kq + e;
      const uint16_t h0 = f32_to_bf16(p0), h1 = f32_to_bf16(p1);
      phi[row * kPStr + r] = h0;
      phi[row * kPStr + 16 + r] = h1;
      plo[row * kPStr + r] = f32_to_bf16(p0 - bf16_to_f32(h0));
      plo[row * kPStr + 16 + r] = f32_to_bf16(p1 - bf16_to_f32(h1));
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int nt = 0; nt < kDV / 16; nt++)
#pragma unroll
      for (int e = 0; e < 4; e++) o[nt][e] *= alpha[e];
    // O += P V: A = P[head r][tokens 8kq .. 8kq+7]; B = V[token 8kq + j][dim 16nt + r]
    const bf16x8 ah = as_bf16x8(*reinterpret_cast<const u32x4*>(phi + r * kPStr + 8 * kq));
    const bf16x8 al = as_bf16x8(*reinterpret_cast<const u32x4*>(plo + r * kPStr + 8 * kq));
    const unsigned char* vb0 = sh.kv + (8 * kq + (r >> 2)) * kRowL * 16 + 8 * (r & 3);
#pragma unroll
    for (int nt = 0; nt < kDV / 16; nt++) {
      s16x4 t[2];
#pragma unroll
      for (int hh = 0; hh < 2; hh++)
        t[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vb0 + 4 * hh * kRowL * 16 + 32 * nt));
      const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3, 4, 5, 6, 7));
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bv, o[nt], 0, 0, 0);
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bv, o[nt], 0, 0, 0);
      // keep the transposed reads in groups of 8 n-tiles (registers)
      if (nt % 8 == 7) __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();  // the tile's rows are read; the next tile may overwrite them
  }

  // normalise and write the partial result: heads 16*wave + 4kq + e
  const int64_t orow0 = (int64_t(split) * a.nq + i) * kH + 16 * wave;
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const int hrow = 4 * kq + e;
    const float inv = l[e] > 0.f ? 1.f / l[e] : 0.f;
    float* op = a.o_part + (orow0 + hrow) * kDV + r;
#pragma unroll
    for (int nt = 0; nt < kDV / 16; nt++) op[16 * nt] = o[nt][e] * inv;
    if (r == 0) a.lse_part[orow0 + hrow] = l[e] > 0.f ? (m[e] + log2f(l[e])) * kLn2 : -INFINITY;
  }
}

// Barrier without a memory fence (a fence would wait for the gathers in
// flight): each wait for data is an explicit s_waitcnt, and an empty asm with
// a memory clobber keeps the compiler from moving LDS accesses across.
__device__ __forceinline__ void pipe_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---- transposed form, two tile buffers: attend_part_t
// S^T = K Q^T (K rows from LDS as the A operand, the wave's 16 queries as
// the B operand), so after the MFMA lane (kq, r) holds the scores of head r
// for tokens 4kq + e and 16 + 4kq + e (e < 4). The softmax of head r runs
// on its lane column (row reductions across the four 16-lane rows with
// permlane swaps), and the lane's eight probabilities are, as they stand,
// the B operand of O^T += V^T P^T when the 32 tokens of the tile enter the
// contraction in the order {4kq .. 4kq+3, 16+4kq .. 16+4kq+3} for k-group
// kq; V^T is read in that order by the transposed LDS reads. P never goes
// through LDS, so a work-group needs only its tile buffers: two (75 KB), one
// tile gathered while the other is computed, and two work-groups per CU.
// The selection entries of a tile also arrive by LDS DMA, two tiles ahead,
// so no register load (and no wait for it) sits in the loop. Per tile t:
// wait for everything this wave has in flight (tile t's rows, the entries of
// tile t + 1), barrier (tile t visible to all; everyone done with tile
// t - 1), gather tile t + 1 into the other buffer and the entries of tile
// t + 2 into the entry slot tile t used, then compute tile t without
// waiting for either.
constexpr int kSelSlot = 64;  // selection entries per slot (one wave instruction)

struct LdsT {
  __attribute__((aligned(16))) unsigned char kv[2][kTileC * 16];
  int selbuf[2][kSelSlot];
  float lsum[kH];
  int cnt[kNTPART / 64];
};

// max of a and b, both finite or -inf, as one med3 against FLT_MAX (fmaxf
// would first canonicalise both operands of the lane swap)
__device__ __forceinline__ float max2(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, FLT_MAX); }
__device__ __forceinline__ float rows_max(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = max2(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max2(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// A part's list for token-level selection (block 1: list entry p is the
// selected token sel[p], no trailing tokens): its selection row from P0 on.
struct TList {
  const int* sel;  // the query's selection row (topk entries)
  int topk, ctx, P0, n_list;
  bool dma_sel = true;  // entries gathered by sel_dma (else already in LDS)
  // token of row j of tile t, from the entries of the tile (clamped into the context)
  __device__ __forceinline__ int tok(const int* ent, int j) const {
    const int b = ent[j];
    return b < 0 ? 0 : (b >= ctx ? ctx - 1 : b);
  }
  __device__ __forceinline__ int cnt(int t) const {
    const int c = n_list - kTT * t;
    return c <= 0 ? 0 : (c < kTT ? c : kTT);
  }
};

struct TLane {
  int wave, lane, r, kq;
};

// DMA of the selection entries of tile t into a slot (wave 0; the entries
// past the row are clamped to its last one and never used).
__device__ __forceinline__ void sel_dma(const TLane& tl, const TList& ls, int t, int* slot) {
  if (!ls.dma_sel || tl.wave != 0 || ls.cnt(t) == 0) return;
  int e = ls.P0 + kTT * t + tl.lane;
  e = e < ls.topk ? e : ls.topk - 1;
  __builtin_amdgcn_global_load_lds(ls.sel + e, (__attribute__((address_space(3))) void*)slot, 4, 0, 0);
}

// Tile layout of the two-buffer form: the first 512 columns (64 chunks, V
// and the first 16 k-steps of K) of row j at j * kRowM chunks, then the
// rotary tails (chunks 64 .. 71) of all 32 rows, 8 chunks per row, chunk c
// of row j at position c ^ tail_swz(j). Bank model as above: 66 j mod 32 =
// 2 j, so the K reads of rows r = 0..15 at chunks c and c + 1 fall on 32
// distinct (chunk mod 32), and the transposed V reads of rows 4kq + r/4 on
// 16 distinct multiples of 4 eight-byte units; in the tail region the
// swizzle spreads the 4 rows that share (8 j mod 32) over 4 chunk pairs.
// The buffer is exactly as large as 32 rows at kRowL chunks.
constexpr int kMainC = 64;                     // chunks of columns 0 .. 511
constexpr int kRowM = kMainC + 2;              // LDS chunks per row in the main region (1056 bytes)
constexpr int kTailC = kRowC - kMainC;         // 8 chunks of columns 512 .. 575
constexpr int kTailOff = kTT * kRowM * 16;     // byte offset of the tail region
static_assert(kTailOff + kTT * kTailC * 16 <= kTileC * 16, "main rows and tails fit one tile buffer");
__device__ __forceinline__ int tail_swz(int j) { return 2 * ((j >> 2) & 3); }

// DMA of the latent rows of tile t into a buffer, tokens from its entries.
// Wave w gathers rows 8w .. 8w+7: per row, the first 1024 bytes in one wave
// instruction whose token is the same on every lane (lane l loads chunk l),
// so the address is a scalar base plus the lane's offset; then the 8 rows'
// tails in one more instruction (lane l: row 8w + l / 8, tail position
// l % 8). Rows past the tile's count repeat its last row (they are never
// weighted, but their values must be finite); tokens are clamped into
// [0, ctx).
__device__ __forceinline__ void rows_dma(const TLane& tl, const TList& ls, int t, const int* __restrict__ ent,
                                         unsigned char* __restrict__ buf, const uint16_t* kvbase,
                                         int64_t tok_stride) {
  const int n = ls.cnt(t);
  if (n == 0) return;
  const unsigned char* gb = reinterpret_cast<const unsigned char*>(kvbase);
  const uint64_t row_bytes = uint64_t(tok_stride) * 2u;
  // (the wave index through readfirstlane: the compiler then keeps the LDS
  // destinations, which the instruction takes from a scalar register, in
  // scalar arithmetic)
  const int lane = tl.lane, r8 = 8 * __builtin_amdgcn_readfirstlane(tl.wave);
  const int ra = r8 + (lane & 7) < n - 1 ? r8 + (lane & 7) : n - 1;  // rows of the row loads
  const int rb = r8 + (lane >> 3) < n - 1 ? r8 + (lane >> 3) : n - 1;  // row of the lane's tail chunk
  const int ta = ls.tok(ent, ra), tb = ls.tok(ent, rb);
  const int cb = kMainC + ((lane & 7) ^ tail_swz(r8 + (lane >> 3)));
  __builtin_amdgcn_global_load_lds(gb + (uint64_t(uint32_t(tb)) * row_bytes + 16u * uint32_t(cb)),
                                   (__attribute__((address_space(3))) void*)(buf + kTailOff + 128 * r8), 16, 0, 0);
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const uint32_t tk = uint32_t(__builtin_amdgcn_readlane(ta, k));
    const uint64_t rp = reinterpret_cast<uint64_t>(gb) + uint64_t(tk) * row_bytes;
    const uint64_t rs = uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(rp)))) |
                        (uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(rp >> 32)))) << 32);
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const unsigned char*>(rs) + 16u * uint32_t(lane),
                                     (__attribute__((address_space(3))) void*)(buf + (r8 + k) * (kRowM * 16)), 16, 0,
                                     0);
  }
}

// One tile: the gathers of tile t + 1 (rows into `nxt`, from the entries in
// `ent_next`) and of the entries of tile t + 2 (into `ent_free`), then the
// tile in `cur`. Every LDS buffer arrives as a __restrict__ pointer, so the
// compiler knows the DMA in flight does not write what this tile reads and
// does not make the reads wait for it.
__device__ __attribute__((always_inline)) inline void tile_t(
    const TLane& tl, const TList& ls, int t, const unsigned char* __restrict__ cur,
    unsigned char* __restrict__ nxt, const int* __restrict__ ent_next, int* __restrict__ ent_free,
    const uint16_t* kvbase, int64_t tok_stride, float sl2, const bf16x8 (&qa)[kDK / 32], float& m, float& l,
    f32x4 (&o)[kDV / 16]) {
  const int r = tl.r, kq = tl.kq;
  rows_dma(tl, ls, t + 1, ent_next, nxt, kvbase, tok_stride);
  sel_dma(tl, ls, t + 2, ent_free);
  const int cnt = ls.cnt(t);
  // S^T for the two 16-token halves, K operands read two k-steps ahead (the
  // group barriers keep the reads ahead of the MFMAs; left to itself the
  // compiler, short of registers, reads each operand just before its MFMA
  // and waits a full LDS latency at every k-step)
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  // k-steps 0 .. 15 from the main rows, 16 and 17 from the tails (chunks
  // kq and 4 + kq of rows r and 16 + r, which share tail_swz)
  const unsigned char* krow0 = cur + (r * kRowM + kq) * 16;
  const unsigned char* krow1 = cur + ((16 + r) * kRowM + kq) * 16;
  const int tq = kq ^ tail_swz(r);
  const unsigned char* ktail0 = cur + kTailOff + (r * kTailC) * 16;
  const unsigned char* ktail1 = ktail0 + 16 * kTailC * 16;
  constexpr int kPD = 2;
  bf16x8 kb[2][kPD + 1];
#pragma unroll
  for (int ks = 0; ks < kDK / 32 + kPD; ks++) {
    if (ks < kMainC / 4) {
      kb[0][ks % (kPD + 1)] = as_bf16x8(*reinterpret_cast<const u32x4*>(krow0 + 64 * ks));
      kb[1][ks % (kPD + 1)] = as_bf16x8(*reinterpret_cast<const u32x4*>(krow1 + 64 * ks));
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    } else if (ks < kDK / 32) {
      const int tc = 16 * (tq ^ (4 * (ks - kMainC / 4)));
      kb[0][ks % (kPD + 1)] = as_bf16x8(*reinterpret_cast<const u32x4*>(ktail0 + tc));
      kb[1][ks % (kPD + 1)] = as_bf16x8(*reinterpret_cast<const u32x4*>(ktail1 + tc));
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    if (ks >= kPD) {
      const int k = ks - kPD;
      acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[0][k % (kPD + 1)], qa[k], acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[1][k % (kPD + 1)], qa[k], acc[1], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
  }
  // online softmax of head r over the tile's tokens 4kq + e (acc[0]) and
  // 16 + 4kq + e (acc[1]); the scores stay unscaled until the exponent
  // (exp2(s * sl2 - m) as one fma; sl2 > 0, so the maximum commutes with
  // the scaling), and positions past the list are masked in the query's
  // last tile only
  float sv[8];
#pragma unroll
  for (int e = 0; e < 4; e++) {
    sv[e] = acc[0][e];
    sv[4 + e] = acc[1][e];
  }
  if (cnt < kTT) {
#pragma unroll
    for (int e = 0; e < 4; e++) {
      sv[e] = 4 * kq + e < cnt ? sv[e] : -INFINITY;
      sv[4 + e] = 16 + 4 * kq + e < cnt ? sv[4 + e] : -INFINITY;
    }
  }
  float tm = max2(sv[0], sv[1]);
#pragma unroll
  for (int j = 2; j < 8; j++) tm = max2(tm, sv[j]);
  tm = rows_max(tm) * sl2;
  // The reference m (the exponent offset of P, l and O) is raised only when
  // the tile's maximum exceeds it by more than kLazyMax, so the rescale of
  // O below is rare once a head's scores have been seen (weights up to
  // 2^kLazyMax: fp32 sums and the hi + lo split of P are relative, so
  // nothing is lost; the result O / l is independent of the reference).
  const float mn = tm > m + kLazyMax ? tm : m;
  // (exp2 of the hardware: results below 2^-126, weights negligible next to
  // the row maximum's, may flush to zero)
  float pv[8];
  float alpha = 1.f, ps = 0.f;
#pragma unroll
  for (int j = 0; j < 8; j++) pv[j] = 0.f;
  if (mn != -INFINITY) {
    alpha = __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
    for (int j = 0; j < 8; j++) {
      pv[j] = __builtin_amdgcn_exp2f(fmaf(sv[j], sl2, -mn));
      ps += pv[j];
    }
  }
  ps = rows_sum(ps);
  l = l * alpha + ps;
  m = mn;
  // P^T as bf16 hi + lo parts (~16 significant bits; both rounded to
  // nearest even by the hardware conversion), the B operands of P V
  bf16x8 bh, bl;
#pragma unroll
  for (int j = 0; j < 8; j++) {
    bh[j] = (__bf16)pv[j];
    bl[j] = (__bf16)(pv[j] - float(bh[j]));
  }
  // rescale (alpha belongs to the lane's head; it is 1 on every lane unless
  // some head's reference was raised, and then nothing is multiplied)
  if (__ballot(alpha != 1.f)) {
#pragma unroll
    for (int nt = 0; nt < kDV / 16; nt++)
#pragma unroll
      for (int e = 0; e < 4; e++) o[nt][e] *= alpha;
  }
  // O^T += V^T P^T: lane (kq, r) reads, for dims 16nt .. 16nt+15, rows
  // 4kq + r/4 (first read) and 16 + 4kq + r/4 (second), dims 16nt + 4(r % 4)
  // .. +3; after the transpose it holds V[rows 4kq .. 4kq+3, then 16+4kq ..
  // 16+4kq+3][dim 16nt + r]
  const unsigned char* va = cur + (4 * kq + (r >> 2)) * kRowM * 16 + 8 * (r & 3);
  const unsigned char* vb = va + 16 * kRowM * 16;
  // two n-tiles at a time; the next pair's reads are issued before this
  // pair's MFMAs, so they complete while those run
  constexpr int kNP = kDV / 32;  // pairs of n-tiles
  s16x4 tv[2][2][2];             // [buffer][n-tile of the pair][read]
  auto load_pair = [&](int np, s16x4 (&t)[2][2]) {
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int nt = 2 * np + j;
      t[j][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(va + 32 * nt));
      t[j][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vb + 32 * nt));
    }
  };
#pragma unroll
  for (int np = 0; np < kNP + 1; np++) {
    if (np < kNP) {
      load_pair(np, tv[np & 1]);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    }
    if (np >= 1) {
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const int nt = 2 * (np - 1) + j;
        const bf16x8 av = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(tv[(np - 1) & 1][j][0], tv[(np - 1) & 1][j][1], 0, 1, 2, 3, 4, 5, 6, 7));
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh, o[nt], 0, 0, 0);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl, o[nt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
  }
}

// kLdsList: the query's ns_lds selected tokens (ascending) are already in
// LDS at sel_lds (the decode layer's own selection); the part takes its
// tiles' entries from there instead of gathering them, and ctx_in / seq_in
// are the query's context and sequence.
template <bool kCoh, bool kLdsList = false>
__device__ __attribute__((always_inline)) inline void attend_part_t(const AttendArgs& a, int split, int i, LdsT& sh,
                                                                    const int* sel_lds = nullptr, int ns_lds = 0,
                                                                    int ctx_in = -1, int seq_in = -1) {
  TLane tl;
  const int tid = threadIdx.x;
  tl.wave = tid >> 6;
  tl.lane = tid & 63;
  tl.r = tl.lane & 15;
  tl.kq = tl.lane >> 4;
  const int wave = tl.wave, r = tl.r, kq = tl.kq;

  const int seq = kLdsList ? seq_in : (a.q_seq ? a.q_seq[i] : 0);
  const int ctx = kLdsList ? ctx_in : clamp_ctx(a.q_ctx[i], a.max_ctx);
  // block 1 (the host sends other block sizes to attend_part): the list is
  // the ns selected tokens, no trailing ones
  att::List<kCoh> lv;
  lv.sel = a.sel + int64_t(i) * a.topk;
  lv.block = 1;
  lv.nblk = ctx;
  const int ns_max = ctx < a.topk ? ctx : a.topk;
  const int ns = kLdsList ? ns_lds : (kCoh ? ns_max : a.n_sel[i]);
  lv.ns = ns < 0 ? 0 : (ns > ns_max ? ns_max : ns);
  lv.L = lv.ns;
  if constexpr (kLdsList) {
    lv.cache = (att::LdsIntPtr)sel_lds;
    lv.has_cache = true;
  }
  int P0_, P1_;
  att::part_range<kCoh, kNTPART>(lv, a, split, ctx, sh.cnt, P0_, P1_);
  TList ls;
  ls.sel = lv.sel;
  ls.topk = a.topk;
  ls.ctx = ctx;
  // the part's range is the same on every lane: keep it (and what derives
  // from it) in scalar registers
  ls.P0 = __builtin_amdgcn_readfirstlane(P0_);
  ls.n_list = __builtin_amdgcn_readfirstlane(P1_) - ls.P0;
  ls.dma_sel = !kLdsList;
  const int n_tiles = (ls.n_list + kTT - 1) / kTT;

  const uint16_t* kvbase = a.k + int64_t(seq) * a.seq_stride;
  const float sl2 = a.scale * kLog2e;

  // B operands: Q[head 16w + r][32ks + 8kq .. +7]
  bf16x8 qa[kDK / 32];
  {
    const uint16_t* qrow = a.q + (int64_t(i) * kH + 16 * wave + r) * kDK + 8 * kq;
#pragma unroll
    for (int ks = 0; ks < kDK / 32; ks++) qa[ks] = as_bf16x8(ld16(qrow + 32 * ks));
  }
  float m = -INFINITY, l = 0.f;
  f32x4 o[kDV / 16];
#pragma unroll
  for (int nt = 0; nt < kDV / 16; nt++) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if constexpr (kLdsList) {
    // the entries are in LDS: tile 0's rows at once; tile t + 1's entries
    // start at list position P0 + kTT (t + 1)
    const int* ents = sel_lds + ls.P0;
    rows_dma(tl, ls, 0, ents, sh.kv[0], kvbase, a.tok_stride);
    for (int t = 0; t < n_tiles; t++) {
      wait_memory();
      pipe_barrier();  // every wave's share of tile t has landed; every wave is done with tile t - 1
      tile_t(tl, ls, t, sh.kv[t & 1], sh.kv[(t + 1) & 1], ents + kTT * (t + 1), sh.selbuf[t & 1], kvbase,
             a.tok_stride, sl2, qa, m, l, o);
    }
  } else {
    // the entries of tiles 0 and 1, then tile 0's rows
    sel_dma(tl, ls, 0, sh.selbuf[0]);
    sel_dma(tl, ls, 1, sh.selbuf[1]);
    wait_memory();
    pipe_barrier();
    rows_dma(tl, ls, 0, sh.selbuf[0], sh.kv[0], kvbase, a.tok_stride);
    for (int t = 0; t < n_tiles; t++) {
      // tile t's rows (this wave's share) and the entries of tile t + 1: all
      // this wave has in flight
      wait_memory();
      pipe_barrier();  // every wave's share of tile t has landed; every wave is done with tile t - 1
      tile_t(tl, ls, t, sh.kv[t & 1], sh.kv[(t + 1) & 1], sh.selbuf[(t + 1) & 1], sh.selbuf[t & 1], kvbase,
             a.tok_stride, sl2, qa, m, l, o);
    }
  }

  // normalise and write: lane (kq, r) holds O^T[dim 16nt + 4kq + e][head 16w + r]
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int64_t orow = (int64_t(split) * a.nq + i) * kH + 16 * wave + r;
  float* op = a.o_part + orow * kDV + 4 * kq;
#pragma unroll
  for (int nt = 0; nt < kDV / 16; nt++)
    *reinterpret_cast<f32x4*>(op + 16 * nt) = f32x4{o[nt][0] * inv, o[nt][1] * inv, o[nt][2] * inv, o[nt][3] * inv};
  if (kq == 0) a.lse_part[orow] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  // the only tile of a prefill (first and last of a running merge): the
  // result is final, and its bf16 copy is written here (what a merge of
  // this single partial would produce: the same value, rounded the same way)
  if (a.acc == 7 && a.o_bf16) {
    uint16_t* ob = a.o_bf16 + orow * kDV + 4 * kq;
#pragma unroll
    for (int nt = 0; nt < kDV / 16; nt++) {
      u32x2 pk;
      pk[0] = uint32_t(f32_to_bf16(o[nt][0] * inv)) | (uint32_t(f32_to_bf16(o[nt][1] * inv)) << 16);
      pk[1] = uint32_t(f32_to_bf16(o[nt][2] * inv)) | (uint32_t(f32_to_bf16(o[nt][3] * inv)) << 16);
      *reinterpret_cast<u32x2*>(ob + 16 * nt) = pk;
    }
  }
}

// ---- FP8 latent rows
// "GLM-5.3 最適化 第2部", footnote 1: the FP8 sparse-MLA row is 656 bytes:
// the 512 latent values as E4M3 codes in 4 groups of 128 with one fp32
// scale each (value = code * scale), then the 64 rotary values in bf16:
//   bytes [0, 512) codes, [512, 528) scales, [528, 656) rotary values.
// Same work-group layout and MFMA tiles as above; per tile:
//   * the 32 rows arrive by LDS DMA in a staging area (656-byte stride);
//   * all threads convert the codes to bf16 (exact, unscaled) into the bf16
//     tile above, copy the rotary values and keep the 4 scales per token;
//     the staging area is then free and the next tile's rows are requested
//     at once, so their gather overlaps this tile's MFMA work;
//   * S: one MFMA chain over the 18 k-steps; the accumulator is kept in
//     units of the current group's scale (rescaled by s_prev / s_g on
//     entering group g, back to real units before the rotary columns), so
//     no second accumulator is live;
//   * O += P' V per group, with P' = P * (the token's group scale) split
//     into bf16 hi + lo parts, so the codes serve as V unscaled.
constexpr int kF8Row = 656;                 // bytes per FP8 row
constexpr int kF8RowC = kF8Row / 16;        // 16-byte chunks per FP8 row (41)
constexpr int kF8TileC = kTT * kF8RowC;     // chunks per staged tile (1312)

struct LdsF8 {
  __attribute__((aligned(16))) unsigned char kv[kTileC * 16];      // bf16 tile (as Lds::kv)
  __attribute__((aligned(16))) unsigned char stage[kF8TileC * 16];  // FP8 rows of the tile in flight
  __attribute__((aligned(16))) uint16_t p[4][2][16 * kPStr];
  __attribute__((aligned(16))) float pf[4][64][8];  // per wave and lane: the tile's P before scaling
  float sc[kTT][4];
  int cnt[kNTPART / 64];
};

template <bool kCoh>
__device__ void attend_part_fp8(const AttendArgs& a, int split, int i, LdsF8& sh) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, kq = lane >> 4;

  const int seq = a.q_seq ? a.q_seq[i] : 0;
  const int ctx = clamp_ctx(a.q_ctx[i], a.max_ctx);
  att::List<kCoh> lv;
  lv.sel = a.sel + int64_t(i) * a.topk;
  lv.block = a.block;
  lv.nblk = ctx / a.block;
  const int ns_max = lv.nblk < a.topk ? lv.nblk : a.topk;
  const int ns = kCoh ? ns_max : a.n_sel[i];
  lv.ns = ns < 0 ? 0 : (ns > ns_max ? ns_max : ns);
  lv.L = lv.ns * a.block + (ctx - lv.nblk * a.block);
  int P0_, P1_;
  att::part_range<kCoh, kNTPART>(lv, a, split, ctx, sh.cnt, P0_, P1_);
  const int P0 = P0_, P1 = P1_;

  // strides in bytes
  const unsigned char* kvbase = reinterpret_cast<const unsigned char*>(a.k) + int64_t(seq) * a.seq_stride;
  const float sl2 = a.scale * kLog2e;

  // the rows of the tile starting at list position pb -> staging area
  auto request = [&](int pb) {
    const int cnt = (P1 - pb) < kTT ? (P1 - pb) : kTT;
    const int tokl = lv.tok(pb + ((lane & 31) < cnt ? (lane & 31) : 0));
    for (int s = wave; s * 64 < kF8TileC; s += 4) {
      const int c = 64 * s + lane;
      const int row = c / kF8RowC, col = c % kF8RowC;
      const int rt = __shfl(tokl, row < kTT ? row : 0);
      if (c < kF8TileC)
        __builtin_amdgcn_global_load_lds(kvbase + int64_t(rt) * a.tok_stride + 16 * col,
                                         (__attribute__((address_space(3))) void*)(sh.stage + 1024 * s), 16, 0, 0);
    }
  };

  bf16x8 qa[kDK / 32];
  {
    const uint16_t* qrow = a.q + (int64_t(i) * kH + 16 * wave + r) * kDK + 8 * kq;
#pragma unroll
    for (int ks = 0; ks < kDK / 32; ks++) qa[ks] = as_bf16x8(ld16(qrow + 32 * ks));
  }
  float m[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; e++) {
    m[e] = -INFINITY;
    l[e] = 0.f;
  }
  f32x4 o[kDV / 16];
#pragma unroll
  for (int nt = 0; nt < kDV / 16; nt++) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint16_t* phi = sh.p[wave][0];
  uint16_t* plo = sh.p[wave][1];

  if (P0 < P1) request(P0);
  for (int pb = P0; pb < P1; pb += kTT) {
    const int cnt = (P1 - pb) < kTT ? (P1 - pb) : kTT;
    wait_memory();
    __syncthreads();  // the staged rows have landed; every wave is done with the previous bf16 tile
    // codes -> bf16 tile (row t, chunks 2cc, 2cc+1 hold columns 16cc .. 16cc+15)
#pragma unroll 1
    for (int k = 0; k < 4; k++) {
      const int u = tid + 256 * k;
      const int row = u >> 5, cc = u & 31;
      const u32x4 w = *reinterpret_cast<const u32x4*>(sh.stage + row * kF8Row + 16 * cc);
      u32x4 lo, hi;
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const bf16x8 b = e4m3x8_bf16(u32x2{w[2 * j], w[2 * j + 1]});
        if (j == 0) lo = __builtin_bit_cast(u32x4, b);
        else hi = __builtin_bit_cast(u32x4, b);
      }
      unsigned char* dst = sh.kv + (row * kRowL + 2 * cc) * 16;
      *reinterpret_cast<u32x4*>(dst) = lo;
      *reinterpret_cast<u32x4*>(dst + 16) = hi;
    }
    {  // rotary values: row tid / 8, chunk tid % 8 -> bf16 tile chunk 64 + tid % 8
      const int row = tid >> 3, rc = tid & 7;
      *reinterpret_cast<u32x4*>(sh.kv + (row * kRowL + 64 + rc) * 16) =
          *reinterpret_cast<const u32x4*>(sh.stage + row * kF8Row + 528 + 16 * rc);
    }
    if (tid < kTT * 4)
      sh.sc[tid >> 2][tid & 3] = *reinterpret_cast<const float*>(sh.stage + (tid >> 2) * kF8Row + 512 + 4 * (tid & 3));
    __syncthreads();  // bf16 tile and scales ready; the staging area is free
    if (pb + kTT < P1) request(pb + kTT);

    // S = Q K^T: lane (kq, r) holds S[head 4kq+e][token 16h + r]
    f32x4 acc[2];
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
      acc[hf] = f32x4{0.f, 0.f, 0.f, 0.f};
      const unsigned char* krow = sh.kv + ((16 * hf + r) * kRowL + kq) * 16;
#pragma unroll
      for (int ks = 0; ks < kDK / 32; ks++) {
        const bf16x8 kb = as_bf16x8(*reinterpret_cast<const u32x4*>(krow + 64 * ks));
        // entering group g = ks / 4: rescale to its units (a zero scale, an
        // all-zero group, keeps the units: its codes add nothing)
        if (ks % 4 == 0 && ks < kDV / 32) {
          const float sg = sh.sc[16 * hf + r][ks / 4];
          const float inv = sg > 0.f ? 1.f / sg : 1.f;
          const float prev = ks == 0 ? 1.f : sh.sc[16 * hf + r][ks / 4 - 1];
#pragma unroll
          for (int e = 0; e < 4; e++) acc[hf][e] = acc[hf][e] * (prev > 0.f ? prev : 1.f) * inv;
        }
        if (ks == kDV / 32) {
          const float prev = sh.sc[16 * hf + r][3];
#pragma unroll
          for (int e = 0; e < 4; e++) acc[hf][e] *= prev > 0.f ? prev : 1.f;
        }
        acc[hf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kb, acc[hf], 0, 0, 0);
      }
    }
    float alpha[4];
    float* pl = sh.pf[wave][lane];
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const float s0 = r < cnt ? acc[0][e] * sl2 : -INFINITY;
      const float s1 = 16 + r < cnt ? acc[1][e] * sl2 : -INFINITY;
      const float tm = row16_max(fmaxf(s0, s1));
      // the reference is raised only past kLazyMax (as in the bf16 form)
      const float mn = tm > m[e] + kLazyMax ? tm : m[e];
      float p0 = 0.f, p1 = 0.f;
      alpha[e] = 1.f;
      if (mn != -INFINITY) {
        p0 = exp2f(s0 - mn);
        p1 = exp2f(s1 - mn);
        alpha[e] = exp2f(m[e] - mn);
      }
      const float ps = row16_sum(p0 + p1);
      l[e] = l[e] * alpha[e] + ps;
      m[e] = mn;
      pl[2 * e] = p0;  // kept in LDS (the lane's own slot) for the four groups below
      pl[2 * e + 1] = p1;
    }
    if (__ballot(alpha[0] != 1.f || alpha[1] != 1.f || alpha[2] != 1.f || alpha[3] != 1.f)) {
#pragma unroll
      for (int nt = 0; nt < kDV / 16; nt++)
#pragma unroll
        for (int e = 0; e < 4; e++) o[nt][e] *= alpha[e];
    }
    // O += P' V, one 128-column group at a time
    const unsigned char* vb0 = sh.kv + (8 * kq + (r >> 2)) * kRowL * 16 + 8 * (r & 3);
#pragma unroll
    for (int g = 0; g < 4; g++) {
      const float sa = sh.sc[r][g], sb = sh.sc[16 + r][g];
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int row = 4 * kq + e;
        const float x0 = pl[2 * e] * sa, x1 = pl[2 * e + 1] * sb;
        const uint16_t h0 = f32_to_bf16(x0), h1 = f32_to_bf16(x1);
        phi[row * kPStr + r] = h0;
        phi[row * kPStr + 16 + r] = h1;
        plo[row * kPStr + r] = f32_to_bf16(x0 - bf16_to_f32(h0));
        plo[row * kPStr + 16 + r] = f32_to_bf16(x1 - bf16_to_f32(h1));
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      const bf16x8 ah = as_bf16x8(*reinterpret_cast<const u32x4*>(phi + r * kPStr + 8 * kq));
      const bf16x8 al = as_bf16x8(*reinterpret_cast<const u32x4*>(plo + r * kPStr + 8 * kq));
#pragma unroll
      for (int nt = 8 * g; nt < 8 * g + 8; nt++) {
        s16x4 t[2];
#pragma unroll
        for (int hh = 0; hh < 2; hh++)
          t[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(vb0 + 4 * hh * kRowL * 16 + 32 * nt));
        const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3, 4, 5, 6, 7));
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bv, o[nt], 0, 0, 0);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bv, o[nt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();  // this group's P' is read before the next one overwrites it
    }
  }

  const int64_t orow0 = (int64_t(split) * a.nq + i) * kH + 16 * wave;
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const int hrow = 4 * kq + e;
    const float inv = l[e] > 0.f ? 1.f / l[e] : 0.f;
    float* op = a.o_part + (orow0 + hrow) * kDV + r;
#pragma unroll
    for (int nt = 0; nt < kDV / 16; nt++) op[16 * nt] = o[nt][e] * inv;
    if (r == 0) a.lse_part[orow0 + hrow] = l[e] > 0.f ? (m[e] + log2f(l[e])) * kLn2 : -INFINITY;
  }
}

}  // namespace mla
}  // namespace qsa
