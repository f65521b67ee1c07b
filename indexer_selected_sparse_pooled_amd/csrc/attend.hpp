// Device code of A4 / A6 for the pooled-block variant (hq 16, hkv 2, head
// dim 256): softmax attention of one query and one kv head over a part of
// its selected tokens, optionally followed by the log-sum-exp merge of all
// parts. Used by the stand-alone attention kernel (attend.hip) and by the
// decode layer (decode_layer.hip).
//
// "3090x3で 314 万コンテキスト": only the indexer-selected K/V rows are read
// (section "なぜ"), addressed per (token, kv head) (section "カーネルを書き換え
// ずに済む"); prefill restricts each query to one history tile and merges the
// tiles' partial results (section "ちなみにこの欠点"). "GLM-5.3 最適化 第2部",
// section "DCP": partial attention results are combined by log-sum-exp.
//
// The query's token list is the tokens of its selected blocks (ascending)
// followed by the trailing tokens of the incomplete block. A work-group
// walks its contiguous part of the list (intersected with [tile_begin,
// tile_end)) in groups of GT tiles of 64 tokens, every load of a group
// issued before any is used:
//   * K rows go straight from global memory to registers as the B operand
//     of S = Q K^T on MFMA 16x16x32 bf16: the GQA group's 8 query heads are
//     the A rows (rows 8..15 zero), each wave computes 16 * GT tokens;
//   * V rows go straight from global memory to LDS (global_load_lds_dwordx4,
//     no registers), two rows per wave instruction;
//   * online softmax in exp2 form per head (one barrier);
//   * O += P V on MFMA 16x16x32: P split into bf16 hi + lo parts (two
//     MFMAs, ~16 significant bits); each wave owns 64 of the 256 output
//     dims and reads V transposed out of LDS with ds_read_tr16_b64.
// Output: normalised partial O (fp32) and its natural-log lse. With a
// counter, the last work-group of each (query, kv head) to finish merges
// all parts into the final O (fp32 and/or bf16) and lse; the parts are
// handed over with agent-coherent stores, so no L2 write-back is needed.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace qsa {
namespace att {

constexpr int kTT = 64;          // token positions per tile
constexpr int kG = 8;            // query heads per kv head
constexpr int kD = 256;          // head dim of K and V
// LDS bytes per pair of V rows (2 x 512 + 32). gfx950's LDS has 128
// four-byte banks; a transposed V read takes one row of each of 16
// consecutive pairs (32 bytes each), and at 1056 bytes (132 eight-byte
// units, 4 mod 64) the 16 pairs start on 16 distinct multiples of 4 units:
// no conflicts. (The two rows of a pair, 512 bytes apart, always share
// banks, so they are never read by the same instruction.)
constexpr int kPair = 1056;
// LDS position of token t of a tile in S and P: within each group of 8
// tokens the even ones first (0 2 4 6 1 3 5 7), the order in which the
// P V contraction takes them (see the V reads)
__device__ __forceinline__ int tok_pos(int t) { return (t & ~7) | ((t & 7) >> 1) | ((t & 1) << 2); }
constexpr unsigned kMergeSpinLimit = 1u << 24;  // polls while the parts of a merge arrive

typedef short s16x4 __attribute__((ext_vector_type(4)));

// LDS of one work-group; a group of GT tiles (64 * GT tokens) is loaded at once.
template <int GT>
struct Lds {
  static constexpr int kTok = kTT * GT;
  static constexpr int kPStr = kTok + 8;  // LDS row of P in elements
  __attribute__((aligned(16))) unsigned char v[kTok / 2 * kPair];
  float s[kG][kTok];
  __attribute__((aligned(16))) uint16_t phi[kG * kPStr];
  __attribute__((aligned(16))) uint16_t plo[kG * kPStr];
  float alpha[kG], m[kG], l[kG];
  int cnt[4];
};

// sel may have been written earlier in the same launch by another
// work-group: then they are read with agent-coherent loads.
template <bool kCoh>
__device__ __forceinline__ int ld_sel(const int* p) {
  if constexpr (kCoh) return int(ld_coherent(reinterpret_cast<const uint32_t*>(p)));
  return *p;
}

// A pointer into LDS, typed as one: reads through it are ds_read (counted by
// lgkmcnt alone). A generic pointer would make them flat loads, which also
// count against vmcnt, so every read would wait for the loads in flight.
typedef const __attribute__((address_space(3))) int* LdsIntPtr;

template <bool kCoh>
struct List {
  const int* sel;
  int ns;    // selected blocks
  int nblk;  // complete blocks
  int block;
  int L;     // list length
  // LDS copy of sel[0 .. ns) when has_cache (a flag, not a null test: LDS
  // offset 0 is a valid address)
  LdsIntPtr cache = nullptr;
  bool has_cache = false;
  __device__ __forceinline__ int sel_at(int j) const { return has_cache ? cache[j] : ld_sel<kCoh>(sel + j); }
  // token of list entry p (0 <= p < L)
  __device__ __forceinline__ int tok(int p) const {
    const int nb_tok = ns * block;
    if (p < nb_tok) {
      int b = sel_at(p / block);
      b = b < 0 ? 0 : (b >= nblk ? nblk - 1 : b);
      return b * block + p % block;
    }
    return nblk * block + (p - nb_tok);
  }
  // the number of list entries whose token is < x (x a multiple of block,
  // or >= ctx) when it follows from the sizes alone (true), else false: x
  // falls among the selected blocks and their count below x / block decides
  __device__ __forceinline__ bool below_known(int64_t x, int ctx, int& val) const {
    if (x <= 0) {
      val = 0;
      return true;
    }
    if (x >= ctx) {
      val = L;
      return true;
    }
    const int nb_tok = nblk * block;
    if (x >= nb_tok) {
      val = ns * block + int(x - nb_tok);
      return true;
    }
    return false;
  }
};

// First list position of part `split` of n_split over a list of L entries:
// split * L / n_split. L < (topk + 1) * block <= 8196 and split <= n_split
// <= 256, so the product fits 32-bit unsigned arithmetic (a 64-bit division
// is a long emulated sequence).
__device__ __forceinline__ int split_point(int split, int L, int n_split) {
  return int(uint32_t(split) * uint32_t(L) / uint32_t(n_split));
}

// The part's list range [P0, P1): its split of the list intersected with
// the positions of the tokens in [tile_begin, tile_end), the same on every
// thread of the work-group (NT threads, all calling). A tile bound that
// falls among the selected blocks is settled by all threads at once: each
// reads ns / NT entries of the (ascending) selection and counts those below
// the bound's block, then one block sum (cnt: NT / 64 ints of LDS, one
// barrier, only when a bound needs it), in place of a binary search of
// dependent loads.
template <bool kCoh, int NT>
__device__ void part_range(const List<kCoh>& lv, const AttendArgs& a, int split, int ctx, int* cnt, int& P0,
                           int& P1) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lo = split_point(split, lv.L, a.n_split);
  const int hi = split_point(split + 1, lv.L, a.n_split);
  int t0, t1;
  const bool k0 = lv.below_known(a.tile_begin, ctx, t0);
  const bool k1 = lv.below_known(a.tile_end, ctx, t1);
  if (!(k0 && k1)) {  // uniform
    const int xb0 = k0 ? 0 : int(a.tile_begin) / lv.block;
    const int xb1 = k1 ? 0 : int(a.tile_end) / lv.block;
    int c = 0;  // below bound 0 in the low half, below bound 1 in the high half (ns <= 2048)
    for (int j = tid; j < lv.ns; j += NT) {
      const int b = lv.sel_at(j);
      c += (b < xb0 ? 1 : 0) + (b < xb1 ? 0x10000 : 0);
    }
    c = __builtin_amdgcn_readlane(wave_incl_sum(c), 63);
    if (lane == 0) cnt[wave] = c;
    __syncthreads();
    int s = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; w++) s += cnt[w];
    if (!k0) t0 = (s & 0xFFFF) * lv.block;
    if (!k1) t1 = (s >> 16) * lv.block;
  }
  P0 = lo > t0 ? lo : t0;
  P1 = hi < t1 ? hi : t1;
}

__device__ __forceinline__ uint64_t shfl64(uint64_t v, int src) {
  const uint32_t lo = __shfl(uint32_t(v), src), hi = __shfl(uint32_t(v >> 32), src);
  return (uint64_t(hi) << 32) | lo;
}

// One part (split, kv head g, query i): see the file comment. With ns_lds >=
// 0, sel_lds holds the query's ns_lds selected blocks in LDS (ascending) and
// replaces sel / n_sel; ctx_in / seq_in, when >= 0, are the query's context
// length and sequence (already loaded by the caller). kCached: rows come from the HBM row cache on a hit
// (the plan in a.src) and from their home (host) memory otherwise, and the
// rows this part may fill are written to the cache after the tile
// (row_cache.hip).
template <bool kCoh, int GT, bool kCached = false, bool kAcc = false>
__device__ void attend_part(const AttendArgs& a, int split, int g, int i, Lds<GT>& sh, LdsIntPtr sel_lds = nullptr,
                            int ns_lds = -1, int ctx_in = -1, int seq_in = -1) {
  const bool sel_lds_given = ns_lds >= 0;
  constexpr int kTok = Lds<GT>::kTok, kPStr = Lds<GT>::kPStr;
  constexpr int kRW = 16 * GT;  // token rows per wave
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, kq = lane >> 4;

  const int seq = seq_in >= 0 ? seq_in : (a.q_seq ? a.q_seq[i] : 0);
  const int ctx = ctx_in >= 0 ? ctx_in : clamp_ctx(a.q_ctx[i], a.max_ctx);
  List<kCoh> lv;
  lv.sel = a.sel + int64_t(i) * a.topk;
  lv.block = a.block;
  lv.nblk = ctx / a.block;
  const int ns_max = lv.nblk < a.topk ? lv.nblk : a.topk;
  // a selection made in this launch (sel_lds, or kCoh) always holds
  // min(complete blocks, topk) entries: no need to read n_sel
  const int ns = sel_lds_given ? ns_lds : (kCoh ? ns_max : a.n_sel[i]);
  lv.ns = ns < 0 ? 0 : (ns > ns_max ? ns_max : ns);
  lv.cache = sel_lds;
  lv.has_cache = sel_lds_given;
  lv.L = lv.ns * a.block + (ctx - lv.nblk * a.block);

  int P0, P1;
  part_range<kCoh, 256>(lv, a, split, ctx, sh.cnt, P0, P1);
  if (tid < kG) {
    sh.m[tid] = -INFINITY;
    sh.l[tid] = 0.f;
  }
  __syncthreads();

  const int64_t kvs = int64_t(seq) * a.seq_stride + int64_t(g) * a.head_stride;
  const uint16_t* kbase = a.k + kvs;
  const uint16_t* vbase = a.v + kvs;
  const float sl2 = a.scale * kLog2e;
  [[maybe_unused]] uint32_t epoch = 0;
  if constexpr (kCached) epoch = *a.c_epoch;
  [[maybe_unused]] const int64_t slot_off = int64_t(g) * (a.dk + a.dv) * 2;  // kv head g's K, V in a slot

  bf16x8 qa[kD / 32];
  {
    const uint16_t* qrow = a.q + (int64_t(i) * a.hq + g * kG + (r < kG ? r : 0)) * kD;
#pragma unroll
    for (int ks = 0; ks < kD / 32; ks++) {
      const u32x4 w = r < kG ? ld16(qrow + 32 * ks + 8 * kq) : u32x4{0u, 0u, 0u, 0u};
      qa[ks] = as_bf16x8(w);
    }
  }
  f32x4 oacc[4];
#pragma unroll
  for (int nt = 0; nt < 4; nt++) oacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // kAcc: the earlier tiles' merged result for this lane's elements (rows
  // 4 kq + e < 8, dims 64 wave + 16 nt + r) and rows, loaded now so that the
  // loads complete while the tile is attended
  [[maybe_unused]] float run_o[4][4], run_lse[4];
  if constexpr (kAcc) {
    const bool first = a.acc & 1;
    const int64_t row0 = int64_t(i) * a.hq + g * kG;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const int row = 4 * kq + e;
      const bool mine = !first && row < kG;
      run_lse[e] = mine ? a.lse_part[row0 + row] : -INFINITY;
#pragma unroll
      for (int nt = 0; nt < 4; nt++)
        run_o[e][nt] = mine ? a.o_part[(row0 + row) * kD + 64 * wave + 16 * nt + r] : 0.f;
    }
  }

  for (int pb = P0; pb < P1; pb += kTok) {
    const int cnt = (P1 - pb) < kTok ? (P1 - pb) : kTok;
    // wave w owns group rows kRW*w .. kRW*w + kRW-1 (its S rows and its V
    // rows); lane l holds the token of row kRW*w + l % kRW. Rows past cnt
    // repeat row 0, so every load reads finite data that the softmax then
    // weights by 0.
    const int row_l = kRW * wave + lane % kRW;
    const int pos_l = pb + (row_l < cnt ? row_l : 0);
    int tokl = 0;
    [[maybe_unused]] uint64_t krow_l = 0, vrow_l = 0, key_l = 0;  // cached: the row's K, V addresses and key
    [[maybe_unused]] int64_t slot_l = 0;
    [[maybe_unused]] bool fill_l = false;
    if constexpr (kCached) {
      const int e = a.src[int64_t(i) * a.src_ld + pos_l];
      if (e < 0) {  // in the cache
        slot_l = -int64_t(e) - 1;
        krow_l = uint64_t(a.c_rows + slot_l * a.row_bytes + slot_off);
        vrow_l = krow_l + 2 * a.dk;
      } else {  // from its home memory; may fill its slot
        krow_l = uint64_t(kbase + int64_t(e) * a.tok_stride);
        vrow_l = uint64_t(vbase + int64_t(e) * a.tok_stride);
        key_l = uint64_t(int64_t(seq) * a.key_stride + e) + 1u;
        slot_l = int64_t((key_l - 1u) % uint64_t(a.n_slots));
        const uint32_t id = uint32_t(int64_t(i) * a.src_ld + pos_l) + 1u;
        fill_l = row_l < cnt && a.c_claim[slot_l] == ((uint64_t(epoch) << 32) | id) && a.c_hit[slot_l] != epoch;
      }
    } else {
      tokl = lv.tok(pos_l);
    }
    // V rows go straight to LDS (no registers) and K rows to registers as
    // the B operands of S. With one tile per group (many work-groups per CU)
    // the V rows are issued first; with several tiles (few, latency-bound
    // work-groups) the K rows are, so that S waits for them alone.
    auto load_v = [&]() {
      const int half = lane >> 5, c = lane & 31;
      // every row address first (cross-lane moves, one wait), then the
      // loads back to back
      const uint16_t* vsrc[8 * GT];
#pragma unroll
      for (int j = 0; j < 8 * GT; j++) {
        if constexpr (kCached) {
          vsrc[j] = reinterpret_cast<const uint16_t*>(shfl64(vrow_l, 2 * j + half)) + 8 * c;
        } else {
          const int vt = __shfl(tokl, 2 * j + half);
          vsrc[j] = vbase + int64_t(vt) * a.tok_stride + 8 * c;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 8 * GT; j++) {
        const int p = 8 * GT * wave + j;
        __builtin_amdgcn_global_load_lds(vsrc[j], (__attribute__((address_space(3))) void*)(sh.v + p * kPair), 16, 0,
                                         0);
      }
    };
    if constexpr (GT == 1) load_v();
    bf16x8 kb[GT][kD / 32];
#pragma unroll
    for (int b = 0; b < GT; b++) {
      const uint16_t* krow;
      if constexpr (kCached) {
        krow = reinterpret_cast<const uint16_t*>(shfl64(krow_l, 16 * b + r)) + 8 * kq;
      } else {
        const int kt = __shfl(tokl, 16 * b + r);
        krow = kbase + int64_t(kt) * a.tok_stride + 8 * kq;
      }
#pragma unroll
      for (int ks = 0; ks < kD / 32; ks++) kb[b][ks] = as_bf16x8(ld16(krow + 32 * ks));
    }
    if constexpr (GT > 1) load_v();
    // S for the wave's rows, 16 at a time: lane (kq, r) holds S[head 4kq+e][row r]
#pragma unroll
    for (int b = 0; b < GT; b++) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kD / 32; ks++)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kb[b][ks], acc, 0, 0, 0);
      const int rr = kRW * wave + 16 * b + r;
      if (kq < 2) {
#pragma unroll
        for (int e = 0; e < 4; e++) sh.s[4 * kq + e][tok_pos(rr)] = rr < cnt ? acc[e] * sl2 : -INFINITY;
      }
    }
    __syncthreads();
    // online softmax: head h = tid / 32, 2 * GT consecutive positions per thread
    {
      constexpr int kE = 2 * GT;
      const int h = tid >> 5;
      const int t0 = (tid & 31) * kE;
      float sv[kE];
#pragma unroll
      for (int e = 0; e < kE; e++) sv[e] = sh.s[h][t0 + e];
      float mt = sv[0];
#pragma unroll
      for (int e = 1; e < kE; e++) mt = fmaxf(mt, sv[e]);
#pragma unroll
      for (int m = 16; m >= 1; m >>= 1) mt = fmaxf(mt, __shfl_xor(mt, m));
      const float m_old = sh.m[h], l_old = sh.l[h];
      const float m_new = fmaxf(m_old, mt);
      float pv[kE];
      float al = 1.f, ps = 0.f;
#pragma unroll
      for (int e = 0; e < kE; e++) pv[e] = 0.f;
      if (m_new != -INFINITY) {
        al = exp2f(m_old - m_new);
#pragma unroll
        for (int e = 0; e < kE; e++) {
          pv[e] = exp2f(sv[e] - m_new);
          ps += pv[e];
        }
      }
#pragma unroll
      for (int m = 16; m >= 1; m >>= 1) ps += __shfl_xor(ps, m);
#pragma unroll
      for (int e = 0; e < kE; e += 2) {
        const uint16_t h0 = f32_to_bf16(pv[e]), h1 = f32_to_bf16(pv[e + 1]);
        const uint16_t l0 = f32_to_bf16(pv[e] - bf16_to_f32(h0)), l1 = f32_to_bf16(pv[e + 1] - bf16_to_f32(h1));
        *reinterpret_cast<uint32_t*>(sh.phi + h * kPStr + t0 + e) = uint32_t(h0) | (uint32_t(h1) << 16);
        *reinterpret_cast<uint32_t*>(sh.plo + h * kPStr + t0 + e) = uint32_t(l0) | (uint32_t(l1) << 16);
      }
      if ((tid & 31) == 0) {
        sh.alpha[h] = al;
        sh.l[h] = al * l_old + ps;
        sh.m[h] = m_new;
      }
    }
    wait_memory();  // this wave's V rows have landed in LDS
    __syncthreads();
    // O += P V for dims 64*wave .. 64*wave+63
    {
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int row = 4 * kq + e;
        const float al = row < kG ? sh.alpha[row] : 1.f;
#pragma unroll
        for (int nt = 0; nt < 4; nt++) oacc[nt][e] *= al;
      }
#pragma unroll
      for (int k2 = 0; k2 < kTok / 32; k2++) {
        // A: P[head r][positions 32*k2 + 8*kq .. +7] (rows 8..15 are zero)
        const bf16x8 ah = r < kG ? as_bf16x8(ld16(sh.phi + r * kPStr + 32 * k2 + 8 * kq)) : bf16x8{};
        const bf16x8 al8 = r < kG ? as_bf16x8(ld16(sh.plo + r * kPStr + 32 * k2 + 8 * kq)) : bf16x8{};
#pragma unroll
        for (int nt = 0; nt < 4; nt++) {
          // B: V[token at position 32*k2 + 8*kq + j][dim 64*wave + 16*nt + r],
          // j = 0..7, as two transposed reads: lane (kq, r') addresses row
          // 32*k2 + 8*kq + 2*(r'/4) + h (the even tokens of the group, then
          // the odd ones: the positions' order), dims 64*wave + 16*nt +
          // 4*(r'%4) .. +3
          const int d0 = 64 * wave + 16 * nt + 4 * (r & 3);
          s16x4 t[2];
#pragma unroll
          for (int hh = 0; hh < 2; hh++) {
            const int row = 32 * k2 + 8 * kq + 2 * (r >> 2) + hh;
            const unsigned char* pa = sh.v + (row >> 1) * kPair + (row & 1) * 512 + 2 * d0;
            t[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)pa);
          }
          const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bv, oacc[nt], 0, 0, 0);
          oacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al8, bv, oacc[nt], 0, 0, 0);
        }
      }
    }
    if constexpr (kCached) {
      // rows this part may fill: K from the registers (lane (kq, r) holds
      // dims 32ks + 8kq .. +7 of wave row 16b + r), V from LDS (as loaded)
#pragma unroll
      for (int b = 0; b < GT; b++) {
        const int sl = 16 * b + r;
        const bool f = __shfl(int(fill_l), sl) != 0;
        const int64_t c = int64_t(shfl64(uint64_t(slot_l), sl));
        const uint64_t key = shfl64(key_l, sl);
        if (f) {
          unsigned char* dst = a.c_rows + c * a.row_bytes + slot_off;
#pragma unroll
          for (int ks = 0; ks < kD / 32; ks++) st16(dst + 2 * (32 * ks + 8 * kq), __builtin_bit_cast(u32x4, kb[b][ks]));
          if (kq == 0 && g == 0) a.c_tag[c] = key;
        }
      }
      const int half = lane >> 5, c32 = lane & 31;
#pragma unroll
      for (int j = 0; j < 8 * GT; j++) {
        const int p = 8 * GT * wave + j;
        const int sl = 2 * j + half;
        const bool f = __shfl(int(fill_l), sl) != 0;
        const int64_t c = int64_t(shfl64(uint64_t(slot_l), sl));
        if (f)
          st16(a.c_rows + c * a.row_bytes + slot_off + 2 * a.dk + 16 * c32,
               *reinterpret_cast<const u32x4*>(sh.v + p * kPair + 512 * half + 16 * c32));
      }
    }
    __syncthreads();
  }

  // normalise and write the partial result
  const int64_t orow0 = (int64_t(split) * a.nq + i) * a.hq + g * kG;
  if constexpr (kAcc) {
    // merge with the earlier tiles (log-sum-exp weights; an empty side
    // weighs 0) and write the running result in place
    const bool last = a.acc & 2;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const int row = 4 * kq + e;
      if (row < kG) {
        const float l = sh.l[row];
        const float lse_t = l > 0.f ? (sh.m[row] + log2f(l)) * kLn2 : -INFINITY;
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const float mx = fmaxf(run_lse[e], lse_t);
        float w_run = 0.f, w_t = 0.f, lse = -INFINITY;
        if (mx != -INFINITY) {
          w_run = expf(run_lse[e] - mx);
          w_t = expf(lse_t - mx);
          lse = mx + logf(w_run + w_t);
        }
        const float norm = w_run + w_t > 0.f ? 1.f / (w_run + w_t) : 0.f;
        const int64_t orow = orow0 + row;
#pragma unroll
        for (int nt = 0; nt < 4; nt++) {
          const float o = (run_o[e][nt] * w_run + oacc[nt][e] * inv * w_t) * norm;
          const int64_t idx = orow * kD + 64 * wave + 16 * nt + r;
          a.o_part[idx] = o;
          if (last && a.o_bf16) a.o_bf16[idx] = f32_to_bf16(o);
        }
        if (r == 0 && wave == 0) a.lse_part[orow] = lse;
      }
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const int row = 4 * kq + e;
    if (row < kG) {
      const float l = sh.l[row];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      float* o = a.o_part + (orow0 + row) * kD + 64 * wave + r;
#pragma unroll
      for (int nt = 0; nt < 4; nt++) {
        if (a.counter)
          st_coherent(reinterpret_cast<uint32_t*>(o + 16 * nt), __float_as_uint(oacc[nt][e] * inv));
        else
          o[16 * nt] = oacc[nt][e] * inv;
      }
    }
  }
  if (tid < kG) {
    const float l = sh.l[tid];
    const float lse = l > 0.f ? (sh.m[tid] + log2f(l)) * kLn2 : -INFINITY;
    if (a.counter)
      st_coherent(reinterpret_cast<uint32_t*>(a.lse_part + orow0 + tid), __float_as_uint(lse));
    else
      a.lse_part[orow0 + tid] = lse;
  }
  if (!a.counter) return;

  // ---- merge: once every part of (query, kv head) has stored its result,
  // part `split` merges dims [256 split / n_split, 256 (split + 1) / n_split)
  // of the 8 heads, each element over all parts, every load of a batch issued
  // before any is used. The parts of a (query, kv head) are resident
  // together (the host checks this), so the wait ends.
  wait_memory();
  __syncthreads();
  uint32_t* arrive = a.counter + size_t(i * a.hkv + g) * 2 * kCounterStride;
  uint32_t* depart = arrive + kCounterStride;
  if (tid == 0) {
    atomicAdd(arrive, 1u);
    unsigned polls = 0;
    while (ld_coherent(arrive) < unsigned(a.n_split)) {
      if (++polls > kMergeSpinLimit) {
        if (a.error) atomicOr(a.error, 2u);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
  const int d0 = kD * split / a.n_split, w = kD * (split + 1) / a.n_split - d0;
  const int64_t pstride = int64_t(a.nq) * a.hq;  // rows per part
  const int64_t row0 = int64_t(i) * a.hq + g * kG;
  constexpr int kMB = 16;  // parts per batch
  for (int e = tid; e < kG * w; e += 256) {
    const int h = e / w, d = d0 + e % w;
    float mx = -INFINITY, tot = 0.f, acc = 0.f;
    for (int p0 = 0; p0 < a.n_split; p0 += kMB) {
      float lp[kMB], op[kMB];
#pragma unroll
      for (int q = 0; q < kMB; q++) {
        const int p = p0 + q;
        const bool ok = p < a.n_split;
        const int64_t r = p * pstride + row0 + h;
        lp[q] = ok ? __uint_as_float(ld_coherent(reinterpret_cast<const uint32_t*>(a.lse_part + r))) : -INFINITY;
        op[q] = ok ? __uint_as_float(ld_coherent(reinterpret_cast<const uint32_t*>(a.o_part + r * kD + d))) : 0.f;
      }
      float bm = mx;
#pragma unroll
      for (int q = 0; q < kMB; q++) bm = fmaxf(bm, lp[q]);
      if (bm == -INFINITY) continue;
      const float sc = expf(mx - bm);
      tot *= sc;
      acc *= sc;
      mx = bm;
#pragma unroll
      for (int q = 0; q < kMB; q++) {
        if (lp[q] == -INFINITY) continue;  // empty part
        const float wq = expf(lp[q] - mx);
        tot += wq;
        acc += wq * op[q];
      }
    }
    const float o = tot > 0.f ? acc / tot : 0.f;
    const int64_t hrow = row0 + h;
    if (a.o_out) a.o_out[hrow * kD + d] = o;
    if (a.o_bf16) a.o_bf16[hrow * kD + d] = f32_to_bf16(o);
    if (a.lse_out && split == 0 && e % w == 0) a.lse_out[hrow] = tot > 0.f ? mx + logf(tot) : -INFINITY;
  }
  // the last part to leave resets both counters for the next call: every
  // part has passed its wait by then
  if (tid == 0 && atomicAdd(depart, 1u) == unsigned(a.n_split - 1)) {
    atomicExch(arrive, 0u);
    atomicExch(depart, 0u);
  }
}

}  // namespace att
}  // namespace qsa
