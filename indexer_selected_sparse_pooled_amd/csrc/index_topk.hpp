// Device code of A2 + A3 for decode: the pooled-key scan and the exact top-k
// of one chunk of one query (index_topk.hip launches it on its own,
// decode_layer.hip as the decode layer's first launch, without the selection).
// "3090x3で 314 万コンテキスト", section "VRAM に残す必要があるもの": every
// pooled key (128 x bf16 per block) is scored at every step, so the scan is
// a bandwidth-bound stream; section "なぜ": the indexer then keeps a fixed
// budget of blocks (all of them when there are at most topk).
//
// A work-group scores one chunk of C = 256 * TPW
// consecutive blocks of one query (wave w takes tiles w*TPW .. w*TPW+TPW-1
// of 64 keys, 16 lanes per key row, 16-byte non-temporal loads, partial dots
// folded by a transposing butterfly), writes the scores, and keeps the
// chunk's best (key, block) pairs (16, or 8 when a query has more than 256
// chunks) plus a bound: the best block it leaves out. Every wave first keeps
// 8 (register threshold search, no barrier), wave 0 then 16 of the 32. The
// lists are chosen on the top 16 bits of the keys (every key above the
// 16-bit threshold, then the first at it), which halves the search; the
// bound is still the best block left out at full precision, which is all
// the selection below relies on.
//
// The last work-group of a query to finish (device-scope counter) selects:
//  * union mode: the topk best of the union of the chunk lists (register
//    radix select, one list per thread). With tau the topk-th best of the
//    union, a chunk can hide a better element only if its bound ranks above
//    tau; if none does, the union's top-k is the exact top-k. Otherwise,
//    and in
//  * stream mode (too few chunks for the union to be safe), an exact select
//    over every score of the query read back from memory;
//  * raw mode (at most 4096 candidates): the register select straight on the
//    query's scores.
// Results are identical in every mode: the unique top-k under (score
// descending, block ascending), written in ascending block order.
//
// Hand-off between work-groups inside the launch: scores, lists and bounds
// are written with agent-coherent (sc1) stores, each thread waits for its
// stores to complete before the work-group's barrier, and only then is the
// counter incremented; the last work-group reads with coherent loads. No
// L2 write-back or invalidate is needed (those cost more than the scan).
#pragma once

#include "common.hpp"
#include "fp8.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace qsa {
namespace itk {

// Selections are written with agent-coherent stores, as every hand-off
// between work-groups of one launch is.
__device__ __forceinline__ void st_sel(int* p, int v) { st_coherent(reinterpret_cast<uint32_t*>(p), uint32_t(v)); }

// Stores of the scan's outputs: agent-coherent when a work-group of the
// same launch reads them (the last arrival's selection), plain when only a
// later launch does (kernel boundaries order those).
template <bool kCoh>
__device__ __forceinline__ void put(uint32_t* p, uint32_t v) {
  if constexpr (kCoh) st_coherent(p, v); else *p = v;
}
template <bool kCoh>
__device__ __forceinline__ void put(uint64_t* p, uint64_t v) {
  if constexpr (kCoh) st_coherent(p, v); else *p = v;
}

// Every thread's stores are complete before the work-group goes on.
__device__ __forceinline__ void publish() {
  wait_memory();
  __syncthreads();
}


constexpr int kNT = 256;
constexpr int kWaveKeep = 8;    // at most, per wave (a.wkeep)
constexpr int kChunkKeep = 16;  // at most, per chunk (a.keep)
constexpr int kRegR = 16;       // union / raw entries per thread in the final select
constexpr int kRegCap = kNT * kRegR;

// One chunk's list step: every wave's candidates (at most WK) and bound.
template <int WK = kWaveKeep>
struct ListLds {
  uint32_t wkey[4 * WK];
  int widx[4 * WK];
  uint64_t wbound[4];
};

struct FinalLds {
  RegSelLds<kNT> rs;
  StreamLds st;
  ListLds<> lst;
  int last;
};

__device__ __forceinline__ uint32_t score_key(const float* sc, int j) {
  return order_key(__uint_as_float(ld_coherent(reinterpret_cast<const uint32_t*>(sc) + j)));
}

__device__ __forceinline__ float dot8(u32x4 k, u32x4 q) {
  float acc = 0.f;
  acc = dot2(k[0], q[0], acc);
  acc = dot2(k[1], q[1], acc);
  acc = dot2(k[2], q[2], acc);
  acc = dot2(k[3], q[3], acc);
  return acc;
}

// A tile is 64 consecutive keys; lane (g, c) = (lane / 16, lane % 16) reads
// bytes 16c .. 16c+15 of keys tile0 + 4k + g, k = 0..15. Rows past n are
// clamped to row n - 1 (read, then ignored), so the loads carry no branch.
__device__ __forceinline__ void load_tile(const uint16_t* kb, int64_t tile0, int64_t n, u32x4 (&v)[16]) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
#pragma unroll
  for (int k = 0; k < 16; k++) {
    const int64_t blk = tile0 + 4 * k + g;
    v[k] = ld16_nt(kb + (blk < n ? blk : n - 1) * 128 + 8 * c);
  }
  // keep the tile's loads together, in issue order: scoring a tile then
  // waits for its own loads only, not for the next tile's
  __builtin_amdgcn_sched_barrier(0);
}

// Scores of the tile loaded by load_tile (keys past n score 0); lane l
// returns the score of key tile0 + l.
__device__ __forceinline__ float tile_scores(const u32x4 (&v)[16], int64_t tile0, int64_t n, u32x4 qv) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
  float p[16];
#pragma unroll
  for (int k = 0; k < 16; k++) p[k] = tile0 + 4 * k + g < n ? dot8(v[k], qv) : 0.f;
  // transposing butterfly over the 16 lanes of a group: afterwards lane
  // (g, c) holds the full dot product of key 4c + g
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const bool up = c & 8;
    const float keep = up ? p[j + 8] : p[j];
    const float send = up ? p[j] : p[j + 8];
    p[j] = keep + __shfl_xor(send, 8);
  }
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
  // key l = 4c + g sits in lane 16 * (l % 4) + l / 4
  return __shfl(p[0], 16 * (lane & 3) + (lane >> 2));
}

// The score of pooled key b of query i computed by one thread, bit for bit
// the scan's (tile_scores / fp8::tile_scores): the same 16-byte chunk dots
// (dot2 chains for bf16 keys, fp32 FMA chains over exact E4M3 values for
// FP8 keys) and the same pairwise tree over the chunks as the scan's
// butterfly (fp32 addition is commutative, so only the pairing matters).
// q: the query's 128 bf16 indexer values; keys: its sequence's key rows
// (bf16) or FP8 pages (fp8). Plain values, not the argument struct: a
// reference to the kernel's argument struct would make the caller copy it
// to private memory.
__device__ __noinline__ float key_score(const uint16_t* q, const void* keys, int fp8, int b) {
  if (fp8) {
    const uint8_t* kb = static_cast<const uint8_t*>(keys);
    const uint8_t* row = kb + fp8_code_off(b, 128);
    float p[8];
#pragma unroll
    for (int c = 0; c < 8; c++) {  // chunk c: codes 16c .. 16c+15
      const u32x4 v = ld16(row + 16 * c);
      const u32x4 qa = ld16(q + 16 * c), qb = ld16(q + 16 * c + 8);
      float qf[16];
#pragma unroll
      for (int j = 0; j < 4; j++) {
        qf[2 * j] = bf16_lo(qa[j]);
        qf[2 * j + 1] = bf16_hi(qa[j]);
        qf[8 + 2 * j] = bf16_lo(qb[j]);
        qf[8 + 2 * j + 1] = bf16_hi(qb[j]);
      }
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; w++) {
        float x0, x1, x2, x3;
        e4m3x4(v[w], x0, x1, x2, x3);
        acc = fmaf(x0, qf[4 * w], acc);
        acc = fmaf(x1, qf[4 * w + 1], acc);
        acc = fmaf(x2, qf[4 * w + 2], acc);
        acc = fmaf(x3, qf[4 * w + 3], acc);
      }
      p[c] = acc;
    }
#pragma unroll
    for (int c = 0; c < 4; c++) p[c] = p[c] + p[c + 4];
#pragma unroll
    for (int c = 0; c < 2; c++) p[c] = p[c] + p[c + 2];
    const float sc = *reinterpret_cast<const float*>(kb + fp8_scale_off(b, 128));
    return (p[0] + p[1]) * sc;
  }
  const uint16_t* row = static_cast<const uint16_t*>(keys) + int64_t(b) * 128;
  float p[16];
#pragma unroll
  for (int c = 0; c < 16; c++) p[c] = dot8(ld16(row + 8 * c), ld16(q + 8 * c));
#pragma unroll
  for (int c = 0; c < 8; c++) p[c] = p[c] + p[c + 8];
#pragma unroll
  for (int c = 0; c < 4; c++) p[c] = p[c] + p[c + 4];
#pragma unroll
  for (int c = 0; c < 2; c++) p[c] = p[c] + p[c + 2];
  return p[0] + p[1];
}

// Exact selection over the scores of query i recomputed from its keys (for
// calls given no score buffer): the streamed select with each key's score
// computed where it is read. Slow (every pass reads the query's keys), but
// only taken where the chunk lists cannot show the selection exact.
template <class Emit>
__device__ void select_streamed_keys(const IndexTopkArgs& a, int i, int n, FinalLds& sh, Emit emit) {
  const int seq = a.q_seq ? a.q_seq[i] : 0;
  const uint16_t* q = a.q_idx + int64_t(i) * 128;
  const int64_t off = a.key_fp8 ? int64_t(seq) * a.keys_ss : int64_t(seq) * a.keys_ss * 2;
  const void* keys = static_cast<const uint8_t*>(a.keys) + off;
  const int fp8 = a.key_fp8;
  auto key_at = [q, keys, fp8](int j) { return order_key(key_score(q, keys, fp8, j)); };
  uint32_t kstar;
  int need;
  stream_select<kNT>(key_at, n, a.topk, sh.st, kstar, need);
  stream_compact<kNT>(key_at, n, kstar, need, sh.st, emit);
}

// Exact selection over the scores of one query, streamed from memory.
template <class Emit>
__device__ void select_streamed(const float* sc, int n, int topk, FinalLds& sh, Emit emit) {
  auto key_at = [&](int j) { return score_key(sc, j); };
  uint32_t kstar;
  int need;
  stream_select<kNT>(key_at, n, topk, sh.st, kstar, need);
  stream_compact<kNT>(key_at, n, kstar, need, sh.st, emit);
}

// Whether query i's exact top-k comes from the union of its chunk lists:
// enough lists for the union to hold the top-k twice over, few enough for
// the registers. Otherwise the scores themselves are selected from.
__device__ __forceinline__ bool use_union(const IndexTopkArgs& a, int n) {
  const int nch = (n + a.chunk_blocks - 1) / a.chunk_blocks;
  return n > kRegCap && nch * a.keep >= 2 * a.topk && nch * a.keep <= kRegCap;
}

// Union entry e = chunk * keep + slot of query i (each list in ascending
// block order, so entry order is block order), as (key << 32 | block), 0 =
// empty; thread t holds entries t * kRegR + r (thread-major). Entries at or
// past u are 0. The lists are stored pair-major (chunk_list), so the 16-byte
// pair loads of neighbouring threads are neighbours in memory. kCoh: written
// by other work-groups of the same launch (else by an earlier launch, and
// plain 16-byte loads see it).
template <bool kCoh = true>
__device__ __forceinline__ void load_union(const IndexTopkArgs& a, int i, int u, uint64_t (&ent)[kRegR]) {
  const uint64_t* ul = a.list + size_t(i) * a.n_chunks * a.keep;
  const int e0 = int(threadIdx.x) * kRegR;
  const int lk = a.keep == 16 ? 4 : 3;  // the list length is 8 or 16
  // u is a multiple of the list length, so pairs are never split
#pragma unroll
  for (int r = 0; r < kRegR; r += 2) {
    const int e = e0 + r;
    const int c = e >> lk, s = e & (a.keep - 1);
    const size_t at = (size_t(s >> 1) * a.n_chunks + c) * 2;
    if constexpr (kCoh) {
      ent[r] = e < u ? ld_coherent(ul + at) : 0ull;
      ent[r + 1] = e < u ? ld_coherent(ul + at + 1) : 0ull;
    } else {
      const u32x4 w = e < u ? ld16(ul + at) : u32x4{0u, 0u, 0u, 0u};
      ent[r] = (uint64_t(w[1]) << 32) | w[0];
      ent[r + 1] = (uint64_t(w[3]) << 32) | w[2];
    }
  }
}

// The topk best of the keys in registers (element j = tid * R + r, in
// block order; 0 = empty): emit(position, block) with position in [0, topk)
// for each selected key, positions ascending in element order, and
// emit(-1, block) for every other key of the thread (emit must ignore or
// redirect those: the loops carry no per-key branch); returns true. Returns
// false, emitting nothing, when in union mode a chunk's bound (the best block
// it left out; my_bound is the largest this thread checked) ranks above the
// union's topk-th, so the union may miss a better block. Positions come from
// one block-wide scan of the per-thread counts of keys above and equal to the
// threshold (packed in one word); the bound check rides on the same
// exchange: a bound key above the threshold fails at once, and only a bound
// key equal to it needs the topk-th's block.
// What select_registers found when it returns false on a tie (no bound key
// above the threshold, but one equal to it that ranks above the topk-th):
// the threshold key and need are then the whole row's, and every key above
// the threshold is in the union (n_gt of them).
struct RegSelOut {
  bool tie_fail;
  uint32_t kstar;
  int need, n_gt;
};

template <int R, bool kAgg = false, class Emit>
__device__ bool select_registers(const IndexTopkArgs& a, bool union_mode, const uint32_t (&ukey)[R],
                                 const int (&uidx)[R], uint64_t my_bound, FinalLds& sh, Emit emit, RegSelOut& out) {
  constexpr int NW = kNT / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t kstar;
  int need;
  regsel_threshold<kNT, R, kAgg>(ukey, a.topk, sh.rs, kstar, need);
  int g = 0, e = 0;
#pragma unroll
  for (int r = 0; r < R; r++) {
    g += ukey[r] > kstar ? 1 : 0;
    e += (ukey[r] == kstar && ukey[r] != 0u) ? 1 : 0;
  }
  static_assert(kNT * R < 65536, "two 16-bit counts in one word");
  const int v = g | (e << 16);  // at most kNT * R each: no carry between the halves
  const int incl = wave_incl_sum(v);
  const uint32_t bkey = uint32_t(my_bound >> 32);
  const uint64_t bfail = __ballot(union_mode && bkey > kstar);
  const uint64_t btie = __ballot(union_mode && my_bound != 0ull && bkey == kstar);
  if (lane == 63) sh.rs.wg[wave] = incl;
  if (lane == 0) sh.rs.we[wave] = (bfail ? 1 : 0) | (btie ? 2 : 0);
  __syncthreads();
  int off = incl - v, flags = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; w++) {
    if (w < wave) off += sh.rs.wg[w];
    tot += sh.rs.wg[w];
    flags |= sh.rs.we[w];
  }
  out.tie_fail = false;
  if (flags & 1) return false;
  const int gb0 = off & 0xFFFF, eb0 = off >> 16;
  if (flags & 2) {  // a bound ties with the threshold key: compare blocks
    int eb = eb0;
#pragma unroll
    for (int r = 0; r < R; r++) {
      const bool eq = ukey[r] == kstar && ukey[r] != 0u;
      if (eq && eb == need - 1) sh.rs.tau_val = uidx[r];
      eb += eq ? 1 : 0;
    }
    __syncthreads();
    const uint64_t tau = rank64(kstar, sh.rs.tau_val);
    if (__syncthreads_or(my_bound > tau)) {
      out.tie_fail = true;
      out.kstar = kstar;
      out.need = need;
      out.n_gt = tot & 0xFFFF;
      return false;
    }
  }
  // keys above kstar, then the first `need` keys equal to it, in element order
  int gb = gb0, eb = eb0;
#pragma unroll
  for (int r = 0; r < R; r++) {
    const bool gt = ukey[r] > kstar;
    const bool eq = ukey[r] == kstar && ukey[r] != 0u;
    const int p = gt ? gb + (eb < need ? eb : need) : ((eq && eb < need) ? gb + eb : -1);
    emit(p, uidx[r]);
    gb += gt ? 1 : 0;
    eb += eq ? 1 : 0;
  }
  return true;
}

template <int R = kRegR, class Emit>
__device__ __forceinline__ bool select_registers(const IndexTopkArgs& a, bool union_mode, const uint32_t (&ukey)[R],
                                                 const int (&uidx)[R], uint64_t my_bound, FinalLds& sh, Emit emit) {
  RegSelOut out;
  return select_registers<R>(a, union_mode, ukey, uidx, my_bound, sh, emit, out);
}

// The exact top-k of query i (n > topk candidates), once every chunk of the
// query has written its scores and list: emit(position, block) for each of
// the topk selected blocks, positions in ascending block order. Lists,
// bounds and scores are read with agent-coherent loads (they may have been
// written earlier in the same launch). Modes:
//  * union: register select over the chunk lists; exact unless a chunk's
//    bound (the best block it left out) ranks above the union's topk-th;
//  * raw (n <= 4096): register select straight over the scores;
//  * streamed: exact select over every score (too many or too few lists,
//    or a failed bound check).
template <class Emit>
__device__ void final_select(const IndexTopkArgs& a, int i, int n, FinalLds& sh, Emit emit) {
  const int tid = threadIdx.x;
  const float* sc = a.scores + int64_t(i) * a.ld;
  const bool union_mode = use_union(a, n);
  if (union_mode || n <= kRegCap) {
    uint32_t ukey[kRegR];
    int uidx[kRegR];
    uint64_t my_bound = 0ull;
    if (union_mode) {
      const int nch = (n + a.chunk_blocks - 1) / a.chunk_blocks;
      uint64_t ent[kRegR];
      load_union(a, i, nch * a.keep, ent);
#pragma unroll
      for (int r = 0; r < kRegR; r++) {
        ukey[r] = uint32_t(ent[r] >> 32);
        uidx[r] = int(uint32_t(ent[r]));
      }
      for (int c = tid; c < nch; c += kNT) {
        const uint64_t b = ld_coherent(a.list_bound + size_t(i) * a.n_chunks + c);
        my_bound = b > my_bound ? b : my_bound;
      }
    } else {
      // thread-major raw scores: element j = tid * kRegR + r
#pragma unroll
      for (int r = 0; r < kRegR; r++) {
        const int j = tid * kRegR + r;
        ukey[r] = j < n ? score_key(sc, j) : 0u;
        uidx[r] = j;
      }
    }
    if (select_registers(a, union_mode, ukey, uidx, my_bound, sh, [&](int pos, int blk) {
          if (pos >= 0) emit(pos, blk);
        }))
      return;
  }
  select_streamed(sc, n, a.topk, sh, emit);
}

// The list of one chunk (union mode): every wave keeps its a.wkeep (<= WK)
// best keys (a register threshold search on their top 16 bits, no barrier)
// and the best block it leaves out; wave 0 then keeps the chunk's `keep`
// best of the 4 WK and writes them (ascending block order, 0 past the kept
// ones) with the chunk's bound: the best block it left out, at full
// precision. key[t] holds the order key of block w0 + 64 t + lane (0 past
// n). One barrier; the caller keeps L untouched until every wave has passed
// the next one. kCoh: the list is read by another work-group of the same
// launch. kPairMajor: the query's lists are stored pair-major (entry
// (chunk c, slot s) at ((s / 2) * n_chunks + c) * 2 + s % 2 of the query's
// region), so that thread c loading list c's pairs reads contiguously
// across lanes; otherwise list by list.
template <int TPW, bool kCoh, int WK = kWaveKeep, bool kPairMajor = false>
__device__ void chunk_list(const IndexTopkArgs& a, int i, int chunk, int n, int64_t w0, const uint32_t (&key)[TPW],
                           ListLds<WK>& L) {
  static_assert(4 * WK <= 64, "wave 0 holds the 4 WK candidates one per lane");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int keep = a.keep, wkeep = a.wkeep;
  const int64_t m64 = int64_t(n) - w0;
  const int m = m64 <= 0 ? 0 : (m64 >= TPW * 64 ? TPW * 64 : int(m64));
  if (lane < WK) {
    L.wkey[wave * WK + lane] = 0u;
    L.widx[wave * WK + lane] = -1;
  }
  uint32_t kh[TPW];  // top 16 bits (nonzero for every nonzero key)
#pragma unroll
  for (int t = 0; t < TPW; t++) kh[t] = key[t] >> 16;
  uint32_t kstar = 0u;
  int need = wkeep;
  if (m > wkeep) wave_select<TPW, 16>(kh, wkeep, kstar, need);
  wave_compact<TPW>(kh, kstar, need, [&](int pos, int r) {
    L.wkey[wave * WK + pos] = key[r];
    L.widx[wave * WK + pos] = int(w0) + 64 * r + lane;
  });
  const uint64_t wb = wave_best_excluded<TPW>(kh, key, kstar, need, [&](int j) { return int(w0) + j; });
  if (lane == 0) L.wbound[wave] = wb;
  __syncthreads();
  if (wave == 0) {
    const uint32_t k1[1] = {lane < 4 * WK ? L.wkey[lane] : 0u};
    const uint32_t h1[1] = {k1[0] >> 16};
    const int i1 = lane < 4 * WK ? L.widx[lane] : -1;
    const int valid = __popcll(__ballot(k1[0] != 0u));
    uint64_t bound = 0ull;
#pragma unroll
    for (int w = 0; w < 4; w++) bound = L.wbound[w] > bound ? L.wbound[w] : bound;
    uint32_t ks = 0u;
    int nd = keep;
    if (valid > keep) wave_select<1, 16>(h1, keep, ks, nd);
    const size_t qbase = size_t(i) * a.n_chunks * keep;
    auto slot = [&](int pos) -> size_t {
      return kPairMajor ? qbase + (size_t(pos >> 1) * a.n_chunks + chunk) * 2 + (pos & 1)
                        : qbase + size_t(chunk) * keep + pos;
    };
    // kept entries (key << 32 | block) go to their list position; the
    // positions past the kept count are cleared (0 = empty)
    wave_compact<1>(h1, ks, nd, [&](int pos, int) {
      put<kCoh>(a.list + slot(pos), (uint64_t(k1[0]) << 32) | uint32_t(i1));
    });
    const int nkept = valid < keep ? valid : keep;
    if (lane >= nkept && lane < keep) put<kCoh>(a.list + slot(lane), 0ull);
    const uint64_t b = wave_best_excluded<1>(h1, k1, ks, nd, [&](int) { return i1; });
    bound = b > bound ? b : bound;
    if (lane == 0) put<kCoh>(a.list_bound + size_t(i) * a.n_chunks + chunk, bound);
  }
}

// One chunk of query i. Returns true in the one work-group that completed
// the query's selection (sel and n_sel written, the stores complete); the
// caller may then hand the selection on.
// kSelect == false: scores and lists only (the selection is made by the
// caller's next kernel), and the function returns false.
// kFp8: the keys are FP8 pages (fp8.hpp) instead of bf16 rows.
template <int TPW, bool kSelect = true, bool kFp8 = false>
__device__ bool chunk_step(const IndexTopkArgs& a, int i, int chunk, FinalLds& sh) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  constexpr int C = kNT * TPW;
  const int seq = a.q_seq ? a.q_seq[i] : 0;
  const int n = clamp_ctx(a.q_ctx[i], a.max_ctx) / 4;
  const int topk = a.topk;
  int* sel = a.sel + int64_t(i) * topk;
  const int64_t lo = int64_t(chunk) * C;
  if (lo >= n) {
    if (kSelect && chunk == 0) {  // n == 0: nothing to score
      for (int j = tid; j < topk; j += kNT) st_sel(sel + j, -1);
      if (tid == 0) st_sel(a.n_sel + i, 0);
      publish();
      return true;
    }
    return false;
  }
  const int nch = (n + C - 1) / C;

  // ---- scan: scores of this chunk (the lists-only scan writes them only
  // when given a score buffer)
  const bool store = kSelect || a.scores != nullptr;
  float* out = store ? a.scores + int64_t(i) * a.ld : nullptr;
  const int64_t w0 = lo + int64_t(wave) * TPW * 64;
  uint32_t key[TPW];
  // two tiles in flight per wave: the next tile's loads are issued before
  // the current one is scored. The loads are unconditional (tiles past n
  // re-read row n - 1): on a branch, scoring would have to wait for every
  // load in flight, the next tile's included.
  auto keep_score = [&](int t, int64_t tile0, float s) {
    const int64_t blk = tile0 + lane;
    if (blk < n) {
      if (store) put<kSelect>(reinterpret_cast<uint32_t*>(out) + blk, __float_as_uint(s));
      key[t] = order_key(s);
    }
  };
  if constexpr (kFp8) {
    float qf[16];
    fp8::load_query(a.q_idx + int64_t(i) * 128, qf);
    const uint8_t* kb = static_cast<const uint8_t*>(a.keys) + int64_t(seq) * a.keys_ss;
    u32x4 v[2][8];
    float sc[2];
    fp8::load_tile(kb, w0, n, v[0], sc[0]);
#pragma unroll
    for (int t = 0; t < TPW; t++) {
      const int64_t tile0 = w0 + 64 * t;
      if (t + 1 < TPW) fp8::load_tile(kb, tile0 + 64, n, v[(t + 1) & 1], sc[(t + 1) & 1]);
      key[t] = 0u;
      if (tile0 < n) keep_score(t, tile0, fp8::tile_scores(v[t & 1], sc[t & 1], tile0, n, qf));  // wave-uniform
    }
  } else {
    const u32x4 qv = ld16(a.q_idx + int64_t(i) * 128 + 8 * (lane & 15));
    const uint16_t* kb = static_cast<const uint16_t*>(a.keys) + int64_t(seq) * a.keys_ss;
    u32x4 v[2][16];
    load_tile(kb, w0, n, v[0]);
#pragma unroll
    for (int t = 0; t < TPW; t++) {
      const int64_t tile0 = w0 + 64 * t;
      if (t + 1 < TPW) load_tile(kb, tile0 + 64, n, v[(t + 1) & 1]);
      key[t] = 0u;
      if (tile0 < n) keep_score(t, tile0, tile_scores(v[t & 1], tile0, n, qv));  // wave-uniform
    }
  }

  if (n <= topk) {  // every block is selected
    if (kSelect && chunk == 0) {
      for (int j = tid; j < topk; j += kNT) st_sel(sel + j, j < n ? j : -1);
      if (tid == 0) st_sel(a.n_sel + i, n);
      publish();
      return true;
    }
    return false;
  }
  const bool union_mode = use_union(a, n);

  // ---- chunk list: 8 best per wave, then 16 best of the 32
  if (union_mode) chunk_list<TPW, kSelect, kWaveKeep, true>(a, i, chunk, n, w0, key, sh.lst);

  if (!kSelect) return false;
  // ---- the last work-group of this query selects
  wait_memory();  // this thread's coherent stores are complete
  __syncthreads();
  uint32_t* cnt = a.counter + size_t(i) * kCounterStride;
  if (tid == 0) sh.last = atomicAdd(cnt, 1u) == unsigned(nch - 1);
  __syncthreads();
  if (!sh.last) return false;
  if (tid == 0) {
    atomicExch(cnt, 0u);  // ready for the next call
    st_sel(a.n_sel + i, topk);
  }
  final_select(a, i, n, sh, [&](int pos, int blk) { st_sel(sel + pos, blk); });
  publish();
  return true;
}

}  // namespace itk
}  // namespace qsa
