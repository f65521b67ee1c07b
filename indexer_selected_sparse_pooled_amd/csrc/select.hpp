// Exact top-k selection building blocks (wave64, gfx950).
//
// Ranking ("125B MoE を 3090 3 枚で運用する vLLM 最適化編", section 3.3: the
// top-k there ranks an order-preserving integer image of each value and
// gives equal values to the smaller id): every fp32 score becomes an
// order-preserving 32-bit key (order_key, never 0 for a finite score, so 0
// marks an empty slot) and elements rank by (key descending, index
// ascending). The k best elements are therefore unique, and so is the
// selection. As a single 64-bit value, rank64(key, index) orders elements
// the same way (larger ranks better).
//
// Three kinds of selectors:
//  * wave_*:   one wave, keys in registers, no barrier (bit-by-bit
//              threshold search with ballot counts);
//  * regsel_*: one work-group, keys in registers, threshold found by 8-bit
//              radix passes over LDS histograms that start below the common
//              prefix of the largest and smallest key (one barrier a pass);
//  * stream_*: one work-group, keys read through a functor (global memory),
//              any count; slow path.
#pragma once

#include "common.hpp"

namespace qsa {

__device__ __forceinline__ uint64_t rank64(uint32_t key, int idx) {
  return (uint64_t(key) << 32) | uint32_t(~uint32_t(idx));
}

__device__ __forceinline__ uint64_t lanes_below() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}


// ------------------------------------------------------------------ wave ----
// Keys key[r] of lane l are element r*64 + l of the wave's range; empty slots
// hold 0 and never count (every candidate threshold is >= 1).

// k-th largest key among the wave's nonzero keys; need = k - #{key > kstar}.
// Keys hold kBits bits (the bits above are zero): one ballot step per bit.
// Requires 1 <= k <= number of nonzero keys. Wave-uniform results.
template <int R, int kBits = 32>
__device__ __forceinline__ void wave_select(const uint32_t (&key)[R], int k, uint32_t& kstar, int& need) {
  uint32_t t = 0;
#pragma unroll 1
  for (int bit = kBits - 1; bit >= 0; bit--) {
    const uint32_t cand = t | (1u << bit);
    int c = 0;
#pragma unroll
    for (int r = 0; r < R; r++) c += __popcll(__ballot(key[r] >= cand));
    if (c >= k) t = cand;
  }
  int gt = 0;
  if (t != 0xFFFFFFFFu) {
#pragma unroll
    for (int r = 0; r < R; r++) gt += __popcll(__ballot(key[r] > t));
  }
  kstar = t;
  need = k - gt;
}

// Emit, in element order, every key > kstar and the first `need` keys equal
// to kstar: emit(position, r) for key[r] of the calling lane. Returns the
// element that is the need-th one equal to kstar (wave-uniform), or -1 if
// there is none.
template <int R, class Emit>
__device__ __forceinline__ int wave_compact(const uint32_t (&key)[R], uint32_t kstar, int need, Emit emit) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt = lanes_below();
  int base_g = 0, base_e = 0, tau = -1;
#pragma unroll
  for (int r = 0; r < R; r++) {
    const bool fg = key[r] > kstar;
    const bool fe = key[r] == kstar && key[r] != 0u;
    const uint64_t bg = __ballot(fg), be = __ballot(fe);
    const int gb = base_g + __popcll(bg & lt);
    const int eb = base_e + __popcll(be & lt);
    if (fg || (fe && eb < need)) emit(gb + (eb < need ? eb : need), r);
    const uint64_t tm = __ballot(fe && eb == need - 1);
    if (tm) tau = r * 64 + int(__ffsll(static_cast<unsigned long long>(tm)) - 1);
    base_g += __popcll(bg);
    base_e += __popcll(be);
  }
  return tau;
}

// rank64 of the best element that wave_compact(key, kstar, need) leaves out
// (0 if it keeps every nonzero key), ranked by its full key fkey[r] (key may
// be a coarser image of it, e.g. its top bits); idx_of(j) is element j's
// index. Wave-uniform.
template <int R, class IdxOf>
__device__ __forceinline__ uint64_t wave_best_excluded(const uint32_t (&key)[R], const uint32_t (&fkey)[R],
                                                       uint32_t kstar, int need, IdxOf idx_of) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt = lanes_below();
  int base_e = 0;
  uint64_t best = 0ull;
#pragma unroll
  for (int r = 0; r < R; r++) {
    const bool fe = key[r] == kstar && key[r] != 0u;
    const uint64_t be = __ballot(fe);
    const int eb = base_e + __popcll(be & lt);
    const bool out = key[r] != 0u && (key[r] < kstar || (fe && eb >= need));
    if (out) {
      const uint64_t k64 = rank64(fkey[r], idx_of(r * 64 + lane));
      best = k64 > best ? k64 : best;
    }
    base_e += __popcll(be);
  }
  return wave_max_u64(best);
}

// --------------------------------------------------------- work-group, regs --
// Element j = tid * R + r lives in key[r] of thread tid (so element order is
// thread order, then register order). Empty slots hold 0.

// Once the threshold digit's bin holds at most this many keys, they move
// to LDS and one wave finds the exact threshold among them bit by bit (one
// ballot per bit), instead of more histogram passes over every key.
constexpr int kRegSelCand = 64;

// LDS histogram increment of bin b (< 256) for the lanes with `in`: the
// lanes that share the first such lane's bin add their count in one atomic
// (scores cluster, and identical keys all fall in one bin, so one bin often
// takes most of a wave and would otherwise serialize on one address); every
// other lane adds to its own bin, or to its dummy bin 256 + lane, so the
// instruction carries no branch.
__device__ __forceinline__ void hist_add(uint32_t* h, bool in, uint32_t b) {
  const int lane = threadIdx.x & 63;
  const uint64_t act = __ballot(in);
  const int first = act ? int(__ffsll(static_cast<unsigned long long>(act))) - 1 : 0;
  const uint32_t b0 = uint32_t(__builtin_amdgcn_readlane(int(b), first));
  const uint64_t same = __ballot(in && b == b0);
  const bool lead = in && lane == first;
  const bool own = lead || (in && b != b0);
  atomicAdd(&h[own ? b : 256u + lane], lead ? uint32_t(__popcll(same)) : 1u);
}

// Histogram bins 256 + lane and counters / slots past the candidates are
// per-lane dummies: keys that take no part in a pass still issue their LDS
// atomic or store (to a lane of their own, so no two lanes of one
// instruction collide), which keeps the per-key loops free of branches.
template <int NT>
struct RegSelLds {
  uint32_t hist[3][256 + 64];
  uint32_t wmax[NT / 64], wmin[NT / 64];
  int wg[NT / 64], we[NT / 64];
  int pg[64], pe[64];  // register-major positions: counts per (register, wave)
  uint32_t cand[kRegSelCand + 64];
  uint32_t n_cand[1 + 64];
  int eqmx[NT / 64];  // (kAgg) per wave: keys equal to the largest
  uint32_t res_key;
  int res_need;
  int tau_slot;
  int tau_val;
};

// The k-th largest nonzero key (kstar) and need = k - #{key > kstar} >= 1.
// Requires 1 <= k <= number of nonzero keys. 8-bit radix passes narrow the
// threshold to one bin; as soon as that bin holds at most kRegSelCand keys,
// they are gathered in LDS and wave 0 settles the remaining low bits.
// kAgg: histogram increments go through hist_add (worth its extra
// instructions where many keys are equal, e.g. scores that are exact zeros),
// and the first pass also counts the keys equal to the largest: with k or
// more of them the threshold is found without further passes.
template <int NT, int R, bool kAgg = false>
__device__ void regsel_threshold(const uint32_t (&key)[R], int k, RegSelLds<NT>& sh, uint32_t& kstar, int& need) {
  constexpr int NW = NT / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t mx = 0u, mn = 0xFFFFFFFFu;
#pragma unroll
  for (int r = 0; r < R; r++) {
    if (key[r] != 0u) {
      mx = key[r] > mx ? key[r] : mx;
      mn = key[r] < mn ? key[r] : mn;
    }
  }
  mx = wave_max_u32(mx);
  mn = wave_min_u32(mn);
  if (lane == 0) {
    sh.wmax[wave] = mx;
    sh.wmin[wave] = mn;
  }
  for (int b = threadIdx.x; b < 256; b += NT) sh.hist[0][b] = 0u;
  if (threadIdx.x == 0) sh.n_cand[0] = 0u;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; w++) {
    mx = sh.wmax[w] > mx ? sh.wmax[w] : mx;
    mn = sh.wmin[w] < mn ? sh.wmin[w] : mn;
  }
  const uint32_t diff = mx ^ mn;
  if (diff == 0u) {  // every nonzero key is equal
    kstar = mx;
    need = k;
    return;
  }
  int lo = 32 - __clz(diff);  // bits [lo, 32) are common to every nonzero key
  uint32_t mask = lo >= 32 ? 0u : ~((1u << lo) - 1u);
  uint32_t prefix = mx & mask;
  int remaining = k;
  int pass = 0;
  int dcnt = 0;  // keys in the bin chosen last
  while (lo > 0) {
    const int width = lo < 8 ? lo : 8;
    const int shift = lo - width;
    const uint32_t dmask = (1u << width) - 1u;
    uint32_t* h = sh.hist[pass % 3];
    uint32_t* hz = sh.hist[(pass + 1) % 3];
    for (int b = threadIdx.x; b < 256; b += NT) hz[b] = 0u;
#pragma unroll
    for (int r = 0; r < R; r++) {
      const bool in = key[r] != 0u && (key[r] & mask) == prefix;
      if constexpr (kAgg)
        hist_add(h, in, (key[r] >> shift) & dmask);
      else
        atomicAdd(&h[in ? (key[r] >> shift) & dmask : 256u + lane], 1u);
    }
    if constexpr (kAgg) {
      if (pass == 0) {  // keys equal to the largest (many equal keys: e.g. exact-zero scores)
        int eq = 0;
#pragma unroll
        for (int r = 0; r < R; r++) eq += key[r] == mx ? 1 : 0;
        eq = wave_incl_sum(eq);
        if (lane == 63) sh.eqmx[wave] = eq;
      }
    }
    __syncthreads();
    if constexpr (kAgg) {
      if (pass == 0) {  // at least k of them: the threshold is the largest key itself
        int te = 0;
#pragma unroll
        for (int w = 0; w < NW; w++) te += sh.eqmx[w];
        if (te >= k) {
          kstar = mx;
          need = k;
          return;
        }
      }
    }
    // every wave finds the digit (same result everywhere): lane holds the
    // bins 255 - 4*lane - e, e = 0..3, i.e. digits in descending order
    int cnt[4];
    int lsum = 0;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      cnt[e] = int(h[255 - (4 * lane + e)]);
      lsum += cnt[e];
    }
    int above = wave_incl_sum(lsum) - lsum;
    int my_digit = -1, my_above = 0, my_cnt = 0;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      if (my_digit < 0 && above < remaining && remaining <= above + cnt[e]) {
        my_digit = 255 - (4 * lane + e);
        my_above = above;
        my_cnt = cnt[e];
      }
      above += cnt[e];
    }
    const uint64_t hit = __ballot(my_digit >= 0);
    const int src = int(__ffsll(static_cast<unsigned long long>(hit)) - 1);
    const uint32_t digit = uint32_t(__builtin_amdgcn_readlane(my_digit, src));
    remaining -= __builtin_amdgcn_readlane(my_above, src);
    dcnt = __builtin_amdgcn_readlane(my_cnt, src);
    prefix |= digit << shift;
    mask |= dmask << shift;
    lo = shift;
    pass++;
    if (dcnt <= kRegSelCand) break;
  }
  if (lo == 0) {  // every bit settled by the passes
    kstar = prefix;
    need = remaining;
    return;
  }
  // the dcnt keys of the chosen bin (1 <= remaining <= dcnt of them are
  // still needed): the largest t with #{bin keys >= t} >= remaining is the
  // threshold, found from the top remaining bit down
  uint32_t slot[R];
#pragma unroll
  for (int r = 0; r < R; r++) {
    const bool in = key[r] != 0u && (key[r] & mask) == prefix;
    slot[r] = atomicAdd(&sh.n_cand[in ? 0 : 1 + lane], 1u);
    slot[r] = in ? slot[r] : uint32_t(kRegSelCand + lane);
  }
#pragma unroll
  for (int r = 0; r < R; r++) sh.cand[slot[r]] = key[r];
  __syncthreads();
  if (wave == 0) {
    const uint32_t c = lane < dcnt ? sh.cand[lane] : 0u;
    uint32_t t = prefix;
    for (int bit = lo - 1; bit >= 0; bit--) {
      const uint32_t cd = t | (1u << bit);
      if (__popcll(__ballot(c >= cd)) >= remaining) t = cd;
    }
    const int gt = __popcll(__ballot(c > t));
    if (lane == 0) {
      sh.res_key = t;
      sh.res_need = remaining - gt;
    }
  }
  __syncthreads();
  kstar = sh.res_key;
  need = sh.res_need;
}

// Output position of every element (-1 if not selected): keys > kstar and
// the first `need` keys equal to kstar in element order. Also records the
// element that is the need-th equal one (the k-th best): its slot in
// sh.tau_slot and its val[] entry in sh.tau_val. Ends with a barrier.
template <int NT, int R>
__device__ void regsel_positions(const uint32_t (&key)[R], const int (&val)[R], uint32_t kstar, int need,
                                 RegSelLds<NT>& sh, int (&pos)[R]) {
  constexpr int NW = NT / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int g = 0, e = 0;
#pragma unroll
  for (int r = 0; r < R; r++) {
    g += key[r] > kstar ? 1 : 0;
    e += (key[r] == kstar && key[r] != 0u) ? 1 : 0;
  }
  const int ig = wave_incl_sum(g), ie = wave_incl_sum(e);
  if (lane == 63) {
    sh.wg[wave] = ig;
    sh.we[wave] = ie;
  }
  __syncthreads();
  int gb = ig - g, eb = ie - e;
#pragma unroll
  for (int w = 0; w < NW; w++) {
    if (w < wave) {
      gb += sh.wg[w];
      eb += sh.we[w];
    }
  }
#pragma unroll
  for (int r = 0; r < R; r++) {
    pos[r] = -1;
    if (key[r] > kstar) {
      pos[r] = gb + (eb < need ? eb : need);
      gb++;
    } else if (key[r] == kstar && key[r] != 0u) {
      if (eb < need) pos[r] = gb + eb;
      if (eb == need - 1) {
        sh.tau_slot = threadIdx.x * R + r;
        sh.tau_val = val[r];
      }
      eb++;
    }
  }
  __syncthreads();
}

// regsel_positions for the register-major layout: element j = r * NT + tid
// lives in key[r] of thread tid (consecutive threads hold consecutive
// elements, so loading them is coalesced). Same results and the same
// sh.tau_slot / sh.tau_val; ends with a barrier. Each wave counts its
// greater / equal keys per register with ballots; one exchange of those
// counts gives every (register, wave) pair its offset.
template <int NT, int R>
__device__ void regsel_positions_rm(const uint32_t (&key)[R], const int (&val)[R], uint32_t kstar, int need,
                                    RegSelLds<NT>& sh, int (&pos)[R]) {
  constexpr int NW = NT / 64;
  static_assert(R * NW <= 64, "one lane per (register, wave) pair");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const uint64_t lt = lanes_below();
  uint64_t bg[R], be[R];
  int cg = 0, ce = 0;  // lane r: this wave's counts for register r
#pragma unroll
  for (int r = 0; r < R; r++) {
    bg[r] = __ballot(key[r] > kstar);
    be[r] = __ballot(key[r] == kstar && key[r] != 0u);
    if (lane == r) {
      cg = __popcll(bg[r]);
      ce = __popcll(be[r]);
    }
  }
  if (lane < R) {
    sh.pg[lane * NW + wave] = cg;
    sh.pe[lane * NW + wave] = ce;
  }
  __syncthreads();
  // lane l holds pair l = r * NW + w (element order); exclusive prefix sums
  const int xg = lane < R * NW ? sh.pg[lane] : 0, xe = lane < R * NW ? sh.pe[lane] : 0;
  const int og = wave_incl_sum(xg) - xg, oe = wave_incl_sum(xe) - xe;
#pragma unroll
  for (int r = 0; r < R; r++) {
    const int gb = __builtin_amdgcn_readlane(og, r * NW + wave) + __popcll(bg[r] & lt);
    const int eb = __builtin_amdgcn_readlane(oe, r * NW + wave) + __popcll(be[r] & lt);
    pos[r] = -1;
    if (key[r] > kstar) {
      pos[r] = gb + (eb < need ? eb : need);
    } else if (key[r] == kstar && key[r] != 0u) {
      if (eb < need) pos[r] = gb + eb;
      if (eb == need - 1) {
        sh.tau_slot = r * NT + int(threadIdx.x);
        sh.tau_val = val[r];
      }
    }
  }
  __syncthreads();
}

// ---------------------------------------------------- work-group, streamed --

struct StreamLds {
  uint32_t hist[256];
  int wsum[2][16];
  int digit;
  int above;
};

// Block-wide sums of two per-wave counters (up to 16 waves): this wave's
// exclusive offsets and the totals.
template <int NT>
__device__ __forceinline__ void wave_offsets(int a, int b, StreamLds& sh, int& off_a, int& off_b, int& tot_a,
                                             int& tot_b) {
  constexpr int NW = NT / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    sh.wsum[0][wave] = a;
    sh.wsum[1][wave] = b;
  }
  __syncthreads();
  off_a = 0, off_b = 0, tot_a = 0, tot_b = 0;
#pragma unroll
  for (int w = 0; w < NW; w++) {
    const int x = sh.wsum[0][w], y = sh.wsum[1][w];
    if (w < wave) {
      off_a += x;
      off_b += y;
    }
    tot_a += x;
    tot_b += y;
  }
  __syncthreads();
}

// The k-th largest key among key_at(0..n) and need = k - #{key > kstar}.
// Radix passes of up to 8 bits, each reading every key once, that start
// below the common prefix of the largest and smallest key (one extra read
// finds them): scores cluster in their top bits, and a pass over bits every
// key shares would send them all to one histogram bin. Requires
// 1 <= k <= n.
template <int NT, class KeyAt>
__device__ void stream_select(KeyAt key_at, int n, int k, StreamLds& sh, uint32_t& kstar, int& need) {
  constexpr int NW = NT / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t mx = 0u, mn = 0xFFFFFFFFu;
  for (int j = threadIdx.x; j < n; j += NT) {
    const uint32_t key = key_at(j);
    mx = key > mx ? key : mx;
    mn = key < mn ? key : mn;
  }
  mx = wave_max_u32(mx);
  mn = wave_min_u32(mn);
  if (lane == 0) {
    sh.wsum[0][wave] = int(mx);
    sh.wsum[1][wave] = int(mn);
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; w++) {
    const uint32_t x = uint32_t(sh.wsum[0][w]), y = uint32_t(sh.wsum[1][w]);
    mx = x > mx ? x : mx;
    mn = y < mn ? y : mn;
  }
  __syncthreads();
  const uint32_t diff = mx ^ mn;
  if (diff == 0u) {  // every key is equal
    kstar = mx;
    need = k;
    return;
  }
  int lo = 32 - __clz(diff);  // bits [lo, 32) are common to every key
  uint32_t mask = lo >= 32 ? 0u : ~((1u << lo) - 1u);
  uint32_t prefix = mx & mask;
  int remaining = k;
  while (lo > 0) {
    const int width = lo < 8 ? lo : 8;
    const int shift = lo - width;
    const uint32_t dmask = (1u << width) - 1u;
    for (int b = threadIdx.x; b < 256; b += NT) sh.hist[b] = 0;
    __syncthreads();
    for (int j = threadIdx.x; j < n; j += NT) {
      const uint32_t key = key_at(j);
      if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      int cnt[4];
      int lsum = 0;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        cnt[e] = int(sh.hist[255 - (4 * lane + e)]);
        lsum += cnt[e];
      }
      int above = wave_incl_sum(lsum) - lsum;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        if (above < remaining && remaining <= above + cnt[e]) {
          sh.digit = 255 - (4 * lane + e);
          sh.above = above;
        }
        above += cnt[e];
      }
    }
    __syncthreads();
    remaining -= sh.above;
    prefix |= uint32_t(sh.digit) << shift;
    mask |= dmask << shift;
    lo = shift;
    __syncthreads();
  }
  kstar = prefix;
  need = remaining;
}

// Emit, in ascending index order, every j with key > kstar plus the first
// `need` j with key == kstar: emit(position, j). Each round a thread takes
// kB consecutive keys, so a block-wide prefix (two barriers) covers NT * kB
// keys at once.
template <int NT, class KeyAt, class Emit>
__device__ void stream_compact(KeyAt key_at, int n, uint32_t kstar, int need, StreamLds& sh, Emit emit) {
  constexpr int kB = 16;
  const int lane = threadIdx.x & 63;
  int base_g = 0, base_e = 0;
  for (int r0 = 0; r0 < n; r0 += NT * kB) {
    const int j0 = r0 + kB * int(threadIdx.x);
    uint32_t fg = 0u, fe = 0u;  // bit r: key j0 + r is greater / equal
#pragma unroll
    for (int r = 0; r < kB; r++) {
      const int j = j0 + r;
      const uint32_t key = j < n ? key_at(j) : 0u;
      fg |= uint32_t(j < n && key > kstar) << r;
      fe |= uint32_t(j < n && key == kstar) << r;
    }
    const int cg = __popc(fg), ce = __popc(fe);
    // inclusive scan of (cg, ce) over the wave
    const int ig = wave_incl_sum(cg), ie = wave_incl_sum(ce);
    int wg_off, we_off, tg, te;
    wave_offsets<NT>(__builtin_amdgcn_readlane(ig, 63), __builtin_amdgcn_readlane(ie, 63), sh, wg_off, we_off, tg, te);
    int gb = base_g + wg_off + ig - cg;
    int eb = base_e + we_off + ie - ce;
#pragma unroll
    for (int r = 0; r < kB; r++) {
      if ((fg >> r) & 1u) {
        emit(gb + (eb < need ? eb : need), j0 + r);
        gb++;
      } else if ((fe >> r) & 1u) {
        if (eb < need) emit(gb + eb, j0 + r);
        eb++;
      }
    }
    base_g += tg;
    base_e += te;
  }
}

// Index of the need-th (1-based) element equal to kstar, in index order.
template <int NT, class KeyAt>
__device__ int stream_nth_equal(KeyAt key_at, int n, uint32_t kstar, int need, StreamLds& sh, int* out) {
  const uint64_t lt = lanes_below();
  int base_e = 0;
  for (int r0 = 0; r0 < n; r0 += NT) {
    const int j = r0 + threadIdx.x;
    const bool fe = j < n && key_at(j) == kstar;
    const uint64_t be = __ballot(fe);
    int og, oe, tg, te;
    wave_offsets<NT>(0, __popcll(be), sh, og, oe, tg, te);
    if (fe && base_e + oe + __popcll(be & lt) == need - 1) *out = j;
    base_e += te;
    if (base_e >= need) break;
  }
  __syncthreads();
  return *out;
}

}  // namespace qsa
