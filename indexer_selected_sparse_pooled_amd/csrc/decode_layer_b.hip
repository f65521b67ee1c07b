// One decode layer of the shared-latent variant in one call: A2 + A3 + A4 +
// A5 in three launches. "GLM-5.3 最適化 第2部", section "PCP": the
// token-level indexer (4 heads of 64 dims, ReLU-weighted) scores every
// earlier token and its top-2048 feed the sparse MLA; section "DCP": the
// parts' results are merged by log-sum-exp.
//
// Launch 1 (index_lists_b): each work-group scores one chunk of 512 keys of
// one query (scores_b.hpp, one wave per 128 keys), writes the scores (the
// exact fallback below reads them), and, when the query's selection comes
// from the chunk lists, keeps the chunk's list: the waves' scores are
// exchanged into key order, every wave keeps its 16 best keys and the best
// one it leaves out, wave 0 then the chunk's 32 best of the 64 and the
// chunk's bound (itk::chunk_list; the lists stored pair-major, so the
// select below loads them with contiguous lanes).
//
// Launch 2 (attend_select_b): one work-group per (query, split). Every
// work-group selects its query's exact top-k itself into LDS: from the union
// of the chunk lists (up to 8192 entries; thread t holds chunk t's list),
// exact when no chunk's bound (the best key it left out) ranks above the
// union's k-th, else from the scores (one pass when only a tie at the k-th
// key failed: the threshold is then known); a query with at most 8192 keys
// selects straight from its scores in registers, and one with too few or
// too many chunks for the union by radix passes over its scores. Split 0 also writes
// the selection to sel / n_sel. Each part then attends its split of the
// selected tokens (attend_mla.hpp, transposed form, the rows gathered
// straight from the LDS selection) and writes its partial result.
//
// Launch 3: the log-sum-exp merge of the splits (merge.hip).
#include "attend_mla.hpp"
#include "index_topk.hpp"
#include "scores_b.hpp"

namespace qsa {
namespace {

constexpr int kWaveKeepB = 16;                 // candidates per wave (128 keys)
constexpr int kRegRB = kDecodeBKeep;           // union or raw entries per thread: one chunk list
constexpr int kUnionCapB = itk::kNT * kRegRB;  // 8192
constexpr int kMaxTopkB = 2048;
static_assert(kDecodeBChunk == 4 * 128, "one wave per 128 keys");
static_assert(kDecodeBMaxChunks == itk::kNT, "thread t holds chunk t's list");

// Whether a query with n > topk keys selects from the union of its chunk
// lists: more keys than the registers hold, lists enough to hold the top-k
// twice over, and one list per thread at most.
__host__ __device__ inline bool union_b(int n, int topk) {
  const int nch = (n + kDecodeBChunk - 1) / kDecodeBChunk;
  return n > kUnionCapB && nch * kDecodeBKeep >= 2 * topk && nch <= kDecodeBMaxChunks;
}

template <bool kFp8>
__global__ __launch_bounds__(256) void index_lists_b(ScoreArgs sa, IndexTopkArgs la) {
  __shared__ itk::ListLds<kWaveKeepB> lst;
  const int i = blockIdx.y, chunk = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int seq = sa.q_seq ? sa.q_seq[i] : 0;
  const int n = clamp_ctx(sa.q_ctx[i], sa.max_ctx);
  const int64_t lo = int64_t(chunk) * kDecodeBChunk;
  if (lo >= n) return;  // the whole work-group
  const int64_t tile0 = lo + 128 * wave;
  float s[2] = {0.f, 0.f};
  if (tile0 < n) sb::tile_scores<kFp8>(sa, i, seq, n, tile0, s);
  float* out = sa.scores + int64_t(i) * sa.ld;
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int64_t tok = sb::tile_token(tile0, lane, j);
    if (tok < n) out[tok] = s[j];
  }
  if (n <= la.topk || !union_b(n, la.topk)) return;
  // key order: lane holds keys tile0 + 64 t + lane (0 past n). Key x of the
  // tile is score (x >> 3) & 1 of lane 8 (x & 7) + (x >> 4).
  uint32_t key[2];
#pragma unroll
  for (int t = 0; t < 2; t++) {
    const int x = 64 * t + lane;
    const int src = ((x & 7) << 3) | (x >> 4);
    const float v0 = __shfl(s[0], src), v1 = __shfl(s[1], src);
    const float v = ((x >> 3) & 1) ? v1 : v0;
    key[t] = tile0 + x < n ? order_key(v) : 0u;
  }
  itk::chunk_list<2, false, kWaveKeepB, true>(la, i, chunk, n, tile0, key, lst);
}

// ---- exact selection over a query's score row (written by the first
// launch: plain loads). A pass reads the row in rounds of 16,384 keys:
// thread t works on keys [64 t, 64 t + 64) of the round. Wave w loads its
// 4096 keys with contiguous lanes (16 bytes each, 1 KiB per instruction)
// and passes them through a padded LDS area into that layout; the loads of
// the next round are issued before the current one is processed.
constexpr int kSB = 64;
constexpr int kRound = itk::kNT * kSB;
constexpr int kTrRow = kSB + 4;  // floats per lane row of the transpose (padded: no bank conflicts)

struct RowLds {
  uint32_t hist[256 + 64];  // then one dummy bin per lane
  int wsum[2][itk::kNT / 64];
  uint32_t wmax[itk::kNT / 64], wmin[itk::kNT / 64];
  int digit, above;
  __attribute__((aligned(16))) float tr[itk::kNT / 64][64 * kTrRow];
};

// Barrier for LDS data only: global loads of the next round stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS accesses are done
  mla::pipe_barrier();
}

typedef const __attribute__((address_space(1))) u32x4* GlobalU32x4Ptr;
typedef const __attribute__((address_space(1))) float* GlobalF32Ptr;

// The wave's loads of the round starting at r0: v[q] holds keys
// r0 + 4096 w + 256 q + 4 lane .. + 3 (the values of keys past n are
// unspecified). vec: the row is 16-byte aligned and `lim` (its allocated
// length, >= n) a multiple of 4, so 16-byte loads at addresses clamped
// below lim cover every key below n; else one clamped load per key.
// No branch per load, so all of them are in flight together.
__device__ __forceinline__ void row_fetch(const float* __restrict__ sc, int n, int64_t lim, int r0, bool vec,
                                          u32x4 (&v)[16]) {
  const int x0 = r0 + (int(threadIdx.x) >> 6) * (64 * kSB) + 4 * (int(threadIdx.x) & 63);
  if (vec) {
    const int64_t xmax = lim - 4;
#pragma unroll
    for (int q = 0; q < 16; q++) {
      const int64_t x = x0 + 256 * q;
      v[q] = *(GlobalU32x4Ptr)(sc + (x < xmax ? x : xmax));
    }
  } else {
#pragma unroll
    for (int q = 0; q < 16; q++)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int x = x0 + 256 * q + e;
        v[q][e] = __float_as_uint(*(GlobalF32Ptr)(sc + (x < n ? x : n - 1)));
      }
  }
}

// Order keys of keys r0 + 64 tid .. + 63 (0 past n), from the wave's loads.
__device__ __forceinline__ void row_conv(int n, int r0, const u32x4 (&v)[16], RowLds& sh, uint32_t (&key)[kSB]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* tr = sh.tr[wave];
  // key 256 q + 4 lane of the wave's range belongs to lane 4 q + lane / 16, slot 4 (lane % 16)
#pragma unroll
  for (int q = 0; q < 16; q++)
    *reinterpret_cast<u32x4*>(tr + (4 * q + (lane >> 4)) * kTrRow + 4 * (lane & 15)) = v[q];
  const int j0 = r0 + kSB * int(threadIdx.x);
#pragma unroll
  for (int q = 0; q < 16; q++) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(tr + lane * kTrRow + 4 * q);
#pragma unroll
    for (int e = 0; e < 4; e++) key[4 * q + e] = j0 + 4 * q + e < n ? order_key(__uint_as_float(w[e])) : 0u;
  }
}

// one round's keys, loaded and converted
__device__ __forceinline__ void row_keys(const float* __restrict__ sc, int n, int64_t lim, int r0, bool vec,
                                         RowLds& sh, uint32_t (&key)[kSB]) {
  u32x4 v[16];
  row_fetch(sc, n, lim, r0, vec, v);
  row_conv(n, r0, v, sh, key);
}

// whether row_fetch may use 16-byte loads on this row
__device__ __forceinline__ bool row_vec(const float* sc, int64_t lim) {
  return (reinterpret_cast<uintptr_t>(sc) & 15u) == 0u && (lim & 3) == 0;
}

// Emit every key above kstar and the first `need` equal to it, in index
// order: emit(position, token) for the selected keys only. n_gt >= 0: the
// number of keys above kstar, known in advance; the pass then stops once it
// has them all and `need` equal ones.
template <class Emit>
__device__ void row_compact(const float* __restrict__ sc, int n, int64_t lim, uint32_t kstar, int need, int n_gt,
                            RowLds& sh, Emit emit) {
  constexpr int NW = itk::kNT / 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool vec = row_vec(sc, lim);
  int base_g = 0, base_e = 0;
  int par = 0;
  u32x4 v[16];
  row_fetch(sc, n, lim, 0, vec, v);
  for (int r0 = 0; r0 < n; r0 += kRound, par ^= 1) {
    const int j0 = r0 + kSB * tid;
    uint32_t key[kSB];
    row_conv(n, r0, v, sh, key);
    if (r0 + kRound < n) row_fetch(sc, n, lim, r0 + kRound, vec, v);  // the next round in flight meanwhile
    uint64_t fg = 0ull, fe = 0ull;  // bit r: key j0 + r above / equal to kstar (kstar != 0)
#pragma unroll
    for (int r = 0; r < kSB; r++) {
      fg |= uint64_t(key[r] > kstar) << r;
      fe |= uint64_t(key[r] == kstar) << r;
    }
    const int cg = __popcll(fg), ce = __popcll(fe);
    static_assert(kRound < 65536, "two 16-bit counts in one word");
    const int v = cg | (ce << 16);
    const int incl = wave_incl_sum(v);
    if (lane == 63) sh.wsum[par][wave] = incl;
    lds_barrier();  // (the other buffer is next written after the next barrier)
    int off = incl - v, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; w++) {
      const int x = sh.wsum[par][w];
      off += w < wave ? x : 0;
      tot += x;
    }
    // keys above kstar before this thread's, and equal ones
    const int gb = base_g + (off & 0xFFFF), eb = base_e + (off >> 16);
    // the thread's equal keys still needed are its first ones; a selected
    // key's position is then gb + min(eb, need) + the selected keys before
    // it in the thread
    const int take = need - eb <= 0 ? 0 : (need - eb >= ce ? ce : need - eb);
    uint64_t keep_e = take >= ce ? fe : 0ull;
    if (take > 0 && take < ce) {  // the one thread the need runs out in: its lowest `take` equal keys
      uint64_t rest = fe;
      for (int c = 0; c < take; c++) rest &= rest - 1ull;
      keep_e = fe ^ rest;
    }
    const uint64_t s_all = fg | keep_e;
    const int p0 = gb + (eb < need ? eb : need);
    uint64_t s = s_all;
    while (s) {
      const int r = int(__ffsll(static_cast<unsigned long long>(s))) - 1;
      emit(p0 + __popcll(s_all & ((1ull << r) - 1ull)), j0 + r);
      s &= s - 1ull;
    }
    base_g += tot & 0xFFFF;
    base_e += tot >> 16;
    if (n_gt >= 0 && base_g >= n_gt && base_e >= need) break;  // the same on every thread
  }
}

// The exact top-k (1 <= k < n) of the row: 8-bit radix passes below the
// common prefix of the largest and smallest key, then the compaction.
template <class Emit>
__device__ void row_select(const float* __restrict__ sc, int n, int64_t lim, int k, RowLds& sh, Emit emit) {
  constexpr int NW = itk::kNT / 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool vec = row_vec(sc, lim);
  uint32_t mx = 0u, mn = 0xFFFFFFFFu;
  for (int r0 = 0; r0 < n; r0 += kRound) {
    uint32_t key[kSB];
    row_keys(sc, n, lim, r0, vec, sh, key);
#pragma unroll
    for (int r = 0; r < kSB; r++) {
      mx = key[r] > mx ? key[r] : mx;
      mn = (key[r] != 0u && key[r] < mn) ? key[r] : mn;
    }
  }
  mx = wave_max_u32(mx);
  mn = wave_min_u32(mn);
  if (lane == 0) {
    sh.wmax[wave] = mx;
    sh.wmin[wave] = mn;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; w++) {
    mx = sh.wmax[w] > mx ? sh.wmax[w] : mx;
    mn = sh.wmin[w] < mn ? sh.wmin[w] : mn;
  }
  uint32_t kstar = mx;
  int need = k;
  if (mx != mn) {
    int lo = 32 - __clz(mx ^ mn);  // bits [lo, 32) are common to every key
    uint32_t mask = lo >= 32 ? 0u : ~((1u << lo) - 1u);
    uint32_t prefix = mx & mask;
    int remaining = k;
    while (lo > 0) {
      const int width = lo < 8 ? lo : 8;
      const int shift = lo - width;
      const uint32_t dmask = (1u << width) - 1u;
      for (int b = tid; b < 256; b += itk::kNT) sh.hist[b] = 0u;
      __syncthreads();
      for (int r0 = 0; r0 < n; r0 += kRound) {
        uint32_t key[kSB];
        row_keys(sc, n, lim, r0, vec, sh, key);
#pragma unroll
        for (int r = 0; r < kSB; r++) {
          const bool in = key[r] != 0u && (key[r] & mask) == prefix;
          hist_add(sh.hist, in, (key[r] >> shift) & dmask);
        }
      }
      __syncthreads();
      if (wave == 0) {  // lane holds bins 255 - 4 lane - e: digits in descending order
        int cnt[4], lsum = 0;
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
    }
    kstar = prefix;
    need = remaining;
  }
  row_compact(sc, n, lim, kstar, need, -1, sh, emit);
}

struct SelAttnLdsB {
  int sel[kMaxTopkB + 64];  // the query's selected tokens, ascending (then one dummy slot per lane)
  union {
    itk::FinalLds f;
    RowLds r;
    mla::LdsT t;
  } u;
};

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void attend_select_b(IndexTopkArgs la,
                                                                                       AttendArgs at) {
  __shared__ SelAttnLdsB sh;
  const int tid = threadIdx.x;
  const int i = int(blockIdx.x) / at.n_split, split = int(blockIdx.x) % at.n_split;
  // thread t's chunk list (t < the plan's chunk count) and bound, loaded
  // before the query's context arrives (one round trip instead of two);
  // lists past the query's own chunks are dropped below
  const bool in0 = tid < la.n_chunks;
  u32x4 ul[kRegRB / 2];
  {
    // pair-major lists: pair p of list t at (p * n_chunks + t) * 2
    const uint64_t* lp = la.list + size_t(i) * la.n_chunks * kDecodeBKeep + 2 * (in0 ? tid : 0);
#pragma unroll
    for (int r = 0; r < kRegRB / 2; r++)
      ul[r] = in0 ? ld16(lp + size_t(r) * la.n_chunks * 2) : u32x4{0u, 0u, 0u, 0u};
  }
  const uint64_t ub = in0 ? la.list_bound[size_t(i) * la.n_chunks + tid] : 0ull;
  const int n = clamp_ctx(la.q_ctx[i], la.max_ctx);
  const int aseq = at.q_seq ? at.q_seq[i] : 0;
  const int topk = la.topk;
  const int ns = n < topk ? n : topk;
  const float* sc = la.scores + int64_t(i) * la.ld;
  // selectors call emit(-1, token) for keys they leave out: those go to the
  // lane's dummy slot
  int* const lsel = sh.sel;
  const int dummy = kMaxTopkB + (tid & 63);
  auto emit = [lsel, dummy](int pos, int tok) { lsel[pos >= 0 ? pos : dummy] = tok; };
  const bool um = n > topk && union_b(n, topk);
  if (n <= topk) {  // every earlier token
    for (int j = tid; j < ns; j += 256) lsel[j] = j;
  } else if (um || n <= kUnionCapB) {
    uint32_t ukey[kRegRB];
    int uidx[kRegRB];
    uint64_t my_bound = 0ull;
    if (um) {
      // thread t: chunk t's list (ascending token order, 0 = empty), and its bound
      const bool in = tid < (n + kDecodeBChunk - 1) / kDecodeBChunk;
#pragma unroll
      for (int r = 0; r < kRegRB; r += 2) {
        const u32x4 w = ul[r / 2];
        uidx[r] = int(w[0]);
        ukey[r] = in ? w[1] : 0u;
        uidx[r + 1] = int(w[2]);
        ukey[r + 1] = in ? w[3] : 0u;
      }
      my_bound = in ? ub : 0ull;
    } else {
      // raw: element j = tid * kRegRB + r is key j
#pragma unroll
      for (int r = 0; r < kRegRB; r++) {
        const int j = tid * kRegRB + r;
        ukey[r] = j < n ? order_key(sc[j]) : 0u;
        uidx[r] = j;
      }
    }
    itk::RegSelOut ro;
    if (!itk::select_registers<kRegRB, true>(la, um, ukey, uidx, my_bound, sh.u.f, emit, ro)) {
      // the union cannot show the top-k exact: from the scores (when only a
      // tie failed, the threshold is known and one pass settles it)
      __syncthreads();  // the select's LDS is free
      if (ro.tie_fail)
        row_compact(sc, n, la.ld, ro.kstar, ro.need, ro.n_gt, sh.u.r, emit);
      else
        row_select(sc, n, la.ld, topk, sh.u.r, emit);
    }
  } else {
    row_select(sc, n, la.ld, topk, sh.u.r, emit);
  }
  __syncthreads();
  if (split == 0) {  // the query's selection, padded with -1
    int* gsel = la.sel + int64_t(i) * topk;
    for (int j = tid; j < topk; j += 256) gsel[j] = j < ns ? lsel[j] : -1;
    if (tid == 0) la.n_sel[i] = ns;
  }
  mla::attend_part_t<false, true>(at, split, i, sh.u.t, sh.sel, ns, n, aseq);
}

}  // namespace

DecodeLayerBPlan plan_decode_layer_b(int nq, int max_ctx, int hq, int dv, int n_split) {
  DecodeLayerBPlan p{};
  const int64_t nc = (int64_t(max_ctx) + kDecodeBChunk - 1) / kDecodeBChunk;
  p.n_chunks = int(nc < 1 ? 1 : nc);
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  size_t off = 0;
  p.off_list = off;
  off += up(size_t(nq) * p.n_chunks * kDecodeBKeep * 8);
  p.off_bound = off;
  off += up(size_t(nq) * p.n_chunks * 8);
  p.off_o = off;
  off += up(size_t(n_split) * nq * hq * dv * 4);
  p.off_lse = off;
  off += up(size_t(n_split) * nq * hq * 4);
  p.ws_bytes = off;
  return p;
}

hipError_t launch_decode_layer_b(ScoreArgs sa, AttendArgs att, const DecodeLayerBPlan& p, void* ws,
                                 hipStream_t s) {
  if (sa.nq <= 0) return hipSuccess;
  char* w = static_cast<char*>(ws);
  IndexTopkArgs la{};
  la.q_seq = sa.q_seq;
  la.q_ctx = sa.q_ctx;
  la.max_ctx = sa.max_ctx;
  la.nq = sa.nq;
  la.scores = sa.scores;
  la.ld = sa.ld;
  la.topk = att.topk;
  la.sel = const_cast<int*>(att.sel);
  la.n_sel = const_cast<int*>(att.n_sel);
  la.list = reinterpret_cast<uint64_t*>(w + p.off_list);
  la.list_bound = reinterpret_cast<uint64_t*>(w + p.off_bound);
  la.n_chunks = p.n_chunks;
  la.chunk_blocks = kDecodeBChunk;
  la.keep = kDecodeBKeep;
  la.wkeep = kWaveKeepB;
  att.o_part = reinterpret_cast<float*>(w + p.off_o);
  att.lse_part = reinterpret_cast<float*>(w + p.off_lse);
  const dim3 g1(unsigned(p.n_chunks), unsigned(sa.nq));
  if (sa.key_fp8)
    hipLaunchKernelGGL(index_lists_b<true>, g1, dim3(256), 0, s, sa, la);
  else
    hipLaunchKernelGGL(index_lists_b<false>, g1, dim3(256), 0, s, sa, la);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attend_select_b, dim3(unsigned(int64_t(sa.nq) * att.n_split)), dim3(256), 0, s, la, att);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = int64_t(att.nq) * att.hq;
  return launch_merge(att.n_split, rows, att.dv, att.o_part, rows * att.dv, att.lse_part, rows, att.o_out, att.o_bf16,
                      att.lse_out, s);
}

}  // namespace qsa
