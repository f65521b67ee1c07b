// A2: indexer scores of every candidate block.
// "3090x3で 314 万コンテキスト", section "VRAM に残す必要があるもの": the
// pooled keys (128 x bf16 per block) are the only read that grows with the
// context and are scanned in full at every decode step, so the decode
// kernel is a bandwidth-bound stream: each wave reads 64 consecutive keys
// (16 KiB) with 16-byte non-temporal loads, 16 lanes per key row, and folds
// the 16 partial dot products of a lane group with a transposing butterfly
// (15 lane exchanges per 16 keys instead of 60).
// "GLM-5.3 最適化 第2部", section "PCP": the token-level indexer of the
// MLA-like variant scores every earlier token with several heads; the score
// is the weighted sum of the heads' ReLU'd dot products.
// A prefill chunk (all queries in one sequence) uses MFMA 16x16x32 bf16
// tiles: 16 queries x 16 keys x 32 dims per instruction.
#include <cfloat>

#include "common.hpp"
#include "fp8.hpp"
#include "kernels.hpp"
#include "scores_b.hpp"
#include "select.hpp"

namespace qsa {
namespace {

__device__ __forceinline__ float dot8(u32x4 k, u32x4 q) {
  float acc = 0.f;
  acc = dot2(k[0], q[0], acc);
  acc = dot2(k[1], q[1], acc);
  acc = dot2(k[2], q[2], acc);
  acc = dot2(k[3], q[3], acc);
  return acc;
}

// Variant A decode: 128-d keys, one head. A wave owns 64 consecutive keys
// per tile; lane (g = lane/16, c = lane%16) loads dims [8c, 8c+8) of keys
// 4k+g (k = 0..15) and after the butterfly holds the score of key 4c+g.
template <int TPW>
__global__ __launch_bounds__(256) void scores_gemv_a(ScoreArgs a) {
  const int i = blockIdx.y;
  const int seq = a.q_seq ? a.q_seq[i] : 0;
  const int64_t n = clamp_ctx(a.q_ctx[i], a.max_ctx) / a.block;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
  const int64_t wg0 = int64_t(blockIdx.x) * (4 * TPW * 64);
  if (wg0 >= n) return;
  const u32x4 qv = ld16(a.q_idx + int64_t(i) * 128 + 8 * c);
  const uint16_t* kb = static_cast<const uint16_t*>(a.keys) + int64_t(seq) * a.keys_ss;
  float* out = a.scores + int64_t(i) * a.ld;
  for (int t = 0; t < TPW; t++) {
    const int64_t tile0 = wg0 + int64_t(wave * TPW + t) * 64;
    if (tile0 >= n) break;
    u32x4 v[16];
#pragma unroll
    for (int k = 0; k < 16; k++) {
      const int64_t blk = tile0 + 4 * k + g;
      v[k] = blk < n ? ld16_nt(kb + blk * 128 + 8 * c) : u32x4{0u, 0u, 0u, 0u};
    }
    float p[16];
#pragma unroll
    for (int k = 0; k < 16; k++) p[k] = dot8(v[k], qv);
    // transposing butterfly over the 16 lanes of a group
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
    const int64_t blk = tile0 + 4 * c + g;
    if (blk < n) out[blk] = p[0];
  }
}

// Variant A decode with FP8 keys (fp8.hpp): 64 keys per tile, 8 lanes per
// 128-byte code row, the key's scale applied to the dot product.
template <int TPW>
__global__ __launch_bounds__(256) void scores_gemv_a_fp8(ScoreArgs a) {
  const int i = blockIdx.y;
  const int seq = a.q_seq ? a.q_seq[i] : 0;
  const int64_t n = clamp_ctx(a.q_ctx[i], a.max_ctx) / a.block;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t wg0 = int64_t(blockIdx.x) * (4 * TPW * 64);
  if (wg0 >= n) return;
  float qf[16];
  fp8::load_query(a.q_idx + int64_t(i) * 128, qf);
  const uint8_t* kb = static_cast<const uint8_t*>(a.keys) + int64_t(seq) * a.keys_ss;
  float* out = a.scores + int64_t(i) * a.ld;
  for (int t = 0; t < TPW; t++) {
    const int64_t tile0 = wg0 + int64_t(wave * TPW + t) * 64;
    if (tile0 >= n) break;
    u32x4 v[8];
    float sc;
    fp8::load_tile(kb, tile0, n, v, sc);
    const float sv = fp8::tile_scores(v, sc, tile0, n, qf);
    if (tile0 + lane < n) out[tile0 + lane] = sv;
  }
}

// Variant B decode: one wave per 128 consecutive keys (scores_b.hpp).
template <bool kFp8>
__global__ __launch_bounds__(256) void scores_gemv_b(ScoreArgs a) {
  const int i = blockIdx.y;
  const int seq = a.q_seq ? a.q_seq[i] : 0;
  const int64_t n = clamp_ctx(a.q_ctx[i], a.max_ctx) / a.block;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t tile0 = (int64_t(blockIdx.x) * 4 + wave) * 128;
  if (tile0 >= n) return;
  float s[2];
  sb::tile_scores<kFp8>(a, i, seq, n, tile0, s);
  float* out = a.scores + int64_t(i) * a.ld;
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int64_t tok = sb::tile_token(tile0, lane, j);
    if (tok < n) out[tok] = s[j];
  }
}

// Largest candidate count among the 64 queries of a work-group.
__device__ __forceinline__ int64_t wg_max_n(const ScoreArgs& a, int q0, int* red) {
  int n = 0;
  if (threadIdx.x < 64) {
    const int q = q0 + threadIdx.x;
    n = q < a.nq ? clamp_ctx(a.q_ctx[q], a.max_ctx) / a.block : 0;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) n = max(n, __shfl_xor(n, m));
    if (threadIdx.x == 0) red[0] = n;
  }
  __syncthreads();
  return red[0];
}

// Prefill chunk, variant A: work-group = 64 queries (16 per wave) x 128 keys.
// MFMA 16x16x32 bf16: A = q_idx rows, B = key rows (dims contiguous).
__global__ __launch_bounds__(256) void scores_gemm_a(ScoreArgs a) {
  __shared__ int red[1];
  const int q0 = blockIdx.y * 64;
  const int64_t b0 = int64_t(blockIdx.x) * 128;
  const int64_t nmax = wg_max_n(a, q0, red);
  if (b0 >= nmax) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, kq = lane >> 4;
  const int qa_row = q0 + 16 * wave + r;
  bf16x8 qa[4];
#pragma unroll
  for (int ks = 0; ks < 4; ks++) {
    u32x4 w = qa_row < a.nq ? ld16(a.q_idx + int64_t(qa_row) * 128 + 32 * ks + 8 * kq)
                            : u32x4{0u, 0u, 0u, 0u};
    qa[ks] = as_bf16x8(w);
  }
  int64_t nrow[4];
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const int q = q0 + 16 * wave + 4 * kq + e;
    nrow[e] = q < a.nq ? clamp_ctx(a.q_ctx[q], a.max_ctx) / a.block : 0;
  }
  for (int nt = 0; nt < 8; nt++) {
    const int64_t blk = b0 + 16 * nt + r;
    if (b0 + 16 * nt >= nmax) break;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      u32x4 w = blk < nmax ? ld16(static_cast<const uint16_t*>(a.keys) + blk * 128 + 32 * ks + 8 * kq)
                           : u32x4{0u, 0u, 0u, 0u};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], as_bf16x8(w), acc, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const int q = q0 + 16 * wave + 4 * kq + e;
      if (blk < nrow[e]) a.scores[int64_t(q) * a.ld + blk] = acc[e];
    }
  }
}

// Prefill chunk, variant A with FP8 keys: the same tiles, the B operand
// converted from E4M3 to bf16 (exact) and each key column scaled after the
// MFMA: score = scale_b * (q . codes_b).
__global__ __launch_bounds__(256) void scores_gemm_a_fp8(ScoreArgs a) {
  __shared__ int red[1];
  const int q0 = blockIdx.y * 64;
  const int64_t b0 = int64_t(blockIdx.x) * 128;
  const int64_t nmax = wg_max_n(a, q0, red);
  if (b0 >= nmax) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, kq = lane >> 4;
  const int qa_row = q0 + 16 * wave + r;
  const uint8_t* kb = static_cast<const uint8_t*>(a.keys);
  bf16x8 qa[4];
#pragma unroll
  for (int ks = 0; ks < 4; ks++) {
    u32x4 w = qa_row < a.nq ? ld16(a.q_idx + int64_t(qa_row) * 128 + 32 * ks + 8 * kq)
                            : u32x4{0u, 0u, 0u, 0u};
    qa[ks] = as_bf16x8(w);
  }
  int64_t nrow[4];
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const int q = q0 + 16 * wave + 4 * kq + e;
    nrow[e] = q < a.nq ? clamp_ctx(a.q_ctx[q], a.max_ctx) / a.block : 0;
  }
  for (int nt = 0; nt < 8; nt++) {
    const int64_t blk = b0 + 16 * nt + r;
    if (b0 + 16 * nt >= nmax) break;
    const int64_t bc = blk < nmax ? blk : nmax - 1;
    const uint8_t* row = kb + fp8_code_off(bc, 128);
    const float sc = *reinterpret_cast<const float*>(kb + fp8_scale_off(bc, 128));
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(row + 32 * ks + 8 * kq);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], e4m3x8_bf16(w), acc, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const int q = q0 + 16 * wave + 4 * kq + e;
      if (blk < nrow[e]) a.scores[int64_t(q) * a.ld + blk] = acc[e] * sc;
    }
  }
}

// Prefill chunk, variant B: 4 heads x 64 dims, score = sum_h w_h relu(dot_h).
// kFp8: B operands converted from E4M3 codes, the key scale applied last.
// Work-group = 64 queries (16 per wave) x 128 columns; column t scores key
// t * tok_step (the sample pass of the one-call selection strides). kList
// (the one-call selection, prefill_select.hip): 8 x 128 columns per
// work-group, and instead of storing scores each query row keeps the
// entries ranked at or above its threshold in a per-query list.
// The key rows of tile t + 2 are fetched before tile t is computed.
constexpr int kListBatches = 8;  // list mode: 8 x 128 columns per work-group
constexpr int kStage = 64;       // list mode: LDS entries staged per query row

template <bool kFp8, bool kList>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void scores_gemm_b(ScoreArgs a) {
  __shared__ int red[2];
  const int q0 = blockIdx.y * 64;
  if (a.only) {  // only the tiles that hold a flagged query
    if (threadIdx.x == 0) red[1] = 0;
    __syncthreads();
    if (threadIdx.x < 64 && q0 + int(threadIdx.x) < a.nq && a.only[q0 + threadIdx.x]) red[1] = 1;
    __syncthreads();
    if (red[1] == 0) return;
  }
  // (list mode never strides)
  const int64_t step = kList ? 1 : (a.tok_step > 0 ? a.tok_step : 1);
  // a span is 128 columns, or kListBatches x 128 in list mode; work-group x
  // covers spans x, x + gridDim.x, ... (one span each unless the launch
  // narrows the grid)
  const int64_t span = 128 * (kList ? kListBatches : 1);
  const int64_t nmax = (wg_max_n(a, q0, red) + step - 1) / step;  // in units of tok_step
  if (int64_t(blockIdx.x) * span >= nmax) return;
  [[maybe_unused]] __shared__ uint64_t stage[kList ? 64 : 1][kList ? kStage : 1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, kq = lane >> 4;
  const int qa_row = q0 + 16 * wave + r;
  bf16x8 qa[4][2];
#pragma unroll
  for (int h = 0; h < 4; h++)
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
      u32x4 w = qa_row < a.nq ? ld16(a.q_idx + (int64_t(qa_row) * 4 + h) * 64 + 32 * ks + 8 * kq)
                              : u32x4{0u, 0u, 0u, 0u};
      qa[h][ks] = as_bf16x8(w);
    }
  int64_t nrow[4];
  float wr[4][4];
  [[maybe_unused]] uint64_t th[4];
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const int q = q0 + 16 * wave + 4 * kq + e;
    const int64_t n = q < a.nq ? clamp_ctx(a.q_ctx[q], a.max_ctx) / a.block : 0;
    nrow[e] = (n + step - 1) / step;
    if (a.only && q < a.nq && !a.only[q]) nrow[e] = 0;
#pragma unroll
    for (int h = 0; h < 4; h++) wr[e][h] = q < a.nq ? a.w_idx[int64_t(q) * 4 + h] : 0.f;
    if constexpr (kList) th[e] = q < a.nq ? a.theta[q] : ~0ull;
  }
  for (int64_t b00 = int64_t(blockIdx.x) * span; b00 < nmax; b00 += int64_t(gridDim.x) * span) {
  // Column tiles t = 0 .. T-1 of the span (tokens b00 + 16 t + r); the key
  // rows of tile t + 2 are fetched before tile t is computed, so loads stay
  // two tiles ahead of the MFMAs. Columns past nmax read a valid row (the
  // last) and are ignored.
  struct KRaw {
    u32x4 w[2];
    float sc;
  };
  auto fetch = [&](int t) {
    KRaw k;
    const int64_t tok = b00 + 16 * t + r;
    const int64_t kt = (tok < nmax ? tok : nmax - 1) * step;  // the key row of column tok
    k.sc = 1.f;
    if constexpr (kFp8) {
      const uint8_t* kb8 = static_cast<const uint8_t*>(a.keys);
      k.sc = *reinterpret_cast<const float*>(kb8 + fp8_scale_off(kt, 64));
#pragma unroll
      for (int ks = 0; ks < 2; ks++) {
        const u32x2 c = *reinterpret_cast<const u32x2*>(kb8 + fp8_code_off(kt, 64) + 32 * ks + 8 * kq);
        k.w[ks] = u32x4{c[0], c[1], 0u, 0u};
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ks++) k.w[ks] = ld16(static_cast<const uint16_t*>(a.keys) + kt * 64 + 32 * ks + 8 * kq);
    }
    return k;
  };
  auto compute = [&](const KRaw& k, float (&sc)[4]) {
    bf16x8 kb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
      if constexpr (kFp8)
        kb[ks] = e4m3x8_bf16(u32x2{k.w[ks][0], k.w[ks][1]});
      else
        kb[ks] = as_bf16x8(k.w[ks]);
    }
    float acc_s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 4; h++) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[h][0], kb[0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[h][1], kb[1], acc, 0, 0, 0);
      // ReLU as one med3 clamp to [0, FLT_MAX] (fmaxf would first
      // canonicalise the MFMA result; the same for every finite dot); the
      // sum starts at +0, so the sign of a zero never reaches a score
#pragma unroll
      for (int e = 0; e < 4; e++) acc_s[e] += wr[e][h] * __builtin_amdgcn_fmed3f(acc[e], 0.f, FLT_MAX);
    }
#pragma unroll
    for (int e = 0; e < 4; e++) sc[e] = acc_s[e] * k.sc;
  };
  constexpr int kTiles = 8 * (kList ? kListBatches : 1);
  const int T = int((nmax - b00 + 15) / 16 < kTiles ? (nmax - b00 + 15) / 16 : kTiles);  // >= 1
  [[maybe_unused]] int staged[4] = {0, 0, 0, 0};  // list mode: uniform in the lane group
  // list mode: the threshold as a float and an index, 32-bit counts, and the
  // lane group's ballot masks
  [[maybe_unused]] float thf[4];
  [[maybe_unused]] int thi[4], nrow32[4];
  [[maybe_unused]] const uint32_t below16 = (1u << r) - 1u;  // lanes of the group below this one
  [[maybe_unused]] const uint32_t gshift = 16u * kq;         // the group's bits in a ballot
  if constexpr (kList) {
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const uint32_t tk = uint32_t(th[e] >> 32);
      // the float whose order key is tk (tk >= 0x80000000: non-negative)
      thf[e] = __uint_as_float(tk & 0x80000000u ? tk & 0x7FFFFFFFu : ~tk);
      const uint64_t ti = th[e] & 0xFFFFFFFFull;
      thi[e] = ti > 0x7FFFFFFFull ? 0x7FFFFFFF : int(ti);
      nrow32[e] = int(nrow[e]);
      if (tk == 0xFFFFFFFFu) nrow32[e] = 0;  // keep none
      if (tk == 0u) { thf[e] = -INFINITY; thi[e] = 0x7FFFFFFF; }  // keep every score
    }
  }
  // list mode: query row 16 wave + 4 kq + e belongs to the 16 lanes of group
  // kq of one wave; they stage its kept entries in LDS (ballot prefix, no
  // atomics) and, when the stage might not hold another tile's entries and
  // after the span, reserve list slots with one atomic and copy
  [[maybe_unused]] auto flush = [&](int e) {
    const int q = q0 + 16 * wave + 4 * kq + e;
    const int row = 16 * wave + 4 * kq + e;
    uint32_t base = 0u;
    if (r == 0) base = atomicAdd(a.counts + int64_t(q) * kCountStride, uint32_t(staged[e]));
    base = uint32_t(__shfl(int(base), 16 * kq));
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int jj = 0; jj < kStage / 16; jj++) {  // straight-line: at most kStage entries
      const int j = r + 16 * jj;
      if (j < staged[e] && base + uint32_t(j) < uint32_t(a.list_cap))
        a.lists[int64_t(q) * a.list_cap + base + j] = stage[row][j];
    }
    __builtin_amdgcn_wave_barrier();
    staged[e] = 0;
  };
  // per-tile work on tile t's scores: list staging or score stores
  auto work = [&](int t, const float (&sc)[4]) {
    const int64_t tok = b00 + 16 * t + r;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      if constexpr (kList) {
        // keep the scores ranked at least as high as the query's threshold
        // (score descending, index ascending; float order equals key order);
        // bitwise, not short-circuit, so no branch per test
        // a tile adds at most 16 entries to the row; the test comes first so
        // that no branch separates the ballot from the stores
        if (staged[e] > kStage - 16) flush(e);  // rare; uniform in the group
        const int tk32 = int(tok);
        const bool keep = (tk32 < nrow32[e]) & ((sc[e] > thf[e]) | ((sc[e] == thf[e]) & (tk32 <= thi[e])));
        const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
        const uint32_t g16 = uint32_t(bal >> gshift) & 0xFFFFu;  // the 16 ballot bits of the lane's group
        const int c = __popc(g16);                                // kept in the lane's group
        const int before = __popc(g16 & below16);                 // ... ahead of the lane
        if (keep)
          stage[16 * wave + 4 * kq + e][staged[e] + before] =
              (uint64_t(__float_as_uint(sc[e])) << 32) | uint64_t(uint32_t(tk32));
        staged[e] += c;
      } else {
        const int q = q0 + 16 * wave + 4 * kq + e;
        if (tok < nrow[e]) a.scores[int64_t(q) * a.ld + tok] = sc[e];
      }
    }
  };
  // two fetch buffers with fixed roles (unrolled by two, no copies of
  // registers still being loaded); with T odd the last step computes the
  // tile past the span's keys, whose columns are all past nmax and ignored
  // (in this order: the waits at the loop head count the loads issued
  // after a tile's keys, on the way in as on the way round)
  KRaw ka = fetch(0);
  __builtin_amdgcn_sched_barrier(0);
  KRaw kb = fetch(T > 1 ? 1 : 0);
  __builtin_amdgcn_sched_barrier(0);
  for (int t = 0; t < T; t += 2) {
    float sc[4];
    compute(ka, sc);
    ka = fetch(t + 2 < T ? t + 2 : T - 1);
    __builtin_amdgcn_sched_barrier(0);  // keep the fetches in program order
    work(t, sc);
    compute(kb, sc);
    kb = fetch(t + 3 < T ? t + 3 : T - 1);
    __builtin_amdgcn_sched_barrier(0);
    work(t + 1, sc);
  }
  if constexpr (kList) {
#pragma unroll
    for (int e = 0; e < 4; e++)
      if (staged[e] > 0) flush(e);
  }
  }  // spans
}

}  // namespace

hipError_t launch_scores_gemm_b(const ScoreArgs& a, int64_t n_cols, bool lists, hipStream_t s) {
  if (a.nq <= 0 || n_cols <= 0) return hipSuccess;
  const int64_t span = 128 * (lists ? kListBatches : 1);
  dim3 grid(unsigned((n_cols + span - 1) / span), unsigned((a.nq + 63) / 64));
  // a pass over flagged queries only: few work-groups per query tile, each
  // walking many spans, so that a pass with nothing flagged (the usual case)
  // costs a small grid of work-groups that exit at once
  if (a.only && grid.x > 64) grid.x = 64;
  if (lists) {
    if (a.key_fp8)
      hipLaunchKernelGGL(HIP_KERNEL_NAME(scores_gemm_b<true, true>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(HIP_KERNEL_NAME(scores_gemm_b<false, true>), grid, dim3(256), 0, s, a);
  } else {
    if (a.key_fp8)
      hipLaunchKernelGGL(HIP_KERNEL_NAME(scores_gemm_b<true, false>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(HIP_KERNEL_NAME(scores_gemm_b<false, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_scores(const ScoreArgs& a, hipStream_t s) {
  if (a.nq <= 0) return hipSuccess;
  const int64_t nmax = int64_t(a.max_ctx) / a.block;
  if (nmax <= 0) return hipSuccess;
  const bool chunk = a.q_seq == nullptr && a.nq >= 16;
  if (a.idx_heads == 1 && a.key_fp8) {
    if (chunk) {
      dim3 grid(unsigned((nmax + 127) / 128), unsigned((a.nq + 63) / 64));
      hipLaunchKernelGGL(scores_gemm_a_fp8, grid, dim3(256), 0, s, a);
    } else {
      const int64_t wgs1 = ((nmax + 255) / 256) * a.nq;
      if (wgs1 >= 8192) {
        dim3 grid(unsigned((nmax + 511) / 512), unsigned(a.nq));
        hipLaunchKernelGGL(scores_gemv_a_fp8<2>, grid, dim3(256), 0, s, a);
      } else {
        dim3 grid(unsigned((nmax + 255) / 256), unsigned(a.nq));
        hipLaunchKernelGGL(scores_gemv_a_fp8<1>, grid, dim3(256), 0, s, a);
      }
    }
  } else if (a.idx_heads == 1) {
    if (chunk) {
      dim3 grid(unsigned((nmax + 127) / 128), unsigned((a.nq + 63) / 64));
      hipLaunchKernelGGL(scores_gemm_a, grid, dim3(256), 0, s, a);
    } else {
      const int64_t per_wg1 = 256;  // keys per work-group with one tile per wave
      const int64_t wgs1 = ((nmax + per_wg1 - 1) / per_wg1) * a.nq;
      if (wgs1 >= 8192) {
        dim3 grid(unsigned((nmax + 511) / 512), unsigned(a.nq));
        hipLaunchKernelGGL(scores_gemv_a<2>, grid, dim3(256), 0, s, a);
      } else {
        dim3 grid(unsigned((nmax + 255) / 256), unsigned(a.nq));
        hipLaunchKernelGGL(scores_gemv_a<1>, grid, dim3(256), 0, s, a);
      }
    }
  } else {
    if (chunk) {
      return launch_scores_gemm_b(a, nmax, false, s);
    } else {
      dim3 grid(unsigned((nmax + 511) / 512), unsigned(a.nq));
      if (a.key_fp8)
        hipLaunchKernelGGL(scores_gemv_b<true>, grid, dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL(scores_gemv_b<false>, grid, dim3(256), 0, s, a);
    }
  }
  return hipGetLastError();
}

}  // namespace qsa
