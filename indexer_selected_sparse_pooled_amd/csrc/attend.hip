// A4 / A6: softmax attention of each query over its selected tokens.
// "3090x3で 314 万コンテキスト": only the indexer-selected K/V rows are read
// (section "なぜ"), addressed per (token, kv head) (section "カーネルを書き換え
// ずに済む"); prefill restricts each query to one history tile and merges the
// tiles' partial results afterwards (section "ちなみにこの欠点").
//
// One work-group per (query, kv head, split). The query's token list is the
// tokens of its selected blocks (ascending) followed by the trailing tokens
// of the incomplete block; a work-group walks its contiguous part of that
// list (intersected with [tile_begin, tile_end)) in tiles of 64 tokens:
//   * V rows of the tile are staged in LDS (coalesced 16-byte loads);
//   * S = Q K^T on MFMA 16x16x32 bf16: the GQA group's 8 query heads are the
//     A rows (rows 8..15 zero), each wave computes 16 tokens with K rows as
//     the B operand, loaded straight from global memory;
//   * online softmax in exp2 form per head;
//   * O += P V on MFMA, P split into bf16 hi + lo parts (two MFMAs) so the
//     weights keep ~16 bits; each wave owns 64 of the 256 output dims and
//     reads V transposed out of LDS.
// Output: normalised partial O (fp32) and its natural-log lse.
#include "common.hpp"
#include "kernels.hpp"

namespace qsa {
namespace {

constexpr int TT = 64;            // token positions per tile
constexpr int GROUP_A = 8;        // query heads per kv head
constexpr int DK_A = 256;
constexpr int DV_A = 256;
constexpr int VSTR = DV_A + 4;    // LDS row of V: 520 bytes (rows 8 apart hit distinct banks)
constexpr int PSTR = TT + 8;      // LDS row of P: 144 bytes, 16-byte aligned

struct ListView {
  const int* sel;
  int ns;        // selected blocks
  int nblk;      // complete blocks
  int block;
  int64_t L;     // list length
  // token position of list entry p (0 <= p < L)
  __device__ __forceinline__ int64_t tok(int64_t p) const {
    const int64_t nb_tok = int64_t(ns) * block;
    if (p < nb_tok) {
      int b = sel[p / block];
      b = b < 0 ? 0 : (b >= nblk ? nblk - 1 : b);
      return int64_t(b) * block + p % block;
    }
    return int64_t(nblk) * block + (p - nb_tok);
  }
  // number of list entries whose token is < x (x a multiple of block, or >= ctx)
  __device__ int64_t count_below(int64_t x, int ctx) const {
    if (x <= 0) return 0;
    if (x >= ctx) return L;
    const int64_t nb_tok = int64_t(nblk) * block;
    if (x >= nb_tok) return int64_t(ns) * block + (x - nb_tok);
    const int xb = int(x / block);
    int lo = 0, hi = ns;  // first selected block >= xb
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (sel[mid] < xb) lo = mid + 1; else hi = mid;
    }
    return int64_t(lo) * block;
  }
};

__global__ __launch_bounds__(256) void attend_a(AttendArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t vsh[TT * VSTR];
  __shared__ float ssh[GROUP_A][TT];
  __shared__ __attribute__((aligned(16))) uint16_t phi[16 * PSTR];
  __shared__ __attribute__((aligned(16))) uint16_t plo[16 * PSTR];
  __shared__ float alpha_sh[16];
  __shared__ float m_sh[GROUP_A], l_sh[GROUP_A];
  __shared__ int64_t range_sh[2];

  const int split = blockIdx.x % a.n_split, g = blockIdx.y;
  const int i = blockIdx.x / a.n_split;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, kq = lane >> 4;

  const int seq = a.q_seq ? a.q_seq[i] : 0;
  const int ctx = clamp_ctx(a.q_ctx[i], a.max_ctx);
  ListView lv;
  lv.sel = a.sel + int64_t(i) * a.topk;
  lv.block = a.block;
  lv.nblk = ctx / a.block;
  int ns = a.n_sel[i];
  const int ns_max = lv.nblk < a.topk ? lv.nblk : a.topk;
  lv.ns = ns < 0 ? 0 : (ns > ns_max ? ns_max : ns);
  lv.L = int64_t(lv.ns) * a.block + (ctx - lv.nblk * a.block);

  if (tid == 0) {
    const int64_t lo = int64_t(split) * lv.L / a.n_split;
    const int64_t hi = int64_t(split + 1) * lv.L / a.n_split;
    const int64_t t0 = lv.count_below(a.tile_begin, ctx);
    const int64_t t1 = lv.count_below(a.tile_end, ctx);
    range_sh[0] = lo > t0 ? lo : t0;
    range_sh[1] = hi < t1 ? hi : t1;
  }
  if (tid < GROUP_A) {
    m_sh[tid] = -INFINITY;
    l_sh[tid] = 0.f;
  }
  // rows 8..15 of P stay zero (padding rows of the MFMA A operand)
  for (int e = tid; e < 16 * PSTR; e += 256) {
    phi[e] = 0;
    plo[e] = 0;
  }
  __syncthreads();
  const int64_t P0 = range_sh[0], P1 = range_sh[1];

  const int64_t kvs = int64_t(seq) * a.seq_stride + int64_t(g) * a.head_stride;
  const uint16_t* kbase = a.k + kvs;
  const uint16_t* vbase = a.v + kvs;
  const float sl2 = a.scale * kLog2e;

  bf16x8 qa[DK_A / 32];
  {
    const uint16_t* qrow = a.q + (int64_t(i) * a.hq + g * GROUP_A + (r < GROUP_A ? r : 0)) * DK_A;
#pragma unroll
    for (int ks = 0; ks < DK_A / 32; ks++) {
      const u32x4 w = r < GROUP_A ? ld16(qrow + 32 * ks + 8 * kq) : u32x4{0u, 0u, 0u, 0u};
      qa[ks] = as_bf16x8(w);
    }
  }
  f32x4 oacc[4];
#pragma unroll
  for (int nt = 0; nt < 4; nt++) oacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t pb = P0; pb < P1; pb += TT) {
    const int cnt = int((P1 - pb) < TT ? (P1 - pb) : TT);
    // token positions first, then every K and V load of the tile, so that
    // all of them are in flight together
    const int c = tid & 31;
    int64_t vtok[TT / 8];
#pragma unroll
    for (int ps = 0; ps < TT / 8; ps++) {
      const int row = ps * 8 + (tid >> 5);
      vtok[ps] = row < cnt ? lv.tok(pb + row) : -1;
    }
    const int rr = 16 * wave + r;
    const bool valid = rr < cnt;
    const int64_t kt = lv.tok(pb + (valid ? rr : 0));
    u32x4 vw[TT / 8];
#pragma unroll
    for (int ps = 0; ps < TT / 8; ps++)
      vw[ps] = vtok[ps] >= 0 ? ld16(vbase + vtok[ps] * a.tok_stride + 8 * c) : u32x4{0u, 0u, 0u, 0u};
    bf16x8 kb[DK_A / 32];
    {
      const uint16_t* krow = kbase + kt * a.tok_stride + 8 * kq;
#pragma unroll
      for (int ks = 0; ks < DK_A / 32; ks++) kb[ks] = as_bf16x8(ld16(krow + 32 * ks));
    }
    // V tile -> LDS: 8 passes of 8 rows x 32 chunks of 16 bytes
#pragma unroll
    for (int ps = 0; ps < TT / 8; ps++) {
      const int row = ps * 8 + (tid >> 5);
      u32x2* dst = reinterpret_cast<u32x2*>(vsh + row * VSTR + 8 * c);
      dst[0] = u32x2{vw[ps][0], vw[ps][1]};
      dst[1] = u32x2{vw[ps][2], vw[ps][3]};
    }
    // S for tokens 16*wave .. 16*wave+15
    {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DK_A / 32; ks++)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kb[ks], acc, 0, 0, 0);
      if (kq < 2) {
#pragma unroll
        for (int e = 0; e < 4; e++) ssh[4 * kq + e][rr] = valid ? acc[e] * sl2 : -INFINITY;
      }
    }
    __syncthreads();
    // online softmax: head h = tid / 32, two tokens per thread
    {
      const int h = tid >> 5;
      const int t2 = (tid & 31) * 2;
      const float s0 = ssh[h][t2], s1 = ssh[h][t2 + 1];
      float mt = fmaxf(s0, s1);
#pragma unroll
      for (int m = 16; m >= 1; m >>= 1) mt = fmaxf(mt, __shfl_xor(mt, m));
      const float m_old = m_sh[h], l_old = l_sh[h];
      const float m_new = fmaxf(m_old, mt);
      float p0 = 0.f, p1 = 0.f, al = 1.f;
      if (m_new != -INFINITY) {
        al = exp2f(m_old - m_new);
        p0 = exp2f(s0 - m_new);
        p1 = exp2f(s1 - m_new);
      }
      float ps = p0 + p1;
#pragma unroll
      for (int m = 16; m >= 1; m >>= 1) ps += __shfl_xor(ps, m);
      const uint16_t h0 = f32_to_bf16(p0), h1 = f32_to_bf16(p1);
      phi[h * PSTR + t2] = h0;
      phi[h * PSTR + t2 + 1] = h1;
      plo[h * PSTR + t2] = f32_to_bf16(p0 - bf16_to_f32(h0));
      plo[h * PSTR + t2 + 1] = f32_to_bf16(p1 - bf16_to_f32(h1));
      if ((tid & 31) == 0) {
        alpha_sh[h] = al;
        l_sh[h] = al * l_old + ps;
        m_sh[h] = m_new;
      }
    }
    __syncthreads();
    // O += P V for dims 64*wave .. 64*wave+63
    {
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int row = 4 * kq + e;
        const float al = row < GROUP_A ? alpha_sh[row] : 1.f;
#pragma unroll
        for (int nt = 0; nt < 4; nt++) oacc[nt][e] *= al;
      }
#pragma unroll
      for (int k2 = 0; k2 < TT / 32; k2++) {
        const bf16x8 ah = as_bf16x8(ld16(phi + r * PSTR + 32 * k2 + 8 * kq));
        const bf16x8 al8 = as_bf16x8(ld16(plo + r * PSTR + 32 * k2 + 8 * kq));
        const int tok0 = 32 * k2 + 8 * kq;
#pragma unroll
        for (int nt = 0; nt < 4; nt++) {
          const int d = 64 * wave + 16 * nt + r;
          u32x4 bw;
#pragma unroll
          for (int q2 = 0; q2 < 4; q2++) {
            const uint32_t lo = vsh[(tok0 + 2 * q2) * VSTR + d];
            const uint32_t hi = vsh[(tok0 + 2 * q2 + 1) * VSTR + d];
            bw[q2] = lo | (hi << 16);
          }
          const bf16x8 bv = as_bf16x8(bw);
          oacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bv, oacc[nt], 0, 0, 0);
          oacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al8, bv, oacc[nt], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  // normalise and write the partial result
  const int64_t orow0 = (int64_t(split) * a.nq + i) * a.hq + g * GROUP_A;
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const int row = 4 * kq + e;
    if (row < GROUP_A) {
      const float l = l_sh[row];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      float* o = a.o_part + (orow0 + row) * DV_A + 64 * wave + r;
#pragma unroll
      for (int nt = 0; nt < 4; nt++) o[16 * nt] = oacc[nt][e] * inv;
    }
  }
  if (tid < GROUP_A) {
    const float l = l_sh[tid];
    a.lse_part[orow0 + tid] = l > 0.f ? (m_sh[tid] + log2f(l)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
  if (a.nq <= 0) return hipSuccess;
  if (a.hq == 16 && a.hkv == 2 && a.dk == 256 && a.dv == 256) {
    dim3 grid(unsigned(int64_t(a.nq) * a.n_split), unsigned(a.hkv));
    hipLaunchKernelGGL(attend_a, grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace qsa
