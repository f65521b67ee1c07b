// A4 / A6: the stand-alone attention launches (device code in attend.hpp
// for the pooled-block variant, attend_mla.hpp for the shared latent).
// One work-group per (query, split) and kv head; each writes one partial
// (O, lse). Decode combines the splits with qsa_lse_merge; prefill calls it
// once per history tile ("3090x3で 314 万コンテキスト", section "ちなみにこの
// 欠点") and merges the tiles the same way.
#include "attend.hpp"
#include "attend_mla.hpp"

namespace qsa {
namespace {

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8))) void attend_a(AttendArgs a) {
  __shared__ att::Lds<1> sh;
  const int split = blockIdx.x % a.n_split, i = blockIdx.x / a.n_split;
  att::attend_part<false, 1>(a, split, blockIdx.y, i, sh);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void attend_b(AttendArgs a) {
  __shared__ mla::Lds sh;
  const int split = blockIdx.x % a.n_split, i = blockIdx.x / a.n_split;
  mla::attend_part<false>(a, split, i, sh);
}

// Transposed form with two tile buffers: two work-groups per CU, each
// gathering its next tile while it computes the current one.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void attend_b_t(AttendArgs a) {
  __shared__ mla::LdsT sh;
  const int split = blockIdx.x % a.n_split, i = blockIdx.x / a.n_split;
  mla::attend_part_t<false>(a, split, i, sh);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void attend_b_fp8(AttendArgs a) {
  __shared__ mla::LdsF8 sh;
  const int split = blockIdx.x % a.n_split, i = blockIdx.x / a.n_split;
  mla::attend_part_fp8<false>(a, split, i, sh);
}

// The pooled-block variant, one history tile merged into the running result
// of the earlier tiles (AttendArgs::acc).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) void attend_a_acc(AttendArgs a) {
  __shared__ att::Lds<1> sh;
  const int split = blockIdx.x % a.n_split, i = blockIdx.x / a.n_split;
  att::attend_part<false, 1, false, true>(a, split, blockIdx.y, i, sh);
}

// The pooled-block variant over K/V in host memory with the HBM row cache.
__global__ __launch_bounds__(256) void attend_a_cached(AttendArgs a) {
  __shared__ att::Lds<1> sh;
  const int split = blockIdx.x % a.n_split, i = blockIdx.x / a.n_split;
  att::attend_part<false, 1, true>(a, split, blockIdx.y, i, sh);
}

}  // namespace

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
  if (a.nq <= 0) return hipSuccess;
  if (a.hq == 16 && a.hkv == 2 && a.dk == 256 && a.dv == 256) {
    dim3 grid(unsigned(int64_t(a.nq) * a.n_split), unsigned(a.hkv));
    if (a.src)
      hipLaunchKernelGGL(attend_a_cached, grid, dim3(256), 0, s, a);
    else if (a.acc)
      hipLaunchKernelGGL(attend_a_acc, grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(attend_a, grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  if (a.hq == mla::kH && a.hkv == 1 && a.dk == mla::kDK && a.dv == mla::kDV) {
    const dim3 grid(unsigned(int64_t(a.nq) * a.n_split));
    if (a.kv_fp8)
      hipLaunchKernelGGL(attend_b_fp8, grid, dim3(256), 0, s, a);
    else if (a.block == 1)  // token-level selection (the indexer of this shape)
      hipLaunchKernelGGL(attend_b_t, grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(attend_b, grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace qsa
