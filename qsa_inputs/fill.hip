// GPU side of the seeded input generator (definition in qsa_inputs/__init__.py):
// element i of stream (seed, stream) is NORMAL_TABLE[c], where c is 16-bit
// lane (i % 4) (most significant first) of the (i / 4)-th SplitMix64 output
// started at key = mix64(seed * G ^ stream * H). Integer-only, so it matches
// the numpy implementation bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kG = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kH = 0xD1B54A32D192ED03ull;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Each thread writes 4 consecutive elements (one 64-bit word) per step.
__global__ __launch_bounds__(256) void fill_kernel(uint64_t key, uint64_t start, int64_t n,
                                                   const uint16_t* __restrict__ table,
                                                   uint16_t* __restrict__ out) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  // 8-byte stores need the word's first element 8-byte aligned in `out`
  const bool aligned = (start & 3u) == 0 && (reinterpret_cast<uintptr_t>(out) & 7u) == 0;
  // elements [start, start + n): word w covers elements 4w .. 4w+3
  const uint64_t w0 = start >> 2;
  const uint64_t w1 = (start + uint64_t(n) + 3) >> 2;
  for (uint64_t w = w0 + uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; w < w1; w += uint64_t(stride)) {
    const uint64_t u = mix64(key + (w + 1) * kG);
    const uint64_t e0 = 4 * w;
    if (aligned && e0 >= start && e0 + 4 <= start + uint64_t(n)) {
      // whole word inside the range: one 8-byte store
      const uint64_t v = uint64_t(table[(u >> 48) & 0xFFFFu]) | (uint64_t(table[(u >> 32) & 0xFFFFu]) << 16) |
                         (uint64_t(table[(u >> 16) & 0xFFFFu]) << 32) | (uint64_t(table[u & 0xFFFFu]) << 48);
      *reinterpret_cast<uint64_t*>(out + (e0 - start)) = v;
      continue;
    }
#pragma unroll
    for (int l = 0; l < 4; l++) {
      const uint64_t e = e0 + l;
      if (e >= start && e < start + uint64_t(n)) out[e - start] = table[(u >> (48 - 16 * l)) & 0xFFFFu];
    }
  }
}

}  // namespace

extern "C" int qsa_fill_normal_bf16(uint64_t seed, uint64_t stream, uint64_t start, int64_t n,
                                    const uint16_t* table, uint16_t* out, void* hip_stream) {
  if (n <= 0) return 0;
  if (!table || !out) return 1;
  const uint64_t key = mix64(seed * kG ^ stream * kH);
  const int64_t words = (n + 3) / 4 + 1;
  int64_t grid = (words + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(fill_kernel, dim3(unsigned(grid)), dim3(256), 0, static_cast<hipStream_t>(hip_stream), key,
                     start, n, table, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
