// calib.hip — a measured ceiling for the int8 matrix-core roofline.
//
// The GEMM's roofline is priced against the published dense int8 peak; this
// kernel measures what the matrix cores actually sustain on the part at hand
// (same instruction as the GEMM, v_mfma_i32_32x32x32_i8, nothing else in the
// loop) and at what shader clock, from the wave-level cycle counter
// (s_memtime) against the constant-rate counter (s_memrealtime).
#include "internal.hpp"

namespace qk {

typedef int cv4i __attribute__((ext_vector_type(4)));
typedef int cv16i __attribute__((ext_vector_type(16)));

// Every wave runs iters x 16 MFMAs over four independent accumulators (enough
// in flight to keep the matrix pipe busy at two waves per SIMD).  Thread 0 of
// each block records (cycles at start, cycles at end, reference ticks at start,
// reference ticks at end) in clocks[4 b .. 4 b + 3].
__global__ __launch_bounds__(256) void k_mfma_i8_peak(int iters, int seed, uint64_t* __restrict__ clocks,
                                                      int* __restrict__ sink) {
  const int t = threadIdx.x;
  const cv4i a = {seed, seed + t, seed ^ 0x5a5a5a5a, t * 7}, b = {seed * 5, t + 1, 0x01020304, seed - t};
  cv16i c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) c[j][e] = e + j;
  __syncthreads();
  const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[j], 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[j][e];
  __syncthreads();
  const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (s == 0x7fffffff) sink[0] = s;  // keeps the chains live; practically never taken
  if (t == 0) {
    clocks[4 * blockIdx.x + 0] = c0;
    clocks[4 * blockIdx.x + 1] = c1;
    clocks[4 * blockIdx.x + 2] = r0;
    clocks[4 * blockIdx.x + 3] = r1;
  }
}

hipError_t launch_mfma_peak(int blocks, int iters, uint64_t* clocks, int32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(k_mfma_i8_peak, dim3(blocks), dim3(256), 0, s, iters, 3, clocks, sink);
  return hipGetLastError();
}

}  // namespace qk
