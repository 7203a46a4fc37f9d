// trellis.hip — the runtime hash codebook and the decode of trellis-coded
// weights to int8 for the prefill GEMM.
//
// Trellis format (per row): 2-bit symbols c_i, state st <- ((st << 2) | c_i)
// & 0xFFFF from the row's seed, value index h = ((st * 0x9E37) ^ (st >> 7)) &
// 0xFF, value = s64 * V16[h].  The codebook is computed at run time, not
// stored with the weights (the trellis format of [P1] "2.4bit 是个什么量级").
// Because the state is 16 bits and each symbol shifts in 2 bits, the state
// after symbol 4g+j is the 16-bit window of seed||bytes ending with that
// symbol, so every weight decodes independently.
#include <cmath>
#include <mutex>

#include <hip/hip_fp16.h>

#include "internal.hpp"

#pragma clang fp contract(off)

namespace qk {

namespace {
// Inverse standard normal CDF by Newton's method on Phi(z) - p from z = 0.
// Phi is concave on z > 0 and convex on z < 0, so the iterates approach the
// root monotonically from the side of 0.
double inv_norm_cdf(double p) {
  const double inv_sqrt2 = 0.70710678118654752440;
  const double inv_sqrt2pi = 0.39894228040143267794;
  double z = 0.0;
  for (int it = 0; it < 100; ++it) {
    const double f = 0.5 * std::erfc(-z * inv_sqrt2) - p;
    const double fp = inv_sqrt2pi * std::exp(-0.5 * z * z);
    const double zn = z - f / fp;
    if (zn == z) break;
    z = zn;
  }
  return z;
}

struct Tables {
  V16Table v16;
  V8Table v8;
  float gain;
};

const Tables& tables() {
  static Tables t;
  static std::once_flag once;
  std::call_once(once, [] {
    for (int k = 0; k < 256; ++k) t.v16.v[k] = f64_to_f16_bits(inv_norm_cdf((k + 0.5) / 256.0));
    const double top = (double)__half2float(__ushort_as_half(t.v16.v[255]));
    for (int k = 0; k < 256; ++k)
      t.v8.v[k] = (int8_t)std::nearbyint((double)__half2float(__ushort_as_half(t.v16.v[k])) * 127.0 / top);
    t.gain = (float)(top / 127.0);
  });
  return t;
}
}  // namespace

void trellis_tables(V16Table* v16, V8Table* v8, float* gain) {
  const Tables& t = tables();
  if (v16) *v16 = t.v16;
  if (v8) *v8 = t.v8;
  if (gain) *gain = t.gain;
}

// One wave per (row, 256 weights): lane l decodes byte l of the 64-byte run
// (4 weights), then the wave quantizes per oblock (256: whole wave, 32: 8 lanes).
__global__ __launch_bounds__(256) void k_trellis_decode(GemvItem it, int oblock, V16Table v16t, int8_t* __restrict__ wq,
                                                        float* __restrict__ dw) {
  __shared__ uint16_t v16[256];
  v16[threadIdx.x] = v16t.v[threadIdx.x];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int nblk = it.cols / 256;
  const int64_t job = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (job >= (int64_t)it.rows * nblk) return;
  const int64_t row = job / nblk;
  const int blk = (int)(job % nblk);
  const uint8_t* rp = it.codes + row * it.row_bytes;
  const int g = blk * 64 + lane;  // byte index in the row
  const uint32_t seed = it.seeds[row];
  const uint32_t b0 = rp[g];
  const uint32_t b1 = g >= 1 ? rp[g - 1] : (seed & 0xFFu);
  const uint32_t b2 = g >= 2 ? rp[g - 2] : (g == 1 ? (seed & 0xFFu) : (seed >> 8));
  const uint32_t w24 = (b2 << 16) | (b1 << 8) | b0;
  const float s = __half2float(__ushort_as_half(it.scales[scale_index(QFMT_TRELLIS2, it.cols, row, (4 * g) / 64)]));
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t st = (w24 >> (6 - 2 * j)) & 0xFFFFu;
    const uint32_t h = ((st * 0x9E37u) ^ (st >> 7)) & 0xFFu;
    v[j] = s * __half2float(__ushort_as_half(v16[h]));  // exact: 11-bit x 11-bit significands
  }
  // Q8 over `oblock` values = oblock/4 lanes
  const int width = oblock / 4;
  float am = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
  for (int m = 1; m < width; m <<= 1) am = fmaxf(am, __shfl_xor(am, m));
  const float dd = am / 127.0f;
  const float id = am == 0.0f ? 0.0f : 1.0f / dd;
  uint32_t packed = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float r = rintf(v[j] * id);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    packed |= ((uint32_t)((int)r & 0xFF)) << (8 * j);
  }
  *(uint32_t*)(wq + row * it.cols + 4 * (int64_t)g) = packed;
  if (lane % width == 0) dw[row * (it.cols / oblock) + (4 * g) / oblock] = dd;
}

hipError_t launch_trellis_decode(const GemvItem& it, int oblock, int8_t* wq, float* dw, hipStream_t s) {
  V16Table v16;
  trellis_tables(&v16, nullptr, nullptr);
  const int64_t jobs = (int64_t)it.rows * (it.cols / 256);
  hipLaunchKernelGGL(k_trellis_decode, dim3((unsigned)((jobs + 3) / 4)), dim3(256), 0, s, it, oblock, v16, wq, dw);
  return hipGetLastError();
}

}  // namespace qk
