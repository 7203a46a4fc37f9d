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
#include <algorithm>
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

// Decode of one 1024-weight unit ub of row `row` by a whole wave: lane l takes
// code bytes 4l .. 4l+3 of the unit (16 weights, one 16-lane quarter per
// 256-block) with one 4-byte load; the two bytes before its first byte come
// from the previous lane (lane 0: from memory, or the seed at the row start).
// Per weight: the state st is the 16-bit window ending at its symbol, and
// 4 h = ((220 st) ^ (st >> 5)) & 0x3FC is the table byte offset (the low 8 bits
// of 0x9E37 st are those of 55 st, so bits 2..9 of 220 st are bits 0..7 of
// 0x9E37 st, and bits 2..9 of st >> 5 are bits 0..7 of st >> 7); a multiply
// takes only the window's low 24 bits, and bits above the state land outside
// the mask.  v = s * V16[h] exactly (both fp16).  Returns whether the lane's
// 256-block exists (its v are zeros otherwise); a unit wholly past the row's
// end (the per-row kernel's spare waves) reads no memory.
__device__ __forceinline__ bool decode_unit(const GemvItem& it, int row, int ub, int lane, uint32_t lds_base,
                                            float v[16]) {
  const int nblk = it.cols / 256;
  const bool ok = ub * 4 + (lane >> 4) < nblk;  // this lane's 256-block exists
  const uint8_t* rp = it.codes + (int64_t)row * it.row_bytes;
  const int g0 = ub * 256 + 4 * lane;  // first code byte of the lane
  const uint32_t cur = ok ? *(const uint32_t*)(rp + g0) : 0u;
  uint32_t prev = __shfl_up(cur, 1);
  if (lane == 0 && ub * 4 < nblk) {  // (a unit past the row's end reads nothing)
    const uint32_t seed = it.seeds[row];
    // bytes -1 and -2 of a row are the seed's low and high byte
    prev = ub == 0 ? ((seed & 0xFFu) << 24) | (((seed >> 8) & 0xFFu) << 16) : *(const uint32_t*)(rp + g0 - 4);
  }
  const uint64_t x = ((uint64_t)cur << 32) | prev;
  const float s = ok ? __half2float(__ushort_as_half(it.scales[scale_index(QFMT_TRELLIS2, it.cols, row, g0 / 16)]))
                     : 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // bytes g-2, g-1, g (g = g0 + k) as the big-endian window g-2 | g-1 | g
    const uint32_t y3 = (uint32_t)(x >> (16 + 8 * k));
    const uint32_t w24 = ((y3 & 0xFFu) << 16) | (y3 & 0xFF00u) | ((y3 >> 16) & 0xFFu);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t a = w24 >> (6 - 2 * j);      // st in the low 16 bits
      const uint32_t off = ((a * 220u) ^ (a >> 5)) & 0x3FCu;  // 4 h
      const float val = *(const __attribute__((address_space(3))) float*)(uintptr_t)(lds_base + off);
      v[4 * k + j] = s * val;  // exact: 11-bit x 11-bit significands
    }
  }
  return ok;
}

// Q8 codes of 16 values through the 1.5 * 2^23 sum (its low byte is
// rint(v * (1 / d)) in two's complement, ties to even; no clamp: |v| <= amax,
// so |v * (1 / d)| <= 127 (1 + 3 ulp) and q stays in [-127, 127]), packed.
__device__ __forceinline__ float q8_inv(float d) {  // 1 / d, or 0 where it overflows (a zero block)
  const float r = 1.0f / d;  // +inf when d = 0 or d <= 2^-128
  return r < __builtin_inff() ? r : 0.0f;
}
__device__ __forceinline__ void q8_pack16(const float v[16], float id, uint32_t pk[4]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = __builtin_bit_cast(uint32_t, v[4 * w + j] * id + 12582912.0f);
    const uint32_t lo = __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u);  // q0 | q1 << 8
    const uint32_t hi = __builtin_amdgcn_perm(b[3], b[2], 0x0C0C0400u);  // q2 | q3 << 8
    pk[w] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
  }
}

// One wave per (row, 1024 weights) (decode_unit), then Q8 per oblock (WIDTH
// lanes: 16 for 256, 2 for 32) and one 16-byte store per lane.  Waves walk the
// units in a grid-stride loop (the unit's row and position advance by a fixed
// quotient and remainder, no division per unit), so the codebook is copied to
// LDS once per workgroup, as fp32 (exact for fp16 values).
template <int WIDTH>
__global__ __launch_bounds__(256) void k_trellis_decode(GemvItem it, V16Table v16t, int8_t* __restrict__ wq,
                                                        float* __restrict__ dw, int upr, int step_rows,
                                                        int step_units) {
  __shared__ float v32[256];
  v32[threadIdx.x] = __half2float(__ushort_as_half(v16t.v[threadIdx.x]));
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nblk = it.cols / 256;
  constexpr int OBLOCK = 16 * WIDTH;
  const bool vec = ((uintptr_t)wq & 15) == 0;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)v32;
  // this wave's first unit, then (row, ub) += (step_rows, step_units) per turn
  const int u0 = blockIdx.x * 4 + wave;
  int row = u0 / upr, ub = u0 - row * upr;
  for (; row < it.rows;) {
    float v[16];
    const bool ok = decode_unit(it, row, ub, lane, lds_base, v);
    const int g0 = ub * 256 + 4 * lane;  // first code byte of the lane
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(v[i]));
    am = fmaxf(am, xlane<1>(am));
    if constexpr (WIDTH > 2) {
      am = fmaxf(am, xlane<2>(am));
      am = fmaxf(am, xlane<4>(am));
      am = fmaxf(am, xlane<8>(am));
    }
    const float dd = am / 127.0f;
    const float id = q8_inv(dd);
    uint32_t pk[4];
    q8_pack16(v, id, pk);
    if (ok) {
      int8_t* o = wq + (int64_t)row * it.cols + 4 * (int64_t)g0;
      if (vec) {
        *(uint4*)o = uint4{pk[0], pk[1], pk[2], pk[3]};
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) ((uint32_t*)o)[w] = pk[w];
      }
      if (lane % WIDTH == 0) dw[(int64_t)row * (it.cols / OBLOCK) + (4 * g0) / OBLOCK] = dd;
    }
    ub += step_units;
    row += step_rows;
    if (ub >= upr) {
      ub -= upr;
      ++row;
    }
  }
}


// Q8 with one scale per weight row (oblock = cols): a workgroup of W waves
// takes rows blockIdx.x, blockIdx.x + gridDim.x, ... (one codebook copy for all
// of them); the W waves decode a row's units w, w + W, ... (NB each at most,
// kept in registers), and the row's amax is reduced over each wave and then
// over the W waves (LDS, double-buffered by row parity so one barrier per row
// suffices).
template <int NB>
__global__ __launch_bounds__(1024) void k_trellis_decode_row(GemvItem it, V16Table v16t, int8_t* __restrict__ wq,
                                                             float* __restrict__ dw) {
  __shared__ float v32[256];
  __shared__ float s_am[2][16];
  for (int i = threadIdx.x; i < 256; i += blockDim.x) v32[i] = __half2float(__ushort_as_half(v16t.v[i]));
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)v32;
  const bool vec = ((uintptr_t)wq & 15) == 0;
  int par = 0;
  for (int row = blockIdx.x; row < it.rows; row += gridDim.x, par ^= 1) {
    float v[NB][16];
    bool ok[NB];
    float am = 0.0f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      ok[b] = decode_unit(it, row, w + W * b, lane, lds_base, v[b]);
#pragma unroll
      for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(v[b][i]));
    }
    for (int m = 1; m < 64; m <<= 1) am = fmaxf(am, __shfl_xor(am, m));
    if (lane == 0) s_am[par][w] = am;
    __syncthreads();  // (the other parity's slots were last read before this barrier's previous pass)
    am = s_am[par][0];
    for (int k = 1; k < W; ++k) am = fmaxf(am, s_am[par][k]);
    const float dd = am / 127.0f;
    const float id = q8_inv(dd);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      uint32_t pk[4];
      q8_pack16(v[b], id, pk);
      if (ok[b]) {
        int8_t* o = wq + (int64_t)row * it.cols + 4 * (int64_t)((w + W * b) * 256 + 4 * lane);
        if (vec) {
          *(uint4*)o = uint4{pk[0], pk[1], pk[2], pk[3]};
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) ((uint32_t*)o)[k] = pk[k];
        }
      }
    }
    if (w == 0 && lane == 0) dw[row] = dd;
  }
}

hipError_t launch_trellis_decode(const GemvItem& it, int oblock, int8_t* wq, float* dw, hipStream_t s) {
  V16Table v16;
  trellis_tables(&v16, nullptr, nullptr);
  const int upr = (it.cols / 256 + 3) / 4;  // 1024-weight units per row
  if (oblock == it.cols && oblock != 32 && oblock != 256) {  // one scale per row
    const int nb = (upr + 15) / 16;                          // units per wave (<= 16 waves per row)
    const int W = (upr + nb - 1) / nb;                       // waves per row
    const dim3 grid(std::min(it.rows, 2048)), block(64 * W);
    if (nb == 1) hipLaunchKernelGGL(k_trellis_decode_row<1>, grid, block, 0, s, it, v16, wq, dw);
    else if (nb == 2) hipLaunchKernelGGL(k_trellis_decode_row<2>, grid, block, 0, s, it, v16, wq, dw);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  const int64_t units = (int64_t)it.rows * upr;
  const int grid = (int)std::min<int64_t>((units + 3) / 4, 8192);
  const int stride = grid * 4;  // units per turn of the grid
  if (oblock == 256)
    hipLaunchKernelGGL(k_trellis_decode<16>, dim3(grid), dim3(256), 0, s, it, v16, wq, dw, upr, stride / upr,
                       stride % upr);
  else
    hipLaunchKernelGGL(k_trellis_decode<2>, dim3(grid), dim3(256), 0, s, it, v16, wq, dw, upr, stride / upr,
                       stride % upr);
  return hipGetLastError();
}

}  // namespace qk
