// act.hip — activation quantization to int8 (per 32 or 256 values) and the
// block-randomized Walsh-Hadamard rotation that precedes it for prefill.
//
// Both kernels are bit-exact against their definitions: every float op below
// is one IEEE fp32 op in the definition's order (contraction off), division
// and reciprocal correctly rounded, rint rounds half to even.
#include <algorithm>
#include <type_traits>

#include "internal.hpp"

#pragma clang fp contract(off)

namespace qk {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Butterfly reduction over the `width` lanes of a group (width a power of 2).
__device__ __forceinline__ float group_max(float v, int width) {
  for (int m = 1; m < width; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ int group_sum(int v, int width) {
  for (int m = 1; m < width; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

// Reciprocal of the Q8 step d: 1 / d when finite, else 0.  1 / d is +inf for a
// zero block (d = 0) and whenever d <= 2^-128 (the reciprocal overflows); such
// blocks quantize to q = 0 and qsum = 0, with d kept.
__device__ __forceinline__ float q8_inv(float d) {
  const float r = 1.0f / d;
  return r < __builtin_inff() ? r : 0.0f;
}

// Q8 of four values held by this lane, whose block spans `width` lanes.
// Writes the 4 int8 codes to q4 and, from the block's first lane, d and qsum.
__device__ __forceinline__ void q8_lane4(f32x4 v, int width, bool first, uint32_t* q4, float* d, int32_t* qsum) {
  float am = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  am = group_max(am, width);
  const float dd = am / 127.0f;
  const float id = q8_inv(dd);
  const float e[4] = {v.x, v.y, v.z, v.w};
  uint32_t packed = 0;
  int s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float r = rintf(e[i] * id);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    const int qi = (int)r;
    s += qi;
    packed |= ((uint32_t)(qi & 0xFF)) << (8 * i);
  }
  s = group_sum(s, width);
  *q4 = packed;
  if (first) {
    *d = dd;
    *qsum = s;
  }
}

// One thread per 4 consecutive values; qblock/4 lanes per block.
__global__ __launch_bounds__(256) void k_act_quant(const float* __restrict__ x, int64_t n4, int qblock,
                                                   int8_t* __restrict__ q, float* __restrict__ d,
                                                   int32_t* __restrict__ qsum) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int width = qblock / 4;
  // Every lane of a block takes part in the shuffles, so out-of-range lanes
  // (only possible in the last workgroup) use zeros and store nothing.
  const bool ok = i < n4;
  const f32x4 v = ok ? *(const f32x4*)(x + 4 * i) : f32x4{0.f, 0.f, 0.f, 0.f};
  uint32_t q4;
  float dd;
  int32_t s;
  const int64_t blk = (4 * i) / qblock;
  const bool first = (threadIdx.x % width) == 0;
  q8_lane4(v, width, first, &q4, &dd, &s);
  if (ok) {
    *(uint32_t*)(q + 4 * i) = q4;
    if (first) {
      d[blk] = dd;
      qsum[blk] = s;
    }
  }
}

hipError_t launch_act_quant(const float* x, int B, int K, int qblock, int8_t* q, float* d, int32_t* qsum,
                            hipStream_t s) {
  const int64_t n4 = (int64_t)B * K / 4;
  const int64_t grid = (n4 + 255) / 256;
  hipLaunchKernelGGL(k_act_quant, dim3((unsigned)grid), dim3(256), 0, s, x, n4, qblock, q, d, qsum);
  return hipGetLastError();
}

// 4-bit planes of int8 activations: one thread per output word.  Word w of a
// 32-block (8 words) covers values 8g .. 8g+7, g = w % 4: w < 4 takes the low
// nibble of each byte (x mod 16), w >= 4 the high one (floor(x / 16) as a
// two's complement nibble); value n of the group goes to nibble n.
__global__ __launch_bounds__(256) void k_act_planes(const uint32_t* __restrict__ q, int64_t nwords,
                                                    uint32_t* __restrict__ planes) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nwords) return;
  const int w = (int)(i & 7), g = w & 3;
  const int64_t src = (i >> 3) * 8 + 2 * g;  // the group's two q words (4 values each)
  const uint32_t a0 = q[src], a1 = q[src + 1];
  const int sh = w < 4 ? 0 : 4;
  // nibble of byte k of a word, moved to nibble k (k = 0..3)
  auto nib4 = [&](uint32_t a) {
    const uint32_t t = (a >> sh) & 0x0F0F0F0Fu;  // nibbles at bits 8k
    return (t & 0xFu) | ((t >> 4) & 0xF0u) | ((t >> 8) & 0xF00u) | ((t >> 12) & 0xF000u);
  };
  planes[i] = nib4(a0) | (nib4(a1) << 16);
}

hipError_t launch_act_planes(const int8_t* q, int B, int K, uint32_t* planes, hipStream_t s) {
  const int64_t nwords = (int64_t)B * K / 4;  // 8 words per 32 values
  const int64_t grid = (nwords + 255) / 256;
  hipLaunchKernelGGL(k_act_planes, dim3((unsigned)grid), dim3(256), 0, s, (const uint32_t*)q, nwords, planes);
  return hipGetLastError();
}

// Batched Q8 per 32 + planes: job j owns threads [start[j], start[j + 1]) (one
// per 16 values, starts multiples of 256, so a workgroup serves one job).  Lanes
// 2k and 2k + 1 hold the two halves of 32-block k (DPP partners for the block's
// max and sum); q = rint(v * (1 / d)) comes from the low byte of the fp32 sum
// 1.5 * 2^23 + v * (1 / d) (unit ulp: nearest integer, ties to even; |q| <= 127,
// so no clamp), and each lane writes plane words g (lo nibbles) and 4 + g (hi
// nibbles) of its two 8-value groups g as k_act_planes does.
struct ActBatch {
  int n;
  int64_t start[QACT_BATCH_MAX + 1];
  qact_job_t job[QACT_BATCH_MAX];
};

__global__ __launch_bounds__(256) void k_act_quant_batch(const ActBatch b) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int j = 0;
  while (j + 1 < b.n && t >= b.start[j + 1]) ++j;  // uniform over the workgroup
  const qact_job_t& J = b.job[j];
  const int64_t i = t - b.start[j];                 // 16-value chunk of the job
  const int64_t n16 = (int64_t)J.B * J.K / 16;
  const bool ok = i < n16;  // both lanes of a block agree
  float v[16];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const f32x4 x4 = ok ? *(const f32x4*)(J.x + 16 * i + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
    v[4 * c] = x4.x;
    v[4 * c + 1] = x4.y;
    v[4 * c + 2] = x4.z;
    v[4 * c + 3] = x4.w;
  }
  float am = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) am = fmaxf(am, fabsf(v[k]));
  am = fmaxf(am, xlane<1>(am));
  const float dd = am / 127.0f;
  const float id = q8_inv(dd);
  uint32_t pk[4];
  uint32_t bsum = 0;  // 16 x 0x4B400000 + the sum of the 16 codes, mod 2^32
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t bb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      bb[k] = __builtin_bit_cast(uint32_t, v[4 * w + k] * id + 12582912.0f);
      bsum += bb[k];
    }
    const uint32_t lo = __builtin_amdgcn_perm(bb[1], bb[0], 0x0C0C0400u);
    const uint32_t hi = __builtin_amdgcn_perm(bb[3], bb[2], 0x0C0C0400u);
    pk[w] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
  }
  int sum = (int)(bsum - 16u * 0x4B400000u);
  sum += xlane_i<1>(sum);
  if (!ok) return;
  const int64_t blk = i >> 1;
  const int half = (int)(i & 1);
  if (J.q) {
    int8_t* o = J.q + 16 * i;
    if (((uintptr_t)o & 15) == 0) {
      *(uint4*)o = uint4{pk[0], pk[1], pk[2], pk[3]};
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) ((uint32_t*)o)[w] = pk[w];
    }
  }
  if (half == 0) {
    J.d[blk] = dd;
    J.qsum[blk] = sum;
  }
  if (J.planes) {
    // nibbles at bits 8k + sh of a code word, moved to nibble k
    auto nib4 = [](uint32_t a, int sh) {
      const uint32_t u = (a >> sh) & 0x0F0F0F0Fu;
      return (u & 0xFu) | ((u >> 4) & 0xF0u) | ((u >> 8) & 0xF00u) | ((u >> 12) & 0xF000u);
    };
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      const int g = 2 * half + gg;  // values 8g .. 8g + 7 of the block: code words 2gg, 2gg + 1 of this lane
      J.planes[blk * 8 + g] = nib4(pk[2 * gg], 0) | (nib4(pk[2 * gg + 1], 0) << 16);
      J.planes[blk * 8 + 4 + g] = nib4(pk[2 * gg], 4) | (nib4(pk[2 * gg + 1], 4) << 16);
    }
  }
}

hipError_t launch_act_quant_batch(const qact_job_t* jobs, int n, hipStream_t s) {
  ActBatch b{};
  b.n = n;
  int64_t acc = 0;
  for (int j = 0; j < n; ++j) {
    b.job[j] = jobs[j];
    b.start[j] = acc;
    const int64_t n16 = (int64_t)jobs[j].B * jobs[j].K / 16;
    acc += (n16 + 255) / 256 * 256;
  }
  b.start[n] = acc;
  if (acc == 0) return hipSuccess;
  hipLaunchKernelGGL(k_act_quant_batch, dim3((unsigned)(acc / 256)), dim3(256), 0, s, b);
  return hipGetLastError();
}


// The rotation of one 256-block by its 16-lane group: lane t holds elements
// 16t .. 16t+15 (xk = the lane's 16 inputs, k0 their first feature index), so
// stages h = 1, 2, 4, 8 run inside the lane and h = 16, 32, 64, 128 pair lanes
// t ^ 1, t ^ 2, t ^ 4, t ^ 8.  (Every stage adds and subtracts the same pairs
// in the same order as the definition, so the rounding is the same: a cross
// stage forms fma(own, +-1, partner's), which is the partner's value plus or
// minus its own, rounded once.)  Then every element is multiplied by 1/16, as
// the definition does (the product rounds only where it is subnormal, and must
// then round the same way).  Lanes whose group has no block (ok false) compute
// on zeros: the cross-lane steps need the whole wave.
__device__ __forceinline__ void rotate256(const float* __restrict__ xk, const uint32_t* __restrict__ sign_bits,
                                          int k0, int t, bool ok, float u[16]) {
  if (ok) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 v = *(const f32x4*)(xk + 4 * c);
      u[4 * c] = v.x;
      u[4 * c + 1] = v.y;
      u[4 * c + 2] = v.z;
      u[4 * c + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) u[i] = 0.0f;
  }
  const uint32_t sw = ok ? sign_bits[k0 >> 5] >> (k0 & 31) : 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i)  // sign bit i of the word onto element i
    u[i] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, u[i]) ^ ((sw << (31 - i)) & 0x80000000u));
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if ((i & h) == 0) {
        const float a = u[i], b = u[i + h];
        u[i] = a + b;
        u[i + h] = a - b;
      }
  // lower element: u_i + u_{i+h}; upper element: u_i - u_{i+h} (u_i the lower partner's)
  auto cross = [&](auto m_c) {
    constexpr int m = decltype(m_c)::value;
    const float sg = (t & m) != 0 ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) u[i] = __builtin_fmaf(u[i], sg, xlane<m>(u[i]));
  };
  cross(std::integral_constant<int, 1>{});
  cross(std::integral_constant<int, 2>{});
  cross(std::integral_constant<int, 4>{});
  cross(std::integral_constant<int, 8>{});
#pragma unroll
  for (int i = 0; i < 16; ++i) u[i] *= 0.0625f;
}

// Q8 codes of 16 values (u * id rounded through the 1.5 * 2^23 sum: its low
// byte is q in two's complement, ties to even, |q| <= 127 without a clamp when
// |u| <= amax) packed into four words; returns the sum of the 16 codes.
__device__ __forceinline__ int q8_pack16(const float u[16], float id, uint32_t pk[4]) {
  uint32_t bsum = 0;  // 16 * 0x4B400000 + sum of q, mod 2^32
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      b[j] = __builtin_bit_cast(uint32_t, u[4 * w + j] * id + 12582912.0f);
      bsum += b[j];
    }
    const uint32_t lo = __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u);  // q0 | q1 << 8
    const uint32_t hi = __builtin_amdgcn_perm(b[3], b[2], 0x0C0C0400u);  // q2 | q3 << 8
    pk[w] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
  }
  return (int)(bsum - 16u * 0x4B400000u);
}

// One 256-block per 16 lanes, four per wave, in a grid-stride loop: the
// rotation (rotate256), then Q8 per qblock over WIDTH = qblock / 16 lanes and
// one 16-byte store per lane.  Each lane's block advances by a fixed quotient
// and remainder per turn of the grid (no division per block).
template <int WIDTH>
__global__ __launch_bounds__(256) void k_hadamard_quant(const float* __restrict__ x, int K, int nblocks,
                                                        const uint32_t* __restrict__ sign_bits,
                                                        int8_t* __restrict__ q, float* __restrict__ d,
                                                        int32_t* __restrict__ qsum, int step_tok, int step_kb) {
  constexpr int QBLOCK = 16 * WIDTH;
  const int lane = threadIdx.x & 63, t = lane & 15;
  const int nkb = K / 256;
  const bool vec = ((uintptr_t)q & 15) == 0;
  int blk = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
  int tok = blk / nkb, kb = blk - tok * nkb;
  const int step = gridDim.x * 16;  // blocks per turn of the grid
  for (int base = (blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * 4; base < nblocks;
       base += step) {
    const bool ok = blk < nblocks;  // the whole 16-lane group agrees
    const int64_t off = (int64_t)tok * K + kb * 256 + 16 * t;
    float u[16];
    rotate256(x + off, sign_bits, kb * 256 + 16 * t, t, ok, u);
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(u[i]));
    am = fmaxf(am, xlane<1>(am));
    if constexpr (WIDTH > 2) {
      am = fmaxf(am, xlane<2>(am));
      am = fmaxf(am, xlane<4>(am));
      am = fmaxf(am, xlane<8>(am));
    }
    const float dd = am / 127.0f;
    const float id = q8_inv(dd);
    uint32_t pk[4];
    int sum = q8_pack16(u, id, pk);
    sum += xlane_i<1>(sum);
    if constexpr (WIDTH > 2) {
      sum += xlane_i<2>(sum);
      sum += xlane_i<4>(sum);
      sum += xlane_i<8>(sum);
    }
    if (ok) {
      int8_t* o = q + off;
      if (vec) {
        *(uint4*)o = uint4{pk[0], pk[1], pk[2], pk[3]};
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) ((uint32_t*)o)[w] = pk[w];
      }
      if ((t & (WIDTH - 1)) == 0) {
        const int64_t qi = (int64_t)tok * (K / QBLOCK) + (kb * 256 + 16 * t) / QBLOCK;
        d[qi] = dd;
        qsum[qi] = sum;
      }
    }
    blk += step;
    kb += step_kb;
    tok += step_tok;
    if (kb >= nkb) {
      kb -= nkb;
      ++tok;
    }
  }
}


// Q8 with one scale per token row (qblock = K): one workgroup per row, of as
// many waves as it takes for its G = blockDim / 16 groups of 16 lanes to rotate
// all blocks g, g + G, ... (NB each at most, kept in registers); the row's amax
// and code sum are reduced over the wave and then the workgroup (LDS).
template <int NB>
__global__ __launch_bounds__(1024) void k_hadamard_quant_row(const float* __restrict__ x, int K,
                                                             const uint32_t* __restrict__ sign_bits,
                                                             int8_t* __restrict__ q, float* __restrict__ d,
                                                             int32_t* __restrict__ qsum) {
  __shared__ float s_am[16];
  __shared__ int s_sum[16];
  const int tok = blockIdx.x;
  const int lane = threadIdx.x & 63, t = lane & 15, g = threadIdx.x >> 4, wave = threadIdx.x >> 6;
  const int G = blockDim.x >> 4, nw = blockDim.x >> 6;
  const int nkb = K / 256;
  const float* const xr = x + (int64_t)tok * K;
  float u[NB][16];
  float am = 0.0f;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int kb = g + G * b;
    const bool ok = kb < nkb;  // the whole 16-lane group agrees
    rotate256(xr + kb * 256 + 16 * t, sign_bits, kb * 256 + 16 * t, t, ok, u[b]);
#pragma unroll
    for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(u[b][i]));
  }
  for (int m = 1; m < 64; m <<= 1) am = fmaxf(am, __shfl_xor(am, m));
  if (lane == 0) s_am[wave] = am;
  __syncthreads();
  am = s_am[0];
  for (int w = 1; w < nw; ++w) am = fmaxf(am, s_am[w]);
  const float dd = am / 127.0f;
  const float id = q8_inv(dd);
  const bool vec = ((uintptr_t)q & 15) == 0;
  int sum = 0;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int kb = g + G * b;
    uint32_t pk[4];
    const int sb = q8_pack16(u[b], id, pk);
    if (kb < nkb) {
      sum += sb;
      int8_t* o = q + (int64_t)tok * K + kb * 256 + 16 * t;
      if (vec) {
        *(uint4*)o = uint4{pk[0], pk[1], pk[2], pk[3]};
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) ((uint32_t*)o)[w] = pk[w];
      }
    }
  }
  for (int m = 1; m < 64; m <<= 1) sum += __shfl_xor(sum, m);
  if (lane == 0) s_sum[wave] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    int tot = 0;
    for (int w = 0; w < nw; ++w) tot += s_sum[w];
    d[tok] = dd;
    qsum[tok] = tot;
  }
}

hipError_t launch_hadamard_quant(const float* x, int B, int K, const uint32_t* sign_bits, int qblock, int8_t* q,
                                 float* d, int32_t* qsum, hipStream_t s) {
  if (qblock == K && qblock != 32 && qblock != 256) {  // one scale per row
    const int nkb = K / 256;
    const int nb = (nkb + 63) / 64;                      // blocks per 16-lane group (<= 64 groups)
    const int threads = ((nkb + nb - 1) / nb * 16 + 63) / 64 * 64;
    const dim3 grid(B), block(threads);
    if (nb == 1) hipLaunchKernelGGL(k_hadamard_quant_row<1>, grid, block, 0, s, x, K, sign_bits, q, d, qsum);
    else if (nb == 2) hipLaunchKernelGGL(k_hadamard_quant_row<2>, grid, block, 0, s, x, K, sign_bits, q, d, qsum);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  const int64_t nblocks = (int64_t)B * (K / 256);
  if (nblocks >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const int grid = (int)std::min<int64_t>((nblocks + 15) / 16, 8192);
  const int nkb = K / 256, step = grid * 16;
  if (qblock == 256)
    hipLaunchKernelGGL(k_hadamard_quant<16>, dim3(grid), dim3(256), 0, s, x, K, (int)nblocks, sign_bits, q, d, qsum,
                       step / nkb, step % nkb);
  else
    hipLaunchKernelGGL(k_hadamard_quant<2>, dim3(grid), dim3(256), 0, s, x, K, (int)nblocks, sign_bits, q, d, qsum,
                       step / nkb, step % nkb);
  return hipGetLastError();
}

}  // namespace qk
