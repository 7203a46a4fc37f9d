// encode.hip — the trellis encoder: per row, the symbol path of the 2^16-state
// bit-shift trellis whose decoded values are closest to the weights in
// squared error (Viterbi).
//
// The trellis format codes each row jointly rather than weight by weight
// ([P2] "12 GB 装下 27B，靠的是什么取舍": trellis coding of rows in groups of
// weights, after QTIP).  A step shifts a 2-bit symbol into the 16-bit state,
// st_i = ((st_{i-1} << 2) | c_i) & 0xFFFF, so the 4 predecessors of state s are
// (s >> 2) + 16384 a, a = 0..3, and the value of state s at step i is
// s64 * V16[hash(s)].  The recursion, fp32 with each operation rounded once:
//   d = fma(-s64, V16[hash(s)], w_i)                       (s64 * V16 is exact)
//   C_i[s] = fma(d, d, min_a C_{i-1}[(s >> 2) + 16384 a])   (C_{-1} = 0)
// with the predecessor chosen pairwise: within {a, a + 2} by cost, then by its
// own incoming minimum, then the smaller a; between the two pair winners by
// cost, then the pair {0, 2}; the last state is the smallest s of minimum cost.
// Any first state is allowed; the seed is st_0 >> 2.
//
// GPU form.  The 4 states 4j .. 4j+3 share one predecessor set, so only
//   M_i[j] = min_a C_i[j + 16384 a],   j = 0 .. 16383,
// is carried from step to step (64 KB of fp32), with the choice A_i[j] (2 bits)
// written out for the backtrack:
//   C_i[j + 16384 a] = fma(d, d, M_{i-1}[(j >> 2) + 4096 a]).
// One workgroup of 1024 threads per row holds M double-buffered in LDS
// (128 KB); thread t owns j = 16 t .. 16 t + 15, so it reads M_{i-1} at
// 4 t .. 4 t + 3 (+ 4096 a) as four 16-byte loads, keeps the 32 distinct values
// V16[hash] of its 64 states in registers, decides each pair of states with
// equal values on their incoming minima (one compare) before adding the branch
// term, writes its 16 new M as four 16-byte stores and its 16 choices as one
// 32-bit word: 4 KB of choices per row and step, coalesced.
// The backtrack then walks each row's choices from the end, one lane per row.
#include <type_traits>

#include <hip/hip_fp16.h>

#include "internal.hpp"

#pragma clang fp contract(off)

namespace qk {

namespace {

constexpr int kEncThreads = 1024;
constexpr int kEncGroups = 16384;  // predecessor sets j = s mod 2^14

// Per (row, 64-block) scale: the given one, or fp16(sqrt(sum w^2 / 64)) with the
// sum accumulated in index order by fused multiply-adds.
__global__ __launch_bounds__(256) void k_enc_scales(const float* __restrict__ w, int rows, int cols,
                                                    const uint16_t* __restrict__ given,
                                                    uint16_t* __restrict__ out) {
  const int nb = cols / 64;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)rows * nb) return;
  if (given) {
    out[idx] = given[idx];
    return;
  }
  const float* p = w + (idx / nb) * (int64_t)cols + (idx % nb) * 64;
  float acc = 0.0f;
  for (int k = 0; k < 64; ++k) acc = __builtin_fmaf(p[k], p[k], acc);
  out[idx] = __half_as_ushort(__float2half_rn(__builtin_sqrtf(acc * 0.015625f)));
}

// Lexicographic (cost, state) minimum: the smaller cost, on equal costs the
// smaller state.
__device__ __forceinline__ void take_min(float& c, uint32_t& s, float c2, uint32_t s2) {
  if (c2 < c || (c2 == c && s2 < s)) {
    c = c2;
    s = s2;
  }
}

// Forward pass over one row per workgroup (rows row0 .. row0 + gridDim.x - 1).
// dec [pass row][cols - 1][1024] words; fin [pass row] = (last state, cost).
__global__ __launch_bounds__(kEncThreads) void k_enc_forward(const float* __restrict__ w, int cols, int row0,
                                                             const uint16_t* __restrict__ scales, V16Table v16t,
                                                             uint32_t* __restrict__ dec,
                                                             uint2* __restrict__ fin) {
  __shared__ __attribute__((aligned(16))) float M[2][kEncGroups];
  __shared__ float v32[256];
  __shared__ float wbuf[2][64];
  __shared__ float red_c[kEncThreads / 64];
  __shared__ uint32_t red_s[kEncThreads / 64];

  const int t = threadIdx.x;
  const int pr = blockIdx.x;
  const int64_t row = row0 + pr;
  const float* wr = w + row * cols;
  const uint16_t* sr = scales + row * (cols / 64);
  if (t < 256) v32[t] = __half2float(__ushort_as_half(v16t.v[t]));
  if (t < 64) wbuf[0][t] = wr[t];
  __syncthreads();

  // values of this thread's 64 states s = 16 t + u + 16384 a; the hash ignores
  // bit 15, so a and a + 2 share one (kept once, index a & 1)
  float v[16][2];
#pragma unroll
  for (int u = 0; u < 16; ++u)
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const uint32_t s = 16u * t + u + 16384u * a;
      v[u][a] = v32[((s * 0x9E37u) ^ (s >> 7)) & 0xFFu];
    }

  uint32_t* drow = dec + (int64_t)pr * (cols - 1) * kEncThreads + t;
  float sb = 0.0f;
  float lc = 0.0f;  // after the last step: this thread's best (cost, state)
  uint32_t ls = 0;

  // One step: C_i of this thread's 64 states from M_{i-1}, then M_i and A_i of
  // its 16 predecessor sets (LAST: the (cost, state) minimum instead of A_i).
  auto step = [&](int i, auto last_c) {
    constexpr bool LAST = decltype(last_c)::value;
    if ((i & 63) == 0) {
      sb = __half2float(__ushort_as_half(sr[i >> 6]));
      // the other buffer was last read in the previous block, before a barrier
      if (t < 64 && i + 64 < cols) wbuf[((i >> 6) + 1) & 1][t] = wr[i + 64 + t];
    }
    const float wi = wbuf[(i >> 6) & 1][i & 63];
    float4 mp[4];
    if (i == 0) {
#pragma unroll
      for (int a = 0; a < 4; ++a) mp[a] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    } else {
      const float* mprev = M[(i - 1) & 1];
#pragma unroll
      for (int a = 0; a < 4; ++a) mp[a] = *(const float4*)(mprev + 4 * t + 4096 * a);
    }
    float* mo = M[i & 1] + 16 * t;
    uint32_t word = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float m[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) m[a] = q == 0 ? mp[a].x : q == 1 ? mp[a].y : q == 2 ? mp[a].z : mp[a].w;
      if constexpr (LAST) {
        // every state's cost, for the smallest state of minimum cost
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int u = 4 * q + r;
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const float d = __builtin_fmaf(-sb, v[u][a & 1], wi);
            const float c = __builtin_fmaf(d, d, m[a]);
            const uint32_t st = 16u * t + u + 16384u * a;
            if (u == 0 && a == 0) {
              lc = c;
              ls = st;
            } else {
              take_min(lc, ls, c, st);
            }
          }
        }
      } else {
        // States j and j + 32768 differ only in bit 15, which the hash ignores:
        // equal branch terms, so each pair {a, a + 2} is decided by the incoming
        // minima (the smaller, a on equality) before the branch term is added;
        // then the two pair winners by cost (the pair {0, 2} on equality).
        const bool t0 = m[2] < m[0], t1 = m[3] < m[1];
        const float mm0 = t0 ? m[2] : m[0], mm1 = t1 ? m[3] : m[1];
        const uint32_t w0 = t0 ? 2u : 0u, w1 = t1 ? 3u : 1u;
        float nm[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int u = 4 * q + r;
          const float d0 = __builtin_fmaf(-sb, v[u][0], wi), d1 = __builtin_fmaf(-sb, v[u][1], wi);
          const float c0 = __builtin_fmaf(d0, d0, mm0), c1 = __builtin_fmaf(d1, d1, mm1);
          const bool lt = c1 < c0;
          nm[r] = lt ? c1 : c0;
          word |= (lt ? w1 : w0) << (2 * u);
        }
        *(float4*)(mo + 4 * q) = make_float4(nm[0], nm[1], nm[2], nm[3]);
      }
    }
    if constexpr (!LAST) drow[(int64_t)i * kEncThreads] = word;
  };
  for (int i = 0; i < cols - 1; ++i) {
    step(i, std::false_type{});
    __syncthreads();
  }
  step(cols - 1, std::true_type{});

  // workgroup minimum of (cost, state)
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float oc = __shfl_xor(lc, off);
    const uint32_t os = __shfl_xor(ls, off);
    take_min(lc, ls, oc, os);
  }
  if ((t & 63) == 0) {
    red_c[t >> 6] = lc;
    red_s[t >> 6] = ls;
  }
  __syncthreads();
  if (t == 0) {
    float c = red_c[0];
    uint32_t s = red_s[0];
    for (int k = 1; k < kEncThreads / 64; ++k) take_min(c, s, red_c[k], red_s[k]);
    fin[pr] = make_uint2(s, __float_as_uint(c));
  }
}

// Backtrack, one lane per row: from the last state, s_{i-1} = (s_i >> 2) +
// 16384 A_{i-1}[s_i >> 2]; symbols c_i = s_i & 3 packed four to a byte, first
// symbol in the top bits; seed = s_0 >> 2; padding bytes of the row zeroed.
// Each step waits for the word the previous step chose (a dependent load per
// weight): the kernel's time does not depend on how many rows a pass holds.
__global__ __launch_bounds__(64) void k_enc_backtrack(int cols, int row0, int nrows,
                                                      const uint32_t* __restrict__ dec,
                                                      const uint2* __restrict__ fin, uint8_t* __restrict__ codes,
                                                      int64_t row_bytes, uint16_t* __restrict__ seeds,
                                                      float* __restrict__ cost) {
  const int pr = blockIdx.x * blockDim.x + threadIdx.x;
  if (pr >= nrows) return;
  const int64_t row = row0 + pr;
  uint8_t* crow = codes + row * row_bytes;
  const uint32_t* d = dec + (int64_t)pr * (cols - 1) * kEncThreads;
  const uint2 f = fin[pr];
  uint32_t s = f.x;
  uint32_t byte = 0;
  for (int i = cols - 1; i >= 0; --i) {
    byte |= (s & 3u) << (6 - 2 * (i & 3));
    if ((i & 3) == 0) {
      crow[i >> 2] = (uint8_t)byte;
      byte = 0;
    }
    if (i > 0) {
      const uint32_t j = s >> 2;
      const uint32_t wd = d[(int64_t)(i - 1) * kEncThreads + (j >> 4)];
      s = j | (((wd >> (2 * (j & 15))) & 3u) << 14);
    }
  }
  seeds[row] = (uint16_t)(s >> 2);
  for (int64_t b = cols / 4; b < row_bytes; ++b) crow[b] = 0;
  if (cost) cost[row] = __uint_as_float(f.y);
}

}  // namespace

int64_t encode_workspace_bytes(int rows, int cols, int rows_per_pass) {
  const int64_t a = 256;
  const int64_t sc = ((int64_t)rows * (cols / 64) * 2 + a - 1) / a * a;
  const int64_t fin = ((int64_t)rows_per_pass * 8 + a - 1) / a * a;
  return sc + fin + (int64_t)rows_per_pass * (cols - 1) * kEncThreads * 4;
}

hipError_t launch_trellis_encode(const float* w, int rows, int cols, const uint16_t* scales_in, uint8_t* codes,
                                 int64_t row_bytes, uint16_t* seeds, uint16_t* scales, float* cost,
                                 int rows_per_pass, void* ws, hipStream_t s) {
  const int64_t a = 256;
  uint8_t* base = (uint8_t*)ws;
  uint16_t* sc_rm = (uint16_t*)base;
  const int64_t sc_bytes = ((int64_t)rows * (cols / 64) * 2 + a - 1) / a * a;
  uint2* fin = (uint2*)(base + sc_bytes);
  uint32_t* dec = (uint32_t*)(base + sc_bytes + ((int64_t)rows_per_pass * 8 + a - 1) / a * a);

  const int64_t nsc = (int64_t)rows * (cols / 64);
  hipLaunchKernelGGL(k_enc_scales, dim3((unsigned)((nsc + 255) / 256)), dim3(256), 0, s, w, rows, cols, scales_in,
                     sc_rm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_scales_from_rows(QFMT_TRELLIS2, rows, cols, sc_rm, scales, s);
  if (e != hipSuccess) return e;
  V16Table v16;
  trellis_tables(&v16, nullptr, nullptr);
  for (int r0 = 0; r0 < rows; r0 += rows_per_pass) {
    const int n = rows - r0 < rows_per_pass ? rows - r0 : rows_per_pass;
    hipLaunchKernelGGL(k_enc_forward, dim3(n), dim3(kEncThreads), 0, s, w, cols, r0, sc_rm, v16, dec, fin);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_enc_backtrack, dim3((n + 63) / 64), dim3(64), 0, s, cols, r0, n, dec, fin, codes,
                       row_bytes, seeds, cost);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qk
