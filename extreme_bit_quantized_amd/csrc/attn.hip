// attn.hip — the KV cache in Q8 / Q4 and decode attention over it with the
// query heads of each KV head packed into one workgroup.
//
// The KV cache grows with the context and is held in 4 or 8 bits per value
// ([P1] "12G 的账本要这么算"); decode attention of a grouped-KV model reads the
// same K and V rows for every query head of a group, so the pages pack the six
// query heads of a KV head into one block ([P1] "把非标准格式塞进 llama.cpp，难在哪",
// 27.9 -> 35.2 tok/s at a 64K context).  Here a workgroup takes one KV head and
// a chunk of 256 cached tokens for G query rows at once, so each cached byte is
// read once per G rows; a second kernel merges the chunks (flash-decoding).
//
// Cache layout (per KV head h, token t): codes [h][t][row bytes] (Q8: D int8;
// Q4: D/2 bytes, value 2j in the low nibble of byte j of its 32-block and 2j+1
// in the high one), scales [h][t][D/32] fp16, rows of t_cap tokens per head.
// Values: Q8 c * s, Q4 (nibble - 8) * s.
//
// Chunk kernel (256 threads, chunk of C = 256 tokens, D = 256):
//   1. q rows times 1/16 (= 1/sqrt(D), exact) into LDS;
//   2. scores: thread = token; per 32-block the fp32 dot of q with the codes,
//      times the block scale, summed over the blocks;
//   3. softmax statistics of the chunk: m = max s, p = exp(s - m), l = sum p;
//   4. p V: thread = 4 dimensions, wave = 64 tokens; per token and row the
//      weight p * (scale of the lane's block) times the codes; the four
//      waves' sums added in LDS.
// The merge kernel: M = max over chunks of m, out = sum_c exp(m_c - M) O_c /
// sum_c exp(m_c - M) l_c.
#include <hip/hip_fp16.h>

#include "internal.hpp"

#pragma clang fp contract(off)

namespace qk {

namespace {

constexpr int kD = 256;       // head dimension
constexpr int kChunk = 256;   // cached tokens per workgroup

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }

// Q8 / Q4 of one 32-value block per thread, the activation-Q8 rules with the
// scale stored as fp16.
template <int FMT>
__global__ __launch_bounds__(256) void k_kv_quant(const float* __restrict__ x, int64_t nblocks,
                                                  uint8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nblocks) return;
  const float4* p = (const float4*)(x + i * 32);
  float v[32];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float4 f = p[k];
    v[4 * k] = f.x;
    v[4 * k + 1] = f.y;
    v[4 * k + 2] = f.z;
    v[4 * k + 3] = f.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 32; ++k) amax = fmaxf(amax, fabsf(v[k]));
  constexpr float top = FMT == QKV_Q8 ? 127.0f : 7.0f;
  const float d = amax / top;
  const float r = 1.0f / d;
  const float id = r < __builtin_inff() ? r : 0.0f;
  scales[i] = __half_as_ushort(__float2half_rn(d));
  int c[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) c[k] = (int)fminf(fmaxf(__builtin_rintf(v[k] * id), -top), top);
  if constexpr (FMT == QKV_Q8) {
    uint4* o = (uint4*)(codes + i * 32);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int* cc = c + 16 * k + 4 * j;
        w[j] = (uint32_t)(cc[0] & 255) | ((uint32_t)(cc[1] & 255) << 8) | ((uint32_t)(cc[2] & 255) << 16) |
               ((uint32_t)(cc[3] & 255) << 24);
      }
      o[k] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  } else {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t a = 0;
#pragma unroll
      for (int n = 0; n < 8; ++n) a |= (uint32_t)(c[8 * j + n] + 8) << (4 * n);
      w[j] = a;
    }
    *(uint4*)(codes + i * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// The codes of a 32-bit word as signed floats: Q8 4 values, Q4 8 values (low
// nibble first; nibble ^ 8 is the code's 4-bit two's complement).
template <int FMT>
__device__ __forceinline__ void codes_f32(uint32_t w, float* f) {
  if constexpr (FMT == QKV_Q8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) f[j] = (float)(int32_t)(int8_t)(uint8_t)(w >> (8 * j));
  } else {
    const uint32_t x = w ^ 0x88888888u;
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = (float)(((int32_t)(x << (28 - 4 * j))) >> 28);
  }
}

template <int FMT>
struct KvGeo {
  static constexpr int row_bytes = FMT == QKV_Q8 ? kD : kD / 2;
};

// One (KV head, chunk of tokens) for G query rows.  Grid (chunks, row groups);
// row group y covers query rows y G .. y G + G - 1 of KV head y G / group.
// part: [row group][chunk][G][kD + 2] floats (O, then m and l).
template <int FMT, int G>
__global__ __launch_bounds__(256) void k_attn_chunk(const float* __restrict__ q, int group, int T, int64_t t_cap,
                                                    const uint8_t* __restrict__ kc, const uint16_t* __restrict__ ks,
                                                    const uint8_t* __restrict__ vc, const uint16_t* __restrict__ vs,
                                                    float* __restrict__ part) {
  constexpr int RB = KvGeo<FMT>::row_bytes;
  __shared__ __attribute__((aligned(16))) float qs[G][kD];
  __shared__ __attribute__((aligned(16))) float P[kChunk][8];  // weights of each token, rows padded to 8
  __shared__ float red[4][G][kD];
  __shared__ float stat[2][4][G];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int chunk = blockIdx.x, y = blockIdx.y;
  const int row0 = y * G;
  const int h = row0 / group;
  const int t0 = chunk * kChunk;
  const int nt = T - t0 < kChunk ? T - t0 : kChunk;

#pragma unroll
  for (int g = 0; g < G; ++g) qs[g][tid] = q[(int64_t)(row0 + g) * kD + tid] * 0.0625f;
  __syncthreads();

  // ---- scores: thread = token ----
  float s[G];
#pragma unroll
  for (int g = 0; g < G; ++g) s[g] = -__builtin_inff();
  if (tid < nt) {
    const int64_t t = (int64_t)h * t_cap + t0 + tid;
    const uint8_t* krow = kc + t * RB;
    const uint16_t* srow = ks + t * (kD / 32);
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = 0.0f;
#pragma unroll 1
    for (int b = 0; b < kD / 32; ++b) {
      constexpr int WORDS = FMT == QKV_Q8 ? 8 : 4;
      uint32_t w[WORDS];
      if constexpr (FMT == QKV_Q8) {
        const uint4 a = *(const uint4*)(krow + 32 * b), c = *(const uint4*)(krow + 32 * b + 16);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = c.x; w[5] = c.y; w[6] = c.z; w[7] = c.w;
      } else {
        const uint4 a = *(const uint4*)(krow + 16 * b);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
      }
      const float sc = h2f(srow[b]);
      float acc[G];
#pragma unroll
      for (int g = 0; g < G; ++g) acc[g] = 0.0f;
      constexpr int PER = FMT == QKV_Q8 ? 4 : 8;
#pragma unroll
      for (int k = 0; k < WORDS; ++k) {
        float f[8];
        codes_f32<FMT>(w[k], f);
#pragma unroll
        for (int j = 0; j < PER; ++j)
#pragma unroll
          for (int g = 0; g < G; ++g) acc[g] = __builtin_fmaf(qs[g][32 * b + PER * k + j], f[j], acc[g]);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) s[g] = __builtin_fmaf(sc, acc[g], s[g]);
    }
  }

  // ---- softmax statistics of the chunk ----
  float m[G], l[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float v = s[g];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    if (lane == 0) stat[0][wv][g] = v;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) m[g] = fmaxf(fmaxf(stat[0][0][g], stat[0][1][g]), fmaxf(stat[0][2][g], stat[0][3][g]));
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float p = tid < nt ? expf(s[g] - m[g]) : 0.0f;
    P[tid][g] = p;
    float v = p;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) stat[1][wv][g] = v;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) l[g] = (stat[1][0][g] + stat[1][1][g]) + (stat[1][2][g] + stat[1][3][g]);

  // ---- p V: lane = 4 dimensions, wave = 64 tokens ----
  float o[G][4];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < 4; ++j) o[g][j] = 0.0f;
  const int tb = wv * 64;
  const int tn = nt - tb < 64 ? (nt - tb > 0 ? nt - tb : 0) : 64;
  const int blk = lane >> 3;  // the lane's 32-block
  const int64_t tbase = (int64_t)h * t_cap + t0 + tb;
#pragma unroll 2
  for (int k = 0; k < tn; ++k) {
    const int64_t t = tbase + k;
    uint32_t w;
    if constexpr (FMT == QKV_Q8) w = *(const uint32_t*)(vc + t * RB + 4 * lane);
    else w = *(const uint16_t*)(vc + t * RB + 2 * lane);
    const float sc = h2f(vs[t * (kD / 32) + blk]);
    float f[8];
    codes_f32<FMT>(w, f);
    const float4 pa = *(const float4*)&P[tb + k][0];
    const float4 pb = *(const float4*)&P[tb + k][4];
    const float pp[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float wgt = pp[g] * sc;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[g][j] = __builtin_fmaf(wgt, f[j], o[g][j]);
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < 4; ++j) red[wv][g][4 * lane + j] = o[g][j];
  __syncthreads();
  float* pout = part + ((int64_t)y * gridDim.x + chunk) * G * (kD + 2);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    pout[g * (kD + 2) + tid] = (red[0][g][tid] + red[1][g][tid]) + (red[2][g][tid] + red[3][g][tid]);
    if (tid == 0) {
      pout[g * (kD + 2) + kD] = m[g];
      pout[g * (kD + 2) + kD + 1] = l[g];
    }
  }
}

// Merge the chunks of each query row: thread = dimension.
__global__ __launch_bounds__(256) void k_attn_merge(const float* __restrict__ part, int G, int nchunk,
                                                    float* __restrict__ out) {
  __shared__ float e[1024];
  __shared__ float mx[4];
  const int row = blockIdx.x;  // query row = y G + g
  const int y = row / G, g = row % G;
  const int tid = threadIdx.x;
  const float* base = part + (int64_t)y * nchunk * G * (kD + 2) + g * (kD + 2);
  const int64_t cstride = (int64_t)G * (kD + 2);
  float M = -__builtin_inff();
  for (int c = tid; c < nchunk; c += 256) M = fmaxf(M, base[c * cstride + kD]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if ((tid & 63) == 0) mx[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
  float L = 0.0f, acc = 0.0f;
  for (int c0 = 0; c0 < nchunk; c0 += 1024) {
    const int n = nchunk - c0 < 1024 ? nchunk - c0 : 1024;
    __syncthreads();
    for (int c = tid; c < n; c += 256) e[c] = expf(base[(c0 + c) * cstride + kD] - M);
    __syncthreads();
    for (int c = 0; c < n; ++c) {
      const float f = e[c];
      L = __builtin_fmaf(f, base[(c0 + c) * cstride + kD + 1], L);
      acc = __builtin_fmaf(f, base[(c0 + c) * cstride + tid], acc);
    }
  }
  out[(int64_t)row * kD + tid] = acc / L;
}

template <int FMT, int G>
hipError_t launch_chunks(const float* q, int n_kv, int group, int T, int64_t t_cap, const void* kc,
                         const uint16_t* ks, const void* vc, const uint16_t* vs, float* part, hipStream_t s) {
  const int nchunk = (T + kChunk - 1) / kChunk;
  const int ny = n_kv * group / G;
  hipLaunchKernelGGL((k_attn_chunk<FMT, G>), dim3(nchunk, ny), dim3(256), 0, s, q, group, T, t_cap,
                     (const uint8_t*)kc, ks, (const uint8_t*)vc, vs, part);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_chunks_g(int G, const float* q, int n_kv, int group, int T, int64_t t_cap, const void* kc,
                           const uint16_t* ks, const void* vc, const uint16_t* vs, float* part, hipStream_t s) {
  switch (G) {
    case 1: return launch_chunks<FMT, 1>(q, n_kv, group, T, t_cap, kc, ks, vc, vs, part, s);
    case 2: return launch_chunks<FMT, 2>(q, n_kv, group, T, t_cap, kc, ks, vc, vs, part, s);
    case 3: return launch_chunks<FMT, 3>(q, n_kv, group, T, t_cap, kc, ks, vc, vs, part, s);
    case 4: return launch_chunks<FMT, 4>(q, n_kv, group, T, t_cap, kc, ks, vc, vs, part, s);
    case 5: return launch_chunks<FMT, 5>(q, n_kv, group, T, t_cap, kc, ks, vc, vs, part, s);
    case 6: return launch_chunks<FMT, 6>(q, n_kv, group, T, t_cap, kc, ks, vc, vs, part, s);
    case 7: return launch_chunks<FMT, 7>(q, n_kv, group, T, t_cap, kc, ks, vc, vs, part, s);
    case 8: return launch_chunks<FMT, 8>(q, n_kv, group, T, t_cap, kc, ks, vc, vs, part, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int64_t attn_workspace_bytes(int n_kv, int group, int T) {
  const int64_t nchunk = (T + kChunk - 1) / kChunk;
  return (int64_t)n_kv * group * nchunk * (kD + 2) * 4;
}

hipError_t launch_kv_quant(int fmt, const float* x, int64_t rows, uint8_t* codes, uint16_t* scales, hipStream_t s) {
  const int64_t nb = rows * (kD / 32);
  if (nb == 0) return hipSuccess;
  const dim3 grid((unsigned)((nb + 255) / 256));
  if (fmt == QKV_Q8) hipLaunchKernelGGL(k_kv_quant<QKV_Q8>, grid, dim3(256), 0, s, x, nb, codes, scales);
  else hipLaunchKernelGGL(k_kv_quant<QKV_Q4>, grid, dim3(256), 0, s, x, nb, codes, scales);
  return hipGetLastError();
}

hipError_t launch_attn_decode(int fmt, const float* q, int n_kv, int group, int heads_per_block, int T,
                              int64_t t_cap, const void* kc, const uint16_t* ks, const void* vc,
                              const uint16_t* vs, float* out, void* ws, hipStream_t s) {
  float* part = (float*)ws;
  const hipError_t e = fmt == QKV_Q8
                           ? launch_chunks_g<QKV_Q8>(heads_per_block, q, n_kv, group, T, t_cap, kc, ks, vc, vs, part, s)
                           : launch_chunks_g<QKV_Q4>(heads_per_block, q, n_kv, group, T, t_cap, kc, ks, vc, vs, part, s);
  if (e != hipSuccess) return e;
  const int nchunk = (T + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(k_attn_merge, dim3(n_kv * group), dim3(256), 0, s, part, heads_per_block, nchunk, out);
  return hipGetLastError();
}

}  // namespace qk
