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
//   2. scores on the matrix cores (v_mfma_f32_16x16x32_f16, 16 rows x 16 tokens
//      x one 32-value block): the codes are exact in fp16, each q row is scaled
//      by a power of two and split into fp16 high and low halves (two MFMAs,
//      about 22 bits of q); each block's result times the token's block scale,
//      summed over the blocks in fp32, the row scale taken off;
//   3. softmax statistics of the chunk: m = max s, p = exp(s - m), l = sum p;
//   4. p V: thread = 4 dimensions, wave = 64 tokens; per token and row the
//      weight p * (scale of the lane's block) times the codes; the four
//      waves' sums added in LDS.
// The merge kernel: M = max over chunks of m, out = sum_c exp(m_c - M) O_c /
// sum_c exp(m_c - M) l_c, each row's chunks split over 16 waves.
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

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef float f4_t __attribute__((ext_vector_type(4)));

// Two codes as exact fp16 values: the halves 0x6400 | u (= 1024 + u, u the
// unsigned code byte) minus 1024 + the code offset (packed fp16 add; every
// value is an integer below 2048, so all of it is exact).
__device__ __forceinline__ uint32_t halves_minus(uint32_t magic_pair, float off) {
  const h2_t v = __builtin_bit_cast(h2_t, magic_pair) - (h2_t){(_Float16)(1024.0f + off), (_Float16)(1024.0f + off)};
  return __builtin_bit_cast(uint32_t, v);
}

// The 8 codes of a lane's share of a 32-value block as an fp16 MFMA operand.
// Q8: 8 bytes (w0, w1), code c as the byte c + 128; Q4: 4 bytes (w0), low nibble
// first, code c as the nibble c + 8.
template <int FMT>
__device__ __forceinline__ h8_t codes_f16(uint32_t w0, uint32_t w1) {
  uint32_t o[4];
  if constexpr (FMT == QKV_Q8) {
    const uint32_t a = w0 ^ 0x80808080u, b = w1 ^ 0x80808080u;
    o[0] = halves_minus(__builtin_amdgcn_perm(0x64646464u, a, 0x04010400u), 128.0f);
    o[1] = halves_minus(__builtin_amdgcn_perm(0x64646464u, a, 0x04030402u), 128.0f);
    o[2] = halves_minus(__builtin_amdgcn_perm(0x64646464u, b, 0x04010400u), 128.0f);
    o[3] = halves_minus(__builtin_amdgcn_perm(0x64646464u, b, 0x04030402u), 128.0f);
  } else {
    const uint32_t lo = w0 & 0x0F0F0F0Fu, hi = (w0 >> 4) & 0x0F0F0F0Fu;  // values 2j, 2j + 1
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // bytes: value 2j, 0x64, value 2j + 1, 0x64
      const uint32_t pair = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u + 0x00010001u * j) | 0x64006400u;
      o[j] = halves_minus(pair, 8.0f);
    }
  }
  h8_t r;
  __builtin_memcpy(&r, o, 16);
  return r;
}

// One (KV head, chunk of tokens) for G query rows.  Grid (chunks, row groups);
// row group y covers query rows y G .. y G + G - 1 of KV head y G / group.
// part: [row group][chunk][G][kD + 2] floats (O, then m and l).
template <int FMT, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_attn_chunk(const float* __restrict__ q, int group, int T, int64_t t_cap,
                                                    const uint8_t* __restrict__ kc, const uint16_t* __restrict__ ks,
                                                    const uint8_t* __restrict__ vc, const uint16_t* __restrict__ vs,
                                                    float* __restrict__ part) {
  constexpr int RB = KvGeo<FMT>::row_bytes;
  // LDS: the q rows, their MFMA operands and the scores live only until the
  // softmax, so the waves' p V sums reuse that space at the end.
  constexpr int QS_BYTES = G * kD * 4, QA_BYTES = (kD / 32) * 2 * 64 * 16, SC_BYTES = G * kChunk * 4;
  constexpr int RED_BYTES = 4 * G * kD * 4;
  constexpr int PH1 = QS_BYTES + QA_BYTES + SC_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t ubuf[PH1 > RED_BYTES ? PH1 : RED_BYTES];
  float(&qs)[G][kD] = *reinterpret_cast<float(*)[G][kD]>(ubuf);
  uint4(&qa)[kD / 32][2][64] = *reinterpret_cast<uint4(*)[kD / 32][2][64]>(ubuf + QS_BYTES);
  float(&Sc)[G][kChunk] = *reinterpret_cast<float(*)[G][kChunk]>(ubuf + QS_BYTES + QA_BYTES);
  float(&red)[4][G][kD] = *reinterpret_cast<float(*)[4][G][kD]>(ubuf);
  __shared__ float rsc[G][2];                                  // row scale 2^e and 2^-e
  __shared__ __attribute__((aligned(16))) float P[kChunk][8];  // weights of each token, rows padded to 8
  __shared__ float stat[2][4][G];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int chunk = blockIdx.x, y = blockIdx.y;
  const int row0 = y * G;
  const int h = row0 / group;
  const int t0 = chunk * kChunk;
  const int nt = T - t0 < kChunk ? T - t0 : kChunk;

  // Scales issued first, so their latency overlaps the q set-up: this thread's
  // token of the chunk for the V scales (staged through LDS for the p V pass),
  // and the K scales of the lane's token in each of its wave's four tiles.
  const int r16 = lane & 15, jq = lane >> 4;
  uint4 vsr = make_uint4(0u, 0u, 0u, 0u);
  if (tid < nt) vsr = *(const uint4*)(vs + ((int64_t)h * t_cap + t0 + tid) * (kD / 32));
  uint4 ksr[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int kl = 64 * wv + 16 * tt + r16;
    ksr[tt] = make_uint4(0u, 0u, 0u, 0u);
    if (kl < nt) ksr[tt] = *(const uint4*)(ks + ((int64_t)h * t_cap + t0 + kl) * (kD / 32));
  }
#pragma unroll
  for (int g = 0; g < G; ++g) qs[g][tid] = q[(int64_t)(row0 + g) * kD + tid] * 0.0625f;
  __syncthreads();

  // ---- scores on the matrix cores ----
  // Row scales: 2^(15 - E) with max |q row| in [2^(E-1), 2^E), so the scaled row
  // peaks in [2^14, 2^15): its fp16 high halves stay finite and its fp16 low
  // halves (the rest) stay normal down to 2^-17 of the peak.
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float v = fabsf(qs[g][tid]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    if (lane == 0) stat[0][wv][g] = v;
  }
  __syncthreads();
  if (tid < G) {
    const float mxq = fmaxf(fmaxf(stat[0][0][tid], stat[0][1][tid]), fmaxf(stat[0][2][tid], stat[0][3][tid]));
    int e = 0;
    if (mxq > 0.0f) (void)frexpf(mxq, &e);
    rsc[tid][0] = ldexpf(1.0f, 15 - e);
    rsc[tid][1] = ldexpf(1.0f, e - 15);
  }
  __syncthreads();
  // A operands (lane: row lane % 16, values 8 (lane / 16) .. + 7 of each block),
  // q = hi + lo in fp16 after the row scale, rows G .. 15 zero; built once into
  // LDS, each thread two (block, lane) slots.
  for (int slot = tid; slot < (kD / 32) * 64; slot += 256) {
    const int b = slot >> 6, ln = slot & 63, r = ln & 15, jq = ln >> 4;
    h8_t hi8, lo8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = r < G ? qs[r < G ? r : 0][32 * b + 8 * jq + j] * rsc[r < G ? r : 0][0] : 0.0f;
      const _Float16 hi = (_Float16)x;
      hi8[j] = hi;
      lo8[j] = (_Float16)(x - (float)hi);
    }
    qa[b][0][ln] = __builtin_bit_cast(uint4, hi8);
    qa[b][1][ln] = __builtin_bit_cast(uint4, lo8);
  }
  __syncthreads();
  {
    // wave wv: four 16-token tiles, two at a time (16 code loads in flight per
    // lane); lane: token lane % 16 of the tile, values 8 (lane / 16) .. + 7 of
    // each block (the B operand)
#pragma unroll 1
    for (int tp = 0; tp < 2; ++tp) {
      uint32_t kw[2][8][2];
      // tokens past the end read token 0 of the chunk (no branch per load);
      // their scores are dropped below
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int kl = 64 * wv + 16 * (2 * tp + i) + r16;
        const int64_t t = (int64_t)h * t_cap + t0 + (kl < nt ? kl : 0);
#pragma unroll
        for (int b = 0; b < kD / 32; ++b) {
          if constexpr (FMT == QKV_Q8) {
            const uint2 v = *(const uint2*)(kc + t * RB + 32 * b + 8 * jq);
            kw[i][b][0] = v.x;
            kw[i][b][1] = v.y;
          } else {
            kw[i][b][0] = *(const uint32_t*)(kc + t * RB + 16 * b + 4 * jq);
            kw[i][b][1] = 0u;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int tt = 2 * tp + i;
        const int kl = 64 * wv + 16 * tt + r16;
        const uint4 kq = tp == 0 ? ksr[i] : ksr[2 + i];  // (no run-time index into the array)
        const uint32_t sw[4] = {kq.x, kq.y, kq.z, kq.w};
        f4_t sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int b = 0; b < kD / 32; ++b) {
          const h8_t kb = codes_f16<FMT>(kw[i][b][0], kw[i][b][1]);
          const h8_t qhi = __builtin_bit_cast(h8_t, qa[b][0][lane]), qlo = __builtin_bit_cast(h8_t, qa[b][1][lane]);
          f4_t c = {0.0f, 0.0f, 0.0f, 0.0f};
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(qhi, kb, c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(qlo, kb, c, 0, 0, 0);
          const float sc = h2f((uint16_t)(sw[b >> 1] >> (16 * (b & 1))));
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) sacc[i4] = __builtin_fmaf(sc, c[i4], sacc[i4]);
        }
        // C lane: token lane % 16, rows 4 (lane / 16) + i
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int row = 4 * jq + i4;
          if (row < G) Sc[row][kl] = sacc[i4] * rsc[row][1];
        }
      }
    }
  }
  __syncthreads();
  // V scales of the chunk's tokens (zero past the end) over the q operands,
  // which the scores no longer need
  uint16_t(&vsc)[kChunk][kD / 32] = *reinterpret_cast<uint16_t(*)[kChunk][kD / 32]>(ubuf + QS_BYTES);
  *(uint4*)&vsc[tid][0] = vsr;
  float s[G];
#pragma unroll
  for (int g = 0; g < G; ++g) s[g] = tid < nt ? Sc[g][tid] : -__builtin_inff();

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
  // 16 tokens' codes in flight per lane; tokens past the end read the chunk's
  // last token (no branch per load) and add 0: their p and scale are 0 and
  // every code is finite
  const int64_t tlast = (int64_t)h * t_cap + t0 + nt - 1;
#pragma unroll 1
  for (int k0 = 0; k0 < 64; k0 += 16) {
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t t = k0 + i < tn ? tbase + k0 + i : tlast;
      if constexpr (FMT == QKV_Q8) w[i] = *(const uint32_t*)(vc + t * RB + 4 * lane);
      else w[i] = *(const uint16_t*)(vc + t * RB + 2 * lane);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int k = k0 + i;
      const float sc = h2f(vsc[tb + k][blk]);
      float f[8];
      codes_f32<FMT>(w[i], f);
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
  }
  __syncthreads();  // every wave's scale reads are done before the sums overwrite them
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < 4; ++j) red[wv][g][4 * lane + j] = o[g][j];  // over qs / qa / Sc, read before a barrier
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

// Merge the chunks of each query row.  Grid (rows, kD / 64): a workgroup takes
// 64 dimensions of one row; its 16 waves take every 16th chunk (lane =
// dimension), then the waves' sums are added in LDS.  M = max over chunks of m,
// out = sum_c exp(m_c - M) O_c / sum_c exp(m_c - M) l_c.
constexpr int kMergeWaves = 16;

__global__ __launch_bounds__(64 * kMergeWaves) void k_attn_merge(const float* __restrict__ part, int G, int nchunk,
                                                                 float* __restrict__ out) {
  __shared__ float mx[kMergeWaves];
  __shared__ float accs[kMergeWaves][64];
  __shared__ float ls[kMergeWaves];
  const int row = blockIdx.x;  // query row = y G + g
  const int y = row / G, g = row % G;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int d = blockIdx.y * 64 + lane;
  const float* base = part + (int64_t)y * nchunk * G * (kD + 2) + g * (kD + 2);
  const int64_t cstride = (int64_t)G * (kD + 2);
  float M = -__builtin_inff();
  for (int c = threadIdx.x; c < nchunk; c += 64 * kMergeWaves) M = fmaxf(M, base[c * cstride + kD]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if (lane == 0) mx[wv] = M;
  __syncthreads();
  M = mx[0];
#pragma unroll
  for (int w = 1; w < kMergeWaves; ++w) M = fmaxf(M, mx[w]);
  float L = 0.0f, acc = 0.0f;
#pragma unroll 4
  for (int c = wv; c < nchunk; c += kMergeWaves) {
    const float* pc = base + c * cstride;
    const float f = expf(pc[kD] - M);
    L = __builtin_fmaf(f, pc[kD + 1], L);
    acc = __builtin_fmaf(f, pc[d], acc);
  }
  accs[wv][lane] = acc;
  if (lane == 0) ls[wv] = L;
  __syncthreads();
  if (wv == 0) {
    float a = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) {
      a += accs[w][lane];
      l += ls[w];
    }
    out[(int64_t)row * kD + d] = a / l;
  }
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
  hipLaunchKernelGGL(k_attn_merge, dim3(n_kv * group, kD / 64), dim3(64 * kMergeWaves), 0, s, part, heads_per_block,
                     nchunk, out);
  return hipGetLastError();
}

}  // namespace qk
