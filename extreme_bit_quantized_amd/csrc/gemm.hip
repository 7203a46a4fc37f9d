// gemm.hip — block-scaled int8 GEMM on the gfx950 matrix cores.
//
// y[m][n] = sum_kb dx[m][kb] * dw[n][kb] * I[m][n][kb], I the exact int32 dot of
// xq[m] and wq[n] over K-block kb.  Both operands are K-contiguous rows, which
// is exactly what v_mfma_i32_32x32x32_i8 wants per lane (16 int8 of one row).
//
// Tiling: a 256-thread workgroup computes a 128 x 128 tile of y; each wave a
// 64 x 64 quarter as 2 x 2 MFMA tiles.  K advances in 64-wide stages staged
// through LDS (double buffered, rows padded to 80 bytes so the 8 lanes of a
// 16-byte LDS read phase hit different banks); the next stage's global loads
// are in flight while the current one runs on the matrix cores.  At the end of
// each K-block the int32 accumulators are scaled into fp32 accumulators.
#include "internal.hpp"

namespace qk {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int GBM = 128, GBN = 128, GBK = 64, GPITCH = 80;

template <int KB>
__global__ __launch_bounds__(256) void k_gemm_i8(const int8_t* __restrict__ xq, const float* __restrict__ dx, int M,
                                                 const int8_t* __restrict__ wq, const float* __restrict__ dw, int N,
                                                 int K, float* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) int8_t As[2][GBM * GPITCH];
  __shared__ __attribute__((aligned(16))) int8_t Bs[2][GBN * GPITCH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * GBM, n0 = blockIdx.x * GBN;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int nkb = K / KB;

  // Global -> LDS loader: chunk c = tid + 256 h (h = 0, 1): row c / 4, 16-byte column c % 4.
  int lrow[2], lcol[2];
  bool aok[2], bok[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = tid + 256 * h;
    lrow[h] = c >> 2;
    lcol[h] = (c & 3) * 16;
    aok[h] = m0 + lrow[h] < M;
    bok[h] = n0 + lrow[h] < N;
  }
  const int8_t* ag[2];
  const int8_t* bg[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    ag[h] = xq + (int64_t)(aok[h] ? m0 + lrow[h] : 0) * K + lcol[h];
    bg[h] = wq + (int64_t)(bok[h] ? n0 + lrow[h] : 0) * K + lcol[h];
  }
  v4i ra[2], rb[2];
  auto gload = [&](int k0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ra[h] = aok[h] ? *(const v4i*)(ag[h] + k0) : v4i{0, 0, 0, 0};
      rb[h] = bok[h] ? *(const v4i*)(bg[h] + k0) : v4i{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *(v4i*)(&As[buf][lrow[h] * GPITCH + lcol[h]]) = ra[h];
      *(v4i*)(&Bs[buf][lrow[h] * GPITCH + lcol[h]]) = rb[h];
    }
  };

  v16i acc[2][2];
  float facc[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        acc[i][j][e] = 0;
        facc[i][j][e] = 0.0f;
      }

  // Rows / columns of this lane's accumulator entries.
  const int lm = lane & 31, lg = lane >> 5;
  auto epilogue = [&](int kb) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn + 32 * j + lm;
      const float sw = n < N ? dw[(int64_t)n * nkb + kb] : 0.0f;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + wm + 32 * i + 8 * (e >> 2) + 4 * lg + (e & 3);
          const float sx = m < M ? dx[(int64_t)m * nkb + kb] : 0.0f;
          facc[i][j][e] = __builtin_fmaf(sx * sw, (float)acc[i][j][e], facc[i][j][e]);
          acc[i][j][e] = 0;
        }
    }
  };

  const int nstage = K / GBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int s = 0; s < nstage; ++s) {
    const int buf = s & 1;
    if (s + 1 < nstage) gload((s + 1) * GBK);
#pragma unroll
    for (int kk = 0; kk < GBK; kk += 32) {
      v4i fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[i] = *(const v4i*)(&As[buf][(wm + 32 * i + lm) * GPITCH + kk + 16 * lg]);
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = *(const v4i*)(&Bs[buf][(wn + 32 * j + lm) * GPITCH + kk + 16 * lg]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
      if (KB == 32) epilogue((s * GBK + kk) / 32);
    }
    if (KB == 256 && ((s + 1) * GBK) % 256 == 0) epilogue((s * GBK) / 256);
    if (s + 1 < nstage) {
      lstore(buf ^ 1);
      __syncthreads();
    }
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn + 32 * j + lm;
      if (n >= N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm + 32 * i + 8 * (e >> 2) + 4 * lg + (e & 3);
        if (m < M) y[(int64_t)m * N + n] = facc[i][j][e];
      }
    }
}

hipError_t launch_gemm(const int8_t* xq, const float* dx, int M, const int8_t* wq, const float* dw, int N, int K,
                       int kblock, float* y, hipStream_t s) {
  const dim3 grid((N + GBN - 1) / GBN, (M + GBM - 1) / GBM), block(256);
  if (kblock == 256) hipLaunchKernelGGL(k_gemm_i8<256>, grid, block, 0, s, xq, dx, M, wq, dw, N, K, y);
  else hipLaunchKernelGGL(k_gemm_i8<32>, grid, block, 0, s, xq, dx, M, wq, dw, N, K, y);
  return hipGetLastError();
}

}  // namespace qk
