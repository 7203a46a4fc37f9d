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
typedef float v4f __attribute__((ext_vector_type(4)));

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

// ---- pipelined GEMM for 256-blocks ---------------------------------------------------------------
// Workgroup tile 256 (M) x 128 (N), 8 waves (two per SIMD) of 64 x 64 (2 x 2
// MFMA 32x32x32 tiles).  K advances 64 at a time.  Each stage (256 + 128 rows
// of 64 bytes, 3 x 16 bytes per thread) is loaded into registers two stages
// ahead, written to a double-buffered LDS tile and read back as MFMA operands.
// A row's four 16-byte chunks are stored XOR-swizzled by (row >> 2) & 3.  gfx950
// LDS behaves as 64 four-byte banks with a 16-byte access served 16 lanes at a
// time, so the 16 lanes of a phase (rows r..r+15, one chunk) must land in 16
// different 16-byte slots modulo 256 bytes: (row % 4, chunk ^ ((row >> 2) % 4))
// does that (measured: no conflicts; (row >> 1) & 3 gave one conflict cycle per
// access cycle, no swizzle three).  dx / dw of a 256-block go through a 2-slot
// LDS ring, loaded at the previous block's first stage.  Workgroups are dealt to
// the 8 XCDs round robin; each XCD takes a contiguous run of the tiles in M-major
// order, so an XCD keeps one 256-row activation slab in its L2 while the XCDs
// walk the weight slabs in step (shared through the last-level cache).
constexpr int PBM = 256, PBN = 128, PBK = 64, PTHREADS = 512;

__global__ __launch_bounds__(PTHREADS)
void k_gemm_i8_p256(const int8_t* __restrict__ xq, const float* __restrict__ dx, int M,
                    const int8_t* __restrict__ wq, const float* __restrict__ dw, int N, int K,
                    float* __restrict__ y, int n_tiles, int m_tiles) {
  __shared__ __attribute__((aligned(16))) int8_t As[2][PBM * PBK];
  __shared__ __attribute__((aligned(16))) int8_t Bs[2][PBN * PBK];
  __shared__ __attribute__((aligned(16))) float Sx[2][PBM];
  __shared__ __attribute__((aligned(16))) float Sw[2][PBN];

  const int b = blockIdx.x, xcd = b & 7, kx = b >> 3;
  const int per = (m_tiles * n_tiles + 7) / 8;
  const int t = xcd * per + kx;
  if (kx >= per || t >= m_tiles * n_tiles) return;
  const int mt = t / n_tiles, nt = t % n_tiles;
  const int m0 = mt * PBM, n0 = nt * PBN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int nkb = K / 256;

  // This thread's loads: A rows (tid >> 2) and 128 + (tid >> 2), B row (tid >> 2),
  // 16-byte chunk tid & 3; rows clamped into the matrix (clamped rows are
  // computed and never stored).
  const int lr = tid >> 2, lc = tid & 3;
  const int8_t* asrc[2];
  int adst[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = lr + 128 * j;
    asrc[j] = xq + (int64_t)min(m0 + r, M - 1) * K + lc * 16;
    adst[j] = r * PBK + ((lc ^ ((r >> 2) & 3)) << 4);
  }
  const int8_t* bsrc = wq + (int64_t)min(n0 + lr, N - 1) * K + lc * 16;
  const int bdst = lr * PBK + ((lc ^ ((lr >> 2) & 3)) << 4);
  // scales: threads 0..255 carry dx rows, 256..383 dw rows
  const bool sx_thr = tid < PBM, sw_thr = tid >= PBM && tid < PBM + PBN;
  const float* ssrc = sx_thr ? dx + (int64_t)min(m0 + tid, M - 1) * nkb
                             : dw + (int64_t)min(n0 + (sw_thr ? tid - PBM : 0), N - 1) * nkb;
  float* sdst0 = sx_thr ? &Sx[0][tid] : &Sw[0][sw_thr ? tid - PBM : 0];
  float* sdst1 = sx_thr ? &Sx[1][tid] : &Sw[1][sw_thr ? tid - PBM : 0];
  const bool s_thr = sx_thr || sw_thr;

  v4i ra[2][2], rb[2];
  auto gload = [&](int st, v4i (&a)[2], v4i& bb) {
    const int k0 = min(st, K / PBK - 1) * PBK;  // past the end: reload the last stage
#pragma unroll
    for (int j = 0; j < 2; ++j) a[j] = *(const v4i*)(asrc[j] + k0);
    bb = *(const v4i*)(bsrc + k0);
  };
  auto lstore = [&](int buf, const v4i (&a)[2], const v4i& bb) {
#pragma unroll
    for (int j = 0; j < 2; ++j) *(v4i*)(&As[buf][adst[j]]) = a[j];
    *(v4i*)(&Bs[buf][bdst]) = bb;
  };

  // MFMA operand offsets (row r, 16-byte chunk c = 2 kk + lane / 32).
  const int l32 = lane & 31, lhi = lane >> 5;
  int aoff[2][2], boff[2][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int c = 2 * kk + lhi;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = wm * 64 + 32 * i + l32;
      aoff[i][kk] = r * PBK + ((c ^ ((r >> 2) & 3)) << 4);
      const int rn = wn * 64 + 32 * i + l32;
      boff[i][kk] = rn * PBK + ((c ^ ((rn >> 2) & 3)) << 4);
    }
  }

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

  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      v4i fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[i] = *(const v4i*)(&As[buf][aoff[i][kk]]);
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = *(const v4i*)(&Bs[buf][boff[j][kk]]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  };
  // After the last stage of K-block kb: T = dx * dw * I into the fp32 sums.
  auto epilogue = [&](int slot) {
    float sw[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) sw[j] = Sw[slot][wn * 64 + 32 * j + l32];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4f sx4 = *(const v4f*)(&Sx[slot][wm * 64 + 32 * i + 8 * q + 4 * lhi]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int e = 4 * q + t;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            facc[i][j][e] = __builtin_fmaf(sx4[t] * sw[j], (float)acc[i][j][e], facc[i][j][e]);
            acc[i][j][e] = 0;
          }
        }
      }
  };

  // prologue: stages 0 and 1 in registers, block 0's scales in slot 0
  gload(0, ra[0], rb[0]);
  gload(1, ra[1], rb[1]);
  if (s_thr) *sdst0 = ssrc[0];
  float sn = 0.0f;
  for (int kb = 0; kb < nkb; ++kb) {
    const int s0 = 4 * kb;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = u & 1;  // stage parity: LDS buffer and register set
      lstore(p, ra[p], rb[p]);
      gload(s0 + u + 2, ra[p], rb[p]);
      if (u == 0 && s_thr) sn = ssrc[min(kb + 1, nkb - 1)];
      if (u == 2 && s_thr) *((kb & 1) ? sdst0 : sdst1) = sn;  // slot (kb + 1) & 1
      __syncthreads();
      compute(p);
    }
    epilogue(kb & 1);
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + 32 * j + l32;
      if (n >= N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * 64 + 32 * i + 8 * (e >> 2) + 4 * lhi + (e & 3);
        if (m < M) y[(int64_t)m * N + n] = facc[i][j][e];
      }
    }
}

hipError_t launch_gemm(const int8_t* xq, const float* dx, int M, const int8_t* wq, const float* dw, int N, int K,
                       int kblock, float* y, hipStream_t s) {
  // 256-blocks: the pipelined kernel.
  if (kblock == 256) {
    const int n_tiles = (N + PBN - 1) / PBN, m_tiles = (M + PBM - 1) / PBM;
    const int blocks = 8 * ((n_tiles * m_tiles + 7) / 8);
    hipLaunchKernelGGL(k_gemm_i8_p256, dim3(blocks), dim3(PTHREADS), 0, s, xq, dx, M, wq, dw, N, K, y, n_tiles,
                       m_tiles);
    return hipGetLastError();
  }
  const dim3 grid((N + GBN - 1) / GBN, (M + GBM - 1) / GBM), block(256);
  if (kblock == 256) hipLaunchKernelGGL(k_gemm_i8<256>, grid, block, 0, s, xq, dx, M, wq, dw, N, K, y);
  else hipLaunchKernelGGL(k_gemm_i8<32>, grid, block, 0, s, xq, dx, M, wq, dw, N, K, y);
  return hipGetLastError();
}

}  // namespace qk
