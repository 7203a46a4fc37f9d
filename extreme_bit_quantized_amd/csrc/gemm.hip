// gemm.hip — block-scaled int8 GEMM on the gfx950 matrix cores.
//
// y[m][n] = sum_kb dx[m][kb] * dw[n][kb] * I[m][n][kb], I the exact int32 dot of
// xq[m] and wq[n] over K-block kb.  Both operands are K-contiguous rows, which
// is exactly what v_mfma_i32_32x32x32_i8 wants per lane (16 int8 of one row).
//
// Generic kernel (any shape): a 256-thread workgroup computes a 128 x 128 tile
// of y (64 x 256 when M <= 64); each wave a 64 x 64 part as 2 x 2 MFMA tiles.
// K advances in 64-wide stages staged through LDS (double buffered, rows padded
// to 80 bytes so the 8 lanes of a 16-byte LDS read phase hit different banks);
// the next stage's global loads are in flight while the current one runs on
// the matrix cores.  At the end of each K-block the int32 accumulators are
// scaled into fp32 accumulators.  256-blocks with K a multiple of 1024 take the
// pipelined kernel further below.
#include <algorithm>
#include <type_traits>

#include "internal.hpp"

namespace qk {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int GBK = 64, GPITCH = 80;

// Workgroup tile (64 MW) x (256 / MW): MW = 2 gives 128 x 128 (waves 2 x 2),
// MW = 1 gives 64 x 256 (waves 1 x 4, for M <= 64: no idle rows).  The scales of
// the K-blocks that end in a stage travel with its tiles (register-staged into
// LDS, block-major, so four consecutive rows' dx are one 16-byte read).
template <int KB, int MW>
__global__ __launch_bounds__(256, KB == 256 ? 2 : 1) void k_gemm_i8(const int8_t* __restrict__ xq, const float* __restrict__ dx, int M,
                                                 const int8_t* __restrict__ wq, const float* __restrict__ dw, int N,
                                                 int K, float* __restrict__ y) {
  constexpr int TM = 64 * MW, TN = 256 / MW;
  constexpr int AH = TM * 4 / 256, BH = TN * 4 / 256;  // 16-byte chunks per thread and stage
  constexpr int NSB = KB == 32 ? GBK / 32 : 1;         // scale blocks staged per stage
  constexpr int NS = (NSB * (TM + TN) + 255) / 256;    // scale values per thread and stage
  __shared__ __attribute__((aligned(16))) int8_t As[2][TM * GPITCH];
  __shared__ __attribute__((aligned(16))) int8_t Bs[2][TN * GPITCH];
  __shared__ __attribute__((aligned(16))) float Sx[2][NSB][TM];
  __shared__ __attribute__((aligned(16))) float Sw[2][NSB][TN];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * TM, n0 = blockIdx.x * TN;
  const int wm = (wave / (4 / MW)) * 64, wn = (wave % (4 / MW)) * 64;
  const int nkb = K / KB;

  // Global -> LDS loader: chunk c = tid + 256 h: row c / 4, 16-byte column c % 4.
  const int8_t* ag[AH];
  const int8_t* bg[BH];
  bool aok[AH], bok[BH];
  int aoffl[AH], boffl[BH];
#pragma unroll
  for (int h = 0; h < AH; ++h) {
    const int c = tid + 256 * h, r = c >> 2, col = (c & 3) * 16;
    aok[h] = m0 + r < M;
    ag[h] = xq + (int64_t)(aok[h] ? m0 + r : 0) * K + col;
    aoffl[h] = r * GPITCH + col;
  }
#pragma unroll
  for (int h = 0; h < BH; ++h) {
    const int c = tid + 256 * h, r = c >> 2, col = (c & 3) * 16;
    bok[h] = n0 + r < N;
    bg[h] = wq + (int64_t)(bok[h] ? n0 + r : 0) * K + col;
    boffl[h] = r * GPITCH + col;
  }
  v4i ra[AH], rb[BH];
  float rs[NS];
  // the scale blocks of stage st: KB = 32: 2 st, 2 st + 1; KB = 256: the block of stage st
  auto gload = [&](int st) {
    const int k0 = st * GBK;
#pragma unroll
    for (int h = 0; h < AH; ++h) ra[h] = aok[h] ? *(const v4i*)(ag[h] + k0) : v4i{0, 0, 0, 0};
#pragma unroll
    for (int h = 0; h < BH; ++h) rb[h] = bok[h] ? *(const v4i*)(bg[h] + k0) : v4i{0, 0, 0, 0};
    const int kb0 = KB == 32 ? st * NSB : k0 / KB;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int c = tid + 256 * i, blk = c / (TM + TN), r = c % (TM + TN);
      float v = 0.0f;
      if (blk < NSB) {
        if (r < TM) {
          if (m0 + r < M) v = dx[(int64_t)(m0 + r) * nkb + kb0 + blk];
        } else if (n0 + r - TM < N) {
          v = dw[(int64_t)(n0 + r - TM) * nkb + kb0 + blk];
        }
      }
      rs[i] = v;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int h = 0; h < AH; ++h) *(v4i*)(&As[buf][aoffl[h]]) = ra[h];
#pragma unroll
    for (int h = 0; h < BH; ++h) *(v4i*)(&Bs[buf][boffl[h]]) = rb[h];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int c = tid + 256 * i, blk = c / (TM + TN), r = c % (TM + TN);
      if (blk < NSB) {
        if (r < TM) Sx[buf][blk][r] = rs[i];
        else Sw[buf][blk][r - TM] = rs[i];
      }
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

  // Rows / columns of this lane's accumulator entries: row wm + 32 i + 8 (e / 4)
  // + 4 lg + e % 4, column wn + 32 j + lm.
  const int lm = lane & 31, lg = lane >> 5;
  auto epilogue = [&](int buf, int blk) {
    float sw[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) sw[j] = Sw[buf][blk][wn + 32 * j + lm];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const v4f sx = *(const v4f*)&Sx[buf][blk][wm + 32 * i + 8 * q4 + 4 * lg];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int e = 4 * q4 + t;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            facc[i][j][e] = __builtin_fmaf(sx[t] * sw[j], (float)acc[i][j][e], facc[i][j][e]);
            acc[i][j][e] = 0;
          }
        }
      }
  };

  const int nstage = K / GBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int s = 0; s < nstage; ++s) {
    const int buf = s & 1;
    if (s + 1 < nstage) gload(s + 1);
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
      if (KB == 32) epilogue(buf, kk / 32);
    }
    if (KB == 256 && ((s + 1) * GBK) % 256 == 0) epilogue(buf, 0);
    if (s + 1 < nstage) {
      // buffer buf ^ 1 (stage s - 1) was released by the previous barrier
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
// MFMA 32x32x32 tiles).  K advances 128 at a time through a 3-stage LDS ring
// filled by LDS DMA (global_load_lds_dwordx4, no staging registers): each stage
// holds 256 A rows then 128 B rows of 128 bytes.  A row's eight 16-byte chunks
// are stored XOR-swizzled by (row >> 1) & 7.  gfx950 LDS behaves as 64
// four-byte banks with a 16-byte access served 16 lanes at a time, so the 16
// lanes of an MFMA operand read phase (rows r..r+15, one chunk) must land in 16
// different 16-byte slots modulo 256 bytes, which (row % 2, chunk ^ ((row >> 1)
// % 8)) does (measured with 64-byte rows: the matching swizzle had no conflicts,
// a swizzle that paired rows r and r + 8 one conflict cycle per access cycle).
// Every wave issues 6 ring DMA instructions per stage, so "stage s has landed"
// is a fixed vmcnt (extra loads issued in
// between only make that wait stricter); the ring is ordered by a plain
// s_barrier (a __syncthreads() fence would wait for every DMA in flight).  The
// dx / dw values of four consecutive 256-blocks are DMA'd once per 8 stages
// into a 2-slot ring, block-major (Sc[slot][block][row], 4 bytes per lane), so
// the epilogue gets four consecutive rows' scales with one 16-byte read; it
// reads them in one asm block that waits for its own reads (so the compiler
// adds no wait for the DMAs in flight).  The first MFMA of each 256-block
// starts from a zero C operand (no accumulator clearing), and each stage reads
// the operands of step kk + 1 while the MFMAs of step kk run.  Workgroups are dealt to the 8 XCDs round robin; each XCD
// takes a contiguous run of the tiles in M-major order, so an XCD keeps one
// 256-row activation slab in its L2 while the XCDs walk the weight slabs in
// step (shared through the last-level cache).
constexpr int PBM = 256, PBN = 128, PBK = 128, PTHREADS = 512, PST = 3;
constexpr int RING_B = PBM * PBK;             // B rows start here inside a stage
constexpr int RING_STAGE = (PBM + PBN) * PBK; // 24 KB

// LDS-typed views of the ring: every access through them is a ds_* instruction
// whatever the compiler infers about generic pointers (a generic pointer to
// LDS that it once took for a global one turned the operand reads into
// global loads of LDS offsets).
typedef __attribute__((address_space(3))) int8_t lds_i8;
typedef __attribute__((address_space(3))) const v4i lds_v4i;
__device__ __forceinline__ void lds_dma16(const void* g, lds_i8* l) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)l, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma16(const void* g, void* l) {
  lds_dma16(g, (lds_i8*)l);
}
// s_waitcnt vmcnt(n) (n < 64) and lgkmcnt(0)
template <int n>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4));
}
// Workgroup barrier that the compiler may not move memory accesses across (the
// builtin alone carries no memory ordering) and that adds no wait of its own.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ uint32_t lds_addr(const lds_i8* p) { return (uint32_t)(uintptr_t)p; }
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One 128-wide K stage of a wave's 64 x 64 tile, written out as one asm block so
// that every wait is exact: the operands of each 32-wide K step are read while
// the MFMAs of the previous step run (LDS reads return in order, so lgkmcnt(4)
// waits for all but the four just issued), and the stage's six ring DMAs go out
// two at a time between the MFMA groups (issued back to back they stall the
// wave behind the texture path before its first MFMA).  Operand names:
// c00..c11 the accumulators (A tile i, B tile j); x0 x1 y0 y1 and u0 u1 w0 w1
// two operand sets (A rows i = 0, 1 and B rows j = 0, 1 of one K step);
// pa0..pa3 / pb0..pb3 the LDS addresses of the four steps' i = 0 / j = 0 rows
// (rows i, j = 1 are 32 rows = 4096 bytes further, same swizzle); m0..m5,
// v0..v5, sb0 / sb1 the DMAs' LDS destinations, 32-bit source offsets and
// 64-bit source bases (A, B).  An MFMA reads its A / B registers when issued,
// so the next reads into the same set may follow it directly.
#define QG_RD(D, A, OFF) "ds_read_b128 %[" D "], %[" A "]" OFF "\n\t"
#define QG_RD4(X0, X1, Y0, Y1, PA, PB) \
  QG_RD(X0, PA, "") QG_RD(X1, PA, " offset:4096") QG_RD(Y0, PB, "") QG_RD(Y1, PB, " offset:4096")
#define QG_MF(D, A, B, C) "v_mfma_i32_32x32x32_i8 %[" D "], %[" A "], %[" B "], " C "\n\t"
#define QG_MF4(X0, X1, Y0, Y1, C00, C01, C10, C11) \
  QG_MF("c00", X0, Y0, C00) QG_MF("c01", X0, Y1, C01) QG_MF("c10", X1, Y0, C10) QG_MF("c11", X1, Y1, C11)
// (QG_MF4X expands its arguments first, so QG_ACC4 / QG_ZERO4 count as four)
#define QG_MF4X(...) QG_MF4(__VA_ARGS__)
#define QG_ACC4 "%[c00]", "%[c01]", "%[c10]", "%[c11]"
#define QG_ZERO4 "0", "0", "0", "0"
// M0 written by SALU needs one wait state before the LDS DMA reads it
#define QG_DMA(M, V, SB) "s_mov_b32 m0, %[" M "]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[" V "], %[" SB "]\n\t"
#define QG_WAIT(N) "s_waitcnt lgkmcnt(" #N ")\n\t"
// K steps 0..2 and the six DMAs; C0: the first step's C operands
#define QG_STAGE_HEAD(C0)                                                                         \
  QG_RD4("x0", "x1", "y0", "y1", "pa0", "pb0") QG_RD4("u0", "u1", "w0", "w1", "pa1", "pb1") QG_WAIT(4) \
  QG_MF4X("x0", "x1", "y0", "y1", C0) QG_DMA("m0", "v0", "sb0") QG_DMA("m1", "v1", "sb0")         \
  QG_RD4("x0", "x1", "y0", "y1", "pa2", "pb2") QG_WAIT(4)                                         \
  QG_MF4X("u0", "u1", "w0", "w1", QG_ACC4) QG_DMA("m2", "v2", "sb0") QG_DMA("m3", "v3", "sb0")    \
  QG_RD4("u0", "u1", "w0", "w1", "pa3", "pb3") QG_WAIT(4)                                         \
  QG_MF4X("x0", "x1", "y0", "y1", QG_ACC4) QG_DMA("m4", "v4", "sb1") QG_DMA("m5", "v5", "sb1")
// Step 3 of a block's first stage.
#define QG_TAIL_FIRST QG_WAIT(0) QG_MF4X("u0", "u1", "w0", "w1", QG_ACC4)
// Step 3 of a block's last stage, which also brings the epilogue's scales into
// the operand registers as each set frees up (rows i = 0 of dx into x0..y1, rows
// i = 1 into u0..w1, the two dw into pw), then the wait states a VALU read of an
// MFMA result needs (the compiler cannot see the MFMAs in here).
#define QG_TAIL_LAST                                                                                   \
  "ds_read_b128 %[x0], %[xa] offset:0\n\t" "ds_read_b128 %[x1], %[xa] offset:32\n\t"                   \
  "ds_read_b128 %[y0], %[xa] offset:64\n\t" "ds_read_b128 %[y1], %[xa] offset:96\n\t" QG_WAIT(4)        \
  QG_MF4X("u0", "u1", "w0", "w1", QG_ACC4)                                                              \
  "ds_read_b128 %[u0], %[xa] offset:128\n\t" "ds_read_b128 %[u1], %[xa] offset:160\n\t"                \
  "ds_read_b128 %[w0], %[xa] offset:192\n\t" "ds_read_b128 %[w1], %[xa] offset:224\n\t"                \
  "ds_read2_b32 %[pw], %[wa] offset0:0 offset1:32\n\t" QG_WAIT(0) "s_nop 7\n\ts_nop 7\n\ts_nop 3\n\t"
#define QG_OUTS                                                                                       \
  [c00] "+v"(acc[0][0]), [c01] "+v"(acc[0][1]), [c10] "+v"(acc[1][0]), [c11] "+v"(acc[1][1]),       \
  [x0] "=&v"(x0), [x1] "=&v"(x1), [y0] "=&v"(y0), [y1] "=&v"(y1), [u0] "=&v"(u0), [u1] "=&v"(u1),   \
  [w0] "=&v"(w0), [w1] "=&v"(w1)
#define QG_INS                                                                                         \
  [pa0] "v"(pa[0]), [pa1] "v"(pa[1]), [pa2] "v"(pa[2]), [pa3] "v"(pa[3]), [pb0] "v"(pb[0]),           \
  [pb1] "v"(pb[1]), [pb2] "v"(pb[2]), [pb3] "v"(pb[3]), [m0] "s"(dm[0]), [m1] "s"(dm[1]),              \
  [m2] "s"(dm[2]), [m3] "s"(dm[3]), [m4] "s"(dm[4]), [m5] "s"(dm[5]), [v0] "v"(aoff_g[0]),             \
  [v1] "v"(aoff_g[1]), [v2] "v"(aoff_g[2]), [v3] "v"(aoff_g[3]), [v4] "v"(boff_g[0]),                  \
  [v5] "v"(boff_g[1]), [sb0] "s"(sa), [sb1] "s"(sb)

// Work split (stream-K): the T tiles x NG groups of 1024 K are one sequence,
// tile-major, dealt in G equal runs, one per workgroup (G <= T, so a run spans
// at least one tile's worth of groups and a tile is cut at most once).  A tile
// cut by a run boundary gets two partial sums, added into y with fp32 atomics
// after k_gemm_zero_cut has zeroed it: two adds to zero commute, so the result
// does not depend on their order.  Runs are numbered XCD-major, so each XCD
// walks a contiguous stretch of tiles (one 256-row activation slab stays in its
// L2 while the XCDs stream the weight slabs).
__device__ __forceinline__ int64_t run_begin(int64_t total, int c, int G) { return total * c / G; }
__device__ __forceinline__ int run_index(int b, int G) {
  return (G & 7) == 0 ? (b & 7) * (G >> 3) + (b >> 3) : b;
}

__global__ __launch_bounds__(256) void k_gemm_zero_cut(float* __restrict__ y, int M, int N, int n_tiles, int ng,
                                                       int64_t total, int G) {
  const int c = blockIdx.x + 1;  // boundary between runs c - 1 and c
  const int64_t g = run_begin(total, c, G);
  if (g % ng == 0 || g >= total) return;  // on a tile edge: nothing cut
  const int t = (int)(g / ng);
  const int m0 = (t / n_tiles) * PBM, n0 = (t % n_tiles) * PBN;
  if ((N & 3) == 0 && ((uintptr_t)y & 15) == 0) {
    // 16-byte stores (n0 and N are multiples of 4, so a quad is all in or all out)
    for (int i = threadIdx.x; i < PBM * PBN / 4; i += 256) {
      const int m = m0 + i / (PBN / 4), n = n0 + 4 * (i % (PBN / 4));
      if (m < M && n < N) *(float4*)&y[(int64_t)m * N + n] = float4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    return;
  }
  for (int i = threadIdx.x; i < PBM * PBN; i += 256) {
    const int m = m0 + i / PBN, n = n0 + i % PBN;
    if (m < M && n < N) y[(int64_t)m * N + n] = 0.0f;
  }
}

__global__ __launch_bounds__(PTHREADS)
void k_gemm_i8_p256(const int8_t* __restrict__ xq, const float* __restrict__ dx, int M,
                    const int8_t* __restrict__ wq, const float* __restrict__ dw, int N, int K,
                    float* __restrict__ y, int n_tiles, int m_tiles) {
  __shared__ __attribute__((aligned(1024))) int8_t R0[RING_STAGE], R1[RING_STAGE], R2[RING_STAGE];
  // scales of four 256-blocks: rows 0..255 dx of the tile's A rows, rows
  // 256..383 dw of its B rows (one array: the only scale DMA target)
  __shared__ __attribute__((aligned(16))) float Sc[2][4][PBM + PBN];
  lds_i8* const ring[PST] = {(lds_i8*)R0, (lds_i8*)R1, (lds_i8*)R2};

  const int G = gridDim.x;
  const int ng = K / 1024, nkb = K / 256;
  const int64_t total = (int64_t)m_tiles * n_tiles * ng;
  const int c = run_index(blockIdx.x, G);
  const int64_t g_end = run_begin(total, c + 1, G);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // MFMA operand offsets (row r, 16-byte chunk c = 2 kk + lane / 32).
  const int l32 = lane & 31, lhi = lane >> 5;
  int aoff[2][4], boff[2][4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int ch = 2 * kk + lhi;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = wm * 64 + 32 * i + l32;
      aoff[i][kk] = r * PBK + ((ch ^ ((r >> 1) & 7)) << 4);
      const int rn = wn * 64 + 32 * i + l32;
      boff[i][kk] = RING_B + rn * PBK + ((ch ^ ((rn >> 1) & 7)) << 4);
    }
  }
  // This lane's scale-row bases (bytes) in slot 0; rows 4 lhi + 32 i + 8 q + t.
  const uint32_t xbase = lds_addr(&Sc[0][0][wm * 64 + 4 * lhi]);
  const uint32_t wbase = lds_addr(&Sc[0][0][PBM + wn * 64 + l32]);

  for (int64_t g = run_begin(total, c, G); g < g_end;) {
    // one tile's part: groups [ga, gb) of tile t
    const int t = (int)(g / ng);
    const int ga = (int)(g - (int64_t)t * ng);
    const int gb = (int)min((int64_t)ng, ga + (g_end - g));
    g += gb - ga;
    const bool whole = ga == 0 && gb == ng;
    const int mt = t / n_tiles, nt = t % n_tiles;
    const int m0 = mt * PBM, n0 = nt * PBN;
    const int nst = (gb - ga) * 8;      // 128-wide stages of this part
    const int kbase = ga * 1024;        // first K of this part
    const int ngroups = gb - ga;

    // the previous part's LDS reads are done before this part's DMA refills the ring
    wait_vmcnt_lgkm0<0>();
    ring_barrier();

    // DMA sources of this lane: wave w fills A rows 32 w + 8 j + lane / 8 (j < 4)
    // and B rows 16 w + 8 j + lane / 8 (j < 2), chunk lane % 8 (swizzled); rows
    // clamped into the matrix (clamped rows are computed and never stored).
    // (uniform tile bases plus 32-bit per-lane offsets: the tile spans at most
    // 256 rows of K bytes)
    const int8_t* const abase = xq + (int64_t)m0 * K + kbase;
    const int8_t* const bbase = wq + (int64_t)n0 * K + kbase;
    uint32_t aoff_g[4], boff_g[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 32 * wave + 8 * j + (lane >> 3);
      aoff_g[j] = (uint32_t)((min(m0 + r, M - 1) - m0) * K + (((lane & 7) ^ ((r >> 1) & 7)) << 4));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 16 * wave + 8 * j + (lane >> 3);
      boff_g[j] = (uint32_t)((min(n0 + r, N - 1) - n0) * K + (((lane & 7) ^ ((r >> 1) & 7)) << 4));
    }
    // scale rows: waves 0-3 carry dx rows 64 w + lane, waves 4-5 dw rows
    // 64 (w - 4) + lane, waves 6-7 repeat waves 4-5 (same bytes to the same place)
    // so that every wave issues the same loads without a branch.
    const bool sxw = wave < 4;
    const int srow = sxw ? 64 * wave + lane : 64 * (wave & 1) + lane;
    const float* ssrc = (sxw ? dx + (int64_t)min(m0 + srow, M - 1) * nkb : dw + (int64_t)min(n0 + srow, N - 1) * nkb) +
                        ga * 4;
    const int sdst = sxw ? 64 * wave : PBM + 64 * (wave & 1);
    auto issue_scales = [&](int gr) {  // group gr of this part (4 blocks, clamped) into slot gr & 1
      gr = min(gr, ngroups - 1);  // past the end: the last group again, same bytes
#pragma unroll
      for (int b = 0; b < 4; ++b)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(ssrc + 4 * gr + b),
                                         (__attribute__((address_space(3))) void*)&Sc[gr & 1][b][sdst], 4, 0, 0);
    };

    // Ring DMA of stage s (past the end: the last stage again, same count of
    // loads) into buffer R; the first PST - 1 stages are issued here, the rest
    // inside the stage asm.
    auto issue = [&](int s, lds_i8* R) {
      const int k0 = min(s, nst - 1) * PBK;
#pragma unroll
      for (int j = 0; j < 4; ++j) lds_dma16(abase + k0 + aoff_g[j], R + (4 * wave + j) * 1024);
#pragma unroll
      for (int j = 0; j < 2; ++j) lds_dma16(bbase + k0 + boff_g[j], R + RING_B + (2 * wave + j) * 1024);
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
    // Stage s from ring buffer R, issuing the DMA of stage s + PST - 1 into D.
    // Even stages open a 256-block (their first MFMAs start from zero); odd
    // stages close block kb = s / 2 and leave its scales in x0..w1, pw.
    v4i x0, x1, y0, y1, u0, u1, w0, w1;
    v2f pw;
    auto compute = [&](const lds_i8* R, auto last, const lds_i8* D, int s) {
      // named here so that the generic lambda captures them (asm operands alone do not)
      (void)acc, (void)x0, (void)x1, (void)y0, (void)y1, (void)u0, (void)u1, (void)w0, (void)w1, (void)pw;
      (void)aoff_g, (void)boff_g, (void)xbase, (void)wbase;
      const uint32_t rb = lds_addr(R);
      uint32_t pa[4], pb[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        pa[kk] = rb + aoff[0][kk];
        pb[kk] = rb + boff[0][kk];
      }
      const int k0 = min(s + PST - 1, nst - 1) * PBK;
      const int8_t* const sa = abase + k0;
      const int8_t* const sb = bbase + k0;
      const uint32_t db = lds_addr(D);
      uint32_t dm[6];
#pragma unroll
      for (int j = 0; j < 4; ++j) dm[j] = db + (4 * wave + j) * 1024;
#pragma unroll
      for (int j = 0; j < 2; ++j) dm[4 + j] = db + RING_B + (2 * wave + j) * 1024;
      if constexpr (decltype(last)::value) {
        const int kb = s >> 1;
        const uint32_t so = ((kb >> 2) & 1) * (4 * (PBM + PBN) * 4) + (kb & 3) * ((PBM + PBN) * 4);
        const uint32_t xa = xbase + so, wa = wbase + so;
        asm volatile(QG_STAGE_HEAD(QG_ACC4) QG_TAIL_LAST
                     : QG_OUTS, [pw] "=&v"(pw)
                     : QG_INS, [xa] "v"(xa), [wa] "v"(wa)
                     : "memory", "m0");
      } else {
        asm volatile(QG_STAGE_HEAD(QG_ZERO4) QG_TAIL_FIRST
                     : QG_OUTS
                     : QG_INS
                     : "memory", "m0");
      }
    };
    // After block kb's last stage (scales in the operand registers):
    // T = dx * dw * I into the fp32 sums.
    auto epilogue = [&]() {
      const v4f p[2][4] = {{__builtin_bit_cast(v4f, x0), __builtin_bit_cast(v4f, x1), __builtin_bit_cast(v4f, y0),
                            __builtin_bit_cast(v4f, y1)},
                           {__builtin_bit_cast(v4f, u0), __builtin_bit_cast(v4f, u1), __builtin_bit_cast(v4f, w0),
                            __builtin_bit_cast(v4f, w1)}};
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float sx = p[i][e >> 2][e & 3];
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            facc[i][j][e] = __builtin_fmaf(sx * pw[j], (float)acc[i][j][e], facc[i][j][e]);
          }
        }
    };

    // prologue: group 0's scales, stages 0 .. PST-2 in flight
    issue_scales(0);
#pragma unroll
    for (int s = 0; s < PST - 1; ++s) issue(s, ring[s]);
    // main loop, unrolled by 24 stages (ring of 3, scale groups of 8) so every
    // buffer and every scale load has a fixed place
    for (int s0 = 0; s0 < nst; s0 += 24) {
#pragma unroll
      for (int u = 0; u < 24; ++u) {
        const int s = s0 + u;
        if (s >= nst) break;  // the last pass may be partial (uniform)
        // this wave's part of stage s has landed and its reads of stage s-1 are done
        wait_vmcnt_lgkm0<(PST - 2) * 6>();
        ring_barrier();  // ... for every wave: stage s readable, stage s-1's buffer free
        // next group's scales: its slot was last read by the last stages of group
        // (s >> 3) - 1, all before this barrier
        if ((u & 7) == 0) issue_scales((s >> 3) + 1);
        if (u & 1) {
          compute(ring[u % PST], std::true_type{}, ring[(u + PST - 1) % PST], s);
          epilogue();
        } else {
          compute(ring[u % PST], std::false_type{}, ring[(u + PST - 1) % PST], s);
        }
      }
    }
    wait_vmcnt_lgkm0<0>();  // no DMA may still be landing when the part ends

    // a cut tile's partial sums are added (it was zeroed; two adds per entry)
    auto store = [&](auto atomic) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = n0 + wn * 64 + 32 * j + l32;
          if (n >= N) continue;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int m = m0 + wm * 64 + 32 * i + 8 * (e >> 2) + 4 * lhi + (e & 3);
            if (m < M) {
              if constexpr (decltype(atomic)::value) atomicAdd(&y[(int64_t)m * N + n], facc[i][j][e]);
              else y[(int64_t)m * N + n] = facc[i][j][e];
            }
          }
        }
    };
    if (whole) store(std::false_type{});
    else store(std::true_type{});
  }
}

hipError_t launch_gemm(const int8_t* xq, const float* dx, int M, const int8_t* wq, const float* dw, int N, int K,
                       int kblock, float* y, hipStream_t s) {
  // One scale per row of each operand (kblock = K): the plain int8 kernel.  The
  // wave tile is 128 x 128 unless narrower tiles take fewer rounds of
  // workgroups over the compute units for the same work (rounds x tile width).
  if (kblock == K && kblock != 32 && kblock != 256) {
    int cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return hipErrorInvalidDevice;
    const int mt = (M + 255) / 256;
    int best = 128;
    int64_t best_cost = INT64_MAX;
    for (const int wc : {128, 96, 80, 64}) {
      const int64_t tiles = (int64_t)mt * ((N + 2 * wc - 1) / (2 * wc));
      const int64_t cost = (tiles + cus - 1) / cus * wc;
      if (cost < best_cost) best_cost = cost, best = wc;
    }
    return launch_gemm_rs(xq, dx, M, wq, dw, N, K, best, y, s);
  }
  // 256-blocks, K a multiple of 1024 (scales in 16-byte groups of four blocks):
  // the pipelined kernel.
  if (kblock == 256 && K % 1024 == 0) {
    const int n_tiles = (N + PBN - 1) / PBN, m_tiles = (M + PBM - 1) / PBM;
    const int tiles = n_tiles * m_tiles;
    // one run per resident workgroup (one per CU: the ring fills its LDS), at most
    // one per tile; a multiple of 8 so runs can be numbered XCD-major
    const int S = resident_workgroups((const void*)k_gemm_i8_p256, PTHREADS);
    if (S <= 0) return hipErrorInvalidDevice;
    // Whole tiles, one workgroup each, unless the last round would leave more
    // than a quarter of the rounds' time idle: then runs of equal length, one per
    // slot (the idle tail of a short last round is cheaper than cutting tiles:
    // with few CUs busy the clock rises).
    const int rounds = (tiles + S - 1) / S;
    const bool even_runs = tiles > S && 4 * ((int64_t)rounds * S - tiles) > (int64_t)rounds * S;
    const int G = even_runs ? (S >= 8 ? S & ~7 : S) : tiles;
    const int ng = K / 1024;
    const int64_t total = (int64_t)tiles * ng;
    if (G > 1) hipLaunchKernelGGL(k_gemm_zero_cut, dim3(G - 1), dim3(256), 0, s, y, M, N, n_tiles, ng, total, G);
    hipLaunchKernelGGL(k_gemm_i8_p256, dim3(G), dim3(PTHREADS), 0, s, xq, dx, M, wq, dw, N, K, y, n_tiles, m_tiles);
    return hipGetLastError();
  }
  // Other shapes: 64 x 256 workgroup tiles for up to 64 rows (small batches),
  // else 128 x 128.
  const dim3 block(256);
  if (M <= 64) {
    const dim3 grid((N + 255) / 256, 1);
    if (kblock == 256) hipLaunchKernelGGL((k_gemm_i8<256, 1>), grid, block, 0, s, xq, dx, M, wq, dw, N, K, y);
    else hipLaunchKernelGGL((k_gemm_i8<32, 1>), grid, block, 0, s, xq, dx, M, wq, dw, N, K, y);
  } else {
    const dim3 grid((N + 127) / 128, (M + 127) / 128);
    if (kblock == 256) hipLaunchKernelGGL((k_gemm_i8<256, 2>), grid, block, 0, s, xq, dx, M, wq, dw, N, K, y);
    else hipLaunchKernelGGL((k_gemm_i8<32, 2>), grid, block, 0, s, xq, dx, M, wq, dw, N, K, y);
  }
  return hipGetLastError();
}

}  // namespace qk
