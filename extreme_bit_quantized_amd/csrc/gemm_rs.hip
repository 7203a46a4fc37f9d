// gemm_rs.hip — int8 GEMM with one scale per row of each operand, on the gfx950
// matrix cores:
//
//   y[m][n] = dx[m] * dw[n] * I[m][n],   I = exact int32 dot of xq[m] and wq[n]
//
// (the int8 GEMM the pages' prefill runs: activations quantized per token after
// the rotation, weights per output row, the scales applied once to the int32
// result).  Without a scale per K-block nothing but the matrix cores touches
// the accumulators until the tile's last K step, so the design is a plain
// dense int8 GEMM:
//
// - Workgroup tile 256 (M) x 2 WC (N), 4 waves (one per SIMD) in 2 x 2, each a
//   128 x WC tile of v_mfma_i32_16x16x64_i8 tiles (8 x WC/16 accumulators of 4
//   int32 per lane: 256 registers at WC = 128, held in the accumulation
//   registers).  The large wave tile keeps LDS reads at 1/WC + 1/128 bytes per
//   multiply-add.
// - Operands reach LDS by LDS DMA (global_load_lds_dwordx4: 1 KB per
//   instruction), a row's 16-byte chunks XOR-swizzled so the 16 lanes of an
//   operand read phase (16 consecutive rows, one chunk) hit 16 different
//   16-byte slots modulo 256 bytes (conflict free).  Every wave issues the same
//   number of DMA instructions per stage, so "stage s has landed" is a fixed
//   vmcnt, and a plain s_barrier orders the ring.
// - K a multiple of 128 (k_gemm_i8_rs128): 128-byte stages (whole 128-byte
//   lines per row: the DMA path moves about 1.6x the bytes per second it moves
//   with 64-byte rows), A in a ring of 3 slots and B in one of 2, so A's DMAs for
//   stage s + 2 go out one per MFMA group during the first K-step of stage s and
//   B's during the second: a K-step that issued all of a stage's DMAs ran
//   ~1.45x as long as one that issued none (the texture path backs up and stalls
//   the wave, whose matrix core then idles).
// - Other K (k_gemm_i8_rs64): 64-byte stages in one ring of up to 6 slots.
// - The operands of the next K-step are read from LDS while this one's MFMAs run.
// - One workgroup per tile; blocks go round robin to the 8 XCDs, and block b is
//   given the tile that keeps each XCD on one contiguous stretch of an M-fastest
//   tile order: an XCD's resident workgroups then cover all M tiles of a few
//   adjacent N tiles, so each activation and weight K-slice they share is
//   fetched into that XCD's L2 about once per round.
// - Epilogue: the row and column scales are loaded and waited for before the
//   first store (a wait for a load is a wait on the store counter too, so loads
//   interleaved with the stores serialized them: 1.5x the epilogue time).
#include <algorithm>
#include <type_traits>

#include "internal.hpp"

namespace qk {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) int8_t lds_i8;

constexpr int RS_TM = 256;  // workgroup rows

// 64-byte stages (any K a multiple of 64).  SK: K bytes per ring stage.  An LDS
// row holds SK bytes as SK / 16 chunks of 16 bytes, chunk c of row r stored at
// slot c ^ ((r / (256 / SK)) % (SK / 16)): the 16 lanes of an operand read phase
// (16 consecutive rows, one chunk) then hit 16 different 16-byte slots modulo
// 256 bytes.  One DMA instruction lands 1 KB = 1024 / SK rows.
template <int WC, int SK>
struct RsCfg {
  static constexpr int TN = 2 * WC;                    // workgroup columns
  static constexpr int NI = 128 / 16, NJ = WC / 16;    // MFMA tiles of a wave
  static constexpr int HALVES = SK / 64;               // MFMA K-steps per stage
  static constexpr int CH = SK / 16;                   // chunks per row
  static constexpr int RPI = 1024 / SK;                // rows per DMA instruction
  static constexpr int RPW = 256 / SK;                 // rows per 256-byte window
  static constexpr int A_BYTES = RS_TM * SK;
  static constexpr int B_BYTES = TN * SK;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int NST = (144 * 1024) / STAGE < 6 ? (144 * 1024) / STAGE : 6;  // ring stages
  static constexpr int DA = RS_TM / RPI / 4;           // A DMA instructions per wave and stage
  static constexpr int DB = (TN / RPI + 3) / 4;        // B DMA instructions per wave and stage
  static constexpr int D = DA + DB;
  static constexpr int PER = (D + NI - 1) / NI;        // DMA instructions per MFMA group
  static_assert(WC % 16 == 0 && WC <= 128, "wave tile");
  static_assert(NST >= 2 && NST * STAGE <= 144 * 1024, "LDS");
  static_assert((NST - 1) * D < 64, "vmcnt range");
};

// LDS DMA of 16 bytes per lane from base + off (base uniform, off a 32-bit lane
// offset) to LDS address lds + 16 * lane (lds uniform, via M0; an SALU write of
// M0 needs one wait state before the DMA reads it).  Not tracked by the
// compiler's wait counting: the kernel waits for it explicitly.  It writes no
// register, so nothing the compiler allocates can be overwritten in flight.
__device__ __forceinline__ void dma16(const int8_t* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %[m]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[v], %[b]"
               :
               : [m] "s"(lds), [v] "v"(off), [b] "s"(base)
               : "memory", "m0");
}
// s_waitcnt vmcnt(n) (n < 64), lgkmcnt and expcnt left alone
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Workgroup barrier the compiler may not move memory accesses across and that
// adds no wait of its own.
__device__ __forceinline__ void rs_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Tile of block b: XCD x = b % 8 holds blocks x, x + 8, ...; its j-th block takes
// position L = (blocks on XCDs before x) + j of the M-fastest tile order.
__device__ __forceinline__ void rs_tile(int b, int T, int m_tiles, int& mt, int& nt) {
  const int x = b & 7, j = b >> 3, q = T >> 3, r = T & 7;
  const int L = x * q + min(x, r) + j;
  mt = L % m_tiles;
  nt = L / m_tiles;
}

// Loads the scales of a lane's outputs, has them all in registers, then stores
// y = dx[m] dw[n] I: lane holds rows wm*128 + 16 i + 4 (l / 16) + e, column
// wn*WC + 16 j + l % 16 of the tile at (m0, n0).  Called with no DMA in flight,
// right after the last MFMAs.  The compiler does not see the latency of the
// MFMAs (asm), so the wait states before their results are read are explicit,
// and every accumulator passes through an empty asm after them: otherwise the
// copies out of the accumulation registers may be scheduled right behind the
// MFMA that writes them, before its result is there.
template <int NI, int NJ, int WC>
__device__ __forceinline__ void rs_epilogue(v4i (&acc)[NI][NJ], const float* __restrict__ dx,
                                            const float* __restrict__ dw, float* __restrict__ y, int M, int N,
                                            int m0, int n0, int wm, int wn, int lr, int lc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) asm volatile("" : "+a"(acc[i][j]));
  float sx[NI][4], swv[NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) sx[i][e] = dx[min(m0 + wm * 128 + 16 * i + 4 * lc + e, M - 1)];
#pragma unroll
  for (int j = 0; j < NJ; ++j) swv[j] = dw[min(n0 + wn * WC + 16 * j + lr, N - 1)];
  // every scale in a register here (else the compiler sinks loads into the
  // per-row store branches, between stores)
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(sx[i][e]));
#pragma unroll
  for (int j = 0; j < NJ; ++j) asm volatile("" : "+v"(swv[j]));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = m0 + wm * 128 + 16 * i + 4 * lc + e;
      if (m >= M) continue;
      float* const yr = y + (int64_t)m * N;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int n = n0 + wn * WC + 16 * j + lr;
        if (n < N) yr[n] = (sx[i][e] * swv[j]) * (float)acc[i][j][e];
      }
    }
}

template <int WC>
__global__ __launch_bounds__(256, 1) void k_gemm_i8_rs64(const int8_t* __restrict__ xq, const float* __restrict__ dx,
                                                         int M, const int8_t* __restrict__ wq,
                                                         const float* __restrict__ dw, int N, int K,
                                                         float* __restrict__ y, int m_tiles, int n_tiles) {
  constexpr int SK = 64;
  using C = RsCfg<WC, SK>;
  __shared__ __attribute__((aligned(1024))) int8_t ring_mem[C::NST * C::STAGE];
  lds_i8* const ring = (lds_i8*)ring_mem;
  typedef const __attribute__((address_space(3))) v4i lds_v4i;

  int mt, nt;
  rs_tile(blockIdx.x, m_tiles * n_tiles, m_tiles, mt, nt);
  const int m0 = mt * RS_TM, n0 = nt * C::TN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // DMA i of a wave (i < DA: A instruction DA * wave + i; else B instruction
  // DB * wave + i - DA, the last one repeated where the count does not divide:
  // same bytes to the same place) covers rows RPI j .. RPI j + RPI - 1; lane l
  // brings row RPI j + l / CH into slot l % CH, i.e. chunk (l % CH) ^ f(row).
  // Rows past the matrix are clamped to its last row (computed, never stored).
  const int8_t* const abase = xq + (int64_t)m0 * K;
  const int8_t* const bbase = wq + (int64_t)n0 * K;
  const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;
  uint32_t off[C::D], dst[C::D];
#pragma unroll
  for (int i = 0; i < C::D; ++i) {
    const bool a = i < C::DA;
    const int j = a ? C::DA * wave + i : min(C::DB * wave + i - C::DA, C::TN / C::RPI - 1);
    const int r = C::RPI * j + lane / C::CH;
    const int c = (lane % C::CH) ^ ((r / C::RPW) % C::CH);
    off[i] = (uint32_t)(((a ? min(m0 + r, M - 1) - m0 : min(n0 + r, N - 1) - n0)) * K + 16 * c);
    dst[i] = (uint32_t)((a ? 0 : C::A_BYTES) + 1024 * j);
  }
  const int nst = K / SK;
  auto dma = [&](int s, int i) {  // DMA i of stage s (past the end: the last stage again) into its slot
    const int k0 = min(s, nst - 1) * SK;
    dma16((i < C::DA ? abase : bbase) + k0, off[i], ring_lds + (uint32_t)((s % C::NST) * C::STAGE) + dst[i]);
  };

  // Operand reads of K-step h of a stage: A tile i = rows wm*128 + 16 i + l % 16,
  // chunk 4 h + l / 16; B alike.
  const int lr = lane & 15, lc = lane >> 4;
  int a_lane[C::HALVES], b_lane[C::HALVES];
#pragma unroll
  for (int h = 0; h < C::HALVES; ++h) {
    const int sw = ((4 * h + lc) ^ ((lr / C::RPW) % C::CH)) << 4;
    a_lane[h] = (wm * 128 + lr) * SK + sw;
    b_lane[h] = C::A_BYTES + (wn * WC + lr) * SK + sw;
  }
  v4i fa[2][C::NI], fb[2][C::NJ];
  v4i acc[C::NI][C::NJ];
#pragma unroll
  for (int i = 0; i < C::NI; ++i)
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  // Prologue: stages 0 .. NST-1 in flight, stage 0 landed everywhere, its first
  // K-step's operands read.
  for (int s = 0; s < C::NST; ++s)
#pragma unroll
    for (int i = 0; i < C::D; ++i) dma(s, i);
  wait_vm<(C::NST - 1) * C::D>();
  rs_barrier();
#pragma unroll
  for (int i = 0; i < C::NI; ++i) fa[0][i] = *(lds_v4i*)(ring + a_lane[0] + 16 * SK * i);
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) fb[0][j] = *(lds_v4i*)(ring + b_lane[0] + 16 * SK * j);
  wait_lgkm0();

  // K-step h of stage s (operands in set cur): read the next K-step's
  // operands into the other set and run this one's MFMAs.  Before a stage's last
  // K-step: wait for this wave's DMAs of stage s + 1, then a barrier (everyone's
  // have landed, and everyone has read stage s, whose slot is refilled with
  // stage s + NST during this K-step).  With one wave per SIMD any stall of the
  // wave idles its matrix core, so the K-step is cut into 8 groups (one A tile
  // each: its WC/16 MFMAs), each also issuing at most two operand reads and PER
  // DMAs: the LDS and texture queues drain while the MFMAs run instead of
  // stalling the wave up front.  The MFMAs are asm with the accumulators in the
  // accumulation registers ("a"): with the builtin the register allocator moved
  // accumulators between register files inside the loop.  The compiler does
  // not see their latency, so the epilogue waits for the last results
  // explicitly.  The loop is unrolled by two K-steps (one per stage) so the
  // operand sets alternate at fixed registers.
  auto kstep = [&](int s, auto h_c, auto cur_c) {
    constexpr int h = decltype(h_c)::value, cur = decltype(cur_c)::value;
    constexpr bool last = h == C::HALVES - 1;
    if constexpr (last) {
      wait_vm<(C::NST - 2) * C::D>();
      rs_barrier();
    }
    // next K-step: (s, h + 1), or (s + 1, 0) (past the end: unused data)
    constexpr int nh = last ? 0 : h + 1;
    const lds_i8* const Rr = ring + ((last ? s + 1 : s) % C::NST) * C::STAGE;
#pragma unroll
    for (int g = 0; g < C::NI; ++g) {
      fa[cur ^ 1][g] = *(lds_v4i*)(Rr + a_lane[nh] + 16 * SK * g);
      if (g < C::NJ) fb[cur ^ 1][g] = *(lds_v4i*)(Rr + b_lane[nh] + 16 * SK * g);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (last) {
#pragma unroll
        for (int q = 0; q < C::PER; ++q)
          if (C::PER * g + q < C::D) dma(s + C::NST, C::PER * g + q);
      }
#pragma unroll
      for (int j = 0; j < C::NJ; ++j)
        asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc[g][j]) : "v"(fa[cur][g]), "v"(fb[cur][j]));
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_lgkm0();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  static_assert(C::HALVES == 1, "one K-step per stage");
  int s = 0;
  for (; s + 1 < nst; s += 2) {
    kstep(s, I0{}, I0{});
    kstep(s + 1, I0{}, I1{});
  }
  if (s < nst) kstep(s, I0{}, I0{});
  wait_vm<0>();  // no DMA in flight past the loop
  rs_epilogue<C::NI, C::NJ, WC>(acc, dx, dw, y, M, N, m0, n0, wm, wn, lr, lc);
}

// 128-byte stages (K a multiple of 128).  A slot holds 256 A rows or TN B rows of
// 128 bytes, chunk c of row r at slot c ^ ((r / 2) % 8); one DMA instruction
// lands 8 rows.  A has 3 slots and B 2: A(s + 2) goes into the slot of stage
// s - 1 during the first K-step of stage s, B(s + 2) into the slot of stage s
// during the second (after the barrier that ends every wave's reads of it).
template <int WC>
struct Rs128Cfg {
  static constexpr int SK = 128, TN = 2 * WC;
  static constexpr int NI = 128 / 16, NJ = WC / 16;
  static constexpr int A_BYTES = RS_TM * SK, B_BYTES = TN * SK;  // one slot
  static constexpr int NSA = 3, NSB = 2;
  static constexpr int LDS = NSA * A_BYTES + NSB * B_BYTES;
  static constexpr int DA = RS_TM / 8 / 4, DB = TN / 8 / 4;  // DMA instructions per wave and stage
  static_assert(WC % 16 == 0 && WC <= 128 && TN % 32 == 0, "wave tile");
  static_assert(DA <= NI && DB <= NI, "at most one DMA per MFMA group");
  static_assert(LDS <= 160 * 1024, "LDS");
};

template <int WC>
__global__ __launch_bounds__(256, 1) void k_gemm_i8_rs128(const int8_t* __restrict__ xq,
                                                          const float* __restrict__ dx, int M,
                                                          const int8_t* __restrict__ wq,
                                                          const float* __restrict__ dw, int N, int K,
                                                          float* __restrict__ y, int m_tiles, int n_tiles) {
  using C = Rs128Cfg<WC>;
  __shared__ __attribute__((aligned(1024))) int8_t ring_mem[C::LDS];
  lds_i8* const ring_a = (lds_i8*)ring_mem;
  lds_i8* const ring_b = ring_a + C::NSA * C::A_BYTES;
  typedef const __attribute__((address_space(3))) v4i lds_v4i;

  int mt, nt;
  rs_tile(blockIdx.x, m_tiles * n_tiles, m_tiles, mt, nt);
  const int m0 = mt * RS_TM, n0 = nt * C::TN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // A DMA i of a wave covers slot rows 8 j .. 8 j + 7, j = DA * wave + i (B:
  // DB * wave + i); lane l brings row 8 j + l / 8 into slot l % 8, i.e. chunk
  // (l % 8) ^ ((row / 2) % 8).  Rows past the matrix are clamped to its last row
  // (computed, never stored).
  const int8_t* const abase = xq + (int64_t)m0 * K;
  const int8_t* const bbase = wq + (int64_t)n0 * K;
  const uint32_t lds_a = (uint32_t)(uintptr_t)ring_a, lds_b = (uint32_t)(uintptr_t)ring_b;
  const int lrow = lane >> 3, lslot = lane & 7;
  uint32_t off_a[C::DA], off_b[C::DB];
#pragma unroll
  for (int i = 0; i < C::DA; ++i) {
    const int r = 8 * (C::DA * wave + i) + lrow;
    off_a[i] = (uint32_t)((min(m0 + r, M - 1) - m0) * K + 16 * (lslot ^ ((r >> 1) & 7)));
  }
#pragma unroll
  for (int i = 0; i < C::DB; ++i) {
    const int r = 8 * (C::DB * wave + i) + lrow;
    off_b[i] = (uint32_t)((min(n0 + r, N - 1) - n0) * K + 16 * (lslot ^ ((r >> 1) & 7)));
  }
  auto dma_a = [&](int s, int i) {
    dma16(abase + (int64_t)s * C::SK, off_a[i],
          lds_a + (uint32_t)((s % C::NSA) * C::A_BYTES + 1024 * (C::DA * wave + i)));
  };
  auto dma_b = [&](int s, int i) {
    dma16(bbase + (int64_t)s * C::SK, off_b[i],
          lds_b + (uint32_t)((s & 1) * C::B_BYTES + 1024 * (C::DB * wave + i)));
  };

  // Operand reads of K-step h: A tile g = slot rows wm*128 + 16 g + l % 16,
  // chunk 4 h + l / 16 (B alike); the swizzle term depends on l % 16 only.
  const int lr = lane & 15, lc = lane >> 4;
  int a_lane[2], b_lane[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int sw = ((4 * h + lc) ^ ((lr >> 1) & 7)) << 4;
    a_lane[h] = (wm * 128 + lr) * C::SK + sw;
    b_lane[h] = (wn * WC + lr) * C::SK + sw;
  }
  v4i fa[2][C::NI], fb[2][C::NJ];
  v4i acc[C::NI][C::NJ];
#pragma unroll
  for (int i = 0; i < C::NI; ++i)
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  // Prologue: stages 0 and 1 in flight (this wave's DMAs in issue order A0 B0
  // A1 B1), stage 0 landed everywhere, its first K-step's operands read.
  const int nst = K / C::SK;
#pragma unroll
  for (int i = 0; i < C::DA; ++i) dma_a(0, i);
#pragma unroll
  for (int i = 0; i < C::DB; ++i) dma_b(0, i);
  if (nst > 1) {
#pragma unroll
    for (int i = 0; i < C::DA; ++i) dma_a(1, i);
#pragma unroll
    for (int i = 0; i < C::DB; ++i) dma_b(1, i);
    wait_vm<C::DA + C::DB>();
  } else {
    wait_vm<0>();
  }
  rs_barrier();
#pragma unroll
  for (int i = 0; i < C::NI; ++i) fa[0][i] = *(lds_v4i*)(ring_a + a_lane[0] + 2048 * i);
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) fb[0][j] = *(lds_v4i*)(ring_b + b_lane[0] + 2048 * j);
  wait_lgkm0();

  // K-step h of stage s, operands in set h: read the next K-step's operands
  // ((s, 1), or (s + 1, 0)) into set h ^ 1 while this one's MFMAs run, in 8
  // groups (one A tile each: its WC/16 MFMAs) that each also issue at most one
  // operand read of each kind and one DMA.  Modes: FULL issues A(s + 2) in
  // K-step 0 and B(s + 2) in K-step 1; before K-step 1 it waits for stage s + 1
  // (in flight after it in issue order: A(s + 2) only) and a barrier.  NODMA
  // (s = nst - 2) issues nothing and waits for everything; LAST (s = nst - 1)
  // issues nothing, and its K-step 1 neither waits nor reads.  The MFMAs are
  // asm with the accumulators in the accumulation registers ("a"): with the
  // builtin the register allocator moved accumulators between register files
  // inside the loop.
  constexpr int FULL = 0, NODMA = 1, LAST = 2;
  auto kstep = [&](int s, auto h_c, auto mode_c) {
    constexpr int h = decltype(h_c)::value, mode = decltype(mode_c)::value;
    constexpr int nh = h ^ 1;
    constexpr bool reads = !(h == 1 && mode == LAST);
    if constexpr (h == 1 && mode != LAST) {
      if constexpr (mode == FULL) wait_vm<C::DA>();
      else wait_vm<0>();
      rs_barrier();
    }
    const int sn = h == 0 ? s : s + 1;
    const lds_i8* const ra = ring_a + (sn % C::NSA) * C::A_BYTES;
    const lds_i8* const rb = ring_b + (sn & 1) * C::B_BYTES;
#pragma unroll
    for (int g = 0; g < C::NI; ++g) {
      if constexpr (reads) {
        fa[nh][g] = *(lds_v4i*)(ra + a_lane[nh] + 2048 * g);
        if (g < C::NJ) fb[nh][g] = *(lds_v4i*)(rb + b_lane[nh] + 2048 * g);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (mode == FULL) {
        if constexpr (h == 0) {
          if (g < C::DA) dma_a(s + 2, g);
        } else {
          if (g < C::DB) dma_b(s + 2, g);
        }
      }
#pragma unroll
      for (int j = 0; j < C::NJ; ++j)
        asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc[g][j]) : "v"(fa[h][g]), "v"(fb[h][j]));
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (reads) wait_lgkm0();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using MF = std::integral_constant<int, FULL>;
  using MN = std::integral_constant<int, NODMA>;
  using ML = std::integral_constant<int, LAST>;
  for (int s = 0; s < nst - 2; ++s) {
    kstep(s, I0{}, MF{});
    kstep(s, I1{}, MF{});
  }
  if (nst >= 2) {
    kstep(nst - 2, I0{}, MN{});
    kstep(nst - 2, I1{}, MN{});
  }
  kstep(nst - 1, I0{}, ML{});
  kstep(nst - 1, I1{}, ML{});
  rs_epilogue<C::NI, C::NJ, WC>(acc, dx, dw, y, M, N, m0, n0, wm, wn, lr, lc);
}

template <int WC>
hipError_t launch_rs(const int8_t* xq, const float* dx, int M, const int8_t* wq, const float* dw, int N, int K,
                     float* y, hipStream_t s) {
  const int m_tiles = (M + RS_TM - 1) / RS_TM, n_tiles = (N + 2 * WC - 1) / (2 * WC);
  if (K % 128 == 0)
    hipLaunchKernelGGL((k_gemm_i8_rs128<WC>), dim3(m_tiles * n_tiles), dim3(256), 0, s, xq, dx, M, wq, dw, N, K, y,
                       m_tiles, n_tiles);
  else
    hipLaunchKernelGGL((k_gemm_i8_rs64<WC>), dim3(m_tiles * n_tiles), dim3(256), 0, s, xq, dx, M, wq, dw, N, K, y,
                       m_tiles, n_tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_rs(const int8_t* xq, const float* dx, int M, const int8_t* wq, const float* dw, int N,
                          int K, int wc, float* y, hipStream_t s) {
  switch (wc) {
    case 128: return launch_rs<128>(xq, dx, M, wq, dw, N, K, y, s);
    case 96: return launch_rs<96>(xq, dx, M, wq, dw, N, K, y, s);
    case 80: return launch_rs<80>(xq, dx, M, wq, dw, N, K, y, s);
    case 64: return launch_rs<64>(xq, dx, M, wq, dw, N, K, y, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace qk
