// gemv_mfma.hpp — GEMV for 9..64 tokens over packed low-bit weights on the
// matrix cores.
//
// The DPP GEMV (gemv_impl.hpp) spends every dot product on the vector ALUs, so
// its cost grows with the token count; past 8 tokens it re-reads the weights
// once per 8 tokens.  Here each 32-weight block of a row is decoded once into
// signed int8 levels and multiplied against all tokens on the matrix cores:
// v_mfma_i32_16x16x32_i8 with the activations as A (16 tokens x 32 k) and the
// weights as B (32 k x 16 rows) gives the exact int32 block dot I of 16 tokens
// x 16 rows per instruction, so one block is one MFMA per (16 rows, 16 tokens).
//
// Work unit: one wave owns 64 weight rows (four 16-row groups) and all tokens
// (TG groups of 16).  Per 32-weight block:
//   1. decode (lane = row): the lane's row codes -> 8 dwords of signed int8
//      levels (TERN t, INT2 2c-3, SIGN1 2b-1, INT4 2c-15, TRELLIS V8[h]);
//   2. LDS transpose: the 8 dwords go to one of this wave's 2 KB buffers as two
//      16-byte halves (dwords 0..3 at row*16, 4..7 at 1024 + row*16), and lane
//      l reads its B operand, dwords 2j and 2j+1 of row 16G + l%16 (j = l/16),
//      with one 8-byte read per row group; writes (16 lanes per phase, 16 B
//      each) and reads (32 lanes per phase, 8 B each) both cover the 64 banks
//      once, and a wave's LDS operations complete in order, so no wait is
//      needed between its own write and read (two buffers, by block parity,
//      let a block's reads trail the next block's write);
//   3. A operand of token group tg: lane l holds token 16tg + l%16, k = 8j..8j+7
//      of the block (INT2 and SIGN1: rebuilt from the 4-bit activation planes,
//      k in the order 0,2,4,6,1,3,5,7 of each 8-group, which is also the order
//      their code planes give);
//   4. per (row group, token group) one MFMA; C lane l holds weight row
//      16G + l%16 and tokens 4j + i (i = 0..3) of the group;
//   5. epilogue: t = cvt(I) and acc += t * d[token][block], the activation
//      scale arriving by a DPP row broadcast: the d register of a token group
//      holds, in lane 4b + i of 16-lane row j, d of token 4j + i and block
//      kb0 + b of the current quad of blocks, so row_newbcast:(4b + i) gives
//      each lane exactly its element's d;  at the end of a weight-scale block
//      y += s * acc (s of the lane's row).  I is exact; the fp32 sums follow
//      the same terms as the definition in another order.
#pragma once

#include "gemv_impl.hpp"

namespace qk {

typedef int32_t v4i32 __attribute__((ext_vector_type(4)));

// Byte lookup: result byte k = byte sel_k of tab (sel bytes 0..3).
__device__ __forceinline__ uint32_t lut4(uint32_t tab, uint32_t sel) { return __builtin_amdgcn_perm(0u, tab, sel); }

// Bytes of one sub-chunk (256 weights) of a packed row, and of one 32-block.
template <int FMT> struct MGeo;
template <> struct MGeo<QFMT_SIGN1> { static constexpr int SUBB = 32, BLKB = 4; };
template <> struct MGeo<QFMT_INT2> { static constexpr int SUBB = 64, BLKB = 8; };
template <> struct MGeo<QFMT_INT4> { static constexpr int SUBB = 128, BLKB = 16; };
template <> struct MGeo<QFMT_TERN_B3> { static constexpr int SUBB = 52, BLKB = 0; };
template <> struct MGeo<QFMT_TRELLIS2> { static constexpr int SUBB = 64, BLKB = 8; };

// ---- decoders: the lane's row codes of one sub-chunk -> per block 8 level dwords -------------------
// Each calls f(integral_constant<kb>, p) for the 8 blocks kb of the sub-chunk,
// in order.  (Blocks past the end of K decode whatever codes stand there; the
// caller gives them d = 0, so they add exact zeros.)

template <typename F>
__device__ __forceinline__ void mdec_sign1(const uint32_t (&T)[8], F&& f) {
  const uint32_t tab = sgpr_const(0x000001FFu);  // bit 0 -> -1, 1 -> +1
  const uint32_t m = sgpr_const(0x01010101u);
  static_for(std::make_integer_sequence<int, 8>{}, [&](auto kc) {
    const uint32_t W = T[decltype(kc)::value];
    uint32_t p[8];
    // weight 8j + n is bit 4n + j: bits 8b + j hold weights 8j + 2b, bits
    // 8b + 4 + j weights 8j + 2b + 1
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[2 * j] = lut4(tab, (W >> j) & m);
      p[2 * j + 1] = lut4(tab, (W >> (j + 4)) & m);
    }
    f(kc, p);
  });
}

template <typename F>
__device__ __forceinline__ void mdec_int2(const uint32_t (&T)[16], F&& f) {
  const uint32_t tab = sgpr_const(0x0301FFFDu);  // c -> 2c - 3
  const uint32_t m = sgpr_const(0x03030303u);
  static_for(std::make_integer_sequence<int, 8>{}, [&](auto kc) {
    constexpr int kb = decltype(kc)::value;
    uint32_t p[8];
    // weight 8j' + n of a 16-weight word is bits 4n + 2j' .. +1: bits 8b + 2j'
    // hold weights 8j' + 2b, bits 8b + 4 + 2j' weights 8j' + 2b + 1
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t W = T[2 * kb + (j >> 1)];
      const int sh = 2 * (j & 1);
      p[2 * j] = lut4(tab, (W >> sh) & m);
      p[2 * j + 1] = lut4(tab, (W >> (sh + 4)) & m);
    }
    f(kc, p);
  });
}

template <typename F>
__device__ __forceinline__ void mdec_int4(const uint32_t (&T)[32], F&& f) {
  const uint32_t m = sgpr_const(0x1E1E1E1Eu), hi = sgpr_const(0x80808080u), off = sgpr_const(0x0F0F0F0Fu);
  static_for(std::make_integer_sequence<int, 8>{}, [&](auto kc) {
    constexpr int kb = decltype(kc)::value;
    uint32_t p[8];
    // word j of the block: weight 8j + 4h + b in bits 8b + 4h .. +3.  Level
    // 2c - 15 per byte: (2c + 0x80 - 15) ^ 0x80, no borrow since 2c + 0x80 >= 0x80.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t W = T[4 * kb + j];
      p[2 * j] = ((((W << 1) & m) | hi) - off) ^ hi;
      p[2 * j + 1] = ((((W >> 3) & m) | hi) - off) ^ hi;
    }
    f(kc, p);
  });
}

// Ternary: 13 words; the digits of dword g (weights 4g .. 4g+3) come out in
// order g = 5m + i (word m < 12, digit i) and 60 + i (word 12), block kb ending
// with dword 8kb + 7.  Digit values 0, 1, 2 become the trits -1, 0, 1.
template <typename F>
__device__ __forceinline__ void mdec_tern(const uint32_t (&T)[13], F&& f) {
  const uint32_t tab = sgpr_const(0x000100FFu);
  const uint32_t m = sgpr_const(0x00FF00FFu);
  uint32_t p[8];
  static_for(std::make_integer_sequence<int, 13>{}, [&](auto mc) {
    constexpr int mw = decltype(mc)::value;
    const uint32_t W = T[mw];
    uint32_t xl = W & m, xh = (W >> 8) & m;
    constexpr int ndig = mw < 12 ? 5 : 4;
    static_for(std::make_integer_sequence<int, ndig>{}, [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const uint32_t yl = xl * 3u, yh = xh * 3u;
      constexpr int g = mw < 12 ? 5 * mw + i : 60 + i;
      p[g & 7] = lut4(tab, __builtin_amdgcn_perm(yh, yl, 0x07030501u));
      if constexpr (i + 1 < ndig) {
        xl = yl & m;
        xh = yh & m;
      }
      if constexpr ((g & 7) == 7) f(std::integral_constant<int, (g >> 3)>{}, p);
    });
  });
}

// Trellis: prev = the 16 bits of seed||bytes before the sub-chunk; the state of
// each weight is the 16-bit window ending at its symbol.
template <typename F>
__device__ __forceinline__ void mdec_trellis(const uint32_t (&T)[16], uint32_t& prev, const int8_t* v8, F&& f) {
  static_for(std::make_integer_sequence<int, 8>{}, [&](auto kc) {
    constexpr int kb = decltype(kc)::value;
    uint32_t p[8];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const uint32_t W = T[2 * kb + w];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const uint32_t w24 = (prev << 8) | ((W >> (8 * q4)) & 0xFFu);
        uint32_t L = 0;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const uint32_t st = (w24 >> (6 - 2 * jj)) & 0xFFFFu;
          const uint32_t h = ((st * 0x9E37u) ^ (st >> 7)) & 0xFFu;
          L |= ((uint32_t)(uint8_t)v8[h]) << (8 * jj);
        }
        prev = w24 & 0xFFFFu;
        p[w * 4 + q4] = L;
      }
    }
    f(kc, p);
  });
}

// acc[i] += d_i * t[i] (MUL: acc[i] = d_i * t[i]) for i = 0..3, d_i lane
// B4 + i of the lane's 16-lane row of the d register.  DPP reads d from other
// lanes, so this runs with the whole wave active; the leading nop keeps the
// two wait states a DPP source needs after a VALU write of d.
template <int B4, bool MUL>
__device__ __forceinline__ void fma_bcast4(float (&acc)[4], float d, const float (&t)[4]) {
  if constexpr (MUL)
    asm("s_nop 1\n\t"
        "v_mul_f32_dpp %0, %4, %5 row_newbcast:%c9 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %4, %6 row_newbcast:%c10 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %2, %4, %7 row_newbcast:%c11 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %3, %4, %8 row_newbcast:%c12 row_mask:0xf bank_mask:0xf"
        : "=&v"(acc[0]), "=&v"(acc[1]), "=&v"(acc[2]), "=&v"(acc[3])
        : "v"(d), "v"(t[0]), "v"(t[1]), "v"(t[2]), "v"(t[3]), "n"(B4), "n"(B4 + 1), "n"(B4 + 2), "n"(B4 + 3));
  else
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %4, %5 row_newbcast:%c9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %4, %6 row_newbcast:%c10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %4, %7 row_newbcast:%c11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %4, %8 row_newbcast:%c12 row_mask:0xf bank_mask:0xf"
        : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])
        : "v"(d), "v"(t[0]), "v"(t[1]), "v"(t[2]), "v"(t[3]), "n"(B4), "n"(B4 + 1), "n"(B4 + 2), "n"(B4 + 3));
}

// Blocks of activations a wave loads ahead of the block it multiplies: enough
// to cover the latency of the loads (from L2) with the VALU work of the blocks
// in between, within the same 16 registers (a ring of PD + 1 slots).
constexpr int mfma_prefetch(int tg) { return tg == 1 ? 7 : tg == 2 ? 3 : 1; }

// ---- one 64-row tile for all tokens ------------------------------------------------------------------------
// Segments wk, wk + nwk, ... of K (Seg<FMT>::K weights, as in the DPP GEMV)
// and, for the wave with (nseg % nwk) == wk, the tail past the last whole
// segment are accumulated into y[G][tg][i] = weight row 16G + l%16, token
// t0 + 16tg + 4(l/16) + i (unscaled by the format's final factor).  lds: this
// wave's code tile (Seg<FMT>::CH KB), xbuf: its 4 KB transpose buffers.
//
// Codes: a segment's 64 x 128-byte rows (208 for ternary) come into LDS by
// DMA in whole 128-byte lines (global_load_lds, the DPP GEMV's swizzled tile
// layout; a lane = row global load would touch 64 lines per instruction).
// Each lane reads its row's bytes of a sub-chunk just before the sub-chunk,
// and the next segment's DMA is issued after the last sub-chunk's reads, so it
// lands while that sub-chunk is computed.  The tail is loaded lane = row
// directly.
template <int FMT, int TG>
__device__ __forceinline__ void mfma_tile(const GemvItem& it, int B, int t0, int row0, int wk, int nwk, uint8_t* lds,
                                          uint8_t* xbuf, const int8_t* v8, float (&y)[4][TG][4]) {
  constexpr int CH = Seg<FMT>::CH;
  constexpr int SEGK = Seg<FMT>::K;
  constexpr int SEGB = CH * 16;
  constexpr int NSUB = SEGK / 256;
  constexpr int SUBB = MGeo<FMT>::SUBB;
  constexpr int NT = FMT == QFMT_TERN_B3 ? 13 : SUBB / 4;  // code dwords per sub-chunk
  constexpr int WBLK = Seg<FMT>::WBLK;
  constexpr int SPS = Seg<FMT>::SPS;
  constexpr int BPS = WBLK / 32;                     // activation blocks per weight-scale block
  constexpr int SPB = WBLK >= 256 ? 1 : 256 / WBLK;  // weight-scale blocks per sub-chunk
  constexpr bool PLANES = FMT == QFMT_SIGN1 || FMT == QFMT_INT2;
  constexpr int PD = mfma_prefetch(TG), R = PD + 1;
  static_assert(8 % R == 0, "the activation ring must divide a sub-chunk");
  // Vector-memory loads certainly issued after a segment's DMA and before the
  // top of the next segment of the wave (the activation loads of the last
  // sub-chunk): waiting until at most that many are in flight implies the DMA
  // has landed (loads complete in order), while the latest activation
  // prefetches stay in flight.
  constexpr int VM_AFTER = 8 * TG * (PLANES ? 2 : 1);
  constexpr int VM_WAIT = VM_AFTER < 63 ? VM_AFTER : 63;
  const int lane = threadIdx.x & 63, r16 = lane & 15, j = lane >> 4;
  const int K = it.cols, N = it.rows, kbs = K >> 5;
  const int nseg = K / SEGK;
  const int nsub_all = (K + 255) >> 8;
  const bool own_tail = (K % SEGK) != 0 && (nseg % nwk) == wk;
  const int nvalid = min(64, N - row0);
  const int row = row0 + (lane < nvalid ? lane : nvalid - 1);  // decode lane's row, clamped into the matrix
  const int64_t rb = it.row_bytes;
  g_u8* rowp = gptr<g_u8*>(it.codes) + (int64_t)row * rb;
  g_u8* tile = gptr<g_u8*>(it.codes) + (int64_t)row0 * rb;
  // tokens of this lane's A operand and d register, clamped into the batch
  int ta[TG], td[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    ta[tg] = min(t0 + 16 * tg + r16, B - 1);
    td[tg] = min(t0 + 16 * tg + 4 * j + (lane & 3), B - 1);
  }
  const int nsb = K / WBLK;
  const int64_t ng = (nsb + SPS - 1) / SPS;  // scale groups per row tile
  g_u16* stile = gptr<g_u16*>(it.scales) + (int64_t)(row0 >> 6) * ng * 64 * SPS;

  // DMA of segment sg: load i puts lane l's 16 bytes at slot 64 i + l; slot s
  // holds row s / CH and chunk (s % CH), swizzled as chunk ^ ((row / 2) % 8)
  // for 8-chunk segments (conflict-free row reads).  Rows past the end of the
  // matrix re-read its last row.
  auto issue_tile = [&](int sg) {
    __builtin_amdgcn_sched_barrier(0);
    // the lane offsets are recomputed at each issue (a few VALU per load)
    // rather than hoisted out of the loop as 64-bit pointers
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int f = i * 64 + ln;
      const int r = f / CH, pos = f % CH;
      const int c = CH == 8 ? (pos ^ ((r >> 1) & 7)) : pos;
      const uint32_t off = (uint32_t)(min(r, nvalid - 1) * rb + c * 16);
      if constexpr (TileCachePolicy<FMT>::v == 0)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(tile + (int64_t)sg * SEGB + off),
                                         (__attribute__((address_space(3))) void*)(lds + i * 1024), 16, 0,
                                         0);
      else
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(tile + (int64_t)sg * SEGB + off),
                                         (__attribute__((address_space(3))) void*)(lds + i * 1024), 16, 0,
                                         kTileCachePolicy);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // the lane's row bytes of sub-chunk SUB of the segment in LDS: dwords
  // [NT SUB, NT SUB + NT) of the row, from 16-byte chunks C0 .. C1
  auto read_sub = [&](auto sub_c, uint32_t (&Tc)[NT]) {
    constexpr int SUB = decltype(sub_c)::value;
    constexpr int D0 = NT * SUB, C0 = D0 / 4, C1 = (D0 + NT - 1) / 4;
    uint32_t buf[(C1 - C0 + 1) * 4];
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int k = C0; k <= C1; ++k) {
      const int off = CH == 8 ? ln * 128 + ((k ^ ((ln >> 1) & 7)) << 4) : ln * (CH * 16) + 16 * k;
      const u32x4 v = *(const u32x4*)(lds + off);
      buf[4 * (k - C0)] = v.x;
      buf[4 * (k - C0) + 1] = v.y;
      buf[4 * (k - C0) + 2] = v.z;
      buf[4 * (k - C0) + 3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) Tc[i] = buf[D0 - 4 * C0 + i];
  };
  // tail sub-chunk sc, lane = row (bytes past the end of K are not loaded:
  // zeros stand there)
  auto load_codes = [&](int sc, uint32_t (&T)[NT]) {
    if constexpr (FMT == QFMT_TERN_B3) {
      g_u32* p = (g_u32*)(rowp + (int64_t)sc * SUBB);
#pragma unroll
      for (int i = 0; i < 13; ++i) T[i] = p[i];
    } else {
      const int valid = min(SUBB, (kbs - 8 * sc) * MGeo<FMT>::BLKB);
#pragma unroll
      for (int c = 0; c < SUBB / 16; ++c) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (16 * c < valid) v = *(g_u32x4*)(rowp + (int64_t)sc * SUBB + 16 * c);
        T[4 * c] = v.x;
        T[4 * c + 1] = v.y;
        T[4 * c + 2] = v.z;
        T[4 * c + 3] = v.w;
      }
    }
  };
  // weight scales of sub-chunk sc for the four row groups (row 16G + l%16)
  auto load_scales_sc = [&](int sc, uint32_t (&S)[4][(SPB + 1) / 2]) {
    const int b0 = sc * SPB;  // first scale block of the sub-chunk
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      g_u16* p = stile + (uint32_t)(((b0 / SPS) * 64 + 16 * G + r16) * SPS + b0 % SPS);
      if constexpr (SPB == 1) S[G][0] = p[0];
      else if constexpr (SPB == 2) S[G][0] = *(g_u32*)p;
      else if constexpr (SPB == 4) {
        const u32x2 v = *(g_u32x2*)p;
        S[G][0] = v.x;
        S[G][1] = v.y;
      } else {
        const u32x4 v = *(g_u32x4*)p;
        S[G][0] = v.x;
        S[G][1] = v.y;
        S[G][2] = v.z;
        S[G][3] = v.w;
      }
    }
  };
  // A operand of block kb (global index) for every token group (32-bit lane
  // offsets from the uniform base: B K < 2^31)
  auto load_act = [&](int kb, int64_t (&A)[TG]) {
    kb = min(kb, kbs - 1);
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      if constexpr (PLANES) {
        g_u32* pl = gptr<g_u32*>(it.q) + (uint32_t)((ta[tg] * kbs + kb) * 8 + j);
        const uint32_t L = pl[0], H = pl[4];
        const uint32_t qe = (L & 0x0F0F0F0Fu) | ((H << 4) & 0xF0F0F0F0u);  // values 8j + 0, 2, 4, 6
        const uint32_t qo = ((L >> 4) & 0x0F0F0F0Fu) | (H & 0xF0F0F0F0u);   // values 8j + 1, 3, 5, 7
        A[tg] = (int64_t)(((uint64_t)qo << 32) | qe);
      } else {
        A[tg] = *(const int64_t __attribute__((address_space(1)))*)(gptr<g_u8*>(it.q) +
                                                                       (uint32_t)(ta[tg] * K + 32 * kb + 8 * j));
      }
    }
  };
  // d register of a quad of blocks starting at kb0 (global); 0 for blocks
  // past the end of K, so a partial last sub-chunk's missing blocks add exact
  // zeros (their codes and activations are finite: clamped or zero-filled)
  auto load_d = [&](int kb0, float (&D)[TG]) {
    const int kb = kb0 + (r16 >> 2);
    const int kbc = min(kb, kbs - 1);
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      const float v = gptr<const float __attribute__((address_space(1)))*>(it.d)[(uint32_t)(td[tg] * kbs + kbc)];
      D[tg] = kb < kbs ? v : 0.0f;
    }
  };
  auto trellis_prev = [&](int sc) -> uint32_t {
    if constexpr (FMT == QFMT_TRELLIS2) {
      if (sc == 0) return (uint32_t)gptr<g_u16*>(it.seeds)[row];
      const uint32_t raw = (uint32_t)((g_u16*)(rowp + (int64_t)sc * SUBB))[-1];
      return ((raw & 0xFFu) << 8) | (raw >> 8);
    } else {
      return 0u;
    }
  };
  // the sub-chunk this wave computes after sc (sc itself after its last one)
  auto next_sub = [&](int sc) -> int {
    if (sc >= nseg * NSUB) return sc + 1 < nsub_all ? sc + 1 : sc;  // inside the tail
    if ((sc + 1) % NSUB != 0) return sc + 1;                        // inside a segment
    const int seg = sc / NSUB;
    if (seg + nwk < nseg) return (seg + nwk) * NSUB;
    return own_tail ? nseg * NSUB : sc;
  };

  const int first = wk < nseg ? wk * NSUB : (own_tail ? nseg * NSUB : -1);
  if (first < 0) return;
  if (wk < nseg) issue_tile(wk);
  // Software pipeline over the blocks of a sub-chunk: when block kb has been
  // decoded, its levels go to LDS buffer kb & 1 and block kb - 1 (written one
  // step earlier, so its LDS reads overlap kb's decode) is multiplied; the last
  // block is multiplied after the decode.  Activations of block kb sit in slot
  // kb % R of a ring loaded PD blocks ahead (R = PD + 1, so a slot is reloaded
  // right after its block was used); d registers of a quad of blocks in slot
  // quad & 1, loaded one quad ahead.
  uint32_t S[4][(SPB + 1) / 2];
  int64_t A[R][TG];
  float D[2][TG];
  load_scales_sc(first, S);
  static_for(std::make_integer_sequence<int, PD>{}, [&](auto bc) {
    load_act(8 * first + decltype(bc)::value, A[decltype(bc)::value]);
  });
  load_d(8 * first, D[0]);
  float acc[4][TG][4];
  uint32_t prev = 0;

  auto run_sub = [&](int sc, const uint32_t (&Tc)[NT]) {
    const int kb0 = 8 * sc;
    const int nsc = next_sub(sc);
    uint32_t Sn[4][(SPB + 1) / 2];
    load_scales_sc(nsc, Sn);
    // block kb (compile-time) of this sub-chunk: its B operands from LDS, the MFMAs, the epilogue
    auto multiply = [&](auto kbc) {
      constexpr int kb = decltype(kbc)::value;
      const uint8_t* xb = xbuf + (kb & 1) * 2048;
      int64_t Bw[4];
#pragma unroll
      for (int G = 0; G < 4; ++G) Bw[G] = *(const int64_t*)(xb + (j >> 1) * 1024 + (16 * G + r16) * 16 + (j & 1) * 8);
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {
        // a token group's four MFMAs, then their epilogue (issuing every group's
        // MFMAs first would keep 16 TG result registers live)
        if (tg > 0) __builtin_amdgcn_sched_barrier(0);
        v4i32 c[4];
#pragma unroll
        for (int G = 0; G < 4; ++G)
          c[G] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A[kb % R][tg], Bw[G], v4i32{0, 0, 0, 0}, 0, 0, 0);
        const float d = D[(kb >> 2) & 1][tg];
#pragma unroll
        for (int G = 0; G < 4; ++G) {
          const float t[4] = {(float)c[G][0], (float)c[G][1], (float)c[G][2], (float)c[G][3]};
          if constexpr (BPS == 1) {
            float u[4];
            fma_bcast4<4 * (kb & 3), true>(u, d, t);
            const float s = scale_half(S[G][kb >> 1], kb & 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) y[G][tg][i] = __builtin_fmaf(s, u[i], y[G][tg][i]);
          } else {
            fma_bcast4<4 * (kb & 3), (kb % BPS) == 0>(acc[G][tg], d, t);
            if constexpr ((kb % BPS) == BPS - 1) {
              constexpr int sb = kb / BPS;
              const float s = SPB == 1 ? __half2float(__ushort_as_half((unsigned short)S[G][0]))
                                       : scale_half(S[G][sb >> 1], sb & 1);
#pragma unroll
              for (int i = 0; i < 4; ++i) y[G][tg][i] = __builtin_fmaf(s, acc[G][tg][i], y[G][tg][i]);
            }
          }
        }
      }
    };
    auto consume = [&](auto kbc, const uint32_t (&p)[8]) {
      constexpr int kb = decltype(kbc)::value;
      // one scheduling region per block: interleaving the eight unrolled blocks
      // would keep several blocks' operands live at once
      __builtin_amdgcn_sched_barrier(0);
      uint8_t* xb = xbuf + (kb & 1) * 2048;
      *(u32x4*)(xb + lane * 16) = u32x4{p[0], p[1], p[2], p[3]};
      *(u32x4*)(xb + 1024 + lane * 16) = u32x4{p[4], p[5], p[6], p[7]};
      if constexpr (kb >= 1) multiply(std::integral_constant<int, kb - 1>{});
      // refill the ring slot block kb - 1 used: block kb + PD (past this
      // sub-chunk: the next sub-chunk's block kb + PD - 8)
      constexpr int nb = kb + PD;
      load_act(nb < 8 ? kb0 + nb : 8 * nsc + nb - 8, A[nb % R]);
      if constexpr ((kb & 3) == 1) {
        constexpr int nq = (kb >> 2) + 1;  // the quad after kb's: slot nq & 1 is free again
        load_d(nq < 2 ? kb0 + 4 * nq : 8 * nsc, D[nq & 1]);
      }
    };
    if constexpr (FMT == QFMT_SIGN1) mdec_sign1(Tc, consume);
    else if constexpr (FMT == QFMT_INT2) mdec_int2(Tc, consume);
    else if constexpr (FMT == QFMT_INT4) mdec_int4(Tc, consume);
    else if constexpr (FMT == QFMT_TERN_B3) mdec_tern(Tc, consume);
    else mdec_trellis(Tc, prev, v8, consume);
    multiply(std::integral_constant<int, 7>{});  // the last decoded block
#pragma unroll
    for (int G = 0; G < 4; ++G)
#pragma unroll
      for (int i = 0; i < (SPB + 1) / 2; ++i) S[G][i] = Sn[G][i];
  };

  for (int seg = wk; seg < nseg; seg += nwk) {
    // this segment's tile: the first wait drains everything (the loads before
    // it are fewer than VM_WAIT), the others keep the activation prefetches
    if (seg == wk) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    else __builtin_amdgcn_s_waitcnt(0x0F70 | (VM_WAIT & 15) | ((VM_WAIT >> 4) << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    prev = trellis_prev(seg * NSUB);
    static_for(std::make_integer_sequence<int, NSUB>{}, [&](auto sc_c) {
      constexpr int SUB = decltype(sc_c)::value;
      uint32_t Tc[NT];
      read_sub(sc_c, Tc);
      if constexpr (SUB == NSUB - 1) {
        // the tile reads complete before the next DMA overwrites the region
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        asm volatile("" ::: "memory");
        if (seg + nwk < nseg) issue_tile(seg + nwk);
      }
      run_sub(seg * NSUB + SUB, Tc);
    });
  }
  if (own_tail) {
    prev = trellis_prev(nseg * NSUB);
    for (int sc = nseg * NSUB; sc < nsub_all; ++sc) {
      uint32_t Tc[NT];
      load_codes(sc, Tc);
      run_sub(sc, Tc);
    }
  }
}

// Token groups per pass of a tile: the 2- and 1-bit formats, whose decode is
// cheap, run more than 32 tokens as passes of up to 32 (decoding again per
// pass) rather than hold four token groups' accumulators at once.
constexpr int mfma_pass_groups(int tg, int fmt) {
  return (fmt == QFMT_INT2 || fmt == QFMT_SIGN1) && tg > 2 ? 2 : tg;
}

// Waves per workgroup of the persistent MFMA launch (one workgroup per CU):
// as many as the kernel's registers allow without spilling (8 waves leave a
// wave 256 VGPRs, 4 leave 512 with the AGPRs); the code tile and transpose
// buffers (12 KB of LDS per wave, 17 KB for ternary) allow at most 13 (9).
constexpr int mfma_wpg(int tg, int fmt) {
  if (fmt == QFMT_INT4) return 8;
  if (fmt == QFMT_TERN_B3) return tg <= 2 ? 8 : 4;
  return tg == 1 ? 8 : 4;  // INT2, SIGN1 (in passes of 2 groups), TRELLIS
}

// Single matrix: a workgroup of 4 waves covers 64 rows and splits the
// sub-chunks of K between its waves; partial sums are added in LDS in a fixed
// order (deterministic).
template <int FMT, int TG>
__global__ __launch_bounds__(256) void k_gemv_mfma(GemvItem it, int B, V8Table v8t, float gain) {
  constexpr int TP = mfma_pass_groups(TG, FMT);
  __shared__ __attribute__((aligned(16))) uint8_t ctile[4][Seg<FMT>::CH * 1024];
  __shared__ __attribute__((aligned(16))) uint8_t xb[4][4096];
  __shared__ float red[3][4 * TP * 4][64];
  __shared__ int8_t v8[256];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if constexpr (FMT == QFMT_TRELLIS2) {
    v8[threadIdx.x] = v8t.v[threadIdx.x];
    __syncthreads();
  }
  const int row0 = blockIdx.x * 64;
  const float fs = final_scale<FMT>(gain);
  const int r16 = lane & 15, j = lane >> 4;
  for (int t0 = 0; t0 < B; t0 += 16 * TP) {
    float y[4][TP][4];
#pragma unroll
    for (int G = 0; G < 4; ++G)
#pragma unroll
      for (int tg = 0; tg < TP; ++tg)
#pragma unroll
        for (int i = 0; i < 4; ++i) y[G][tg][i] = 0.0f;
    mfma_tile<FMT, TP>(it, B, t0, row0, wave, 4, ctile[wave], xb[wave], v8, y);
    __builtin_amdgcn_s_waitcnt(0);  // no tile DMA may still be landing when the wave moves on
    if (wave > 0) {
#pragma unroll
      for (int G = 0; G < 4; ++G)
#pragma unroll
        for (int tg = 0; tg < TP; ++tg)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[wave - 1][(G * TP + tg) * 4 + i][lane] = y[G][tg][i];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int G = 0; G < 4; ++G) {
        const int row = row0 + 16 * G + r16;
#pragma unroll
        for (int tg = 0; tg < TP; ++tg)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = (G * TP + tg) * 4 + i;
            const float v = ((y[G][tg][i] + red[0][e][lane]) + red[1][e][lane]) + red[2][e][lane];
            const int t = t0 + 16 * tg + 4 * j + i;
            if (row < it.rows && t < B) gptr<g_f32*>(it.y)[(int64_t)t * it.rows + row] = v * fs;
          }
      }
    }
    __syncthreads();  // red is reused by the next pass
  }
}

// Grouped: persistent workgroups, one per CU, whose waves take the plan's tiles
// of format ONLY in list order through an LDS counter (as k_gemv_grouped).
template <int TG, int ONLY>
__global__ __launch_bounds__(64 * mfma_wpg(TG, ONLY)) void k_gemv_grouped_mfma(const uint8_t* __restrict__ plan,
                                                                              V8Table v8t, float gain) {
  constexpr int TP = mfma_pass_groups(TG, ONLY);
  __shared__ __attribute__((aligned(16))) uint8_t ctile[mfma_wpg(TG, ONLY)][Seg<ONLY>::CH * 1024];
  __shared__ __attribute__((aligned(16))) uint8_t xb[mfma_wpg(TG, ONLY)][4096];
  __shared__ int8_t v8[256];
  __shared__ int next_k;
  const PlanHeader* hp = (const PlanHeader*)plan;
  const GemvItem* items = (const GemvItem*)(plan + hp->items_off);
  const GemvTile* tiles = (const GemvTile*)(plan + hp->tiles_off);
  const int nwk = hp->n_workers;
  const int B = hp->B;
  const int32_t* wb = (const int32_t*)(plan + hp->workers_off) + ONLY * (nwk + 1);
  if constexpr (ONLY == QFMT_TRELLIS2) {
    if (threadIdx.x < 256) v8[threadIdx.x] = v8t.v[threadIdx.x];
  }
  if (threadIdx.x == 0) next_k = 0;
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r16 = lane & 15, j = lane >> 4;
  for (;;) {
    int k = 0;
    if (lane == 0) k = __hip_atomic_fetch_add(&next_k, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    k = __builtin_amdgcn_readfirstlane(k);
    int w = blockIdx.x, t = -1;
    while (w < nwk) {
      const int b0 = wb[w], n = wb[w + 1] - b0;
      if (k < n) {
        t = b0 + k;
        break;
      }
      k -= n;
      w += gridDim.x;
    }
    if (t < 0) break;
    const GemvTile tl = tiles[t];
    const int ii = __builtin_amdgcn_readfirstlane((int)tl.item);
    const int row0 = __builtin_amdgcn_readfirstlane((int)tl.row0);
    const GemvItem it = items[ii];
    const float fs = final_scale<ONLY>(gain);
    for (int t0 = 0; t0 < B; t0 += 16 * TP) {
      float y[4][TP][4];
#pragma unroll
      for (int G = 0; G < 4; ++G)
#pragma unroll
        for (int tg = 0; tg < TP; ++tg)
#pragma unroll
          for (int i = 0; i < 4; ++i) y[G][tg][i] = 0.0f;
      mfma_tile<ONLY, TP>(it, B, t0, row0, 0, 1, ctile[wave], xb[wave], v8, y);
#pragma unroll
      for (int G = 0; G < 4; ++G) {
        const int row = row0 + 16 * G + r16;
#pragma unroll
        for (int tg = 0; tg < TP; ++tg)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tok = t0 + 16 * tg + 4 * j + i;
            if (row < it.rows && tok < B) gptr<g_f32*>(it.y)[(int64_t)tok * it.rows + row] = y[G][tg][i] * fs;
          }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no tile DMA may still be landing when the wave ends
}

}  // namespace qk
