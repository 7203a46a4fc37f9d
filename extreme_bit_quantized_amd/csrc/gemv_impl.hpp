// gemv_impl.hpp — batch-1..8 GEMV over packed low-bit weights for gfx950.
//
// Work unit: one wave owns 64 consecutive weight rows; lane i computes row
// row0 + i.  Weight bytes are streamed in row segments (128 bytes per row, 208
// for ternary): the wave fetches a [64 rows x segment] tile with coalesced,
// non-temporal 16-byte loads (8 rows x 128 bytes per wave instruction), writes
// it to its own LDS region and reads back the 16-byte chunks of its own row, so
// every HBM transaction is a full cache line while each lane ends up with a
// whole row of codes.  Activations are the same for all 64 rows, so they are
// read with scalar loads into SGPRs and enter v_dot4 as the scalar operand;
// the integer block dot I of every 32-block is exact, and the fp32 scaling is
// folded so that the per-row cost per 32 weights is the unpack, 8 dot4 and
// three or four VALU ops.
//
// Decode per format (levels come out as bytes lined up with activation dwords):
//   SIGN1  word w, weight 4j+b at bit 8b+j: (w>>j) & 0x01010101 for j = 0..3
//          and (w>>j) & 0x10101010 (16x, a second dot chain) for j = 4..7.
//   INT2   weight 4j+b at bits 8b+2j: masks 0x03030303 / 0x30303030 of w, w>>2.
//   INT4   weight 4j+b at bits 8b+4j: w & 0x0F0F0F0F, (w>>4) & 0x0F0F0F0F.
//   TERN   byte = fixed-point base-3 fraction of 5 trits: multiplying the byte
//          by 3 brings the next digit into bits 8..9 and leaves the rest below;
//          two bytes per 32-bit register (16-bit lanes), a v_perm gathers the
//          four digits of one activation dword.
//   TRELLIS 16-bit window of seed||bytes, hash, int8 codebook in LDS.
#pragma once

#include <hip/hip_fp16.h>

#include "internal.hpp"

namespace qk {

typedef const int32_t __attribute__((address_space(4))) c_i32;
typedef const float __attribute__((address_space(4))) c_f32;
typedef const uint8_t __attribute__((address_space(4))) c_u8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int dot4(uint32_t w, int32_t a, int acc) {
  return __builtin_amdgcn_sdot4((int)w, a, acc, false);
}

// Geometry of one row segment per format.
template <int FMT> struct Seg;
template <> struct Seg<QFMT_SIGN1> {
  static constexpr int CH = 8, K = 1024, SPS = 8, WBLK = 128;
};
template <> struct Seg<QFMT_INT2> {
  static constexpr int CH = 8, K = 512, SPS = 16, WBLK = 32;
};
template <> struct Seg<QFMT_INT4> {
  static constexpr int CH = 8, K = 256, SPS = 8, WBLK = 32;
};
template <> struct Seg<QFMT_TERN_B3> {
  static constexpr int CH = 13, K = 1024, SPS = 4, WBLK = 256;
};
template <> struct Seg<QFMT_TRELLIS2> {
  static constexpr int CH = 8, K = 512, SPS = 8, WBLK = 64;
};
// LDS row pitch of the transposed tile: an odd number of 16-byte chunks so
// that the 8 lanes of a ds_read_b128 phase hit 8 different bank groups.
template <int CH> struct Pitch { static constexpr int value = (CH % 2 ? CH : CH + 1) * 16; };
constexpr int kMaxWaveLds = 64 * 208;  // largest per-wave tile region (ternary)

// Wave-uniform view of the activations of NB tokens (scalar address space).
struct Act {
  c_i32* q;   // token b, act block kb, dword j at q[b*kq + kb*8 + j]
  c_f32* d;   // d[b*kb_stride + kb]
  c_i32* qs;  // qs[b*kb_stride + kb]
  int kq;     // K / 4
  int kbs;    // K / 32
};

// ---- per-format segment compute ------------------------------------------------------------
// T: the lane's row codes for the segment (dwords), S: its fp16 scales as
// packed pairs, kb0: act block index of the segment start, nkb: valid act
// blocks (FULL: all).  y accumulates the per-format scaled result.

template <int NB, bool FULL, bool WI>
__device__ __forceinline__ void seg_sign1(const uint32_t (&T)[32], const uint32_t (&S)[4], const Act& A,
                                          int kb0, int nkb, float (&y)[NB], int32_t* Iout) {
#pragma unroll
  for (int sb = 0; sb < 8; ++sb) {
    if (!(FULL || sb * 4 < nkb)) continue;
    float acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = 0.0f;
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int kb = sb * 4 + j4;
      const uint32_t W = T[kb];
      uint32_t P[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t t = W >> j;
        P[j] = t & 0x01010101u;
        P[j + 4] = t & 0x10101010u;
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        c_i32* a = A.q + b * A.kq + (kb0 + kb) * 8;
        int x = 0, z = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x = dot4(P[j], a[j], x);
          z = dot4(P[j + 4], a[j + 4], z);
        }
        // 16*S1 - 8*qsum = 8*I with I = 2*S1 - qsum = sum (2b-1) q
        const int i8 = (x << 4) + z - (A.qs[b * A.kbs + kb0 + kb] << 3);
        if (WI && b == 0 && Iout) Iout[kb0 + kb] = i8 >> 3;
        acc[b] = __builtin_fmaf(A.d[b * A.kbs + kb0 + kb], (float)i8, acc[b]);
      }
    }
    const uint32_t sp = S[sb >> 1];
    const float s = __half2float(__ushort_as_half((unsigned short)((sb & 1) ? (sp >> 16) : (sp & 0xFFFF))));
#pragma unroll
    for (int b = 0; b < NB; ++b) y[b] = __builtin_fmaf(s, acc[b], y[b]);
  }
}

template <int NB, bool FULL, bool WI>
__device__ __forceinline__ void seg_int2(const uint32_t (&T)[32], const uint32_t (&S)[8], const Act& A,
                                         int kb0, int nkb, float (&y)[NB], int32_t* Iout) {
#pragma unroll
  for (int kb = 0; kb < 16; ++kb) {
    if (!(FULL || kb < nkb)) continue;
    const uint32_t W0 = T[2 * kb], W1 = T[2 * kb + 1];
    const uint32_t V0 = W0 >> 2, V1 = W1 >> 2;
    const uint32_t p0 = W0 & 0x03030303u, p1 = V0 & 0x03030303u, p4 = W1 & 0x03030303u, p5 = V1 & 0x03030303u;
    const uint32_t p2 = W0 & 0x30303030u, p3 = V0 & 0x30303030u, p6 = W1 & 0x30303030u, p7 = V1 & 0x30303030u;
    const uint32_t sp = S[kb >> 1];
    const float s = __half2float(__ushort_as_half((unsigned short)((kb & 1) ? (sp >> 16) : (sp & 0xFFFF))));
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      c_i32* a = A.q + b * A.kq + (kb0 + kb) * 8;
      int x = dot4(p0, a[0], 0);
      x = dot4(p1, a[1], x);
      x = dot4(p4, a[4], x);
      x = dot4(p5, a[5], x);
      int z = dot4(p2, a[2], 0);
      z = dot4(p3, a[3], z);
      z = dot4(p6, a[6], z);
      z = dot4(p7, a[7], z);
      // 16*sum(c q) - 24*qsum = 8*I with I = sum (2c-3) q
      const int i8 = (x << 4) + z - A.qs[b * A.kbs + kb0 + kb] * 24;
      if (WI && b == 0 && Iout) Iout[kb0 + kb] = i8 >> 3;
      y[b] = __builtin_fmaf(s, A.d[b * A.kbs + kb0 + kb] * (float)i8, y[b]);
    }
  }
}

template <int NB, bool FULL, bool WI>
__device__ __forceinline__ void seg_int4(const uint32_t (&T)[32], const uint32_t (&S)[4], const Act& A,
                                         int kb0, int nkb, float (&y)[NB], int32_t* Iout) {
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    if (!(FULL || kb < nkb)) continue;
    uint32_t P[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t W = T[4 * kb + m];
      P[2 * m] = W & 0x0F0F0F0Fu;
      P[2 * m + 1] = (W >> 4) & 0x0F0F0F0Fu;
    }
    const uint32_t sp = S[kb >> 1];
    const float s = __half2float(__ushort_as_half((unsigned short)((kb & 1) ? (sp >> 16) : (sp & 0xFFFF))));
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      c_i32* a = A.q + b * A.kq + (kb0 + kb) * 8;
      int x = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) x = dot4(P[j], a[j], x);
      // I = sum (2c-15) q = 2*sum(c q) - 15*qsum
      const int I = (x << 1) - A.qs[b * A.kbs + kb0 + kb] * 15;
      if (WI && b == 0 && Iout) Iout[kb0 + kb] = I;
      y[b] = __builtin_fmaf(s, A.d[b * A.kbs + kb0 + kb] * (float)I, y[b]);
    }
  }
}

template <int NB, bool FULL, bool WI>
__device__ __forceinline__ void seg_tern(const uint32_t (&T)[52], const uint32_t (&S)[2], const Act& A,
                                         int kb0, int nkb, float (&y)[NB], int32_t* Iout) {
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {
    if (!(FULL || sb * 8 < nkb)) continue;
    float acc[NB];
    int blk[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      acc[b] = 0.0f;
      blk[b] = 0;
    }
#pragma unroll
    for (int m = 0; m < 13; ++m) {
      const uint32_t W = T[13 * sb + m];
      uint32_t xl = W & 0x00FF00FFu;         // bytes 0, 2 in 16-bit lanes
      uint32_t xh = (W >> 8) & 0x00FF00FFu;  // bytes 1, 3
      const int ndig = m < 12 ? 5 : 4;
#pragma unroll
      for (int i = 0; i < ndig; ++i) {
        const uint32_t yl = xl * 3u, yh = xh * 3u;
        // digits sit in bits 8..9 of every 16-bit lane; gather bytes 1, 5, 3, 7
        const uint32_t D = __builtin_amdgcn_perm(yh, yl, 0x07030501u);
        if (i + 1 < ndig) {
          xl = yl & 0x00FF00FFu;
          xh = yh & 0x00FF00FFu;
        }
        const int g = m < 12 ? 5 * m + i : 60 + i;  // activation dword within the 256-block
        const int kbl = sb * 8 + (g >> 3);
        const int j = g & 7;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          c_i32* a = A.q + b * A.kq + (kb0 + kbl) * 8;
          blk[b] = dot4(D, a[j], blk[b]);
        }
        if (j == 7) {
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            // digits are t + 1: sum d q - qsum = sum t q
            const int I = blk[b] - A.qs[b * A.kbs + kb0 + kbl];
            if (WI && b == 0 && Iout) Iout[kb0 + kbl] = I;
            acc[b] = __builtin_fmaf(A.d[b * A.kbs + kb0 + kbl], (float)I, acc[b]);
            blk[b] = 0;
          }
        }
      }
    }
    const uint32_t sp = S[sb >> 1];
    const float s = __half2float(__ushort_as_half((unsigned short)((sb & 1) ? (sp >> 16) : (sp & 0xFFFF))));
#pragma unroll
    for (int b = 0; b < NB; ++b) y[b] = __builtin_fmaf(s, acc[b], y[b]);
  }
}

// Trellis: `prev` holds the last 16 bits of seed||bytes before the segment.
template <int NB, bool FULL, bool WI>
__device__ __forceinline__ void seg_trellis(const uint32_t (&T)[32], const uint32_t (&S)[4], const Act& A,
                                            int kb0, int nkb, uint32_t prev, const int8_t* v8,
                                            float (&y)[NB], int32_t* Iout) {
#pragma unroll
  for (int sb = 0; sb < 8; ++sb) {  // 64-weight scale blocks = 2 act blocks = 4 dwords
    if (!(FULL || sb * 2 < nkb)) continue;
    float acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = 0.0f;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int kb = sb * 2 + h2;
      int blk[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) blk[b] = 0;
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const uint32_t W = T[kb * 2 + w];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t w24 = (prev << 8) | ((W >> (8 * p)) & 0xFFu);
          uint32_t L = 0;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const uint32_t st = (w24 >> (6 - 2 * jj)) & 0xFFFFu;
            const uint32_t h = ((st * 0x9E37u) ^ (st >> 7)) & 0xFFu;
            L |= ((uint32_t)(uint8_t)v8[h]) << (8 * jj);
          }
          prev = w24 & 0xFFFFu;
          const int j = w * 4 + p;
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            c_i32* a = A.q + b * A.kq + (kb0 + kb) * 8;
            blk[b] = dot4(L, a[j], blk[b]);
          }
        }
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (WI && b == 0 && Iout) Iout[kb0 + kb] = blk[b];
        acc[b] = __builtin_fmaf(A.d[b * A.kbs + kb0 + kb], (float)blk[b], acc[b]);
      }
    }
    const uint32_t sp = S[sb >> 1];
    const float s = __half2float(__ushort_as_half((unsigned short)((sb & 1) ? (sp >> 16) : (sp & 0xFFFF))));
#pragma unroll
    for (int b = 0; b < NB; ++b) y[b] = __builtin_fmaf(s, acc[b], y[b]);
  }
}

// ---- scale loads ---------------------------------------------------------------------------------
// SPS fp16 scales of one lane's row for one segment, as SPS/2 packed pairs.
template <int SPS>
__device__ __forceinline__ void load_scales(const uint16_t* p, bool vec_ok, uint32_t (&S)[SPS / 2]) {
  if (vec_ok) {
    if constexpr (SPS >= 8) {
#pragma unroll
      for (int i = 0; i < SPS / 8; ++i) {
        const u32x4 v = *(const u32x4*)(p + 8 * i);
        S[4 * i] = v.x;
        S[4 * i + 1] = v.y;
        S[4 * i + 2] = v.z;
        S[4 * i + 3] = v.w;
      }
    } else {
      const u32x2 v = *(const u32x2*)p;
      S[0] = v.x;
      S[1] = v.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < SPS / 2; ++i) S[i] = (uint32_t)p[2 * i] | ((uint32_t)p[2 * i + 1] << 16);
  }
}

// Tail segment scales: only nsc of them are valid.
template <int SPS>
__device__ __forceinline__ void load_scales_tail(const uint16_t* p, int nsc, uint32_t (&S)[SPS / 2]) {
#pragma unroll
  for (int i = 0; i < SPS / 2; ++i) {
    const uint32_t lo = 2 * i < nsc ? p[2 * i] : 0u;
    const uint32_t hi = 2 * i + 1 < nsc ? p[2 * i + 1] : 0u;
    S[i] = lo | (hi << 16);
  }
}

template <int FMT, int NB, bool FULL, bool WI>
__device__ __forceinline__ void seg_compute(const uint32_t (&T)[Seg<FMT>::CH * 4], const uint32_t (&S)[Seg<FMT>::SPS / 2],
                                            const Act& A, int kb0, int nkb, uint32_t prev, const int8_t* v8,
                                            float (&y)[NB], int32_t* Iout) {
  if constexpr (FMT == QFMT_SIGN1) seg_sign1<NB, FULL, WI>(T, S, A, kb0, nkb, y, Iout);
  else if constexpr (FMT == QFMT_INT2) seg_int2<NB, FULL, WI>(T, S, A, kb0, nkb, y, Iout);
  else if constexpr (FMT == QFMT_INT4) seg_int4<NB, FULL, WI>(T, S, A, kb0, nkb, y, Iout);
  else if constexpr (FMT == QFMT_TERN_B3) seg_tern<NB, FULL, WI>(T, S, A, kb0, nkb, y, Iout);
  else seg_trellis<NB, FULL, WI>(T, S, A, kb0, nkb, prev, v8, y, Iout);
}

// Result scale applied once per row after accumulation.
template <int FMT>
__device__ __forceinline__ float final_scale(float trellis_gain) {
  if constexpr (FMT == QFMT_SIGN1) return 0.125f;
  else if constexpr (FMT == QFMT_INT2) return 0.0625f;
  else if constexpr (FMT == QFMT_INT4) return 0.5f;
  else if constexpr (FMT == QFMT_TERN_B3) return 1.0f;
  else return trellis_gain;
}

// ---- one 64-row tile ----------------------------------------------------------------------------------
// Accumulates (unscaled by final_scale) into y for segments wk, wk + nwk, ...
// and the tail segment if (nseg % nwk) == wk.  lds: this wave's region.
template <int FMT, int NB, bool WI>
__device__ __forceinline__ void gemv_tile(const GemvItem& it, int row0, int wk, int nwk, uint8_t* lds,
                                          const int8_t* v8, float (&y)[NB], int32_t* Ibase) {
  constexpr int CH = Seg<FMT>::CH;
  constexpr int SEGK = Seg<FMT>::K;
  constexpr int SPS = Seg<FMT>::SPS;
  constexpr int PITCH = Pitch<CH>::value;
  constexpr int SEGB = CH * 16;
  const int lane = threadIdx.x & 63;
  const int K = it.cols;
  const int N = it.rows;
  const int nseg = K / SEGK;
  const int nvalid = min(64, N - row0);
  const int row = row0 + (lane < nvalid ? lane : nvalid - 1);  // clamp: reads stay in bounds
  const int64_t rb = it.row_bytes;
  const int nsb = K / Seg<FMT>::WBLK;

  Act A;
  A.q = (c_i32*)(const void*)it.q;
  A.d = (c_f32*)(const void*)it.d;
  A.qs = (c_i32*)(const void*)it.qsum;
  A.kq = K >> 2;
  A.kbs = K >> 5;

  const uint16_t* srow = it.scales + (int64_t)row * nsb;
  constexpr int SALIGN = SPS * 2 >= 16 ? 16 : SPS * 2;  // bytes per vector scale load
  const bool svec = ((((uintptr_t)it.scales) | (uintptr_t)(nsb * 2)) & (SALIGN - 1)) == 0;
  // Only lanes that own a row write the test-hook output.
  int32_t* Iout = (WI && lane < nvalid) ? Ibase + (int64_t)row * (K >> 5) : nullptr;
  const uint8_t* tile = it.codes + (int64_t)row0 * rb;

  // Per-lane offsets of the coalesced tile load and its LDS slot.
  uint32_t goff[CH], loff[CH];
  uint32_t vmask = 0;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int f = i * 64 + lane;
    const int r = f / CH, c = f % CH;
    goff[i] = (uint32_t)(r * rb + c * 16);
    loff[i] = (uint32_t)(r * PITCH + c * 16);
    if (r < nvalid) vmask |= 1u << i;
  }
  uint8_t* myrow = lds + lane * PITCH;

  u32x4 L[CH];
  uint32_t S[SPS / 2], Sn[SPS / 2];
  int seg = wk;
  if (seg < nseg) {
#pragma unroll
    for (int i = 0; i < CH; ++i)
      L[i] = (vmask >> i) & 1 ? __builtin_nontemporal_load((const u32x4*)(tile + (int64_t)seg * SEGB + goff[i]))
                              : u32x4{0u, 0u, 0u, 0u};
    load_scales<SPS>(srow + seg * SPS, svec, Sn);
  }
  for (; seg < nseg; seg += nwk) {
    // transpose through LDS: write the tile, read back this lane's row
#pragma unroll
    for (int i = 0; i < CH; ++i) *(u32x4*)(lds + loff[i]) = L[i];
    __builtin_amdgcn_wave_barrier();
    uint32_t T[CH * 4];
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const u32x4 v = *(const u32x4*)(myrow + 16 * k);
      T[4 * k] = v.x;
      T[4 * k + 1] = v.y;
      T[4 * k + 2] = v.z;
      T[4 * k + 3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < SPS / 2; ++i) S[i] = Sn[i];
    __builtin_amdgcn_wave_barrier();
    const int nx = seg + nwk;
    if (nx < nseg) {
#pragma unroll
      for (int i = 0; i < CH; ++i)
        L[i] = (vmask >> i) & 1 ? __builtin_nontemporal_load((const u32x4*)(tile + (int64_t)nx * SEGB + goff[i]))
                                : u32x4{0u, 0u, 0u, 0u};
      load_scales<SPS>(srow + nx * SPS, svec, Sn);
    }
    uint32_t prev = 0;
    if constexpr (FMT == QFMT_TRELLIS2) {
      const uint8_t* rp = it.codes + (int64_t)row * rb + (int64_t)seg * SEGB;
      prev = seg == 0 ? (uint32_t)it.seeds[row] : (((uint32_t)rp[-2] << 8) | rp[-1]);
    }
    seg_compute<FMT, NB, true, WI>(T, S, A, seg * (SEGK / 32), SEGK / 32, prev, v8, y, Iout);
  }

  // Tail: fewer than SEGK weights left; this lane loads its own row directly.
  const int tailK = K - nseg * SEGK;
  if (tailK > 0 && (nseg % nwk) == wk) {
    const int64_t tb = packed_row_bytes(FMT, tailK);
    const uint32_t* rp = (const uint32_t*)(it.codes + (int64_t)row * rb + (int64_t)nseg * SEGB);
    uint32_t T[CH * 4];
#pragma unroll
    for (int i = 0; i < CH * 4; ++i) T[i] = 4 * i < tb ? rp[i] : 0u;
    uint32_t St[SPS / 2];
    load_scales_tail<SPS>(srow + nseg * SPS, tailK / Seg<FMT>::WBLK, St);
    uint32_t prev = 0;
    if constexpr (FMT == QFMT_TRELLIS2) {
      const uint8_t* rb8 = (const uint8_t*)rp;
      prev = nseg == 0 ? (uint32_t)it.seeds[row] : (((uint32_t)rb8[-2] << 8) | rb8[-1]);
    }
    seg_compute<FMT, NB, false, WI>(T, St, A, nseg * (SEGK / 32), tailK / 32, prev, v8, y, Iout);
  }
}

// ---- kernels -----------------------------------------------------------------------------------------

// Single matrix: a workgroup of 4 waves covers 64 rows and splits the
// segments of K between its waves; partial sums are added in LDS in a fixed
// order, so results are deterministic.
template <int FMT, int NB, bool WI>
__global__ __launch_bounds__(256) void k_gemv(GemvItem it, V8Table v8t, float gain, int32_t* Iout) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * 64 * Pitch<Seg<FMT>::CH>::value];
  __shared__ float red[4][NB][64];
  __shared__ int8_t v8[256];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if constexpr (FMT == QFMT_TRELLIS2) {
    v8[threadIdx.x] = v8t.v[threadIdx.x];
    __syncthreads();
  }
  const int row0 = blockIdx.x * 64;
  float y[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) y[b] = 0.0f;
  gemv_tile<FMT, NB, WI>(it, row0, wave, 4, lds + wave * 64 * Pitch<Seg<FMT>::CH>::value, v8, y, Iout);
  if (WI) return;
#pragma unroll
  for (int b = 0; b < NB; ++b) red[wave][b][lane] = y[b];
  __syncthreads();
  if (wave == 0 && row0 + lane < it.rows) {
    const float fs = final_scale<FMT>(gain);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float v = ((red[0][b][lane] + red[1][b][lane]) + red[2][b][lane]) + red[3][b][lane];
      it.y[(int64_t)b * it.rows + row0 + lane] = v * fs;
    }
  }
}

// Grouped: persistent waves pull 64-row tiles from an atomic counter.  The
// last wave to leave resets the counters so the scratch is zero again.
template <int NB>
__global__ __launch_bounds__(256) void k_gemv_grouped(const uint8_t* __restrict__ plan, uint32_t* scratch,
                                                      V8Table v8t, float gain) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kMaxWaveLds];
  __shared__ int8_t v8[256];
  const PlanHeader* hp = (const PlanHeader*)plan;
  const int n_tiles = __builtin_amdgcn_readfirstlane(hp->n_tiles);
  const int fmt_mask = __builtin_amdgcn_readfirstlane(hp->fmt_mask);
  const GemvItem* items = (const GemvItem*)(plan + hp->items_off);
  const GemvTile* tiles = (const GemvTile*)(plan + hp->tiles_off);
  if (fmt_mask & (1 << QFMT_TRELLIS2)) {
    v8[threadIdx.x] = v8t.v[threadIdx.x];
    __syncthreads();
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint8_t* my = lds + wave * kMaxWaveLds;
  auto grab = [&]() -> int {
    uint32_t t = 0;
    if (lane == 0) t = atomicAdd(&scratch[0], 1u);
    return __builtin_amdgcn_readfirstlane((int)t);
  };
  int t = grab();
  while (t < n_tiles) {
    const int tn = grab();
    const GemvTile tl = tiles[t];
    const int ii = __builtin_amdgcn_readfirstlane((int)tl.item);
    const int row0 = __builtin_amdgcn_readfirstlane((int)tl.row0);
    const GemvItem it = items[ii];
    const int fmt = __builtin_amdgcn_readfirstlane(it.fmt);
    float y[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) y[b] = 0.0f;
    float fs = 1.0f;
    switch (fmt) {
      case QFMT_SIGN1: gemv_tile<QFMT_SIGN1, NB, false>(it, row0, 0, 1, my, v8, y, nullptr); fs = 0.125f; break;
      case QFMT_INT2: gemv_tile<QFMT_INT2, NB, false>(it, row0, 0, 1, my, v8, y, nullptr); fs = 0.0625f; break;
      case QFMT_INT4: gemv_tile<QFMT_INT4, NB, false>(it, row0, 0, 1, my, v8, y, nullptr); fs = 0.5f; break;
      case QFMT_TERN_B3: gemv_tile<QFMT_TERN_B3, NB, false>(it, row0, 0, 1, my, v8, y, nullptr); fs = 1.0f; break;
      default: gemv_tile<QFMT_TRELLIS2, NB, false>(it, row0, 0, 1, my, v8, y, nullptr); fs = gain; break;
    }
    if (row0 + lane < it.rows) {
#pragma unroll
      for (int b = 0; b < NB; ++b) it.y[(int64_t)b * it.rows + row0 + lane] = y[b] * fs;
    }
    t = tn;
  }
  if (lane == 0) {
    __threadfence();
    const uint32_t done = atomicAdd(&scratch[1], 1u);
    if (done == gridDim.x * 4 - 1) {
      atomicExch(&scratch[0], 0u);
      atomicExch(&scratch[1], 0u);
    }
  }
}

}  // namespace qk
