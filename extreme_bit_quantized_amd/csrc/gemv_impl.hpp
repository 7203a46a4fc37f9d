// gemv_impl.hpp — batch-1..8 GEMV over packed low-bit weights for gfx950.
//
// Work unit: one wave owns 64 consecutive weight rows; lane i computes row
// row0 + i.  Weight bytes are streamed in row segments (128 bytes per row, 208
// for ternary): the wave fetches a [64 rows x segment] tile with coalesced,
// non-temporal 16-byte loads (8 rows x 128 bytes per wave instruction), writes
// it to its own LDS region and reads back the 16-byte chunks of its own row, so
// every HBM transaction is a full cache line while each lane ends up with a
// whole row of codes.  Activations are the same for all 64 rows: they enter
// the dot products as a wave-uniform operand (a scalar register, or a DPP row
// broadcast); the integer block dot I of every 32-block is exact, and the fp32
// scaling costs one convert and one or two FMAs per block.
//
// Decode per format (codes come out lined up with activation words):
//   SIGN1  word w (32 weights): (w >> j) & 0x11111111, j = 0..3, holds weights
//          8j .. 8j+7 one per nibble; multiplied with 8-way nibble dots against
//          the activations split as x = 16 hi + lo.
//   INT2   two words per 32 weights, (w >> 2j) & 0x33333333, the same way.
//   INT4   weight 4j+b at bits 8b+4j: w & 0x0F0F0F0F, (w>>4) & 0x0F0F0F0F, int8 dots.
//   TERN   byte = fixed-point base-3 fraction of 5 trits: multiplying the byte
//          by 3 brings the next digit into bits 8..9 and leaves the rest below;
//          two bytes per 32-bit register (16-bit lanes), a v_perm gathers the
//          four digits of one activation dword.
//   TRELLIS 16-bit window of seed||bytes, hash, int8 codebook in LDS.
#pragma once

#include <hip/hip_fp16.h>

#include <utility>

#include "internal.hpp"

namespace qk {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// Global-address-space views: loads become global_load with an SGPR base and a
// 32-bit VGPR offset instead of flat loads (which also count against lgkmcnt).
typedef const uint8_t __attribute__((address_space(1))) g_u8;
typedef const uint16_t __attribute__((address_space(1))) g_u16;
typedef const uint32_t __attribute__((address_space(1))) g_u32;
typedef const u32x4 __attribute__((address_space(1))) g_u32x4;
typedef const u32x2 __attribute__((address_space(1))) g_u32x2;
typedef float __attribute__((address_space(1))) g_f32;
template <typename T> __device__ __forceinline__ T gptr(const void* p) { return (T)p; }

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

// ---- activation sub-chunks and DPP-broadcast block dots ----------------------------------------
// Activations reach the dot products as the DPP operand of v_dot4c: the 256
// int8 values of one 256-weight sub-chunk sit in four VGPRs, lane i of every
// 16-lane row holding bytes 16i .. 16i+15, and `row_newbcast:i` hands lane i's
// dword to the whole row inside the dot instruction itself.  d and the qsum
// term of the sub-chunk's 8 activation blocks sit in lanes 0..7 of two more
// VGPRs and are broadcast the same way.  Each block is one asm statement that
// starts with s_nop 1: a VALU write to a DPP source needs two wait states;
// and a v_dot4c result needs three wait states (s_nop 2) before any other VALU
// instruction reads it (dependent v_dot4c chains forward without waits).
// Only non-reversed ops take a DPP operand here: for the reversed forms
// (v_subrev_*) the broadcast lands on the other source, so the qsum term is
// stored negated and added with v_add_u32_dpp.
struct ActSub {
  int32_t a[4];  // q dwords (1- and 2-bit: plane words) 4i .. 4i+3 of the sub-chunk in row lane i
  float d;       // lane kb (0..7): scale of activation block kb
  int32_t Q;     // lane kb (0..7): minus the format multiple of the block's qsum
};

// 1-bit extras of one token's sub-chunk, made from d and Q where it is used:
// d I = 2 d (R + Q / 2), and R + Q / 2 is exact in fp32 (a half-integer far
// below 2^23), so a block whose I is 0 adds exactly 0.
struct ActS1 {
  float d2;  // lane kb: 2 d
  float qh;  // lane kb: Q / 2
};
__device__ __forceinline__ ActS1 act_s1(const ActSub& s) {
  ActS1 r;
  r.d2 = s.d + s.d;
  r.qh = (float)s.Q * 0.5f;
  return r;
}

// Global views of one token's activations (token b at offset b * K).
struct ActG {
  g_u8* q;
  const float __attribute__((address_space(1)))* d;
  const int32_t __attribute__((address_space(1)))* qs;
  int K, kbs;
};

// FULL: the sub-chunk lies wholly inside K and kb_base is wave-uniform, so
// each load is a scalar base plus a fixed per-lane offset (no per-lane address
// arithmetic).  Otherwise (a row's tail) offsets are clamped to stay inside K.
template <int QMUL, bool FULL>
__device__ __forceinline__ void load_act(ActSub& s, const ActG& A, int b, int kb_base) {
  const int i = threadIdx.x & 15;
  if constexpr (FULL) {
    g_u8* qb = A.q + ((int64_t)b * A.K + (int64_t)kb_base * 32);
    const u32x4 v = *(g_u32x4*)(qb + (uint32_t)(16 * i));
    s.a[0] = (int32_t)v.x;
    s.a[1] = (int32_t)v.y;
    s.a[2] = (int32_t)v.z;
    s.a[3] = (int32_t)v.w;
    const int64_t kb0 = (int64_t)b * A.kbs + kb_base;
    s.d = (A.d + kb0)[(uint32_t)(i & 7)];
    s.Q = (A.qs + kb0)[(uint32_t)(i & 7)] * -QMUL;
    return;
  }
  // bytes 16i.. of the sub-chunk; a partial last sub-chunk re-reads valid bytes
  const int off = min(kb_base * 32 + 16 * i, A.K - 16);
  const u32x4 v = *(g_u32x4*)(A.q + (int64_t)b * A.K + off);
  s.a[0] = (int32_t)v.x;
  s.a[1] = (int32_t)v.y;
  s.a[2] = (int32_t)v.z;
  s.a[3] = (int32_t)v.w;
  const int kb = min(kb_base + (i & 7), A.kbs - 1);
  s.d = A.d[(int64_t)b * A.kbs + kb];
  s.Q = A.qs[(int64_t)b * A.kbs + kb] * -QMUL;
}

#define QK_DOT(ACC, A, P, L) "v_dot4c_i32_i8_dpp " ACC ", " A ", " P " row_newbcast:" L " row_mask:0xf bank_mask:0xf\n\t"

// One dot chain.  INT4: R = 2x + Q[KB] (Q = -15 qsum), out = d[KB] * R.
template <int KB>
__device__ __forceinline__ int blk_one_chain_mul2(float& out, const ActSub& s, const uint32_t (&p)[8]) {
  int x, t;
  asm("s_nop 1\n\t"
      "v_mov_b32 %1, 0\n\t"
      QK_DOT("%1", "%3", "%7", "%c17") QK_DOT("%1", "%4", "%8", "%c17")
      QK_DOT("%1", "%5", "%9", "%c17") QK_DOT("%1", "%6", "%10", "%c17")
      QK_DOT("%1", "%3", "%11", "%c18") QK_DOT("%1", "%4", "%12", "%c18")
      QK_DOT("%1", "%5", "%13", "%c18") QK_DOT("%1", "%6", "%14", "%c18")
      "s_nop 2\n\t"
      "v_lshlrev_b32 %1, 1, %1\n\t"
      "v_add_u32_dpp %1, %16, %1 row_newbcast:%c19 row_mask:0xf bank_mask:0xf\n\t"
      "v_cvt_f32_i32 %2, %1\n\t"
      "v_mul_f32_dpp %0, %15, %2 row_newbcast:%c19 row_mask:0xf bank_mask:0xf"
      : "=v"(out), "=&v"(x), "=&v"(t)
      : "v"(s.a[0]), "v"(s.a[1]), "v"(s.a[2]), "v"(s.a[3]), "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]),
        "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7]), "v"(s.d), "v"(s.Q), "n"(2 * KB), "n"(2 * KB + 1), "n"(KB));
  return x;
}

// One dot chain.  TERN: R = x + Q[KB] (Q = -qsum, digits are t + 1); TRELLIS:
// Q = 0.  acc += d[KB] * R.  The chain starts from Q[KB] itself (a DPP move),
// so R needs no separate add.
template <int KB>
__device__ __forceinline__ int blk_one_chain_fmac(float& acc, const ActSub& s, const uint32_t (&p)[8]) {
  int x, t;
  asm("s_nop 1\n\t"
      "v_mov_b32_dpp %1, %16 row_newbcast:%c19 row_mask:0xf bank_mask:0xf\n\t"
      QK_DOT("%1", "%3", "%7", "%c17") QK_DOT("%1", "%4", "%8", "%c17")
      QK_DOT("%1", "%5", "%9", "%c17") QK_DOT("%1", "%6", "%10", "%c17")
      QK_DOT("%1", "%3", "%11", "%c18") QK_DOT("%1", "%4", "%12", "%c18")
      QK_DOT("%1", "%5", "%13", "%c18") QK_DOT("%1", "%6", "%14", "%c18")
      "s_nop 2\n\t"
      "v_cvt_f32_i32 %2, %1\n\t"
      "v_fmac_f32_dpp %0, %15, %2 row_newbcast:%c19 row_mask:0xf bank_mask:0xf"
      : "+v"(acc), "=&v"(x), "=&v"(t)
      : "v"(s.a[0]), "v"(s.a[1]), "v"(s.a[2]), "v"(s.a[3]), "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]),
        "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7]), "v"(s.d), "v"(s.Q), "n"(2 * KB), "n"(2 * KB + 1), "n"(KB));
  return x;
}

__device__ __forceinline__ float scale_half(uint32_t pair, int hi) {
  return __half2float(__ushort_as_half((unsigned short)(hi ? (pair >> 16) : (pair & 0xFFFFu))));
}

template <int... I, typename F>
__device__ __forceinline__ void static_for(std::integer_sequence<int, I...>, F&& f) {
  (f(std::integral_constant<int, I>{}), ...);
}

// ---- 1- and 2-bit codes against 4-bit activation planes ------------------------------------------
// Codes are nibble-lane packed: (word >> j*bits) & 0x11111111 (1-bit) or
// & 0x33333333 (2-bit) holds the codes of 8 consecutive weights, one per
// nibble.  Activations come split as x = 16 hi + lo (lo in 0..15, hi a signed
// nibble), 8 words per 32-block: lo of the block's 4 groups of 8 values, then
// hi.  The block's integer dot is 4 unsigned and 4 signed 8-way nibble dots:
//   sum c x = 16 sum c hi + sum c lo,   I = 2 sum c x - m qsum
// (m = 1 for 1-bit levels 2b - 1, m = 3 for 2-bit levels 2c - 3).
//
// Batches up to 2 read the planes, d and qsum of the block with scalar loads
// (wave-uniform) and use them as the scalar operand of v_dot8 / v_fma: no DPP,
// no accumulator initialisation (the first dot adds to an inline 0) and the
// qsum term folds into one shift-add.
typedef const uint32_t __attribute__((address_space(4))) k_u32;
typedef const int32_t __attribute__((address_space(4))) k_i32;
typedef const float __attribute__((address_space(4))) k_f32;
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef const u32x8 __attribute__((address_space(4))) k_u32x8;

struct ActK {  // wave-uniform views of one item's activations (token b at block b * kbs)
  k_u32* pl;   // planes [B][kbs][8] (32-byte aligned)
  k_f32* d;
  k_i32* qs;
  int kbs;
};

// A constant the compiler keeps in an SGPR (a VOP2 operand) instead of a
// 32-bit literal in every instruction that uses it.
__device__ __forceinline__ uint32_t sgpr_const(uint32_t v) {
  uint32_t r;
  asm("s_mov_b32 %0, %1" : "=s"(r) : "i"(v));
  return r;
}

// The scalar operands of one block for one token: its 8 plane words, d and
// qsum (multiplied out where it is used, so that nothing reads the loaded
// values before the wait for their generation).
struct BlkK {
  u32x8 x;
  float d;
  int qs;
};
__device__ __forceinline__ BlkK load_blk(const ActK& A, int b, int kb) {
  const int64_t blk = (int64_t)b * A.kbs + kb;
  BlkK r;
  r.x = *(k_u32x8*)(A.pl + blk * 8);
  r.d = A.d[blk];
  r.qs = A.qs[blk];
  return r;
}

// I of one block from its four code planes p and the token's scalar operands.
template <int M>
__device__ __forceinline__ int nib_I(const uint32_t (&p)[4], const BlkK& k) {
  uint32_t L = __builtin_amdgcn_udot8(k.x[0], p[0], 0u, false);
  // the first signed dot adds to an inline 0 (the compiler's choice, the
  // accumulating VOP2 form, would need a zeroed register first)
  int H;
  asm("v_dot8_i32_i4 %0, %1, %2, 0" : "=v"(H) : "s"(k.x[4]), "v"(p[0]));
  L = __builtin_amdgcn_udot8(k.x[1], p[1], L, false);
  H = __builtin_amdgcn_sdot8((int)k.x[5], (int)p[1], H, false);
  L = __builtin_amdgcn_udot8(k.x[2], p[2], L, false);
  H = __builtin_amdgcn_sdot8((int)k.x[6], (int)p[2], H, false);
  L = __builtin_amdgcn_udot8(k.x[3], p[3], L, false);
  H = __builtin_amdgcn_sdot8((int)k.x[7], (int)p[3], H, false);
  // 32 H + 2 L - m qsum as two shift-adds, -m qsum a scalar operand (written
  // out: the compiler would rather shift and subtract separately)
  int r;
  asm("v_lshl_add_u32 %0, %1, 1, %2\n\t"
      "v_lshl_add_u32 %0, %3, 5, %0"
      : "=&v"(r)
      : "v"(L), "s"(-M * k.qs), "v"(H));
  return r;
}

// Scalar-operand pipeline of the 1- and 2-bit formats at batches up to 2.  A
// wait for any scalar load waits for all of them (they return out of order),
// so the operands of G blocks (every token) travel as one generation: right
// after the wait for generation i the loads of generation i + 1 are issued,
// and they land while generation i is computed.  Two generations of 20 scalar
// registers are live.
template <int NB>
struct KPipe {
  static constexpr int G = NB <= 2 ? 2 / NB : 1;  // blocks per generation (batches up to 2)
  BlkK buf[2][G][NB];
};

template <int M, int PAR, int NB>
__device__ __forceinline__ void kpipe_issue(KPipe<NB>& kp, const ActK& A, int kb) {
  // The generation's base addresses pass through an empty asm: its loads can
  // neither move above this point nor merge with another generation's loads
  // (a merged load would be waited for with the current generation).
  ActK a = A;
  asm volatile("" : "+s"(a.pl), "+s"(a.d), "+s"(a.qs));
  static_for(std::make_integer_sequence<int, KPipe<NB>::G>{}, [&](auto jc) {
    constexpr int j = decltype(jc)::value;
#pragma unroll
    for (int b = 0; b < NB; ++b) kp.buf[PAR][j][b] = load_blk(a, b, kb + j);
  });
}

// Waits for every scalar (and LDS) load of the wave; nothing moves across.
__device__ __forceinline__ void kpipe_wait() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
}

// Generation GI of a sub-chunk (blocks GI*G ..): with PIPE, wait for it and
// issue the next one (the first of the following sub-chunk, kb_after, after
// the last); without, load it and let the compiler wait.
template <int M, int GI, bool PIPE, int NB>
__device__ __forceinline__ void kpipe_step(KPipe<NB>& kp, const ActK& A, int kb0, int kbv, int kb_after) {
  constexpr int G = KPipe<NB>::G, NGS = 8 / G;
  if constexpr (PIPE) {
    kpipe_wait();
    if constexpr (GI + 1 < NGS) kpipe_issue<M, (GI + 1) & 1>(kp, A, kb0 + (GI + 1) * G);
    else kpipe_issue<M, 0>(kp, A, kb_after);
    __builtin_amdgcn_sched_barrier(0);
  } else {
    static_for(std::make_integer_sequence<int, G>{}, [&](auto jc) {
      constexpr int j = decltype(jc)::value;
      if (GI * G + j < kbv)
#pragma unroll
        for (int b = 0; b < NB; ++b) kp.buf[GI & 1][j][b] = load_blk(A, b, kb0 + GI * G + j);
    });
  }
}

#define QK_DOT8(ACC, A, P, L) "v_dot8c_i32_i4_dpp " ACC ", " A ", " P " row_newbcast:" L " row_mask:0xf bank_mask:0xf\n\t"

// Larger batches keep the DPP row-broadcast activations (ActSub, here holding
// planes: lane 2KB of a row the lo words of block KB, lane 2KB+1 the hi words).
// v_dot8c is signed on both sides, so the lo words arrive xor 0x88888888
// (lo - 8 as a signed nibble) and c16 = 16 * (sum of the block's codes) adds
// the 8 sum c back:  I = 2 (16 H + L') + c16 + Q,  Q = -m qsum.
// out = d * I (MUL) or acc += d * I.
template <int KB, bool MUL>
__device__ __forceinline__ void nib_blk_dpp(float& acc, const ActSub& s, const uint32_t (&p)[4], uint32_t c16) {
  int x, z;
  if constexpr (MUL) {
    asm("s_nop 1\n\t"
        "v_mov_b32 %1, 0\n\t"
        "v_mov_b32 %2, 0\n\t"
        QK_DOT8("%1", "%3", "%7", "%c14") QK_DOT8("%2", "%3", "%7", "%c15")
        QK_DOT8("%1", "%4", "%8", "%c14") QK_DOT8("%2", "%4", "%8", "%c15")
        QK_DOT8("%1", "%5", "%9", "%c14") QK_DOT8("%2", "%5", "%9", "%c15")
        QK_DOT8("%1", "%6", "%10", "%c14") QK_DOT8("%2", "%6", "%10", "%c15")
        "s_nop 2\n\t"
        "v_lshl_add_u32 %1, %2, 4, %1\n\t"
        "v_lshl_add_u32 %1, %1, 1, %11\n\t"
        "v_add_u32_dpp %1, %13, %1 row_newbcast:%c16 row_mask:0xf bank_mask:0xf\n\t"
        "v_cvt_f32_i32 %2, %1\n\t"
        "v_mul_f32_dpp %0, %12, %2 row_newbcast:%c16 row_mask:0xf bank_mask:0xf"
        : "=v"(acc), "=&v"(x), "=&v"(z)
        : "v"(s.a[0]), "v"(s.a[1]), "v"(s.a[2]), "v"(s.a[3]), "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]),
          "v"(c16), "v"(s.d), "v"(s.Q), "n"(2 * KB), "n"(2 * KB + 1), "n"(KB));
  } else {
    asm("s_nop 1\n\t"
        "v_mov_b32 %1, 0\n\t"
        "v_mov_b32 %2, 0\n\t"
        QK_DOT8("%1", "%3", "%7", "%c14") QK_DOT8("%2", "%3", "%7", "%c15")
        QK_DOT8("%1", "%4", "%8", "%c14") QK_DOT8("%2", "%4", "%8", "%c15")
        QK_DOT8("%1", "%5", "%9", "%c14") QK_DOT8("%2", "%5", "%9", "%c15")
        QK_DOT8("%1", "%6", "%10", "%c14") QK_DOT8("%2", "%6", "%10", "%c15")
        "s_nop 2\n\t"
        "v_lshl_add_u32 %1, %2, 4, %1\n\t"
        "v_lshl_add_u32 %1, %1, 1, %11\n\t"
        "v_add_u32_dpp %1, %13, %1 row_newbcast:%c16 row_mask:0xf bank_mask:0xf\n\t"
        "v_cvt_f32_i32 %2, %1\n\t"
        "v_fmac_f32_dpp %0, %12, %2 row_newbcast:%c16 row_mask:0xf bank_mask:0xf"
        : "+v"(acc), "=&v"(x), "=&v"(z)
        : "v"(s.a[0]), "v"(s.a[1]), "v"(s.a[2]), "v"(s.a[3]), "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]),
          "v"(c16), "v"(s.d), "v"(s.Q), "n"(2 * KB), "n"(2 * KB + 1), "n"(KB));
  }
}

// 1-bit block KB against DPP planes: acc += 2 d (R + Q / 2) = d I, with
// R = sum b x = 16 H + L.  The lo words arrive as lo - 8, so sum b lo = L' + 8 n
// (n = the block's set bits); the chains start at H = n and L = -8 n, which
// adds exactly 16 n - 8 n.
template <int KB>
__device__ __forceinline__ int nib1_blk_dpp(float& acc, const ActSub& s, const ActS1& s1, const uint32_t (&p)[4],
                                            uint32_t n, int m8n) {
  int x = m8n, z = (int)n;
  asm("s_nop 1\n\t"
      QK_DOT8("%1", "%3", "%7", "%c13") QK_DOT8("%2", "%3", "%7", "%c14")
      QK_DOT8("%1", "%4", "%8", "%c13") QK_DOT8("%2", "%4", "%8", "%c14")
      QK_DOT8("%1", "%5", "%9", "%c13") QK_DOT8("%2", "%5", "%9", "%c14")
      QK_DOT8("%1", "%6", "%10", "%c13") QK_DOT8("%2", "%6", "%10", "%c14")
      "s_nop 2\n\t"
      "v_lshl_add_u32 %1, %2, 4, %1\n\t"
      "v_cvt_f32_i32 %2, %1\n\t"
      "v_add_f32_dpp %2, %12, %2 row_newbcast:%c15 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %11, %2 row_newbcast:%c15 row_mask:0xf bank_mask:0xf"
      : "+v"(acc), "+v"(x), "+v"(z)
      : "v"(s.a[0]), "v"(s.a[1]), "v"(s.a[2]), "v"(s.a[3]), "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]),
        "v"(s1.d2), "v"(s1.qh), "n"(2 * KB), "n"(2 * KB + 1), "n"(KB));
  return x;
}

// 2 R + Q[KB]: the exact block dot I from R (test hook).  Volatile: the
// broadcast reads lane KB, so it must run with the whole wave active (never
// inside a branch on the lane's row).
template <int KB>
__device__ __forceinline__ int blk_I_dpp(int R, const ActSub& s) {
  int t;
  asm volatile("s_nop 1\n\t"
      "v_add_u32_dpp %0, %1, %2 row_newbcast:%c3 row_mask:0xf bank_mask:0xf"
      : "=v"(t)
      : "v"(s.Q), "v"(R), "n"(KB));
  return t + R;
}

// ---- per-format compute of one 256-weight sub-chunk --------------------------------------------------
// T: the lane's row codes of the whole segment (dwords), SUB: sub-chunk index
// in the segment, S: the segment's fp16 scales (pairs).  AS[b]: DPP activations
// of token b (batches above 2 and the byte formats), AK: scalar activation
// views (1- and 2-bit at batches up to 2), kb0: the sub-chunk's first block,
// kbv: its valid blocks (8 except in a tail).  y accumulates (final per-format
// factor applied by the caller).
template <int NB, int SUB, bool WI, bool PIPE>
__device__ __forceinline__ void sub_sign1(const uint32_t (&T)[32], const uint32_t (&S)[4], const ActSub (&AS)[NB],
                                          KPipe<NB>& kp, const ActK& AK, int kb0, int kbv, int kb_after,
                                          float (&y)[NB], int32_t* Iout) {
  const uint32_t m1 = sgpr_const(0x11111111u);
  ActS1 A1[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) A1[b] = act_s1(AS[b]);
  static_for(std::make_integer_sequence<int, 2>{}, [&](auto hc) {  // two 128-weight scale blocks
    constexpr int h = decltype(hc)::value;
    float acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = 0.0f;
    static_for(std::make_integer_sequence<int, 4>{}, [&](auto jc) {
      constexpr int kb = 4 * h + decltype(jc)::value;  // activation block within the sub-chunk
      if (kb < kbv) {
        const uint32_t W = T[SUB * 8 + kb];
        const uint32_t p[4] = {W & m1, (W >> 1) & m1, (W >> 2) & m1, (W >> 3) & m1};
        const uint32_t n = (uint32_t)__builtin_popcount(W);
        int m8n;  // -8 n in one multiply (the compiler would shift and negate)
        asm("v_mul_i32_i24 %0, -8, %1" : "=v"(m8n) : "v"(n));
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int R = nib1_blk_dpp<kb>(acc[b], AS[b], A1[b], p, n, m8n);
          if constexpr (WI) {
            if (b == 0) {
              const int I = blk_I_dpp<kb>(R, AS[0]);
              if (Iout) Iout[SUB * 8 + kb] = I;
            }
          }
        }
      }
    });
    const float s = scale_half(S[SUB], h);
#pragma unroll
    for (int b = 0; b < NB; ++b) y[b] = __builtin_fmaf(s, acc[b], y[b]);
  });
}

template <int NB, int SUB, bool WI, bool PIPE>
__device__ __forceinline__ void sub_int2(const uint32_t (&T)[32], const uint32_t (&S)[8], const ActSub (&AS)[NB],
                                         KPipe<NB>& kp, const ActK& AK, int kb0, int kbv, int kb_after,
                                         float (&y)[NB], int32_t* Iout) {
  const uint32_t m3 = sgpr_const(0x33333333u);
  auto planes = [&](int kb, uint32_t (&p)[4]) {
    const uint32_t W0 = T[SUB * 16 + 2 * kb], W1 = T[SUB * 16 + 2 * kb + 1];
    p[0] = W0 & m3;
    p[1] = (W0 >> 2) & m3;
    p[2] = W1 & m3;
    p[3] = (W1 >> 2) & m3;
  };
  auto scale = [&](int kb) {
    const int si = SUB * 8 + kb;  // scale index within the segment
    return scale_half(S[si >> 1], si & 1);
  };
  if constexpr (NB <= 2) {
    constexpr int G = KPipe<NB>::G;
    static_for(std::make_integer_sequence<int, 8 / G>{}, [&](auto gc) {
      constexpr int GI = decltype(gc)::value;
      kpipe_step<3, GI, PIPE>(kp, AK, kb0, kbv, kb_after);
      static_for(std::make_integer_sequence<int, G>{}, [&](auto jc) {
        constexpr int kb = GI * G + decltype(jc)::value;
        if (kb < kbv) {
          uint32_t p[4];
          planes(kb, p);
          const float s = scale(kb);
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const BlkK& k = kp.buf[GI & 1][kb - GI * G][b];
            const int I = nib_I<3>(p, k);
            if (WI && b == 0 && Iout) Iout[SUB * 8 + kb] = I;
            y[b] = __builtin_fmaf(s, k.d * (float)I, y[b]);
          }
        }
      });
    });
  } else {
    static_for(std::make_integer_sequence<int, 8>{}, [&](auto kc) {
      constexpr int kb = decltype(kc)::value;
      if (kb < kbv) {
        uint32_t p[4];
        planes(kb, p);
        const float s = scale(kb);
        // sum of the block's 32 codes: nibble sums of the 4 planes stay below 16
        const uint32_t csum = __builtin_amdgcn_udot8(p[0] + p[1] + p[2] + p[3], 0x11111111u, 0u, false);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          float t;
          nib_blk_dpp<kb, true>(t, AS[b], p, csum << 4);
          y[b] = __builtin_fmaf(s, t, y[b]);
        }
      }
    });
  }
}

template <int KB, int NB, bool WI, int MODE>
__device__ __forceinline__ void blk_dispatch(float (&out)[NB], const ActSub (&AS)[NB], const uint32_t (&p)[8],
                                             int32_t* Iout, int idx) {
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    int R;
    if constexpr (MODE == 1) R = blk_one_chain_mul2<KB>(out[b], AS[b], p);               // INT4
    else R = blk_one_chain_fmac<KB>(out[b], AS[b], p);                                   // TERN, TRELLIS
    if (WI && b == 0 && Iout) Iout[idx] = R;
  }
}

template <int NB, bool WI, int MODE>
__device__ __forceinline__ void blk_any(int kb, float (&out)[NB], const ActSub (&AS)[NB], const uint32_t (&p)[8],
                                        int32_t* Iout, int idx) {
  switch (kb) {
    case 0: blk_dispatch<0, NB, WI, MODE>(out, AS, p, Iout, idx); break;
    case 1: blk_dispatch<1, NB, WI, MODE>(out, AS, p, Iout, idx); break;
    case 2: blk_dispatch<2, NB, WI, MODE>(out, AS, p, Iout, idx); break;
    case 3: blk_dispatch<3, NB, WI, MODE>(out, AS, p, Iout, idx); break;
    case 4: blk_dispatch<4, NB, WI, MODE>(out, AS, p, Iout, idx); break;
    case 5: blk_dispatch<5, NB, WI, MODE>(out, AS, p, Iout, idx); break;
    case 6: blk_dispatch<6, NB, WI, MODE>(out, AS, p, Iout, idx); break;
    default: blk_dispatch<7, NB, WI, MODE>(out, AS, p, Iout, idx); break;
  }
}

template <int NB, bool WI>
__device__ __forceinline__ void sub_int4(const uint32_t (&T)[32], const uint32_t (&S)[4], const ActSub (&AS)[NB],
                                         float (&y)[NB], int32_t* Iout) {
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    uint32_t p[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t W = T[4 * kb + m];
      p[2 * m] = W & 0x0F0F0F0Fu;
      p[2 * m + 1] = (W >> 4) & 0x0F0F0F0Fu;
    }
    float t[NB];
    blk_any<NB, WI, 1>(kb, t, AS, p, Iout, kb);
    const float s = scale_half(S[kb >> 1], kb & 1);
#pragma unroll
    for (int b = 0; b < NB; ++b) y[b] = __builtin_fmaf(s, t[b], y[b]);
  }
}

// Ternary: 13 words of one 256-weight block; digit dwords come out in
// activation-dword order g = 0..63 (word m < 12: g = 5m + i; word 12: 60 + i).
template <int NB, int SUB, bool WI>
__device__ __forceinline__ void sub_tern(const uint32_t (&T)[52], const uint32_t (&S)[2], const ActSub (&AS)[NB],
                                         float (&y)[NB], int32_t* Iout) {
  float acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = 0.0f;
  // Words and digits are walked with compile-time indices (static_for), so the
  // code words stay in registers even where a loop of this size would not be
  // fully unrolled (an indexed register array would fall back to scratch).
  uint32_t p[8];
  static_for(std::make_integer_sequence<int, 13>{}, [&](auto mc) {
    constexpr int m = decltype(mc)::value;
    const uint32_t W = T[13 * SUB + m];
    uint32_t xl = W & 0x00FF00FFu;         // bytes 0, 2 in 16-bit lanes
    uint32_t xh = (W >> 8) & 0x00FF00FFu;  // bytes 1, 3
    constexpr int ndig = m < 12 ? 5 : 4;
    static_for(std::make_integer_sequence<int, ndig>{}, [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const uint32_t yl = xl * 3u, yh = xh * 3u;
      constexpr int g = m < 12 ? 5 * m + i : 60 + i;
      // the next digit of every byte sits in bits 8..9 of its 16-bit lane
      p[g & 7] = __builtin_amdgcn_perm(yh, yl, 0x07030501u);
      if constexpr (i + 1 < ndig) {
        xl = yl & 0x00FF00FFu;
        xh = yh & 0x00FF00FFu;
      }
      if constexpr ((g & 7) == 7) blk_any<NB, WI, 2>(g >> 3, acc, AS, p, Iout, SUB * 8 + (g >> 3));
    });
  });
  const float s = scale_half(S[SUB >> 1], SUB & 1);
#pragma unroll
  for (int b = 0; b < NB; ++b) y[b] = __builtin_fmaf(s, acc[b], y[b]);
}

// ---- trellis codebook lookups ---------------------------------------------------------------------
// The int8 codebook sits in LDS once per lane of a half-wave, in two
// pre-shifted forms: entry h of copy c = lane % 32 is the dword v << 24 at
// byte h * 256 + 4 c and the dword v << 16 at byte h * 256 + 128 + 4 c
// (v = the entry's byte).  The 32 lanes of a half-wave then read 32 different
// banks whatever their hashes (one shared 256-byte table costs about 1.7x as
// much per read: two of its dwords share each of the 32 banks), and reads of
// different widths and offsets return v alone in byte 0, 1, 2 or 3:
//   u8 at +3: v;  u16 at +2: v << 8;  b32 at +128: v << 16;  b32 at +0: v << 24.
// The table starts at LDS address 0, so a lookup's address register is the
// address itself.
constexpr int kTrellisTableBytes = 65536;

// Lookup state of one wave: the table and 16 standing address registers, each
// holding 4 (lane % 32) in byte 0 and zeros in bytes 2 and 3.  A lookup only
// rewrites byte 1 with the hash, so the address costs two instructions.
struct TrellisCtx {
  const uint8_t* tbl;
  uint32_t ad[16];
};

__device__ __forceinline__ void trellis_ctx_init(TrellisCtx& c, const uint8_t* tbl) {
  c.tbl = tbl;
#pragma unroll
  for (int i = 0; i < 16; ++i) c.ad[i] = (threadIdx.x & 31u) << 2;
}

// Fills the replicated table from the 256 codebook entries (every thread of
// the workgroup takes part; a barrier must follow before any lookup).
__device__ __forceinline__ void trellis_table_fill(uint8_t* tbl, const V8Table& v8t) {
  for (int i = threadIdx.x; i < 256 * 32; i += blockDim.x) {
    const int h = i >> 5, c = i & 31;
    const uint32_t v = (uint8_t)v8t.v[h];
    *(uint32_t*)(tbl + h * 256 + c * 4) = v << 24;
    *(uint32_t*)(tbl + h * 256 + 128 + c * 4) = v << 16;
  }
}

// h = ((st * 0x9E37) ^ (st >> 7)) & 0xFF of the 16-bit states of the four
// weights of one code byte, written into byte 1 of their address registers
// ad[0..3]: the low byte of st * 0x9E37 depends only on lo8 = st & 0xFF, and
// (st >> 7) & 0xFF is mid8 = bits 7..14 of st.  Weight k's lo8 is byte M of
// lo[k] and its mid8 byte M of mid[k] (SDWA byte selects; each multiply writes
// the low 8 bits of lo8 * 0x9E37 into byte 1, each XOR folds mid8 in, both
// leaving the other bytes as they are).  A VALU read of a register right after
// a partial (SDWA dst_sel) write of it sees the unmerged result on this part,
// so the four multiplies come first, then the XORs, then one wait state before
// anything reads the addresses.
template <int M>
__device__ __forceinline__ void trellis_addr4(uint32_t& a0, uint32_t& a1, uint32_t& a2, uint32_t& a3,
                                              const uint32_t (&lo)[4], const uint32_t (&mid)[4], uint32_t mul) {
#define QK_TR_MUL(D, L, B) \
  "v_mul_u32_u24_sdwa " D ", " L ", %12 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_" #B " src1_sel:DWORD\n\t"
#define QK_TR_XOR(D, X, B) \
  "v_xor_b32_sdwa " D ", " D ", " X " dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1 src1_sel:BYTE_" #B "\n\t"
#define QK_TR_ADDR4(B)                                                                                  \
  asm(QK_TR_MUL("%0", "%4", B) QK_TR_MUL("%1", "%5", B) QK_TR_MUL("%2", "%6", B) QK_TR_MUL("%3", "%7", B) \
      QK_TR_XOR("%0", "%8", B) QK_TR_XOR("%1", "%9", B) QK_TR_XOR("%2", "%10", B) QK_TR_XOR("%3", "%11", B) \
      "s_nop 0"                                                                                          \
      : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3)                                                           \
      : "v"(lo[0]), "v"(lo[1]), "v"(lo[2]), "v"(lo[3]), "v"(mid[0]), "v"(mid[1]), "v"(mid[2]), "v"(mid[3]), "s"(mul))
  if constexpr (M == 0) QK_TR_ADDR4(0);
  else if constexpr (M == 1) QK_TR_ADDR4(1);
  else if constexpr (M == 2) QK_TR_ADDR4(2);
  else QK_TR_ADDR4(3);
#undef QK_TR_ADDR4
#undef QK_TR_XOR
#undef QK_TR_MUL
}

typedef const uint8_t __attribute__((address_space(3))) l_u8;
typedef const uint16_t __attribute__((address_space(3))) l_u16;
typedef const uint32_t __attribute__((address_space(3))) l_u32;

// Codebook values of the 16 weights of one code word W (4 code bytes, first
// byte in stream order in the low byte), as 4 dwords of int8 lined up with the
// activation dwords: p[O + g] holds weights 4g .. 4g + 3.  `be` holds the
// previous code bytes big-endian in its low 16 bits and is left holding W's.
// With BE = W byte-reversed, (be : BE) >> s exposes the stream shifted by s
// bits: weight 4g + j has the 16-bit state ((B[g-2] B[g-1] B[g]) >> (6 - 2j)),
// whose lo8 is byte 3 - g of the stream shifted by 6 - 2j and whose mid8 is
// byte 3 - g of the stream shifted by 13 - 2j.
template <int O>
__device__ __forceinline__ void trellis_word(TrellisCtx& c, uint32_t W, uint32_t& be, uint32_t (&p)[8], uint32_t mul) {
  const uint32_t BE = __builtin_amdgcn_perm(W, W, 0x00010203u);
  uint32_t lo[4], mid[4];
  lo[0] = BE;
#pragma unroll
  for (int k = 1; k < 4; ++k) lo[k] = __builtin_amdgcn_alignbit(be, BE, 2 * k);
#pragma unroll
  for (int k = 0; k < 4; ++k) mid[k] = __builtin_amdgcn_alignbit(be, BE, 2 * k + 7);
  l_u8* t = (l_u8*)c.tbl;
  static_for(std::make_integer_sequence<int, 4>{}, [&](auto gc) {
    constexpr int g = decltype(gc)::value, m = 3 - g;
    trellis_addr4<m>(c.ad[4 * g], c.ad[4 * g + 1], c.ad[4 * g + 2], c.ad[4 * g + 3], lo, mid, mul);
    // weight 4g + j uses shift 2k = 6 - 2j; each read lands its value alone in
    // byte j (written out: the compiler would narrow the ORs to 16 bits and mask)
    const uint32_t r0 = t[c.ad[4 * g + 3] + 3];
    const uint32_t r1 = *(l_u16*)(t + c.ad[4 * g + 2] + 2);
    const uint32_t r2 = *(l_u32*)(t + c.ad[4 * g + 1] + 128);
    const uint32_t r3 = *(l_u32*)(t + c.ad[4 * g + 0]);
    uint32_t w;
    asm("v_or3_b32 %0, %1, %2, %3\n\tv_or_b32 %0, %0, %4" : "=&v"(w) : "v"(r0), "v"(r1), "v"(r2), "v"(r3));
    p[O + g] = w;
  });
  be = BE;
}

// Trellis: `prev` holds the last 16 bits of seed||bytes before the sub-chunk
// (big-endian, higher bits ignored).
template <int NB, int SUB, bool WI>
__device__ __forceinline__ void sub_trellis(const uint32_t (&T)[32], const uint32_t (&S)[4], const ActSub (&AS)[NB],
                                            uint32_t& prev, TrellisCtx& tc, float (&y)[NB], int32_t* Iout) {
  const uint32_t mul = sgpr_const(0x9E37u);
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {  // 64-weight scale blocks
    float acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = 0.0f;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int kb = sb * 2 + h2;
      uint32_t p[8];
      trellis_word<0>(tc, T[SUB * 16 + kb * 2], prev, p, mul);
      trellis_word<4>(tc, T[SUB * 16 + kb * 2 + 1], prev, p, mul);
      blk_any<NB, WI, 2>(kb, acc, AS, p, Iout, SUB * 8 + kb);
    }
    const int si = SUB * 4 + sb;
    const float s = scale_half(S[si >> 1], si & 1);
#pragma unroll
    for (int b = 0; b < NB; ++b) y[b] = __builtin_fmaf(s, acc[b], y[b]);
  }
}

// ---- scale loads ---------------------------------------------------------------------------------
// The SPS fp16 scales of one lane's row for one segment: SPS contiguous values
// of the tiled scale layout (16-byte aligned), as SPS/2 packed pairs.
template <int SPS>
__device__ __forceinline__ void load_scales(g_u16* p, uint32_t (&S)[SPS / 2]) {
  if constexpr (SPS >= 8) {
#pragma unroll
    for (int i = 0; i < SPS / 8; ++i) {
      const u32x4 v = *(g_u32x4*)(p + 8 * i);
      S[4 * i] = v.x;
      S[4 * i + 1] = v.y;
      S[4 * i + 2] = v.z;
      S[4 * i + 3] = v.w;
    }
  } else {
    const u32x2 v = *(g_u32x2*)p;
    S[0] = v.x;
    S[1] = v.y;
  }
}

// Multiple of qsum each format's block result subtracts (see the asm blocks).
template <int FMT> struct QMul;
template <> struct QMul<QFMT_SIGN1> { static constexpr int v = 1; };
template <> struct QMul<QFMT_INT2> { static constexpr int v = 3; };
template <> struct QMul<QFMT_INT4> { static constexpr int v = 15; };
template <> struct QMul<QFMT_TERN_B3> { static constexpr int v = 1; };
template <> struct QMul<QFMT_TRELLIS2> { static constexpr int v = 0; };

template <int FMT, int NB, bool FULL = true>
__device__ __forceinline__ void load_act_all(ActSub (&dst)[NB], const ActG& AG, int kb_base, int kbv) {
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    load_act<QMul<FMT>::v, FULL>(dst[b], AG, b, kb_base);
    if constexpr (FMT == QFMT_SIGN1 || FMT == QFMT_INT2) {
      // plane words: even lanes of a row hold lo words, used as lo - 8 (signed)
      const uint32_t f = (threadIdx.x & 1) ? 0u : 0x88888888u;
#pragma unroll
      for (int k = 0; k < 4; ++k) dst[b].a[k] = (int32_t)((uint32_t)dst[b].a[k] ^ f);
    }
    if (kbv < 8 && (int)(threadIdx.x & 7) >= kbv) {  // blocks past the end of K contribute nothing
      dst[b].d = 0.0f;
      dst[b].Q = 0;
    }
  }
}

// One sub-chunk of a segment; Ib: test-hook row output at the sub-chunk's
// first activation block (entries below ivalid are written).
template <int FMT, int NB, int SUB, bool WI, bool PIPE = false>
__device__ __forceinline__ void sub_compute(const uint32_t (&T)[Seg<FMT>::CH * 4], const uint32_t (&S)[Seg<FMT>::SPS / 2],
                                            const ActSub (&AS)[NB], KPipe<NB>& kp, const ActK& AK, int kb0, int kbv,
                                            int kb_after, uint32_t& prev, TrellisCtx& tc, float (&y)[NB],
                                            int32_t* Iseg) {
  if constexpr (FMT == QFMT_SIGN1) sub_sign1<NB, SUB, WI, PIPE>(T, S, AS, kp, AK, kb0, kbv, kb_after, y, Iseg);
  else if constexpr (FMT == QFMT_INT2) sub_int2<NB, SUB, WI, PIPE>(T, S, AS, kp, AK, kb0, kbv, kb_after, y, Iseg);
  else if constexpr (FMT == QFMT_INT4) sub_int4<NB, WI>(T, S, AS, y, Iseg);
  else if constexpr (FMT == QFMT_TERN_B3) sub_tern<NB, SUB, WI>(T, S, AS, y, Iseg);
  else sub_trellis<NB, SUB, WI>(T, S, AS, prev, tc, y, Iseg);
}

// Result scale applied once per row after accumulation.
template <int FMT>
__device__ __forceinline__ float final_scale(float trellis_gain) {
  if constexpr (FMT == QFMT_SIGN1) return 1.0f;
  else if constexpr (FMT == QFMT_INT2) return 0.5f;
  else if constexpr (FMT == QFMT_INT4) return 0.5f;
  else if constexpr (FMT == QFMT_TERN_B3) return 1.0f;
  else return trellis_gain;
}

// Waits for every vector-memory load of this wave, LDS-DMA tile loads
// included, and keeps the compiler from moving memory accesses across the
// wait.  The compiler's own LDS-DMA tracking is not relied on: it can leave out
// the wait before an LDS read of a DMA'd region.
__device__ __forceinline__ void wait_vm_all() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt/lgkmcnt untouched
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Waits for every load of the wave (vector, LDS-DMA, scalar and LDS).
__device__ __forceinline__ void wait_all() {
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Cache policy of the weight-tile loads: non-temporal (weights stream through
// once per call; the activations and scales they would evict are reused) where
// a row segment is whole 128-byte lines.  A ternary segment (208 bytes) is
// not: the line at each boundary belongs to two consecutive segments, and
// non-temporal loads fetched it from memory twice (1.5x the weight bytes);
// ordinary loads find it in L2 for most boundaries.
template <int FMT> struct TileCachePolicy { static constexpr int v = FMT == QFMT_TERN_B3 ? 0 : 2; };
constexpr int kTileCachePolicy = 2;  // nt

// ---- one 64-row tile ----------------------------------------------------------------------------------
// Accumulates (unscaled by final_scale) into y for segments wk, wk + nwk, ...
// and the tail segment if (nseg % nwk) == wk.  lds: this wave's region.
template <int FMT, int NB, bool WI>
__device__ __forceinline__ void gemv_tile(const GemvItem& it, int row0, int wk, int nwk, uint8_t* lds,
                                          const uint8_t* v8, float (&y)[NB], int32_t* Ibase, int sk = 0,
                                          int sn = 1) {
  constexpr int CH = Seg<FMT>::CH;
  constexpr int SEGK = Seg<FMT>::K;
  constexpr int SPS = Seg<FMT>::SPS;
  constexpr int SEGB = CH * 16;
  constexpr int NSUB = SEGK / 256;
  const int lane = threadIdx.x & 63;
  const int K = it.cols;
  const int N = it.rows;
  const int nseg = K / SEGK;
  const int nvalid = min(64, N - row0);
  const int row = row0 + (lane < nvalid ? lane : nvalid - 1);  // clamp: reads stay in bounds
  const int64_t rb = it.row_bytes;
  const int nsb = K / Seg<FMT>::WBLK;

  ActG AG;
  AG.q = gptr<g_u8*>(it.q);
  AG.d = gptr<const float __attribute__((address_space(1)))*>(it.d);
  AG.qs = gptr<const int32_t __attribute__((address_space(1)))*>(it.qsum);
  AG.K = K;
  AG.kbs = K >> 5;
  // 2-bit at batches up to 2: activations by scalar loads only
  constexpr bool KACT = FMT == QFMT_INT2 && NB <= 2;
  ActK AK;
  AK.pl = gptr<k_u32*>(it.q);
  AK.d = gptr<k_f32*>(it.d);
  AK.qs = gptr<k_i32*>(it.qsum);
  AK.kbs = K >> 5;
  KPipe<NB> kp;
  TrellisCtx tc;
  if constexpr (FMT == QFMT_TRELLIS2) trellis_ctx_init(tc, v8);

  // This lane's scales for segment sg: slot `lane` of the tile's group sg (rows
  // past the end read zero padding).
  static_assert(SPS == scale_group(FMT) && SPS * Seg<FMT>::WBLK == SEGK, "scale groups are GEMV segments");
  g_u16* stile = gptr<g_u16*>(it.scales) + (int64_t)(row0 >> 6) * ((nsb + SPS - 1) / SPS) * 64 * SPS + lane * SPS;
  auto sptr = [&](int sg) { return stile + (int64_t)sg * 64 * SPS; };
  // Only lanes that own a row write the test-hook output.
  int32_t* Irow = (WI && lane < nvalid) ? Ibase + (int64_t)row * (K >> 5) : nullptr;
  g_u8* tile = gptr<g_u8*>(it.codes) + (int64_t)row0 * rb;

  // Per-lane offsets of the coalesced tile load and its LDS slot.  Rows past
  // the end of the matrix re-read the last valid row (no branch per load);
  // the lanes that would own them compute on it and store nothing.
  // Tile loads go straight to LDS (global_load_lds_dwordx4): load i puts lane
  // l's 16 bytes at slot 64 i + l of this wave's region.  For 8-chunk segments
  // slot s holds row s / 8, chunk (s % 8) ^ ((row / 2) % 8), so lane r reads its
  // chunk k from slot 8 r + (k ^ ((r / 2) % 8)): the 16 lanes of a 16-byte read
  // phase then hit 16 different 16-byte slots modulo 256 bytes (gfx950 LDS: 64
  // four-byte banks), where (k ^ (r % 8)) pairs lanes r and r + 8 on one slot.
  // 13-chunk segments are plain row-major (13 is odd: conflict free).  Each
  // load instruction still covers whole 128-byte lines.
  auto tile_off = [&](int i) -> uint32_t {
    const int f = i * 64 + lane;
    const int r = f / CH, pos = f % CH;
    const int c = CH == 8 ? (pos ^ ((r >> 1) & 7)) : pos;
    return (uint32_t)(min(r, nvalid - 1) * rb + c * 16);
  };
  // The whole-segment pipeline (batches up to 2) keeps the offsets
  // in registers; the sub-chunk loop, short of registers, recomputes them at
  // each issue (a few VALU per load).
  constexpr int NOFF = NB <= 2 ? CH : 1;
  uint32_t goff[NOFF];
#pragma unroll
  for (int i = 0; i < NOFF; ++i) goff[i] = tile_off(i);
  // real == false: no tile data is needed.  With the offsets in registers
  // (batches up to 2) nothing is loaded (a wave-uniform branch; every segment
  // top waits for all loads in flight, so nothing depends on the count
  // issued), and the lane offsets are made opaque at each issue so that each
  // address stays a scalar base plus a 32-bit lane offset (no 64-bit per-lane
  // pointers hoisted out of the loop).  Otherwise every lane re-reads the
  // tile's first 16 bytes (one cached line), which keeps the register count
  // of the larger batches down.
  auto issue_tile = [&](int sg, bool real) {
    if constexpr (NOFF == CH) {
      if (!real) return;
    }
    g_u8* tseg = tile + (real ? (int64_t)sg * SEGB : 0);
    const uint32_t keep = (NOFF == CH || real) ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if constexpr (NOFF == CH) asm volatile("" : "+v"(goff[i < NOFF ? i : 0]));
      const uint32_t off = NOFF == CH ? goff[i < NOFF ? i : 0] : tile_off(i);
      if constexpr (TileCachePolicy<FMT>::v == 0)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(tseg + (off & keep)),
                                         (__attribute__((address_space(3))) void*)(lds + i * 1024), 16, 0,
                                         0);
      else
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(tseg + (off & keep)),
                                         (__attribute__((address_space(3))) void*)(lds + i * 1024), 16, 0,
                                         kTileCachePolicy);
    }
  };

  uint32_t S[SPS / 2], Sn[SPS / 2];
  int seg = wk;
  auto read_row = [&](uint32_t (&T)[CH * 4]) {
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int off = CH == 8 ? lane * 128 + ((k ^ ((lane >> 1) & 7)) << 4) : lane * (CH * 16) + 16 * k;
      const u32x4 v = *(const u32x4*)(lds + off);
      T[4 * k] = v.x;
      T[4 * k + 1] = v.y;
      T[4 * k + 2] = v.z;
      T[4 * k + 3] = v.w;
    }
  };
  // Trellis state carried into segment sg: the row seed for the first segment,
  // else the last two code bytes before it (big-endian).  Split into the load
  // (issued ahead) and the byte order fix (applied after the segment-top wait),
  // so no wait is needed between the two.
  auto trellis_prev_raw = [&](int sg) -> uint32_t {
    if constexpr (FMT == QFMT_TRELLIS2) {
      if (sg == 0) return (uint32_t)gptr<g_u16*>(it.seeds)[row];
      g_u8* rp = gptr<g_u8*>(it.codes) + (int64_t)row * rb + (int64_t)sg * SEGB;
      return (uint32_t)((g_u16*)rp)[-1];  // rp is 16-byte aligned
    } else {
      return 0u;
    }
  };
  auto trellis_prev_fix = [&](int sg, uint32_t raw) -> uint32_t {
    if constexpr (FMT == QFMT_TRELLIS2) return sg == 0 ? raw : (((raw & 0xFFu) << 8) | (raw >> 8));
    else return 0u;
  };
  constexpr bool SEGPIPE = NB <= 2;
  if constexpr (SEGPIPE) {
    // Whole-segment pipeline: at the top of a segment everything in flight is
    // waited for once; then the next segment's scales and tile DMA are issued
    // and the current segment is computed from registers with no further
    // vector-memory waits.  Each sub-chunk's activation registers are refilled
    // with the next segment's right after the sub-chunk is computed.  (LDS-DMA
    // loads and ordinary loads in flight together make any later wait a full
    // drain, so no ordinary load may be waited for between a DMA issue and the
    // next segment top.)
    ActSub act[NSUB][NB];
    uint32_t prevn = 0;
    if (seg < nseg) {
      if constexpr (KACT) kpipe_issue<QMul<FMT>::v, 0>(kp, AK, seg * (SEGK / 32));  // first generation
#pragma unroll
      for (int sc = 0; sc < NSUB; ++sc)
        if constexpr (!KACT) load_act_all<FMT, NB, FMT != QFMT_TRELLIS2>(act[sc], AG, seg * (SEGK / 32) + sc * 8, 8);
      load_scales<SPS>(sptr(seg), Sn);
      prevn = trellis_prev_raw(seg);
      issue_tile(seg, true);
    }
    for (; seg < nseg; seg += nwk) {
      wait_vm_all();
      uint32_t T[CH * 4];
      read_row(T);
#pragma unroll
      for (int i = 0; i < SPS / 2; ++i) S[i] = Sn[i];
      uint32_t prev = trellis_prev_fix(seg, prevn);
      // the tile reads must be complete before the next DMA overwrites the region
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      const int nx = seg + nwk;
      const bool more_seg = nx < nseg;
      const int nsg = more_seg ? nx : seg;  // a last iteration re-reads valid data
      load_scales<SPS>(sptr(nsg), Sn);
      prevn = trellis_prev_raw(nsg);
      issue_tile(nx, more_seg);
      __builtin_amdgcn_sched_barrier(0);
      static_for(std::make_integer_sequence<int, NSUB>{}, [&](auto scc) {
        constexpr int SUB = decltype(scc)::value;
        // the block the scalar pipeline loads after this sub-chunk
        const int kb_after = SUB + 1 < NSUB ? seg * (SEGK / 32) + (SUB + 1) * 8 : nsg * (SEGK / 32);
        // (sn > 1: this wave computes only sub-chunks SUB % sn == sk; formats
        // without state carried between sub-chunks and without the scalar pipeline)
        if (sn == 1 || SUB % sn == sk)
          sub_compute<FMT, NB, SUB, WI, KACT>(T, S, act[SUB], kp, AK, seg * (SEGK / 32) + SUB * 8, 8, kb_after, prev,
                                              tc, y, Irow ? Irow + seg * (SEGK / 32) : nullptr);
        if constexpr (!KACT) {
          // kept after the sub-chunk's compute: the new values take its registers
          __builtin_amdgcn_sched_barrier(0);
          load_act_all<FMT, NB, FMT != QFMT_TRELLIS2>(act[SUB], AG, nsg * (SEGK / 32) + SUB * 8, 8);
          __builtin_amdgcn_sched_barrier(0);
        }
      });
    }
  } else {
    // Larger batches, short of registers: each 256-weight sub-chunk's codes are
    // read from LDS just before use (the same registers serve every sub-chunk),
    // so the next segment's DMA is issued after the last sub-chunk's reads;
    // activations are prefetched one sub-chunk ahead.
    ActSub cur[NB], nxt[NB];
    uint32_t prevn = 0;
    if (seg < nseg) {
      prevn = trellis_prev_raw(seg);
      issue_tile(seg, true);
      load_scales<SPS>(sptr(seg), Sn);
      load_act_all<FMT, NB, false>(cur, AG, seg * (SEGK / 32), 8);
    }
    for (; seg < nseg; seg += nwk) {
      wait_vm_all();
#pragma unroll
      for (int i = 0; i < SPS / 2; ++i) S[i] = Sn[i];
      const int nx = seg + nwk;
      const bool more_seg = nx < nseg;
      uint32_t prev = trellis_prev_fix(seg, prevn);
      static_for(std::make_integer_sequence<int, NSUB>{}, [&](auto scc) {
        constexpr int SUB = decltype(scc)::value;
        // dwords [D0, D1) of the row feed this sub-chunk: 16-byte chunks C0..C1
        constexpr int D0 = SUB * CH * 4 / NSUB, D1 = (SUB + 1) * CH * 4 / NSUB;
        constexpr int C0 = D0 / 4, C1 = (D1 + 3) / 4;
        uint32_t T[CH * 4];
        static_for(std::make_integer_sequence<int, C1 - C0>{}, [&](auto kc) {
          constexpr int k = C0 + decltype(kc)::value;
          const int off = CH == 8 ? lane * 128 + ((k ^ ((lane >> 1) & 7)) << 4) : lane * (CH * 16) + 16 * k;
          const u32x4 v = *(const u32x4*)(lds + off);
          T[4 * k] = v.x;
          T[4 * k + 1] = v.y;
          T[4 * k + 2] = v.z;
          T[4 * k + 3] = v.w;
        });
        if constexpr (SUB == NSUB - 1) {
          // the tile reads are complete before the next DMA overwrites the region
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
          asm volatile("" ::: "memory");
          __builtin_amdgcn_sched_barrier(0);
          prevn = trellis_prev_raw(more_seg ? nx : seg);
          issue_tile(nx, more_seg);
          load_scales<SPS>(sptr(more_seg ? nx : seg), Sn);
        }
        const int nkb = (SUB + 1 < NSUB) ? seg * (SEGK / 32) + (SUB + 1) * 8
                                         : (more_seg ? nx : seg) * (SEGK / 32);
        load_act_all<FMT, NB, false>(nxt, AG, nkb, 8);
        sub_compute<FMT, NB, SUB, WI>(T, S, cur, kp, AK, seg * (SEGK / 32) + SUB * 8, 8, 0, prev, tc, y,
                                      Irow ? Irow + seg * (SEGK / 32) : nullptr);
#pragma unroll
        for (int b = 0; b < NB; ++b) cur[b] = nxt[b];
      });
    }
  }


  // Tail: fewer than SEGK weights left; this lane loads its own row directly.
  const int tailK = K - nseg * SEGK;
  if (tailK > 0 && (nseg % nwk) == wk) {
    const int64_t tb = packed_row_bytes(FMT, tailK);
    g_u32* rp = (g_u32*)(gptr<g_u8*>(it.codes) + (int64_t)row * rb + (int64_t)nseg * SEGB);
    uint32_t T[CH * 4];
#pragma unroll
    for (int i = 0; i < CH * 4; ++i) T[i] = 4 * i < tb ? rp[i] : 0u;
    uint32_t St[SPS / 2];
    load_scales<SPS>(sptr(nseg), St);  // the group is zero-padded
    uint32_t prev = 0;
    if constexpr (FMT == QFMT_TRELLIS2) {
      g_u8* rb8 = (g_u8*)rp;
      prev = nseg == 0 ? (uint32_t)gptr<g_u16*>(it.seeds)[row] : (((uint32_t)rb8[-2] << 8) | rb8[-1]);
    }
    const int kb0 = nseg * (SEGK / 32);
    const int nkb_tail = tailK / 32;
    int32_t Ib[NSUB * 8];  // test-hook values of the tail segment, copied out below
    static_for(std::make_integer_sequence<int, NSUB>{}, [&](auto sc) {
      constexpr int SUB = decltype(sc)::value;
      const int kbv = nkb_tail - SUB * 8;  // valid activation blocks in this sub-chunk
      if (kbv > 0) {
        ActSub at[NB];
        if constexpr (!KACT) load_act_all<FMT, NB, false>(at, AG, kb0 + SUB * 8, kbv);
        float yt[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) yt[b] = 0.0f;
        // the test hook must not write past the row's last block: bounded copy
        sub_compute<FMT, NB, SUB, WI>(T, St, at, kp, AK, kb0 + SUB * 8, kbv, 0, prev, tc, yt,
                                      WI && Irow ? Ib : nullptr);
        if (WI && Irow) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (j < kbv) Irow[kb0 + SUB * 8 + j] = Ib[SUB * 8 + j];
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) y[b] += yt[b];
      }
    });
  }
}

// ---- kernels -----------------------------------------------------------------------------------------

// Single matrix: a workgroup of 4 waves covers 64 rows and splits the
// segments of K between its waves; partial sums are added in LDS in a fixed
// order, so results are deterministic.
template <int FMT, int NB, bool WI>
__global__ __launch_bounds__(256) void k_gemv(GemvItem it, V8Table v8t, float gain, int32_t* Iout) {
  // One LDS array, so that the trellis table is at address 0: [table][tiles][partial sums]
  constexpr int TBL = FMT == QFMT_TRELLIS2 ? kTrellisTableBytes : 0;
  constexpr int TILES = 4 * Seg<FMT>::CH * 1024;
  __shared__ __attribute__((aligned(16))) uint8_t smem[TBL + TILES + 4 * NB * 64 * 4];
  uint8_t* const v8 = smem;
  uint8_t* const lds = smem + TBL;
  float (*const red)[NB][64] = (float (*)[NB][64])(smem + TBL + TILES);
  // wave-uniform: lets the compiler keep everything derived from it in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if constexpr (FMT == QFMT_TRELLIS2) {
    trellis_table_fill(v8, v8t);
    __syncthreads();
  }
  const int row0 = blockIdx.x * 64;
  float y[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) y[b] = 0.0f;
  // A row of one or two whole segments has fewer segments than waves: the
  // waves of a segment then split its 256-weight sub-chunks.
  constexpr bool SPLIT_OK = !WI && NB <= 2 && FMT != QFMT_INT2 && FMT != QFMT_TRELLIS2;
  const int nseg = it.cols / Seg<FMT>::K;
  if (SPLIT_OK && it.cols % Seg<FMT>::K == 0 && (nseg == 1 || nseg == 2))
    gemv_tile<FMT, NB, WI>(it, row0, wave % nseg, nseg, lds + wave * Seg<FMT>::CH * 1024, v8, y, Iout, wave / nseg,
                           4 / nseg);
  else
    gemv_tile<FMT, NB, WI>(it, row0, wave, 4, lds + wave * Seg<FMT>::CH * 1024, v8, y, Iout);
  wait_all();  // no tile DMA or scalar load may still be landing when the wave ends
  if (WI) return;
#pragma unroll
  for (int b = 0; b < NB; ++b) red[wave][b][lane] = y[b];
  __syncthreads();
  if (wave == 0 && row0 + lane < it.rows) {
    const float fs = final_scale<FMT>(gain);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float v = ((red[0][b][lane] + red[1][b][lane]) + red[2][b][lane]) + red[3][b][lane];
      gptr<g_f32*>(it.y)[(int64_t)b * it.rows + row0 + lane] = v * fs;
    }
  }
}

// Waves per workgroup of the grouped kernel for batch NB and format FMT: every
// wave a CU holds at the kernel's register count (at most 16), so one
// workgroup fills a CU; the ternary tile (13 KB of LDS per wave) allows 12,
// the trellis tiles beside the 64 KB lookup table 11.
// The kernel's launch bound follows from it, and the build fails if that bound
// forces register spills.
constexpr int grouped_wpg(int nb, int fmt) {
  constexpr int t[8][5] = {{12, 16, 16, 16, 11}, {8, 16, 12, 16, 11}, {12, 16, 16, 16, 11}, {12, 12, 16, 12, 11},
                           {8, 12, 12, 12, 11},  {8, 12, 12, 12, 8},  {8, 8, 12, 12, 8},   {8, 8, 8, 8, 8}};
  return t[nb - 1][fmt - 1];
}

// Grouped: persistent workgroups, one per CU.  The plan deals each format's
// tiles to lists of nearly equal bytes (longest first inside a list);
// workgroup g of G works through lists g, g + G, ... and its waves take the
// tiles in that order through an LDS counter.  A fixed share per wave would
// not do: the waves of a SIMD do not progress at equal rates (the instruction
// arbiter favours the oldest), so SIMDs would be left with one wave, or none,
// long before the last one ends.  No counter is shared between workgroups (a
// device-wide atomic per tile caps streaming well below what the HBM delivers).
// One launch serves the plan's tiles of format ONLY (the other formats' code
// is not compiled in, which keeps the register count low).
template <int NB, int ONLY>
__global__ __launch_bounds__(64 * grouped_wpg(NB, ONLY)) void k_gemv_grouped(const uint8_t* __restrict__ plan,
                                                                            V8Table v8t, float gain) {
  static_assert(ONLY >= 1 && ONLY <= 5, "one format per launch");
  constexpr int P = grouped_wpg(NB, ONLY);
  constexpr int WAVE_LDS = Seg<ONLY>::CH * 1024;
  // One LDS array, so that the trellis table is at address 0: [table][tiles][tile counter]
  constexpr int TBL = ONLY == QFMT_TRELLIS2 ? kTrellisTableBytes : 0;
  static_assert(TBL + P * WAVE_LDS + 16 <= 160 * 1024, "LDS per workgroup");
  __shared__ __attribute__((aligned(16))) uint8_t smem[TBL + P * WAVE_LDS + 16];
  uint8_t* const v8 = smem;
  uint8_t* const lds = smem + TBL;
  int& next_k = *(int*)(smem + TBL + P * WAVE_LDS);
  const PlanHeader* hp = (const PlanHeader*)plan;
  const GemvItem* items = (const GemvItem*)(plan + hp->items_off);
  const GemvTile* tiles = (const GemvTile*)(plan + hp->tiles_off);
  const int nwk = hp->n_workers;
  const int32_t* wb = (const int32_t*)(plan + hp->workers_off) + ONLY * (nwk + 1);
  if constexpr (ONLY == QFMT_TRELLIS2) trellis_table_fill(v8, v8t);
  if (threadIdx.x == 0) next_k = 0;
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  uint8_t* my = lds + wave * WAVE_LDS;
  for (;;) {
    int k = 0;
    if (lane == 0) k = __hip_atomic_fetch_add(&next_k, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    k = __builtin_amdgcn_readfirstlane(k);
    // the k-th tile of this workgroup's lists, taken in order
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
    constexpr int fmt = ONLY;
    float y[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) y[b] = 0.0f;
    gemv_tile<fmt, NB, false>(it, row0, 0, 1, my, v8, y, nullptr);
    const float fs = final_scale<fmt>(gain);
    if (row0 + lane < it.rows) {
#pragma unroll
      for (int b = 0; b < NB; ++b) gptr<g_f32*>(it.y)[(int64_t)b * it.rows + row0 + lane] = y[b] * fs;
    }
  }
  wait_all();  // no tile DMA or scalar load may still be landing when the wave ends
}

}  // namespace qk
