// gemv_tern1.hip — grouped ternary GEMV for one token, dot products on the
// matrix cores.
//
// At batch 1 the lane-per-row ternary kernel (gemv_impl.hpp) is bound by its
// vector instructions, not by HBM: pulling the five base-3 digits out of each
// byte costs five instructions per four weights (two multiplies by 3, two
// masks, one byte gather) and the dot products one more.  This kernel spends
// about 0.7 per weight on the digits and about 1.06 in all (counters), from
// two observations.
//
// 1. Telescoped digits.  A byte x holds the base-3 fraction of its 5 trits
//    (ceil(256 b / 243)); with h_j = floor(3^j x / 256) the j-th digit is
//    d_j = h_{j+1} - 3 h_j (h_0 = 0), because 3^(j+1) x = 768 h_j + 256 d_j +
//    (3^(j+1) x mod 256).  The dot product of a word's digits with the
//    activations a_i telescopes:
//        sum_i d_i a_i = sum_{j>=1} h_j a_{j-1} - 3 sum_{j>=1} h_j a_j,
//    so h_j (j = 1..4: at most 80, a signed byte) is needed, not d_j, and
//    h_j of two bytes is ONE multiply: x in two 16-bit lanes times 3^j puts
//    h_j in byte 1 of each lane (3^4 255 < 2^16, no carry between lanes).
//    The last of five digits, whose h_5 would reach 242, is taken directly:
//    d_4 = floor(3 (3^4 x mod 256) / 256), i.e. (Y_4 & 0x00FF00FF) * 3.  The low
//    byte of every 16-bit lane is junk and meets a zero activation: the A
//    operand is 2:4 sparse, which the sparse MFMA skips.
// 2. The matrix core does the dot products, the telescoping and the
//    separation into 32-blocks at once: v_smfmac_i32_16x16x128_i8 with the
//    weights as B (128 k x 16 rows) and the activations as A (16 A-rows x 128 k, 2:4 sparse),
//    A-row 2b + c holding, for the k-bytes of activation block b, the
//    coefficient of the "+a_{j-1}" term (c = 0) or of the "-3 a_j" term (c = 1)
//    and zeros elsewhere.  After the four MFMAs of a 256-weight sub-chunk the
//    accumulator holds, per weight row, 16 sums from which the exact block
//    dots I_b = C[2b] - 3 C[2b+1] - qsum_b follow (the accumulator starts at
//    -qsum_b: digits are trit + 1), so the fp32 epilogue runs once per
//    sub-chunk, not once per block.
//
// Work unit: a wave owns a 64-row tile, four groups G of 16 rows.  Lane l
// provides, for row 16 G + l % 16 and k-quarter q = l / 16 of each sub-chunk,
// the B operand: code words 3q, 3q+1, 3q+2 (ten dwords each: h_1..h_4 and the
// last digit of bytes 0,2 and of bytes 1,3) and h_{q+1} of word 12 (four
// digits: h_1..h_4 telescope it whole, one h per quarter), 32 dwords = four
// sparse MFMAs' worth.  As A operand the same lane is A-row l % 16 of quarter q: the
// activation dwords its quarter's codes meet, masked to its block and
// coefficient.  Codes of a 1024-weight segment (208 bytes per row) come into
// LDS by DMA, 1 KB per instruction, together with the segment's activations, d
// and qsum (double-buffered), and are read lane = (row, quarter) straight from
// there: no transpose.  Ordinary (not non-temporal) loads: a segment shares its
// boundary lines with its neighbours, whose second fetch then mostly hits L2.  The wave's four lane groups end with
// partial sums of the same rows (different blocks), added by lane exchange.
//
// Sources: [P3] §1.2 (ternary weights: add, subtract or skip, bandwidth-bound);
// cfg "5 trits per byte, base 3"; [P1] "把非标准格式塞进 llama.cpp，难在哪"
// (int8 matrix-core products for these formats).
#include "gemv_impl.hpp"

namespace qk {
namespace {

typedef int32_t t1_v4i __attribute__((ext_vector_type(4)));
typedef int32_t t1_v8i __attribute__((ext_vector_type(8)));

constexpr int T1_WAVES = 8;
constexpr int T1_SEGK = 1024;                    // weights per segment
constexpr int T1_SEGB = 208;                     // code bytes per row and segment
constexpr int T1_CODE = 64 * T1_SEGB;            // code tile: 64 rows x one segment
constexpr int T1_ACT = 1024;                     // int8 activations of one segment
constexpr int T1_DQ = 256;                       // d[32] then qsum[32] of its blocks
constexpr int T1_WAVE_LDS = T1_CODE + 2 * T1_ACT + 2 * T1_DQ;
static_assert(T1_WAVES * T1_WAVE_LDS + 16 <= 160 * 1024, "LDS per workgroup");
// Cache policy of the code-tile loads: ordinary, not non-temporal (a 208-byte
// segment shares a line with the next one; TileCachePolicy).
constexpr int T1_TILE_POLICY = TileCachePolicy<QFMT_TERN_B3>::v;

// Operand layout of v_smfmac_i32_16x16x128_i8 (checked against a host
// product): B lane l = column l % 16, its eight dwords k-groups 4 j + d and
// 16 + 4 j + d (d = 0..3, j = l / 16); compressed A lane l = row l % 16,
// elements 2g, 2g+1 from dense k-group 8 j + g at the positions of index bits
// [2i+1:2i].  So compressed A dword i = 4 t + cA of lane group j (sparse MFMA
// t) meets B dwords 8 t + dd, dd = 2 (cA & 1) + 4 (j >> 1) and dd + 1, of lane
// group qB = 2 (j & 1) + (cA >> 1): code slot pair kappa = 4 t + 2 (j >> 1) +
// (cA & 1) of that quarter, whose activation dword is 15 qB + c + kappa
// (kappa < 15) or the word-12 dword 60 + min(qB + c, 3) (kappa = 15).
struct T1Slot {
  int qB, kappa;
};
constexpr T1Slot t1_slot(int i, int j) {
  const int t = i >> 2, cA = i & 3;
  return {2 * (j & 1) + (cA >> 1), 4 * t + 2 * (j >> 1) + (cA & 1)};
}
// Dword offset of compressed A dword i's activation from the lane's base
// 30 (j & 1) + 2 (j >> 1) + c (kappa < 15).
constexpr int t1_off(int i) { return 15 * ((i & 3) >> 1) + (i & 1) + 4 * (i >> 2); }

// Lanes l = (j = l / 16, A-row l % 16 = 2 b + c) whose compressed A dword i
// keeps its activation dword: it lies in block b and the coefficient exists.
// Slot pair kappa % 5 = 0..2 carries h_1..h_3 (both terms), 3 carries h_4 (no
// "-3 a_4" term: the last digit is taken directly), 4 the last digit (first
// term only); in word 12 (four digits, so h_1..h_4 are all at most 80 and no
// digit is taken directly) quarter qB holds h_{qB+1}, whose second term exists
// for qB <= 2.
constexpr uint64_t t1_mask(int i) {
  uint64_t m = 0;
  for (int l = 0; l < 64; ++l) {
    const int j = l >> 4, c = l & 1, b = (l & 15) >> 1;
    const T1Slot sl = t1_slot(i, j);
    bool on;
    if (sl.kappa < 15) on = ((15 * sl.qB + c + sl.kappa) >> 3) == b && !(c == 1 && sl.kappa % 5 >= 3);
    else on = b == 7 && !(c == 1 && sl.qB == 3);
    if (on) m |= 1ull << l;
  }
  return m;
}

// v where the lane's bit of `mask` is set, else 0.
__device__ __forceinline__ uint32_t t1_keep(uint32_t v, uint64_t mask) {
  uint32_t r;
  asm("v_cndmask_b32 %0, 0, %1, %2" : "=v"(r) : "v"(v), "s"(mask));
  return r;
}

__device__ __forceinline__ uint32_t mu24(uint32_t a, uint32_t b) { return __umul24(a, b); }

// Activation dword [a0, a1, a2, a3] as [a0, a2, a1, a3]: the nonzero bytes
// of [0, a0, 0, a2] and of [0, a1, 0, a3] in compressed A order.
__device__ __forceinline__ uint32_t t1_aperm(uint32_t v) { return __builtin_amdgcn_perm(0u, v, 0x03010200u); }

// Ten B dwords of code word W: [Y1l Y1h Y2l Y2h Y3l Y3h Y4l Y4h Dl Dh], Yj =
// 3^j x (x = bytes 0,2 of W in 16-bit lanes for "l", bytes 1,3 for "h"; h_j in
// bytes 1 and 3), D = the last digit in bytes 1 and 3.
__device__ __forceinline__ void t1_word(uint32_t W, uint32_t* b) {
  const uint32_t m = 0x00FF00FFu;
  const uint32_t xl = W & m;
  const uint32_t xh = __builtin_amdgcn_perm(0u, W, 0x0C030C01u);
  b[0] = mu24(xl, 3u);
  b[1] = mu24(xh, 3u);
  b[2] = mu24(xl, 9u);
  b[3] = mu24(xh, 9u);
  b[4] = mu24(xl, 27u);
  b[5] = mu24(xh, 27u);
  b[6] = mu24(xl, 81u);
  b[7] = mu24(xh, 81u);
  b[8] = mu24(b[6] & m, 3u);
  b[9] = mu24(b[7] & m, 3u);
}

// One 256-weight sub-chunk of the tile.  w[G][0..3]: code words 3q, 3q+1, 3q+2
// and 12 of row 16 G + l % 16; ar[16]: the activation dwords of the lane's
// compressed A dwords (t1_slot), bytes in the order 0, 2, 1, 3 (t1_aperm); d0, d1, qs0, qs1: d and qsum of blocks 2q and 2q+1; sw[G]: the
// weight scale of row 16 G + l % 16; acc[G] += sw[G] (d0 I_2q + d1 I_2q+1).
// z1: the lane's word-12 multiplier 3^(q+1).
__device__ __forceinline__ void t1_sub(const uint32_t (&w)[4][4], const uint32_t (&ar)[16], float d0, float d1,
                                       int qs0, int qs1, const float (&sw)[4], uint32_t z1, float (&acc)[4]) {
  // Compressed A: the nonzero bytes of [0, a_p0, 0, a_p2] (against an "l" B
  // dword) and [0, a_p1, 0, a_p3] (against the "h" dword after it), i.e. one
  // dword [a_p0, a_p2, a_p1, a_p3] per pair of B dwords; every group of four
  // k-bytes has its two values at positions 1 and 3 (index 0xD per group).
  uint32_t A[16];
  {
#define T1_KEEP(k)                                                          \
  {                                                                         \
    constexpr uint64_t mk = t1_mask(k);                                     \
    A[k] = t1_keep(ar[k], mk);                                              \
  }
    T1_KEEP(0) T1_KEEP(1) T1_KEEP(2) T1_KEEP(3) T1_KEEP(4) T1_KEEP(5) T1_KEEP(6) T1_KEEP(7)
    T1_KEEP(8) T1_KEEP(9) T1_KEEP(10) T1_KEEP(11) T1_KEEP(12) T1_KEEP(13) T1_KEEP(14) T1_KEEP(15)
#undef T1_KEEP
  }
  const uint32_t m = 0x00FF00FFu;
#pragma unroll
  for (int G = 0; G < 4; ++G) {
    uint32_t Bd[32];
#pragma unroll
    for (int mm = 0; mm < 3; ++mm) t1_word(w[G][mm], Bd + 10 * mm);
    {
      // word 12: quarter q holds h_{q+1} = 3^(q+1) x
      const uint32_t W = w[G][3];
      Bd[30] = mu24(W & m, z1);
      Bd[31] = mu24(__builtin_amdgcn_perm(0u, W, 0x0C030C01u), z1);
    }
    t1_v4i c = {-qs0, 0, -qs1, 0};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const t1_v4i a = {(int)A[4 * t], (int)A[4 * t + 1], (int)A[4 * t + 2], (int)A[4 * t + 3]};
      const t1_v8i b = {(int)Bd[8 * t], (int)Bd[8 * t + 1], (int)Bd[8 * t + 2], (int)Bd[8 * t + 3],
                        (int)Bd[8 * t + 4], (int)Bd[8 * t + 5], (int)Bd[8 * t + 6], (int)Bd[8 * t + 7]};
      c = __builtin_amdgcn_smfmac_i32_16x16x128_i8(a, b, c, (int)0xDDDDDDDDu, 0, 0);
    }
    // rows 4q .. 4q+3 of the result: (block 2q, +), (2q, -3), (2q+1, +), (2q+1, -3)
    // (|C| < 2^23: 24-bit multiply-adds)
    const int I0 = c[0] + __mul24(c[1], -3), I1 = c[2] + __mul24(c[3], -3);
    const float t = __builtin_fmaf(d1, (float)I1, d0 * (float)I0);
    acc[G] = __builtin_fmaf(sw[G], t, acc[G]);
  }
}

// One 64-row tile: y[row0 + i] for i < 64 (rows past the end are not written).
__device__ __forceinline__ void t1_tile(const GemvItem& it, int row0, uint8_t* my) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, q = lane >> 4, c = lane & 1;
  const int K = it.cols, N = it.rows, kbs = K >> 5;
  const int nseg = K / T1_SEGK, nsub = K >> 8;
  const int nvalid = min(64, N - row0);
  const int64_t rb = it.row_bytes;
  g_u8* tile = gptr<g_u8*>(it.codes) + (int64_t)row0 * rb;
  g_u8* qa = gptr<g_u8*>(it.q);
  const float __attribute__((address_space(1)))* dg = gptr<const float __attribute__((address_space(1)))*>(it.d);
  const int32_t __attribute__((address_space(1)))* sg =
      gptr<const int32_t __attribute__((address_space(1)))*>(it.qsum);
  const int nsb = K >> 8;
  g_u16* stile = gptr<g_u16*>(it.scales) + (int64_t)(row0 >> 6) * ((nsb + 3) / 4) * 256;
  // word-12 multiplier of this lane's quarter: 3^(q+1) (h_1..h_4)
  const uint32_t z1 = q == 0 ? 3u : q == 1 ? 9u : q == 2 ? 27u : 81u;
  // activation dwords of the lane's compressed A (t1_slot): base + t1_off(i),
  // except i = 13 and 15, which in lane groups 2 and 3 are word-12 dwords
  const int abase = 30 * (q & 1) + 2 * (q >> 1) + c;
  const int sp13 = q >= 2 ? 60 + min(2 * (q & 1) + c, 3) : abase + t1_off(13);
  const int sp15 = q >= 2 ? 60 + min(2 * (q & 1) + 1 + c, 3) : abase + t1_off(15);
  uint8_t* const codes = my;
  uint8_t* const actb = my + T1_CODE;
  uint8_t* const dqb = my + T1_CODE + 2 * T1_ACT;

  // DMA of segment sg: 13 loads of the 64 x 208-byte code tile (slot f = 64 i
  // + lane holds bytes 16 f of the row-major tile; rows past the end re-read
  // the last valid row), the segment's 1024 activation bytes and its 32 d and
  // 32 qsum words into buffer `bi`.  The lane offsets of the code loads are
  // the same for every segment of the tile (64 rb < 2^24 for K <= 2^20).
  uint32_t toff[13];
#pragma unroll
  for (int i = 0; i < 13; ++i) {
    const uint32_t f = (uint32_t)(i * 64 + lane);
    const uint32_t r = f / 13u, ch = f % 13u;
    toff[i] = __umul24((uint32_t)min((int)r, nvalid - 1), (uint32_t)rb) + ch * 16u;
  }
  auto issue = [&](int sgi, int bi) {
    __builtin_amdgcn_sched_barrier(0);
    int ln = lane;
    asm volatile("" : "+v"(ln));
    g_u8* tseg = tile + (int64_t)sgi * T1_SEGB;
#pragma unroll
    for (int i = 0; i < 13; ++i) {
      asm volatile("" : "+v"(toff[i]));
      const uint32_t off = toff[i];
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(tseg + off),
                                       (__attribute__((address_space(3))) void*)(codes + i * 1024), 16, 0,
                                       T1_TILE_POLICY);
    }
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(qa + (int64_t)sgi * T1_SEGK +
                                                                                      (uint32_t)(16 * ln)),
                                     (__attribute__((address_space(3))) void*)(actb + bi * T1_ACT), 16, 0, 0);
    const void __attribute__((address_space(1)))* dq =
        ln < 32 ? (const void __attribute__((address_space(1)))*)(dg + (int64_t)sgi * 32 + ln)
                : (const void __attribute__((address_space(1)))*)(sg + (int64_t)sgi * 32 + (ln - 32));
    __builtin_amdgcn_global_load_lds(dq, (__attribute__((address_space(3))) void*)(dqb + bi * T1_DQ), 4, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // the four fp16 scales of segment sgi for rows 16 G + r16 (tiled layout, zero padded)
  auto load_scales = [&](int sgi, uint32_t (&S)[4][2]) {
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      const u32x2 v = *(g_u32x2*)(stile + (uint32_t)((sgi * 64 + 16 * G + r16) * 4));
      S[G][0] = v.x;
      S[G][1] = v.y;
    }
  };

  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  uint32_t Sn[4][2];
  if (nseg > 0) {
    issue(0, 0);
    load_scales(0, Sn);
  }
  for (int seg = 0; seg < nseg; ++seg) {
    wait_vm_all();  // this segment's DMA and scales have landed
    uint32_t cw[4][4][4];  // [G][sub-chunk][word 3q, 3q+1, 3q+2, 12]
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      const l_u32* rp = (const l_u32*)(codes + (16 * G + r16) * T1_SEGB);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int mm = 0; mm < 3; ++mm) cw[G][s][mm] = rp[13 * s + 3 * q + mm];
        cw[G][s][3] = rp[13 * s + 12];
      }
    }
    {
      // this segment's activations into compressed-A byte order, in place; a
      // wave's LDS accesses complete in order, so the reads below see it
      u32x4* ap = (u32x4*)(actb + (seg & 1) * T1_ACT + 16 * lane);
      u32x4 v = *ap;
      v = u32x4{t1_aperm(v.x), t1_aperm(v.y), t1_aperm(v.z), t1_aperm(v.w)};
      *ap = v;
    }
    float sw[4][4];
#pragma unroll
    for (int G = 0; G < 4; ++G)
#pragma unroll
      for (int s = 0; s < 4; ++s) sw[G][s] = scale_half(Sn[G][s >> 1], s & 1);
    // the code reads complete before the next DMA overwrites the tile
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (seg + 1 < nseg) {
      issue(seg + 1, (seg + 1) & 1);
      load_scales(seg + 1, Sn);
    }
    const l_u32* ab = (const l_u32*)(actb + (seg & 1) * T1_ACT);
    const l_u32* dqp = (const l_u32*)(dqb + (seg & 1) * T1_DQ);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t ar[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) ar[i] = ab[64 * s + (i == 13 ? sp13 : i == 15 ? sp15 : abase + t1_off(i))];
      const float d0 = __builtin_bit_cast(float, dqp[8 * s + 2 * q]);
      const float d1 = __builtin_bit_cast(float, dqp[8 * s + 2 * q + 1]);
      const int qs0 = (int)dqp[32 + 8 * s + 2 * q], qs1 = (int)dqp[32 + 8 * s + 2 * q + 1];
      uint32_t w[4][4];
#pragma unroll
      for (int G = 0; G < 4; ++G)
#pragma unroll
        for (int k = 0; k < 4; ++k) w[G][k] = cw[G][s][k];
      const float sws[4] = {sw[0][s], sw[1][s], sw[2][s], sw[3][s]};
      t1_sub(w, ar, d0, d1, qs0, qs1, sws, z1, acc);
    }
  }
  // Tail sub-chunks past the last whole segment: codes, activations and scales
  // straight from global memory (rows clamped into the matrix).
  for (int sc = nseg * 4; sc < nsub; ++sc) {
    uint32_t w[4][4];
    float sws[4];
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      const int rr = min(16 * G + r16, nvalid - 1);
      g_u32* rp = (g_u32*)(tile + (int64_t)rr * rb + (int64_t)sc * 52);
#pragma unroll
      for (int mm = 0; mm < 3; ++mm) w[G][mm] = rp[3 * q + mm];
      w[G][3] = rp[12];
      const uint16_t h = stile[(uint32_t)(((sc >> 2) * 64 + 16 * G + r16) * 4 + (sc & 3))];
      sws[G] = __half2float(__ushort_as_half(h));
    }
    g_u32* ag = (g_u32*)(qa + (int64_t)sc * 256);
    uint32_t ar[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) ar[i] = t1_aperm(ag[i == 13 ? sp13 : i == 15 ? sp15 : abase + t1_off(i)]);
    const int kb = 8 * sc + 2 * q;
    const float d0 = dg[kb], d1 = dg[kb + 1];
    const int qs0 = sg[kb], qs1 = sg[kb + 1];
    t1_sub(w, ar, d0, d1, qs0, qs1, sws, z1, acc);
  }
  (void)kbs;
  // the four quarters hold partial sums of the same rows
#pragma unroll
  for (int G = 0; G < 4; ++G) {
    acc[G] += __shfl_xor(acc[G], 16);
    acc[G] += __shfl_xor(acc[G], 32);
  }
  // quarter q writes row group q
  const float v = q == 0 ? acc[0] : q == 1 ? acc[1] : q == 2 ? acc[2] : acc[3];
  const int row = 16 * q + r16;
  if (row < nvalid) gptr<g_f32*>(it.y)[row0 + row] = v;
}

}  // namespace

// Grouped, one token, ternary tiles of the plan: persistent workgroups, one per
// CU, whose waves take the tiles of their lists in order through an LDS
// counter (as k_gemv_grouped).
__global__ __launch_bounds__(64 * T1_WAVES) void k_gemv_grouped_tern1(const uint8_t* __restrict__ plan) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[T1_WAVES * T1_WAVE_LDS + 16];
  int& next_k = *(int*)(smem + T1_WAVES * T1_WAVE_LDS);
  const PlanHeader* hp = (const PlanHeader*)plan;
  const GemvItem* items = (const GemvItem*)(plan + hp->items_off);
  const GemvTile* tiles = (const GemvTile*)(plan + hp->tiles_off);
  const int nwk = hp->n_workers;
  const int32_t* wb = (const int32_t*)(plan + hp->workers_off) + QFMT_TERN_B3 * (nwk + 1);
  if (threadIdx.x == 0) next_k = 0;
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  uint8_t* my = smem + wave * T1_WAVE_LDS;
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
    t1_tile(it, row0, my);
  }
  wait_all();  // no tile DMA may still be landing when the wave ends
}

hipError_t launch_grouped_tern1(const PlanHeader& h, const void* plan, hipStream_t s) {
  const int t0 = h.fmt_begin[QFMT_TERN_B3], t1 = h.fmt_begin[QFMT_TERN_B3 + 1];
  if (t1 <= t0) return hipSuccess;
  constexpr int threads = 64 * T1_WAVES;
  const int grid = resident_workgroups((const void*)k_gemv_grouped_tern1, threads);
  if (grid <= 0) return hipErrorInvalidDevice;
  hipLaunchKernelGGL(k_gemv_grouped_tern1, dim3(grid), dim3(threads), 0, s, (const uint8_t*)plan);
  return hipGetLastError();
}

}  // namespace qk
