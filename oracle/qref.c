/*
 * qref.c — plain CPU oracle.  TEST INFRASTRUCTURE ONLY (see qref.h).
 *
 * Every function follows the definition it cites, in plain loops.  Build:
 *   gcc -std=c11 -O2 -ffp-contract=off -fopenmp -fPIC -shared qref.c -lm
 */
#include "qref.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the parallel loops below use (OpenMP), for timing records. */
int qref_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Set the thread count of the parallel loops (n >= 1). */
void qref_set_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* Format geometry                                                           */
/* ------------------------------------------------------------------------ */

/* Per-block scales: one scale per 64 or 128 weights, value = code x scale
 * ([P4] §2.1).  Block sizes per format are this library's choice: 256 for
 * ternary, 32 for the 2- and 4-bit levels, 128 for 1-bit signs, 64 for the
 * trellis codes. */
int qref_scale_block(int fmt) {
  switch (fmt) {
    case QREF_TERN_B3: return 256;
    case QREF_INT2: return 32;
    case QREF_SIGN1: return 128;
    case QREF_INT4: return 32;
    case QREF_TRELLIS2: return 64;
    default: return 0;
  }
}

/* Bytes per row.  Ternary: a 256-weight block is 48 bytes of 5 trits plus
 * 4 bytes of 4 trits = 52 bytes, 1.625 bits per weight, just above the
 * log2(3) = 1.585 floor ([P3] §1.2).  The others are 2, 1, 4 and 2 bits. */
int64_t qref_packed_row_bytes(int fmt, int K) {
  int blk = qref_scale_block(fmt);
  if (blk == 0 || K <= 0 || K % blk != 0) return -1;
  switch (fmt) {
    case QREF_TERN_B3: return (int64_t)52 * (K / 256);
    case QREF_INT2: return K / 4;
    case QREF_SIGN1: return K / 8;
    case QREF_INT4: return K / 2;
    case QREF_TRELLIS2: return K / 4;
  }
  return -1;
}

int64_t qref_row_stride(int fmt, int K) {
  int64_t b = qref_packed_row_bytes(fmt, K);
  if (b < 0) return b;
  return (b + 15) / 16 * 16;
}

/* ------------------------------------------------------------------------ */
/* fp16 conversion (IEEE binary16, round to nearest even)                    */
/* ------------------------------------------------------------------------ */

uint16_t qref_f64_to_f16(double x) {
  uint16_t sign = signbit(x) ? 0x8000u : 0u;
  if (isnan(x)) return (uint16_t)(sign | 0x7E00u);
  double a = fabs(x);
  if (a == 0.0) return sign;
  /* Largest finite fp16 is 65504; values >= 65520 round to infinity. */
  if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
  int e;
  (void)frexp(a, &e);      /* a = m * 2^e, m in [0.5, 1) */
  int E = e - 1;           /* a in [2^E, 2^(E+1)) */
  if (E < -14) {
    /* Subnormal range: quantum 2^-24.  a / 2^-24 is exact in double. */
    double n = rint(ldexp(a, 24)); /* nearest integer, ties to even */
    /* n == 1024 encodes the smallest normal, which the bit pattern does. */
    return (uint16_t)(sign | (uint16_t)n);
  }
  double n = rint(ldexp(a, 10 - E)); /* in [1024, 2048] */
  if (n >= 2048.0) {
    n = 1024.0;
    E += 1;
  }
  if (E > 15) return (uint16_t)(sign | 0x7C00u);
  return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)n - 1024));
}

double qref_f16_to_f64(uint16_t h) {
  int s = (h >> 15) & 1;
  int e = (h >> 10) & 0x1F;
  int m = h & 0x3FF;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), e - 25);
  return s ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* Activation Q8                                                              */
/* ------------------------------------------------------------------------ */

/* int8 activations are what the pages' int8 dot-product GEMV and int8
 * tensor-core paths consume ([P1] "porting a non-standard format into
 * llama.cpp": decode via DP4A GEMV, batches via INT8 MMA, prefill via INT8
 * GEMM).  One fp32 scale per block of n values:
 *   amax = max |v|;  d = amax / 127 (fp32, IEEE division);
 *   r = 1 / d (fp32);  id = r if r is finite, else 0;
 *   q = clamp(rint(v * id), -127, 127) with rint rounding half to even.
 * r is infinite for a zero block (d = 0) and whenever d <= 2^-128, where the
 * reciprocal overflows (amax below about 3.7e-37): such a block quantizes to
 * q = 0, qsum = 0, and d keeps the value amax / 127.  -128 never occurs.
 * Inputs are finite; v * id is then finite too (|v * id| <= 127 (1 + 2^-22)),
 * and the NaN test below is never taken for them (it only keeps a non-finite
 * input from reaching an undefined float-to-int conversion). */
void qref_q8_block(const float* v, int n, int8_t* q, float* d, int32_t* qsum) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) {
    float a = fabsf(v[i]);
    if (a > amax) amax = a;
  }
  float dd = amax / 127.0f;
  float r = 1.0f / dd;
  float id = isfinite(r) ? r : 0.0f;
  int32_t s = 0;
  for (int i = 0; i < n; ++i) {
    float prod = v[i] * id;
    float t = rintf(prod);
    if (t != t) t = 0.0f;
    if (t > 127.0f) t = 127.0f;
    if (t < -127.0f) t = -127.0f;
    q[i] = (int8_t)t;
    s += q[i];
  }
  *d = dd;
  *qsum = s;
}

void qref_act_quant(const float* x, int B, int K, int qblock, int8_t* q, float* d, int32_t* qsum) {
  int nb = K / qblock;
  for (int b = 0; b < B; ++b)
    for (int kb = 0; kb < nb; ++kb) {
      size_t off = (size_t)b * K + (size_t)kb * qblock;
      qref_q8_block(x + off, qblock, q + off, d + (size_t)b * nb + kb, qsum + (size_t)b * nb + kb);
    }
}

/* Split of int8 activations into 4-bit planes: x = 16 * hi + lo with lo =
 * x mod 16 in [0, 15] and hi = floor(x / 16) in [-8, 7] (two's complement
 * nibble).  For every 32-block and each group g of 8 values (x[8g + n], n =
 * 0..7) the block's 8 words are lo of groups 0..3, then hi of groups 0..3,
 * value n in nibble n.  A layout of the same integers (exact); the 1- and 2-bit
 * GEMV multiplies it nibble by nibble against the codes' planes above. */
void qref_act_planes(const int8_t* q, int B, int K, uint32_t* planes) {
  for (int b = 0; b < B; ++b)
    for (int kb = 0; kb < K / 32; ++kb) {
      const int8_t* x = q + (size_t)b * K + (size_t)kb * 32;
      uint32_t* o = planes + ((size_t)b * (K / 32) + kb) * 8;
      for (int g = 0; g < 4; ++g) {
        uint32_t lo = 0, hi = 0;
        for (int n = 0; n < 8; ++n) {
          int v = x[8 * g + n];
          int h = (v - (((v % 16) + 16) % 16)) / 16; /* floor(v / 16) */
          int l = v - 16 * h;
          lo |= (uint32_t)l << (4 * n);
          hi |= (uint32_t)(h & 15) << (4 * n);
        }
        o[g] = lo;
        o[4 + g] = hi;
      }
    }
}

/* ------------------------------------------------------------------------ */
/* Weight quantizers (host-side data preparation), fp64 decisions            */
/* ------------------------------------------------------------------------ */

/* Ternary quantizer of [P3] §5.1: scale = mean|W| + 1e-8, code =
 * clamp(round(W / scale), -1, 1), dequantized value = code * scale.  The page
 * applies it per tensor; here it runs per 256-weight block, matching the
 * per-block scales of [P4] §2.1.  round = half to even.  The mean is summed in
 * index order in fp64; the stored scale is fp16(scale). */
void qref_quant_tern(const float* w, int N, int K, int8_t* t, uint16_t* s) {
  int nb = K / 256;
#pragma omp parallel for schedule(static)
  for (int n = 0; n < N; ++n)
    for (int kb = 0; kb < nb; ++kb) {
      const float* wb = w + (size_t)n * K + (size_t)kb * 256;
      double sum = 0.0;
      for (int i = 0; i < 256; ++i) sum += fabs((double)wb[i]);
      double sc = sum / 256.0 + 1e-8;
      for (int i = 0; i < 256; ++i) {
        double r = rint((double)wb[i] / sc);
        if (r > 1.0) r = 1.0;
        if (r < -1.0) r = -1.0;
        t[(size_t)n * K + (size_t)kb * 256 + i] = (int8_t)r;
      }
      s[(size_t)n * nb + kb] = qref_f64_to_f16(sc);
    }
}

/* Shared by the 2- and 4-bit quantizers: levels (c - (L-1)/2) * s for
 * c = 0..L-1, i.e. the half-integers +-0.5 .. +-(L-1)/2 times s, with
 * s = fp16(amax / ((L-1)/2)) from the block's absolute maximum.  The code is
 * the nearest level to w / s (s as stored), ties toward the upper level:
 * c = clamp(floor(w/s) + L/2, 0, L-1).  A block with s == 0 gets c = L/2. */
static void quant_levels(const float* w, int N, int K, int L, int8_t* c, uint16_t* s) {
  int nb = K / 32;
  double half_span = (L - 1) / 2.0;
#pragma omp parallel for schedule(static)
  for (int n = 0; n < N; ++n)
    for (int kb = 0; kb < nb; ++kb) {
      const float* wb = w + (size_t)n * K + (size_t)kb * 32;
      double amax = 0.0;
      for (int i = 0; i < 32; ++i) {
        double a = fabs((double)wb[i]);
        if (a > amax) amax = a;
      }
      uint16_t sh = qref_f64_to_f16(amax / half_span);
      double sc = qref_f16_to_f64(sh);
      for (int i = 0; i < 32; ++i) {
        int code;
        if (sc == 0.0) {
          code = L / 2;
        } else {
          double f = floor((double)wb[i] / sc) + L / 2;
          if (f < 0.0) f = 0.0;
          if (f > L - 1) f = L - 1;
          code = (int)f;
        }
        c[(size_t)n * K + (size_t)kb * 32 + i] = (int8_t)code;
      }
      s[(size_t)n * nb + kb] = sh;
    }
}

/* 2 bits hold 4 levels ([P1] "how big is 2.4 bits"): {-1.5,-0.5,0.5,1.5} x s. */
void qref_quant_int2(const float* w, int N, int K, int8_t* c, uint16_t* s) {
  quant_levels(w, N, K, 4, c, s);
}

/* 4 bits hold 16 levels ([P1] "how big is 2.4 bits"): {-7.5..7.5} x s.
 * int4 weights are dequantized and multiplied ([P4] §2.2). */
void qref_quant_int4(const float* w, int N, int K, int8_t* c, uint16_t* s) {
  quant_levels(w, N, K, 16, c, s);
}

/* 1 bit keeps only the sign ([P1] "how big is 2.4 bits"; binarization as the
 * step beyond ternary, [P4] §7).  b = (w >= 0); the scale per 128 weights is
 * the mean |w| of the block (fp64, index order), stored as fp16. */
void qref_quant_sign1(const float* w, int N, int K, int8_t* b, uint16_t* s) {
  int nb = K / 128;
#pragma omp parallel for schedule(static)
  for (int n = 0; n < N; ++n)
    for (int kb = 0; kb < nb; ++kb) {
      const float* wb = w + (size_t)n * K + (size_t)kb * 128;
      double sum = 0.0;
      for (int i = 0; i < 128; ++i) sum += fabs((double)wb[i]);
      for (int i = 0; i < 128; ++i) b[(size_t)n * K + (size_t)kb * 128 + i] = wb[i] >= 0.0f ? 1 : 0;
      s[(size_t)n * nb + kb] = qref_f64_to_f16(sum / 128.0);
    }
}

/* ------------------------------------------------------------------------ */
/* Packers / unpackers                                                        */
/* ------------------------------------------------------------------------ */

/* Ternary byte: 5 trits of one byte form the base-3 number
 *   b = sum_{i=0..4} (t_i + 1) * 3^(4-i)        (digit 0 most significant)
 * stored as the 8-bit fixed-point base-3 fraction q = ceil(256 * b / 243),
 * so b = floor(243 * q / 256).  3 states per weight need log2 3 = 1.585 bits
 * ([P3] §1.2, [P4] §2.1); 5 per byte is 1.6 bits.
 * Within a 256-weight block (13 little-endian 32-bit words, 52 bytes):
 *   word m < 12, byte p, digit i  <->  weight 20m + 4i + p
 *   word 12,     byte p, digit i<4 <->  weight 240 + 4i + p; digit 4 = 1 (t = 0)
 */
static uint8_t tern_encode(const int t[5]) {
  int b = 0;
  for (int i = 0; i < 5; ++i) b = b * 3 + (t[i] + 1);
  return (uint8_t)((256 * b + 242) / 243); /* ceil(256 b / 243) */
}

static void tern_decode(uint8_t q, int t[5]) {
  int b = (243 * (int)q) >> 8; /* floor(243 q / 256) */
  for (int i = 4; i >= 0; --i) {
    t[i] = b % 3 - 1;
    b /= 3;
  }
}

/* Bit position of weight k (within its 32-bit word) for the plane formats.
 * The pages fix the bits per weight, not their order.  1- and 2-bit codes are
 * nibble-lane interleaved: weight 8j + n (n = 0..7) lives in nibble n of the
 * word at bit offset j * bits, so the j-th plane of a word holds the codes of
 * 8 consecutive weights, one per nibble.  4-bit codes are byte-lane
 * interleaved: weight 4j + lane (lane = 0..3) lives in byte `lane` at bit
 * offset 4j.  Words are little-endian. */
static int plane_bitpos(int k_in_word, int bits) {
  if (bits == 4) return 8 * (k_in_word % 4) + 4 * (k_in_word / 4);
  return 4 * (k_in_word % 8) + (k_in_word / 8) * bits;
}

int qref_pack(int fmt, const int8_t* codes, int N, int K, uint8_t* packed) {
  int64_t stride = qref_row_stride(fmt, K);
  if (stride < 0) return -1;
  memset(packed, 0, (size_t)stride * N);
  for (int n = 0; n < N; ++n) {
    const int8_t* c = codes + (size_t)n * K;
    uint8_t* row = packed + (size_t)n * stride;
    switch (fmt) {
      case QREF_TERN_B3:
        for (int blk = 0; blk < K / 256; ++blk) {
          uint8_t* bb = row + 52 * blk;
          const int8_t* cb = c + 256 * blk;
          for (int m = 0; m < 13; ++m)
            for (int p = 0; p < 4; ++p) {
              int t[5];
              for (int i = 0; i < 5; ++i) {
                if (m < 12) t[i] = cb[20 * m + 4 * i + p];
                else t[i] = (i < 4) ? cb[240 + 4 * i + p] : 0;
              }
              bb[4 * m + p] = tern_encode(t);
            }
        }
        break;
      case QREF_INT2:
      case QREF_SIGN1:
      case QREF_INT4: {
        int bits = fmt == QREF_INT2 ? 2 : fmt == QREF_SIGN1 ? 1 : 4;
        int per_word = 32 / bits;
        for (int w = 0; w < K / per_word; ++w) {
          uint32_t word = 0;
          for (int k = 0; k < per_word; ++k)
            word |= (uint32_t)(c[w * per_word + k] & ((1 << bits) - 1)) << plane_bitpos(k, bits);
          for (int by = 0; by < 4; ++by) row[4 * w + by] = (uint8_t)(word >> (8 * by));
        }
        break;
      }
      case QREF_TRELLIS2:
        /* Byte g = c[4g]<<6 | c[4g+1]<<4 | c[4g+2]<<2 | c[4g+3] (first symbol
         * in the top bits). */
        for (int g = 0; g < K / 4; ++g)
          row[g] = (uint8_t)(((c[4 * g] & 3) << 6) | ((c[4 * g + 1] & 3) << 4) |
                             ((c[4 * g + 2] & 3) << 2) | (c[4 * g + 3] & 3));
        break;
      default:
        return -1;
    }
  }
  return 0;
}

int qref_unpack(int fmt, const uint8_t* packed, int N, int K, int8_t* codes) {
  int64_t stride = qref_row_stride(fmt, K);
  if (stride < 0) return -1;
  for (int n = 0; n < N; ++n) {
    int8_t* c = codes + (size_t)n * K;
    const uint8_t* row = packed + (size_t)n * stride;
    switch (fmt) {
      case QREF_TERN_B3:
        for (int blk = 0; blk < K / 256; ++blk) {
          const uint8_t* bb = row + 52 * blk;
          int8_t* cb = c + 256 * blk;
          for (int m = 0; m < 13; ++m)
            for (int p = 0; p < 4; ++p) {
              int t[5];
              tern_decode(bb[4 * m + p], t);
              for (int i = 0; i < 5; ++i) {
                if (m < 12) cb[20 * m + 4 * i + p] = (int8_t)t[i];
                else if (i < 4) cb[240 + 4 * i + p] = (int8_t)t[i];
              }
            }
        }
        break;
      case QREF_INT2:
      case QREF_SIGN1:
      case QREF_INT4: {
        int bits = fmt == QREF_INT2 ? 2 : fmt == QREF_SIGN1 ? 1 : 4;
        int per_word = 32 / bits;
        for (int w = 0; w < K / per_word; ++w) {
          uint32_t word = 0;
          for (int by = 0; by < 4; ++by) word |= (uint32_t)row[4 * w + by] << (8 * by);
          for (int k = 0; k < per_word; ++k)
            c[w * per_word + k] = (int8_t)((word >> plane_bitpos(k, bits)) & ((1u << bits) - 1));
        }
        break;
      }
      case QREF_TRELLIS2:
        for (int g = 0; g < K / 4; ++g)
          for (int j = 0; j < 4; ++j) c[4 * g + j] = (int8_t)((row[g] >> (6 - 2 * j)) & 3);
        break;
      default:
        return -1;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Trellis codes and the hash codebook                                       */
/* ------------------------------------------------------------------------ */

/* The trellis format carries 2-3 bits per weight with a codebook computed at
 * run time from a hash ([P1] "how big is 2.4 bits"), coding each row in groups
 * of 4 weights ([P2] "12 GB 装下 27B，靠的是什么取舍").  This library's
 * variant: 2 bits per weight, a 16-bit state
 *   st <- ((st << 2) | c) & 0xFFFF, starting from a stored per-row seed,
 * the value index h = ((st * 0x9E37) ^ (st >> 7)) & 0xFF computed in uint32
 * on the state after its own symbol is shifted in. */
uint32_t qref_trellis_hash(uint32_t st) {
  return ((st * 0x9E37u) ^ (st >> 7)) & 0xFFu;
}

/* Standard normal CDF through the complementary error function. */
static double norm_cdf(double z) {
  return 0.5 * erfc(-z / sqrt(2.0));
}

/* Inverse standard normal CDF by bisection on norm_cdf: 200 halvings of
 * [-40, 40] reach the double-precision root. */
double qref_norm_ppf(double p) {
  double lo = -40.0, hi = 40.0;
  for (int it = 0; it < 200; ++it) {
    double mid = 0.5 * (lo + hi);
    if (mid == lo || mid == hi) break;
    if (norm_cdf(mid) < p) lo = mid;
    else hi = mid;
  }
  return 0.5 * (lo + hi);
}

/* The 8-bit hash selects one of 256 N(0,1) quantiles at the cell midpoints
 * (k + 0.5) / 256, stored as fp16. */
void qref_codebook_v16(uint16_t v16[256]) {
  for (int k = 0; k < 256; ++k) v16[k] = qref_f64_to_f16(qref_norm_ppf((k + 0.5) / 256.0));
}

/* int8 image of the codebook for the int8 dot-product GEMV:
 * V8[k] = rint(V16[k] * 127 / V16[255]), gain g = V16[255] / 127. */
void qref_codebook_v8(int8_t v8[256], double* g) {
  uint16_t v16[256];
  qref_codebook_v16(v16);
  double top = qref_f16_to_f64(v16[255]);
  for (int k = 0; k < 256; ++k) v8[k] = (int8_t)rint(qref_f16_to_f64(v16[k]) * 127.0 / top);
  if (g) *g = top / 127.0;
}

void qref_trellis_states(const uint8_t* packed, const uint16_t* seeds, int N, int K, uint16_t* st) {
  int64_t stride = qref_row_stride(QREF_TRELLIS2, K);
  for (int n = 0; n < N; ++n) {
    const uint8_t* row = packed + (size_t)n * stride;
    uint32_t s = seeds[n];
    for (int i = 0; i < K; ++i) {
      uint32_t c = (row[i / 4] >> (6 - 2 * (i % 4))) & 3u;
      s = ((s << 2) | c) & 0xFFFFu;
      st[(size_t)n * K + i] = (uint16_t)s;
    }
  }
}

/* Weight value = fp32(s64) * fp32(V16[h]); both factors have 11-bit
 * significands, so the fp32 product is exact. */
void qref_trellis_decode_f32(const uint8_t* packed, const uint16_t* seeds, const uint16_t* scales,
                             int N, int K, float* w) {
  uint16_t v16[256];
  qref_codebook_v16(v16);
  int64_t stride = qref_row_stride(QREF_TRELLIS2, K);
#pragma omp parallel for schedule(static)
  for (int n = 0; n < N; ++n) {
    const uint8_t* row = packed + (size_t)n * stride;
    uint32_t s = seeds[n];
    for (int i = 0; i < K; ++i) {
      uint32_t c = (row[i / 4] >> (6 - 2 * (i % 4))) & 3u;
      s = ((s << 2) | c) & 0xFFFFu;
      float v = (float)qref_f16_to_f64(v16[qref_trellis_hash(s)]);
      float sc = (float)qref_f16_to_f64(scales[(size_t)n * (K / 64) + i / 64]);
      w[(size_t)n * K + i] = sc * v;
    }
  }
}

/* Decode-time Q8 of the exact fp32 weights per (row, oblock) so that an int8
 * GEMM can consume trellis weights (the pages' prefill is an INT8 GEMM,
 * [P1] "porting a non-standard format into llama.cpp"). */
void qref_trellis_decode_i8(const uint8_t* packed, const uint16_t* seeds, const uint16_t* scales,
                            int N, int K, int oblock, int8_t* wq, float* dw) {
  float* w = (float*)malloc(sizeof(float) * (size_t)N * K);
  qref_trellis_decode_f32(packed, seeds, scales, N, K, w);
  int nb = K / oblock;
  for (int n = 0; n < N; ++n)
    for (int kb = 0; kb < nb; ++kb) {
      int32_t qs;
      size_t off = (size_t)n * K + (size_t)kb * oblock;
      qref_q8_block(w + off, oblock, wq + off, dw + (size_t)n * nb + kb, &qs);
    }
  free(w);
}

/* ------------------------------------------------------------------------ */
/* Trellis encoder: Viterbi over the bit-shift trellis                        */
/* ------------------------------------------------------------------------ */

/* Coding a row "jointly, a group of weights at a time" over the trellis
 * ([P2] "12 GB 装下 27B，靠的是什么取舍", after QTIP) means choosing the
 * symbol sequence whose decoded values are closest to the weights.  Closest
 * in squared error is a shortest path through the trellis: the Viterbi
 * algorithm, here in its textbook form over every state.
 *
 * States are L-bit words (2 <= L <= 16); a step shifts a 2-bit symbol c in:
 * st_i = ((st_{i-1} << 2) | c) mod 2^L, so state s has the 4 predecessors
 * (s >> 2) | (a << (L-2)), a = 0..3.  Any first state is allowed (the
 * seed is free).  The value of state s at step i is sc[i] * val[s].
 * Arithmetic, all fp32, each operation rounded once:
 *   d = w[i] - sc[i] * val[s]      (one fused rounding: fmaf(-sc, val, w))
 *   C_0[s] = d * d                 (fmaf(d, d, 0))
 *   C_i[s] = d * d + min_a C_{i-1}[(s >> 2) | (a << (L-2))]   (fmaf)
 * The predecessor taken by each state: within each pair {a, a + 2} (a = 0, 1)
 * the one of smaller cost C_{i-1}, on equal costs the one whose own incoming
 * minimum was smaller, then the smaller a; between the two pair winners the
 * one of smaller cost, on equal costs the winner of the pair {0, 2}.  (Where
 * the two states of a pair have the same value, as in the trellis below whose
 * hash ignores bit 15, a pair's order is that of the incoming minima, which
 * lets an implementation decide a pair before it adds the branch term.)  The
 * last state is the smallest s of minimum cost.  Writes the state path
 * st[0..K-1] and the minimum cost. */
int qref_viterbi(int L, const float* val, const float* w, const float* sc, int K, uint32_t* st,
                 float* cost) {
  if (L < 2 || L > 16 || K < 1) return -1;
  const uint32_t S = 1u << L, top = (uint32_t)(L - 2);
  float* prev = (float*)malloc(sizeof(float) * S);
  float* cur = (float*)malloc(sizeof(float) * S);
  float* inprev = (float*)malloc(sizeof(float) * S);  /* incoming minimum of each state */
  float* incur = (float*)malloc(sizeof(float) * S);
  uint8_t* dec = (uint8_t*)malloc((size_t)K * S);
  if (!prev || !cur || !inprev || !incur || !dec) {
    free(prev); free(cur); free(inprev); free(incur); free(dec);
    return -2;
  }
  for (int i = 0; i < K; ++i) {
    for (uint32_t s = 0; s < S; ++s) {
      float m = 0.0f;
      uint8_t best = 0;
      if (i > 0) {
        uint32_t p[4];
        for (uint32_t a = 0; a < 4; ++a) p[a] = (s >> 2) | (a << top);
        uint32_t win[2];
        for (uint32_t a = 0; a < 2; ++a) {
          const uint32_t x = p[a], y = p[a + 2];
          const int take_y = prev[y] < prev[x] || (prev[y] == prev[x] && inprev[y] < inprev[x]);
          win[a] = take_y ? a + 2 : a;
        }
        best = (uint8_t)(prev[p[win[1]]] < prev[p[win[0]]] ? win[1] : win[0]);
        m = prev[p[best]];
      }
      dec[(size_t)i * S + s] = best;
      incur[s] = m;
      float d = fmaf(-sc[i], val[s], w[i]);
      cur[s] = fmaf(d, d, m);
    }
    float* t = prev;
    prev = cur;
    cur = t;
    t = inprev;
    inprev = incur;
    incur = t;
  }
  uint32_t last = 0;
  for (uint32_t s = 1; s < S; ++s)
    if (prev[s] < prev[last]) last = s;
  *cost = prev[last];
  st[K - 1] = last;
  for (int i = K - 1; i > 0; --i) {
    uint32_t s = st[i];
    st[i - 1] = (s >> 2) | ((uint32_t)dec[(size_t)i * S + s] << top);
  }
  free(prev); free(cur); free(inprev); free(incur); free(dec);
  return 0;
}

/* Per-64 scale of the encoder when none is given: the block's root mean
 * square, so that the scaled values have unit power like the N(0,1)
 * codebook.  fp32: acc = fmaf(w_k, w_k, acc) for k = 0..63 in order, then
 * sqrtf(acc * (1/64)) (the factor is a power of two), stored as fp16 (round
 * to nearest even). */
uint16_t qref_trellis_rms_scale(const float* w64) {
  float acc = 0.0f;
  for (int k = 0; k < 64; ++k) acc = fmaf(w64[k], w64[k], acc);
  return qref_f64_to_f16((double)sqrtf(acc * 0.015625f));
}

/* Encode rows w [N][K] (K a multiple of 64) into the trellis format: scales
 * [N][K/64] fp16 (from scales_in when it is not NULL, else the RMS rule
 * above), then the Viterbi path of each row over the 2^16-state trellis with
 * val[s] = V16[hash(s)] and sc = the block's scale.  The symbols are the low
 * 2 bits of the path's states, packed as qref_pack does; the seed is
 * st_0 >> 2 (its top 2 bits are shifted out by the first symbol, so they are
 * written as 0).  cost [N] = the Viterbi minimum (the fp32 squared error of
 * the row's reconstruction as the recursion accumulates it). */
int qref_trellis_encode(const float* w, int N, int K, const uint16_t* scales_in, uint8_t* packed,
                        uint16_t* seeds, uint16_t* scales, float* cost) {
  if (N < 1 || K < 64 || K % 64) return -1;
  uint16_t v16[256];
  qref_codebook_v16(v16);
  float* val = (float*)malloc(sizeof(float) * 65536);
  int8_t* codes = (int8_t*)malloc((size_t)N * K);
  if (!val || !codes) {
    free(val); free(codes);
    return -2;
  }
  for (uint32_t s = 0; s < 65536; ++s) val[s] = (float)qref_f16_to_f64(v16[qref_trellis_hash(s)]);
  const int nb = K / 64;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (int n = 0; n < N; ++n) {
    const float* row = w + (size_t)n * K;
    float* sc = (float*)malloc(sizeof(float) * K);
    uint32_t* st = (uint32_t*)malloc(sizeof(uint32_t) * K);
    if (!sc || !st) {
      free(sc); free(st);
      err |= 1;
      continue;
    }
    for (int b = 0; b < nb; ++b) {
      uint16_t h = scales_in ? scales_in[(size_t)n * nb + b] : qref_trellis_rms_scale(row + 64 * b);
      scales[(size_t)n * nb + b] = h;
      for (int k = 0; k < 64; ++k) sc[64 * b + k] = (float)qref_f16_to_f64(h);
    }
    if (qref_viterbi(16, val, row, sc, K, st, cost + n)) err |= 1;
    for (int i = 0; i < K; ++i) codes[(size_t)n * K + i] = (int8_t)(st[i] & 3u);
    seeds[n] = (uint16_t)(st[0] >> 2);
    free(sc); free(st);
  }
  if (!err) qref_pack(QREF_TRELLIS2, codes, N, K, packed);
  free(val); free(codes);
  return err ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* KV cache in Q8 / Q4 and decode attention over it                           */
/* ------------------------------------------------------------------------ */

/* The KV cache grows with the context and is kept in 4 or 8 bits ([P1]
 * "12G 的账本要这么算": KV at Q4 or Q8 decides how long a context fits).
 * Each row of D values (one token of one KV head) is cut into 32-value
 * blocks with one fp16 scale each:
 *   Q8: d = amax / 127, r = 1 / d, id = r if finite else 0,
 *       c = clamp(rint(x * id), -127, 127), stored as int8;
 *   Q4: d = amax / 7, id likewise, c = clamp(rint(x * id), -7, 7), stored
 *       as the nibble c + 8 (byte j of a block: value 2j low, 2j+1 high).
 * All fp32, ties to even; the stored scale is fp16(d) (round to nearest
 * even), and the cached value is c * fp16(d). */
int64_t qref_kv_row_bytes(int fmt, int D) {
  if (D < 32 || D % 32) return -1;
  if (fmt == QREF_KV_Q8) return D;
  if (fmt == QREF_KV_Q4) return D / 2;
  return -1;
}

int qref_kv_quant(int fmt, const float* x, int64_t rows, int D, uint8_t* codes, uint16_t* scales) {
  const int64_t rb = qref_kv_row_bytes(fmt, D);
  if (rb < 0) return -1;
  const float top = fmt == QREF_KV_Q8 ? 127.0f : 7.0f;
  const int nb = D / 32;
  for (int64_t r = 0; r < rows; ++r)
    for (int b = 0; b < nb; ++b) {
      const float* v = x + r * D + 32 * b;
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i)
        if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
      const float d = amax / top;
      const float inv = 1.0f / d;
      const float id = isfinite(inv) ? inv : 0.0f;
      scales[r * nb + b] = qref_f64_to_f16((double)d);
      for (int i = 0; i < 32; ++i) {
        float t = rintf(v[i] * id);
        if (t > top) t = top;
        if (t < -top) t = -top;
        const int c = (int)t;
        if (fmt == QREF_KV_Q8) {
          codes[r * rb + 32 * b + i] = (uint8_t)(int8_t)c;
        } else {
          uint8_t* by = codes + r * rb + 16 * b + i / 2;
          if (i % 2 == 0) *by = (uint8_t)(c + 8);
          else *by = (uint8_t)(*by | ((c + 8) << 4));
        }
      }
    }
  return 0;
}

/* Cached values in fp64 (exact: a small integer times an fp16 scale). */
int qref_kv_dequant(int fmt, const uint8_t* codes, const uint16_t* scales, int64_t rows, int D, double* x) {
  const int64_t rb = qref_kv_row_bytes(fmt, D);
  if (rb < 0) return -1;
  const int nb = D / 32;
  for (int64_t r = 0; r < rows; ++r)
    for (int i = 0; i < D; ++i) {
      const double d = qref_f16_to_f64(scales[r * nb + i / 32]);
      int c;
      if (fmt == QREF_KV_Q8) {
        c = (int8_t)codes[r * rb + i];
      } else {
        const uint8_t by = codes[r * rb + i / 2];
        c = (int)((i % 2 == 0) ? (by & 15) : (by >> 4)) - 8;
      }
      x[r * D + i] = c * d;
    }
  return 0;
}

/* Decode attention of one new token with grouped KV heads ([P1]
 * "把非标准格式塞进 llama.cpp，难在哪": the KV heads serve query heads in
 * groups of 6).  Query row i = h * G + g (KV head h, member g) attends over
 * the T cached tokens of KV head h:
 *   s_t = (q_i . k_t) / sqrt(D),  p_t = exp(s_t - max s),
 *   out_i = sum_t p_t v_t / sum_t p_t,
 * with k_t, v_t the cached (dequantized) values; all in fp64.  Cache layout
 * codes [n_kv][t_cap][row bytes], scales [n_kv][t_cap][D/32].
 * bound (may be NULL) gets, per output, an error allowance (first order, a
 * factor 2 of slack) for an fp32 computation that sums each score over its
 * 32-value blocks and then over the D/32 blocks, and sums over tokens in
 * chunks of at most 256 tokens whose results are then summed in turn
 * (flash-decoding order), with u = 2^-24:
 *   sum_t p_t (e_t + 4u + u |s_t - max s|) (|v_t| + |out|) / sum p
 *   + 2 (256 + ceil(T / 256) + D / 32) u sum_t p_t |v_t| / sum p,
 *   e_t = 2 (32 + D / 32 + 8) u sum_d |q_d k_td| / sqrt(D):
 * the score error e_t moves the token's weight by that relative amount, the
 * exponential and the max subtraction add 4u + u |s_t - max s|, and the
 * token sums add the last term. */
int qref_attn_decode(int fmt, const float* q, int n_kv, int G, int D, int T, int64_t t_cap, const uint8_t* kc,
                     const uint16_t* ks, const uint8_t* vc, const uint16_t* vs, double* out, double* bound) {
  const int64_t rb = qref_kv_row_bytes(fmt, D);
  if (rb < 0 || n_kv < 1 || G < 1 || T < 1 || t_cap < T) return -1;
  const int nb = D / 32;
  const double u = ldexp(1.0, -24), isd = 1.0 / sqrt((double)D);
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (int h = 0; h < n_kv; ++h) {
    double* K = (double*)malloc(sizeof(double) * (size_t)T * D);
    double* V = (double*)malloc(sizeof(double) * (size_t)T * D);
    double* s = (double*)malloc(sizeof(double) * (size_t)T);
    double* e = (double*)malloc(sizeof(double) * (size_t)T);
    double* acc_v = (double*)malloc(sizeof(double) * 3 * (size_t)D);
    double* abs_v = acc_v ? acc_v + D : NULL;
    double* err_v = acc_v ? acc_v + 2 * D : NULL;
    if (!K || !V || !s || !e || !acc_v) {
      free(K); free(V); free(s); free(e); free(acc_v);
      err |= 1;
      continue;
    }
    qref_kv_dequant(fmt, kc + (size_t)h * t_cap * rb, ks + (size_t)h * t_cap * nb, T, D, K);
    qref_kv_dequant(fmt, vc + (size_t)h * t_cap * rb, vs + (size_t)h * t_cap * nb, T, D, V);
    for (int g = 0; g < G; ++g) {
      const float* qi = q + ((size_t)h * G + g) * D;
      double m = -INFINITY;
      for (int t = 0; t < T; ++t) {
        double acc = 0.0, aabs = 0.0;
        for (int d = 0; d < D; ++d) {
          acc += (double)qi[d] * K[(size_t)t * D + d];
          aabs += fabs((double)qi[d] * K[(size_t)t * D + d]);
        }
        s[t] = acc * isd;
        e[t] = 2.0 * (32 + D / 32 + 8) * u * aabs * isd;
        if (s[t] > m) m = s[t];
      }
      double L = 0.0;
      for (int t = 0; t < T; ++t) {
        e[t] += 4.0 * u + u * fabs(s[t] - m);  /* the token's relative weight error */
        s[t] = exp(s[t] - m);                   /* from here on s holds p */
        L += s[t];
      }
      double* o = out + ((size_t)h * G + g) * D;
      double* bo = bound ? bound + ((size_t)h * G + g) * D : NULL;
      for (int d = 0; d < D; ++d) acc_v[d] = abs_v[d] = err_v[d] = 0.0;
      for (int t = 0; t < T; ++t)
        for (int d = 0; d < D; ++d) {
          acc_v[d] += s[t] * V[(size_t)t * D + d];
          abs_v[d] += s[t] * fabs(V[(size_t)t * D + d]);
        }
      for (int d = 0; d < D; ++d) o[d] = acc_v[d] / L;
      if (bo) {
        for (int t = 0; t < T; ++t)
          for (int d = 0; d < D; ++d) err_v[d] += s[t] * e[t] * (fabs(V[(size_t)t * D + d]) + fabs(o[d]));
        const double chain = 256.0 + (double)((T + 255) / 256) + D / 32;
        for (int d = 0; d < D; ++d) bo[d] = err_v[d] / L + 2.0 * chain * u * abs_v[d] / L;
      }
    }
    free(K); free(V); free(s); free(e); free(acc_v);
  }
  return err ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* GEMV                                                                       */
/* ------------------------------------------------------------------------ */

/* Integer level of each weight and the fp64 factor that turns the integer
 * block dot into weight units:
 *   TERN_B3  level t            factor s(256-block)
 *   INT2     level 2c - 3       factor s(32-block) / 2
 *   SIGN1    level 2b - 1       factor s(128-block)
 *   INT4     level 2c - 15      factor s(32-block) / 2
 *   TRELLIS2 level V8[h]        factor s(64-block) * g
 * Ternary products reduce to add, subtract or skip ([P3] §1.2, [P4] §2.2);
 * the integer dot below is that sum. */
int qref_gemv(int fmt, const uint8_t* packed, const uint16_t* scales, const uint16_t* seeds,
              int N, int K, const int8_t* q, const float* d, int B,
              int64_t* I, double* y, double* absT) {
  int blk = qref_scale_block(fmt);
  if (blk == 0 || K % blk != 0 || K % 32 != 0) return -1;
  int64_t stride = qref_row_stride(fmt, K);
  int nsb = K / blk, nkb = K / 32;
  int8_t v8[256];
  double g = 0.0;
  if (fmt == QREF_TRELLIS2) qref_codebook_v8(v8, &g);
  int rc = 0;
#pragma omp parallel for schedule(dynamic, 16)
  for (int n = 0; n < N; ++n) {
    int8_t* lev = (int8_t*)malloc((size_t)K);
    int8_t* codes = (int8_t*)malloc((size_t)K);
    const uint8_t* row = packed + (size_t)n * stride;
    if (fmt == QREF_TRELLIS2) {
      uint32_t st = seeds[n];
      for (int i = 0; i < K; ++i) {
        uint32_t c = (row[i / 4] >> (6 - 2 * (i % 4))) & 3u;
        st = ((st << 2) | c) & 0xFFFFu;
        lev[i] = v8[qref_trellis_hash(st)];
      }
    } else {
      qref_unpack(fmt, row, 1, K, codes);
      for (int i = 0; i < K; ++i) {
        int c = codes[i];
        lev[i] = (int8_t)(fmt == QREF_TERN_B3 ? c : fmt == QREF_INT2 ? 2 * c - 3
                          : fmt == QREF_SIGN1 ? 2 * c - 1 : 2 * c - 15);
      }
    }
    for (int b = 0; b < B; ++b) {
      const int8_t* qb = q + (size_t)b * K;
      double acc = 0.0, aacc = 0.0;
      for (int kb = 0; kb < nkb; ++kb) {
        int64_t dot = 0;
        for (int i = 0; i < 32; ++i) dot += (int64_t)lev[kb * 32 + i] * qb[kb * 32 + i];
        double s = qref_f16_to_f64(scales[(size_t)n * nsb + (kb * 32) / blk]);
        double f = (fmt == QREF_INT2 || fmt == QREF_INT4) ? 0.5 * s : fmt == QREF_TRELLIS2 ? s * g : s;
        double T = f * (double)d[(size_t)b * nkb + kb] * (double)dot;
        acc += T;
        aacc += fabs(T);
        if (I) I[((size_t)b * N + n) * nkb + kb] = dot;
      }
      if (y) y[(size_t)b * N + n] = acc;
      if (absT) absT[(size_t)b * N + n] = aacc;
    }
    free(lev);
    free(codes);
  }
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Block-randomized Walsh-Hadamard rotation                                   */
/* ------------------------------------------------------------------------ */

/* Random Hadamard rotation of the QuIP / QuIP# / QTIP line ([P2] "12 GB 装下
 * 27B"): here applied to activations in 256-blocks.  Sylvester (natural)
 * order; stage h = 1, 2, ..., 128 maps (u_i, u_{i+h}) to (u_i + u_{i+h},
 * u_i - u_{i+h}) for every i with (i & h) == 0; then scale by 1/16 so the
 * transform is orthonormal.  fp32, this exact order. */
void qref_fwht256(float* u) {
  for (int h = 1; h < 256; h <<= 1)
    for (int i = 0; i < 256; ++i)
      if ((i & h) == 0) {
        float a = u[i], b = u[i + h];
        u[i] = a + b;
        u[i + h] = a - b;
      }
  for (int i = 0; i < 256; ++i) u[i] = u[i] * 0.0625f;
}

void qref_hadamard_quant(const float* x, int B, int K, const uint32_t* sign_bits, int qblock,
                         int8_t* q, float* d, int32_t* qsum) {
  int nq = K / qblock;
  float u[256];
  for (int b = 0; b < B; ++b) {
    float* rot = (float*)malloc(sizeof(float) * (size_t)K);
    for (int blk = 0; blk < K / 256; ++blk) {
      for (int i = 0; i < 256; ++i) {
        int k = blk * 256 + i;
        float v = x[(size_t)b * K + k];
        u[i] = ((sign_bits[k / 32] >> (k % 32)) & 1u) ? -v : v;
      }
      qref_fwht256(u);
      memcpy(rot + blk * 256, u, sizeof(u));
    }
    for (int kb = 0; kb < nq; ++kb)
      qref_q8_block(rot + kb * qblock, qblock, q + (size_t)b * K + kb * qblock,
                    d + (size_t)b * nq + kb, qsum + (size_t)b * nq + kb);
    free(rot);
  }
}

/* ------------------------------------------------------------------------ */
/* GEMM                                                                       */
/* ------------------------------------------------------------------------ */

/* Prefill as an int8 GEMM with per-block scales on both operands ([P1]
 * "porting a non-standard format into llama.cpp"). */
void qref_gemm_i8(const int8_t* xq, const float* dx, int M, const int8_t* wq, const float* dw,
                  int N, int K, int kblock, double* y, double* absT) {
  int nb = K / kblock;
#pragma omp parallel for schedule(dynamic, 1)
  for (int m = 0; m < M; ++m)
    for (int n = 0; n < N; ++n) {
      double acc = 0.0, aacc = 0.0;
      for (int kb = 0; kb < nb; ++kb) {
        int64_t dot = 0;
        for (int i = 0; i < kblock; ++i)
          dot += (int64_t)xq[(size_t)m * K + kb * kblock + i] * wq[(size_t)n * K + kb * kblock + i];
        double T = (double)dx[(size_t)m * nb + kb] * (double)dw[(size_t)n * nb + kb] * (double)dot;
        acc += T;
        aacc += fabs(T);
      }
      y[(size_t)m * N + n] = acc;
      if (absT) absT[(size_t)m * N + n] = aacc;
    }
}
