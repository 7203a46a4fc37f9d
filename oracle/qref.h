/*
 * qref — the plain CPU oracle for extreme low-bit GEMV/GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this code.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant
 * generator with the HIP library; the two agree only through the format
 * definitions written out below.
 *
 * Arithmetic conventions
 *   - Integer block dot products are computed in int64.
 *   - Every quantity that no page fixes is computed in fp64.
 *   - Where a float decides an integer (activation Q8, the Hadamard rotation
 *     that feeds it, the weight quantizers), the decision is taken in the
 *     precision stated at the function: fp32 for the activation path (the
 *     kernel's precision, with IEEE division and round-half-even), fp64 for
 *     the weight quantizers.
 *   - Build with -O2 -ffp-contract=off and never with -ffast-math.
 *
 * Pages cited (each by title and section):
 *   [P1] "A 27B model at 2.4 bits on a 12 GB RTX 3090" (61893.com)
 *   [P2] "27B 模型压进 12GB 显存的量化实践" (feinterview.poetries.top)
 *   [P3] "为什么'8G显卡跑27B'…" ternary portable pack (pptc.cn)
 *   [P4] "一个 27B 模型被塞进 5.9 GB" (mhpq.cn)
 *   [P5] "升到 4 比特慢了 29%、1 比特快了三倍…" (neodrop.ai)
 *
 * Parity unpinned: nothing here.  Every function is pinned by a test that
 * does not call back into the same arithmetic (see tests/test_oracle_*.py).
 */
#ifndef QREF_H
#define QREF_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight formats.  Values are part of the packed-weight descriptor format. */
enum {
  QREF_TERN_B3 = 1,   /* ternary, 5 trits per byte, scale per 256 */
  QREF_INT2 = 2,      /* 2-bit four-level, scale per 32 */
  QREF_SIGN1 = 3,     /* 1-bit sign, scale per 128 */
  QREF_INT4 = 4,      /* 4-bit sixteen-level, scale per 32 */
  QREF_TRELLIS2 = 5   /* 2-bit bit-shift trellis codes, scale per 64 */
};

/* KV cache formats (values are part of the cache descriptor). */
enum {
  QREF_KV_Q4 = 4,     /* 4-bit, fp16 scale per 32 */
  QREF_KV_Q8 = 8      /* 8-bit, fp16 scale per 32 */
};

/* OpenMP threads of the parallel loops (timing only; results do not depend on it). */
int qref_threads(void);
void qref_set_threads(int n);

/* Scale block along K for a format (0 for an unknown format). */
int qref_scale_block(int fmt);
/* Packed bytes of one row of K weights, without padding (<0 on bad K). */
int64_t qref_packed_row_bytes(int fmt, int K);
/* Row stride of the packed layout: packed bytes rounded up to 16. */
int64_t qref_row_stride(int fmt, int K);

/* fp16 <-> fp64, round to nearest even, subnormals kept. */
uint16_t qref_f64_to_f16(double x);
double qref_f16_to_f64(uint16_t h);

/* Q8 of one block of n fp32 values (fp32 arithmetic, see qref.c). */
void qref_q8_block(const float* v, int n, int8_t* q, float* d, int32_t* qsum);
/* Activation quantization: x [B][K] -> q [B][K], d and qsum [B][K/qblock]. */
void qref_act_quant(const float* x, int B, int K, int qblock, int8_t* q, float* d, int32_t* qsum);
/* 4-bit planes of int8 activations q [B][K] (K a multiple of 32) ->
 * planes [B][K/32][8] (see qref.c). */
void qref_act_planes(const int8_t* q, int B, int K, uint32_t* planes);

/* Weight quantizers: w [N][K] fp32 -> integer codes [N][K] + fp16 scales
 * [N][K/block].  Code meaning per format:
 *   TERN_B3: t in {-1,0,1};  INT2: c in 0..3 (level (2c-3)/2);
 *   SIGN1: b in {0,1} (level 2b-1);  INT4: c in 0..15 (level (2c-15)/2). */
void qref_quant_tern(const float* w, int N, int K, int8_t* t, uint16_t* s);
void qref_quant_int2(const float* w, int N, int K, int8_t* c, uint16_t* s);
void qref_quant_sign1(const float* w, int N, int K, int8_t* b, uint16_t* s);
void qref_quant_int4(const float* w, int N, int K, int8_t* c, uint16_t* s);

/* Packers and unpackers between per-weight codes [N][K] (int8) and the
 * packed rows [N][stride] (stride = qref_row_stride; padding bytes are 0).
 * For TRELLIS2 the codes are the 2-bit trellis symbols 0..3. */
int qref_pack(int fmt, const int8_t* codes, int N, int K, uint8_t* packed);
int qref_unpack(int fmt, const uint8_t* packed, int N, int K, int8_t* codes);

/* Trellis: hash of a 16-bit state, the fp16 N(0,1)-quantile codebook,
 * the int8 codebook for the GEMV and its gain g (value ~= g * V8). */
uint32_t qref_trellis_hash(uint32_t state);
double qref_norm_ppf(double p);
void qref_codebook_v16(uint16_t v16[256]);
void qref_codebook_v8(int8_t v8[256], double* g);
/* States after each symbol, by the literal recurrence: st [N][K] (uint16). */
void qref_trellis_states(const uint8_t* packed, const uint16_t* seeds, int N, int K, uint16_t* st);
/* Decoded fp32 weights w [N][K] = fp32(s64) * fp32(V16[h]). */
void qref_trellis_decode_f32(const uint8_t* packed, const uint16_t* seeds, const uint16_t* scales,
                             int N, int K, float* w);
/* Decode then Q8 per (row, oblock): wq [N][K] int8, dw [N][K/oblock] fp32. */
void qref_trellis_decode_i8(const uint8_t* packed, const uint16_t* seeds, const uint16_t* scales,
                            int N, int K, int oblock, int8_t* wq, float* dw);

/* Viterbi over an L-bit bit-shift trellis (2 bits per step): the state path
 * st [K] minimising the squared error to w with state values sc[i]*val[s],
 * in fp32 (see qref.c for the exact operations and tie rules).  0 or <0. */
int qref_viterbi(int L, const float* val, const float* w, const float* sc, int K, uint32_t* st,
                 float* cost);
/* RMS scale of one 64-block for the encoder, as fp16 bits. */
uint16_t qref_trellis_rms_scale(const float* w64);
/* Trellis encoder: w [N][K] fp32 -> packed [N][stride], seeds [N], scales
 * [N][K/64] fp16 (row-major; scales_in overrides the RMS rule when not
 * NULL), cost [N] fp32.  0 or <0. */
int qref_trellis_encode(const float* w, int N, int K, const uint16_t* scales_in, uint8_t* packed,
                        uint16_t* seeds, uint16_t* scales, float* cost);

/* KV cache: bytes per row of D values, quantization of rows x [rows][D] fp32
 * to codes [rows][row bytes] + fp16 scales [rows][D/32], and the cached values
 * back in fp64.  0 or <0. */
int64_t qref_kv_row_bytes(int fmt, int D);
int qref_kv_quant(int fmt, const float* x, int64_t rows, int D, uint8_t* codes, uint16_t* scales);
int qref_kv_dequant(int fmt, const uint8_t* codes, const uint16_t* scales, int64_t rows, int D, double* x);
/* Decode attention over the cached KV heads, G query rows per KV head:
 * q [n_kv * G][D] fp32 -> out [n_kv * G][D] fp64, bound (may be NULL) the
 * per-output fp32 error allowance (see qref.c).  0 or <0. */
int qref_attn_decode(int fmt, const float* q, int n_kv, int G, int D, int T, int64_t t_cap, const uint8_t* kc,
                     const uint16_t* ks, const uint8_t* vc, const uint16_t* vs, double* out, double* bound);

/* GEMV over packed weights and Q8 activations (per-32 activation blocks).
 *   packed [N][stride], scales fp16 [N][K/block], seeds [N] (TRELLIS2 only)
 *   q [B][K], d [B][K/32]
 * Outputs (any may be NULL):
 *   I    [B][N][K/32] int64 exact block dots
 *   y    [B][N] fp64, absT [B][N] fp64 = sum of |terms|. */
int qref_gemv(int fmt, const uint8_t* packed, const uint16_t* scales, const uint16_t* seeds,
              int N, int K, const int8_t* q, const float* d, int B,
              int64_t* I, double* y, double* absT);

/* Fast Walsh-Hadamard transform of 256 fp32 values in place, natural
 * (Sylvester) order, ascending stages, then x 1/16. */
void qref_fwht256(float* u);
/* Rotation + Q8: x [B][K] fp32, sign_bits [K/32] (bit set = sign -1),
 * per 256-block u = sigma*x, FWHT, then Q8 per qblock (32 or 256). */
void qref_hadamard_quant(const float* x, int B, int K, const uint32_t* sign_bits, int qblock,
                         int8_t* q, float* d, int32_t* qsum);

/* Block-scaled int8 GEMM: y[m][n] = sum_kb dx[m][kb] dw[n][kb] I[m][n][kb].
 * xq [M][K], dx [M][K/kblock], wq [N][K], dw [N][K/kblock]; y, absT [M][N]. */
void qref_gemm_i8(const int8_t* xq, const float* dx, int M, const int8_t* wq, const float* dw,
                  int N, int K, int kblock, double* y, double* absT);

#ifdef __cplusplus
}
#endif
#endif
