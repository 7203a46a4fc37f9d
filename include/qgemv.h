/*
 * qgemv.h — C ABI of libqgemv, extreme low-bit GEMV/GEMM for AMD MI355X (gfx950).
 *
 * What it computes.  Matrix-vector and small-batch products y = W x for LLM
 * weights stored in extreme low-bit packed form, multiplied against int8
 * activations; an int8 GEMM for prefill.  The pages this follows:
 *   [P1] "A 27B model at 2.4 bits on a 12 GB RTX 3090" (61893.com)
 *   [P2] "27B 模型压进 12GB 显存的量化实践" (feinterview.poetries.top)
 *   [P3] "为什么'8G显卡跑27B'…" ternary portable pack (pptc.cn)
 *   [P4] "一个 27B 模型被塞进 5.9 GB" (mhpq.cn)
 *   [P5] "升到 4 比特慢了 29%、1 比特快了三倍…" (neodrop.ai)
 *
 * Conventions for every call below.
 *   - Pointers marked (device) are device memory owned by the caller; the
 *     library never allocates, frees or keeps them.  (host) pointers are read
 *     during the call only.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every device call
 *     is asynchronous on that stream; nothing synchronises the host.
 *   - Return value: 0 on success or a negative QERR_* code.  All argument checks
 *     run on the host before any HIP call, so a rejected call has no effect on
 *     the GPU.  QERR_HIP means a launch failed.  No exception crosses the ABI.
 *   - Calls are reentrant and thread-safe.  The only state kept between calls
 *     is built once and then only read: the trellis codebook tables and, per
 *     device and kernel, the number of workgroups a persistent launch uses
 *     (an occupancy query); both are filled under a lock.
 *   - Codes are dense row-major: weight row n is `row_bytes` bytes at
 *     codes + n*row_bytes.  Scales are fp16 bit patterns in the tiled order
 *     described at qfmt_scales_bytes (convert with qweight_set_scales /
 *     qweight_get_scales).
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- error codes ------------------------------------------------------------- */
#define QERR_OK 0
#define QERR_INVALID_ARG (-1)     /* null pointer, negative size, bad enum value */
#define QERR_UNSUPPORTED_FMT (-2) /* unknown format, or format not valid for the call */
#define QERR_SHAPE (-3)           /* sizes violate the format's block rules */
#define QERR_ALIGNMENT (-4)       /* pointer or stride misaligned */
#define QERR_HIP (-5)             /* a HIP launch or query failed */
#define QERR_BUFFER (-6)          /* caller buffer too small, or not a plan */
#define QERR_TOO_LARGE (-7)       /* exceeds a fixed limit of the library (static plan storage) */

/* Human-readable text for a QERR_* code (static storage, never NULL). */
const char* qstrerror(int err);
/* Name of the HIP error behind the calling thread's most recent QERR_HIP
 * ("hipSuccess" if there was none); static storage, never NULL. */
const char* qhip_error_name(void);

/* ---- weight formats ----------------------------------------------------------- *
 * Level counts: 4 bits hold 16 levels, 2 bits 4, 1 bit only the sign ([P1]
 * "2.4bit 是个什么量级").  Every format carries one fp16 scale per block of
 * `block` weights along a row ([P4] §2.1: value = code x block scale).
 *
 *  QFMT_TERN_B3 (block 256): ternary {-1,0,1}.  Products become add, subtract or
 *    skip ([P3] §1.2, [P4] §2.2).  5 trits per byte in base 3: the trits'
 *    digits d_i = t_i + 1 form b = sum_i d_i 3^(4-i) (digit 0 most significant),
 *    stored as the fixed-point base-3 fraction byte = ceil(256 b / 243).  A
 *    256-weight block is 13 little-endian 32-bit words (52 bytes, 1.625 bits per
 *    weight; log2 3 = 1.585 is the floor, [P3] §1.2): word m < 12, byte p, digit
 *    i holds weight 20m + 4i + p; word 12, byte p, digit i < 4 holds weight
 *    240 + 4i + p and its digit 4 is 1.  Row bytes 52*cols/256.
 *  QFMT_INT2 (block 32): four levels (2c - 3)/2 * s, c = 0..3.  One 32-bit
 *    word per 16 weights; weight 8j + n (j = 0..1, n = 0..7) is bits
 *    4n+2j .. 4n+2j+1 (nibble-lane order: (word >> 2j) & 0x33333333 holds
 *    weights 8j .. 8j+7, one per nibble).
 *  QFMT_SIGN1 (block 128): levels (2b - 1) * s, 8 weights per byte ([P5] §二).
 *    One 32-bit word per 32 weights; weight 8j + n (j = 0..3, n = 0..7) is bit
 *    4n + j (nibble-lane order, as for INT2).
 *  QFMT_INT4 (block 32): sixteen levels (2c - 15)/2 * s.  One 32-bit word per 8
 *    weights; weight 4j + b (j = 0..1) is bits 8b+4j .. 8b+4j+3.
 *  QFMT_TRELLIS2 (block 64): 2-bit bit-shift trellis codes with a codebook
 *    computed at run time from a hash ([P1] "2.4bit 是个什么量级"), each row coded
 *    in groups of 4 weights from a stored seed ([P2] "12 GB 装下 27B，靠的是什么
 *    取舍").  Byte g of a row = c[4g]<<6 | c[4g+1]<<4 | c[4g+2]<<2 | c[4g+3].
 *    State st <- ((st << 2) | c) & 0xFFFF starting at the row's uint16 seed;
 *    h = ((st * 0x9E37) ^ (st >> 7)) & 0xFF; value = s * V16[h] where V16[k] is
 *    the fp16 nearest to the N(0,1) quantile at (k + 0.5)/256.
 */
#define QFMT_TERN_B3 1
#define QFMT_INT2 2
#define QFMT_SIGN1 3
#define QFMT_INT4 4
#define QFMT_TRELLIS2 5

/* Scale block along K for a format, 0 if unknown. */
int32_t qfmt_scale_block(int32_t fmt);
/* Packed bytes of one row (no padding); <0 (QERR_*) on bad arguments.
 * cols must be a positive multiple of the scale block. */
int64_t qfmt_packed_row_bytes(int32_t fmt, int32_t cols);
/* Minimum legal row stride: packed bytes rounded up to 16. */
int64_t qfmt_row_bytes(int32_t fmt, int32_t cols);

/* Scale storage.  The scale of (row r, block b), b < cols/block, lives at
 *   index ((r / 64 * NG + b / G) * 64 + r % 64) * G + b % G
 * with G = qfmt_scale_group(fmt) and NG = ceil((cols/block) / G): tiles of
 * 64 rows x G blocks, tiles in row-major order over (row tile, block group),
 * each tile row-major.  G is the blocks of one GEMV segment (1024 weights for
 * TERN_B3 and SIGN1, 512 for INT2 and TRELLIS2, 256 for INT4), so one
 * segment of a 64-row tile reads one contiguous run of 128 G bytes instead of
 * 2 G bytes from each of 64 rows.  Slots with r >= rows or b >= cols/block
 * must be zero (qweight_quantize and qweight_set_scales write them).
 * qfmt_scales_bytes: bytes of that array (rows, cols as in qweight_t); <0 on
 * bad arguments. */
int32_t qfmt_scale_group(int32_t fmt);
int64_t qfmt_scales_bytes(int32_t fmt, int32_t rows, int32_t cols);

/* Packed-weight descriptor.  All pointers (device). */
typedef struct qweight {
  int32_t fmt;            /* QFMT_* */
  int32_t rows;           /* N >= 1 (output features) */
  int32_t cols;           /* K >= 1 (input features), multiple of block, and of 256 for TERN_B3 */
  int32_t block;          /* must equal qfmt_scale_block(fmt) */
  const void* codes;      /* [rows][row_bytes] bytes, 16-byte aligned */
  int64_t row_bytes;      /* stride, a multiple of 16, >= qfmt_packed_row_bytes */
  const uint16_t* scales; /* qfmt_scales_bytes bytes, tiled (above), 16-byte aligned */
  const uint16_t* seeds;  /* [rows] uint16 trellis seeds; TRELLIS2 only, else NULL */
} qweight_t;

/* Host-only validation of a descriptor (no HIP call).  0 or QERR_*. */
int qweight_check(const qweight_t* w);

/* ---- weight preparation (device) ------------------------------------------------ */

/* Quantize fp32 weights w [rows][cols] (device) and pack them.  Quantizer per
 * format, decisions taken in fp64:
 *   TERN_B3: per 256-block s = mean|w| + 1e-8, t = clamp(round(w / s), -1, 1)
 *            with round half to even ([P3] §5.1, there per tensor);
 *   INT2 / INT4: s = fp16(amax / 1.5) resp. fp16(amax / 7.5) per 32-block,
 *            code = nearest level to w / s, ties to the upper level;
 *   SIGN1:   bit = (w >= 0), s = mean |w| per 128-block.
 * Sums run in index order; stored scale = fp16 (round to nearest even).
 * Output codes [rows][row_bytes] (16-byte aligned, padding zeroed) and
 * scales (qfmt_scales_bytes, tiled, padding zeroed).  TRELLIS2 is not a
 * quantizer target (QERR_UNSUPPORTED_FMT). */
int qweight_quantize(int32_t fmt, const float* w, int32_t rows, int32_t cols,
                     void* codes, int64_t row_bytes, uint16_t* scales, void* stream);

/* Write w->scales (device, tiled) from row-major fp16 scales rowmajor
 * [rows][cols/block] (device); padding slots are zeroed.  Only w's geometry and
 * scales pointer are used. */
int qweight_set_scales(const qweight_t* w, const uint16_t* rowmajor, void* stream);
/* Read w->scales back as row-major rowmajor [rows][cols/block] (device). */
int qweight_get_scales(const qweight_t* w, uint16_t* rowmajor, void* stream);

/* Pack per-weight integer codes levels [rows][cols] int8 (device) into the
 * format's bytes: TERN_B3 trits -1..1; INT2 0..3; SIGN1 0..1; INT4 0..15;
 * TRELLIS2 symbols 0..3.  Out-of-range codes are masked to the field width
 * (ternary values other than -1..1 give undefined bytes).  Padding zeroed. */
int qweight_pack(int32_t fmt, const int8_t* levels, int32_t rows, int32_t cols,
                 void* codes, int64_t row_bytes, void* stream);

/* ---- activation quantization (device) --------------------------------------------- */

/* Q8 per block of `qblock` (32 or 256) values of x [B][K] fp32 (finite):
 *   amax = max|x|; d = amax / 127 (fp32, IEEE division); r = 1/d (fp32);
 *   id = r if r is finite, else 0 (a zero block, or d <= 2^-128 where the
 *   reciprocal overflows: q = 0, qsum = 0, d kept);
 *   q = clamp(rint(x * id), -127, 127) (ties to even); qsum = sum q.
 * int8 activations are what the pages' int8 dot-product GEMV and int8 MMA /
 * GEMM paths consume ([P1] "把非标准格式塞进 llama.cpp，难在哪").
 * Outputs q [B][K] int8, d [B][K/qblock] fp32, qsum [B][K/qblock] int32.
 * Bit-exact: the same fp32 operations as the definition. */
int qact_quant_i8(const float* x, int32_t B, int32_t K, int32_t qblock,
                  int8_t* q, float* d, int32_t* qsum, void* stream);

/* 4-bit planes of int8 activations, the form in which the INT2 and SIGN1 GEMV
 * read the int8 activations of qact_quant_i8 (it multiplies 4-bit code planes
 * against them with 8-way nibble dot products).  q [B][K] int8 (device,
 * 4-byte aligned), K a positive multiple of 32 -> planes [B][K/32][8] uint32
 * (device, 32-byte aligned).  For every 32-block and group g = 0..3 of the
 * values x_n = q[32 kb + 8 g + n], n = 0..7: word g = sum_n (x_n mod 16) << 4n
 * and word 4 + g = sum_n (floor(x_n / 16) mod 16) << 4n, so x_n = 16 hi + lo
 * with lo unsigned and hi a two's complement nibble.  Integer, bit-exact. */
int qact_planes(const int8_t* q, int32_t B, int32_t K, uint32_t* planes, void* stream);

/* One activation input of qact_quant_batch: x [B][K] fp32 (16-byte aligned),
 * K a positive multiple of 32; outputs as qact_quant_i8 with qblock 32 (q
 * 4-byte aligned) and qact_planes (planes 32-byte aligned), either of q and
 * planes may be NULL but not both; d and qsum are required. */
typedef struct qact_job {
  const float* x;
  int32_t B, K;
  int8_t* q;
  uint32_t* planes;
  float* d;
  int32_t* qsum;
} qact_job_t;
#define QACT_BATCH_MAX 16

/* Q8 per 32 values of up to QACT_BATCH_MAX activation inputs in one launch
 * (the inputs of every matrix of a decode step: same results as qact_quant_i8
 * with qblock 32 followed by qact_planes, bit for bit, without the int8
 * round trip).  jobs: host array of n entries (0 <= n <= QACT_BATCH_MAX);
 * QERR_INVALID_ARG for a bad count, size or missing pointer, QERR_SHAPE for
 * K % 32, QERR_ALIGNMENT for misaligned pointers, all before any launch. */
int qact_quant_batch(const qact_job_t* jobs, int32_t n, void* stream);

/* Block-randomized Walsh-Hadamard rotation then Q8 (the random Hadamard
 * rotation of [P2] "12 GB 装下 27B", applied to activations): per token and
 * 256-block, u = sigma * x with sigma_k = -1 where bit k%32 of sign_bits[k/32]
 * is set; stages h = 1, 2, ..., 128 map (u_i, u_{i+h}) to (u_i + u_{i+h},
 * u_i - u_{i+h}) for (i & h) == 0 (Sylvester order); times 1/16; then Q8 per
 * qblock (32, 256, or K: one scale per token row, K <= 32768, else
 * QERR_SHAPE) as in qact_quant_i8; d and qsum [B][K/qblock].  fp32,
 * bit-exact.  K multiple of 256; sign_bits [K/32] (device). */
int qact_hadamard_quant_i8(const float* x, int32_t B, int32_t K, const uint32_t* sign_bits,
                           int32_t qblock, int8_t* q, float* d, int32_t* qsum, void* stream);

/* ---- GEMV ----------------------------------------------------------------------- */

/* y[b][n] = sum_kb T[b][n][kb], T = f * s_w * d[b][kb] * I[b][n][kb], where I is
 * the exact integer dot of the weight levels with q over the 32-block kb:
 *   TERN_B3 level t, f = 1;  INT2 level 2c-3, f = 1/2;  SIGN1 level 2b-1, f = 1;
 *   INT4 level 2c-15, f = 1/2;  TRELLIS2 level V8[h] = rint(V16[h]*127/V16[255]),
 *   f = V16[255]/127.
 * The decode-time GEMV of the pages runs over int8 activations with 4-way int8
 * dot products ([P1] "把非标准格式塞进 llama.cpp，难在哪"); with batch B the
 * weights are decoded once for all tokens ([P5] §五: checking 16 tokens costs
 * about as much as 1 when the product is bandwidth-bound).
 * Inputs (device): q [B][K] int8 (16-byte aligned), d [B][K/32] fp32,
 * qsum [B][K/32] int32 (block sums of q, as written by qact_quant_i8), and
 * planes [B][K/32][8] (32-byte aligned, qact_planes of q).  INT2 and SIGN1
 * read planes and may get q = NULL; the other formats read q and may get
 * planes = NULL.
 * Output y [B][rows] fp32 (device), overwritten.  1 <= B <= 64
 * (QERR_INVALID_ARG otherwise).  Up to 6 tokens each lane decodes one row and
 * takes 4-way int8 dot products per token; from 7 tokens the decoded 32-weight
 * blocks go, as int8 operands, to the int8 matrix cores in groups of 16 tokens
 * (large batches on INT8 MMA, [P1] "把非标准格式塞进 llama.cpp，难在哪"), each
 * block's integer dot scaled in fp32 as above.  Both read the weights once per
 * call whatever B is.
 * Accuracy: I exact; |y - y_exact| <= 1e-4 * sum|T| (fp32 accumulation). */
int qgemv(const qweight_t* w, const int8_t* q, const uint32_t* planes, const float* d,
          const int32_t* qsum, int32_t B, float* y, void* stream);

/* Test hook: the exact integer block dots I [rows][cols/32] int32 (device) of
 * the GEMV above for a single token (B = 1), written by the same decode
 * (q and planes as for qgemv). */
int qgemv_blockdots(const qweight_t* w, const int8_t* q, const uint32_t* planes,
                    const int32_t* qsum, int32_t* out, void* stream);

/* ---- grouped GEMV: many matrices in one persistent launch --------------------------
 * Fusing many small single-token kernels was part of the 3x decode gain of the
 * pages' 1-bit kernel ([P5] §二).  Use: build a plan on the host, copy the
 * plan bytes to device memory, then run it as often as wanted.  The plan
 * stores the device pointers of every item (codes, scales, seeds, q, planes,
 * d, qsum, y): the caller keeps all of them allocated, at the same addresses,
 * for as long as it may run the plan; running a plan whose buffers were freed
 * reads and writes freed memory. */
typedef struct qgemv_item {
  qweight_t w;
  const int8_t* q;          /* [B][w.cols] (device); may be NULL for INT2, SIGN1 */
  const uint32_t* planes;   /* [B][w.cols/32][8] (device); may be NULL except for INT2, SIGN1 */
  const float* d;           /* [B][w.cols/32] (device) */
  const int32_t* qsum;  /* [B][w.cols/32] (device) */
  float* y;             /* [B][w.rows] (device), must not overlap another item's y */
} qgemv_item_t;

/* Bytes of the plan for these items (host); <0 on invalid items.  Every item
 * has B tokens, 1 <= B <= 64, and runs on the same kernels as qgemv would run
 * it at that B. */
int64_t qgemv_grouped_plan_bytes(const qgemv_item_t* items, int32_t n, int32_t B);
/* Validate the items and write the plan to host_plan [plan_bytes] (host).
 * The work is cut into 64-row tiles; inside each format they are dealt,
 * longest first, to 256 lists of nearly equal bytes (one per CU of the
 * part). */
int qgemv_grouped_plan(const qgemv_item_t* items, int32_t n, int32_t B,
                       void* host_plan, int64_t plan_bytes);
/* Run a plan: host_plan (host) is the plan as written by qgemv_grouped_plan,
 * dev_plan (device, 16-byte aligned) a byte copy of it.  The launch needs no
 * scratch memory: one workgroup per CU works through its lists, its waves
 * taking the tiles in list order through a counter in LDS.  Each tile is
 * computed whole by one wave, so results do not depend on which wave takes
 * it: runs are deterministic (bit-identical) and independent of one another.
 * QERR_BUFFER if host_plan is not a plan (of this library's version). */
int qgemv_grouped_run(const void* host_plan, const void* dev_plan, void* stream);

/* Run a plan from the library's own static plan storage, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same results as qgemv_grouped_run
 * with a device copy of the plan, bit for bit: the call copies host_plan (a
 * plan written by qgemv_grouped_plan) into a fixed device array of
 * QGEMV_STATIC_PLAN_BYTES bytes with hipMemcpyAsync on `stream`, then launches.
 * It calls no hipMalloc, hipFree or other allocating routine.  host_plan is
 * read by the stream at this call: keep it unchanged until the stream has
 * passed the call.  Each GPU holds one such array for the life of the process,
 * shared by every call on that GPU and holding the last call's plan; calls
 * that overlap on one GPU (other streams or threads) race on it and must be
 * ordered by the caller.  QERR_TOO_LARGE (before any HIP call) for a plan of
 * more than QGEMV_STATIC_PLAN_BYTES bytes (qgemv_grouped_plan_bytes gives the
 * size; the 448-matrix 64-layer 27B-shaped stack needs about 0.45 MiB). */
#define QGEMV_STATIC_PLAN_BYTES (1 << 20)
int qgemv_grouped_run_static(const void* host_plan, void* stream);

/* ---- trellis encoder ----------------------------------------------------------------- */

/* Encode fp32 weights into TRELLIS2: per row, the symbol path through the
 * 2^16-state bit-shift trellis whose decoded values are closest to the row in
 * squared error, found by the Viterbi algorithm (the format codes each row
 * jointly over a trellis, [P2] "12 GB 装下 27B，靠的是什么取舍", after QTIP;
 * its codebook is hashed at run time, [P1] "2.4bit 是个什么量级").
 *   Scales: s [rows][cols/64] fp16 = scales_in when it is not NULL (device,
 *   row-major), else fp16(sqrt(acc / 64)) with acc = fma(w_k, w_k, acc) over
 *   the block's 64 weights in order (fp32, round to nearest even).  Blocks
 *   whose root mean square exceeds the fp16 range get an infinite scale.
 *   Path: states st_i = ((st_{i-1} << 2) | c_i) & 0xFFFF, any first state;
 *   fp32 recursion d = fma(-s, V16[hash(st)], w_i) (s * V16 is exact),
 *   C_i[st] = fma(d, d, min over the 4 predecessors of C_{i-1}), C_{-1} = 0;
 *   on equal costs the predecessor with the smaller top 2 bits, and the
 *   smallest last state.  seed = st_0 >> 2 (top 2 bits 0).
 * Inputs: w [rows][cols] fp32 (device, finite), cols a multiple of 64, at most
 * 2^20.  Outputs (device): codes [rows][row_bytes] (16-byte aligned, padding
 * zeroed), seeds [rows], scales (tiled, qfmt_scales_bytes(QFMT_TRELLIS2, rows,
 * cols) bytes, 16-byte aligned), and cost [rows] fp32 = the recursion's
 * minimum (the row's squared reconstruction error; may be NULL).  Bit-exact:
 * the same fp32 operations in the same order, so the codes are unique.
 * Rows are encoded rows_per_pass at a time (one compute unit each); the
 * caller's workspace (device, 256-byte aligned) holds the scales and each
 * pass's choices, 4 KB per row and weight:
 * qtrellis_encode_workspace_bytes gives its size (QERR_BUFFER if smaller). */
int64_t qtrellis_encode_workspace_bytes(int32_t rows, int32_t cols, int32_t rows_per_pass);
int qtrellis_encode(const float* w, int32_t rows, int32_t cols, const uint16_t* scales_in, void* codes,
                    int64_t row_bytes, uint16_t* seeds, uint16_t* scales, float* cost, int32_t rows_per_pass,
                    void* workspace, int64_t workspace_bytes, void* stream);

/* ---- KV cache and decode attention ------------------------------------------------------- */

/* KV cache formats: the cache grows with the context, and holding it in 4 or
 * 8 bits decides how long a context fits ([P1] "12G 的账本要这么算").  Rows of
 * D = QATTN_HEAD_DIM values (one token of one KV head) in 32-value blocks
 * with an fp16 scale each:
 *   QKV_Q8: d = amax / 127, codes c = clamp(rint(x * id), -127, 127) int8;
 *   QKV_Q4: d = amax / 7,   codes c = clamp(rint(x * id), -7, 7) stored as the
 *           nibble c + 8 (byte j of a block: value 2j low, value 2j + 1 high);
 * fp32 with r = 1 / d, id = r if finite else 0, ties to even; the stored scale
 * is fp16(d) (round to nearest even) and the cached value c * fp16(d). */
#define QKV_Q4 4
#define QKV_Q8 8
#define QATTN_HEAD_DIM 256

/* Bytes of one cached row of QATTN_HEAD_DIM values: 256 (Q8) or 128 (Q4);
 * <0 for an unknown format. */
int64_t qkv_row_bytes(int32_t fmt);
/* Quantize rows x [rows][QATTN_HEAD_DIM] fp32 (device, 16-byte aligned, finite)
 * into codes [rows][qkv_row_bytes] (16-byte aligned) and fp16 scales
 * [rows][QATTN_HEAD_DIM / 32] (device).  Bit-exact to the rule above. */
int qkv_quant(int32_t fmt, const float* x, int64_t rows, void* codes, uint16_t* scales, void* stream);

/* Decode attention of one new token over a cached context, with the query
 * heads grouped per KV head (grouped-query attention, 6 query heads per KV
 * head in the pages' model, [P1] "把非标准格式塞进 llama.cpp，难在哪"):
 * query row i = h * group + g attends over tokens 0 .. T-1 of KV head h,
 *   s_t = (q_i . k_t) / sqrt(QATTN_HEAD_DIM),  p_t = exp(s_t - max s),
 *   out_i = sum_t p_t v_t / sum_t p_t,
 * k_t, v_t the cached values, fp32 arithmetic.  heads_per_block query rows of
 * a KV head share each read of the cache: group (the pages' packing of the six
 * heads into one block) or 1 (each row reads the cache on its own, for
 * comparison).  Inputs (device): q [n_kv * group][QATTN_HEAD_DIM] fp32;
 * kcodes, vcodes [n_kv][t_cap][qkv_row_bytes] (16-byte aligned); kscales,
 * vscales [n_kv][t_cap][QATTN_HEAD_DIM / 32] fp16 (16-byte aligned: each
 * token's scales are read as one 16-byte row).  Output out
 * [n_kv * group][QATTN_HEAD_DIM] fp32.  1 <= group <= 8, 1 <= T <= t_cap.
 * Workspace (device, 16-byte aligned) of qattn_decode_workspace_bytes: the
 * per-chunk partial sums (256 tokens a chunk).  Accuracy: each output within
 * the fp32 error allowance of the same sums in any order (score dot products,
 * exponentials, sums over tokens); deterministic. */
int64_t qattn_decode_workspace_bytes(int32_t n_kv, int32_t group, int32_t T);
int qattn_decode(int32_t fmt, const float* q, int32_t n_kv, int32_t group, int32_t heads_per_block, int32_t T,
                 int64_t t_cap, const void* kcodes, const uint16_t* kscales, const void* vcodes,
                 const uint16_t* vscales, float* out, void* workspace, int64_t workspace_bytes, void* stream);

/* ---- prefill: trellis decode to int8 and the int8 MFMA GEMM --------------------------- */

/* Decode TRELLIS2 weights to int8 for the GEMM.  The codebook is computed at
 * run time from the hash ([P1] "2.4bit 是个什么量级": trellis codes of 2 to 3
 * bits per weight, codebook hashed on the fly), and the pages' prefill runs as
 * an INT8 GEMM ([P1] "把非标准格式塞进 llama.cpp，难在哪"), so the exact fp32
 * values s * V16[h] of each row (both fp16, so the product is exact) are
 * re-quantized by Q8 per (row, oblock) as in qact_quant_i8.  Output wq
 * [rows][cols] int8, dw [rows][cols/oblock] fp32 (device).  oblock 256, 32,
 * or cols (one scale per row, cols <= 32768, else QERR_SHAPE); cols a
 * multiple of 256. */
int qtrellis_decode_i8(const qweight_t* w, int32_t oblock, int8_t* wq, float* dw, void* stream);

/* Unpack TERN_B3 / INT2 / SIGN1 / INT4 weights to int8 levels for the GEMM:
 * wq [rows][cols] = the format's integer level, dw [rows][cols/32] = the
 * fp32 factor f * s of each 32-block (so W = dw * wq exactly). */
int qweight_unpack_i8(const qweight_t* w, int8_t* wq, float* dw, void* stream);

/* Block-scaled int8 GEMM on the matrix cores (the pages' prefill is an INT8 GEMM
 * and large batches run on INT8 tensor-core MMA, [P1] "把非标准格式塞进
 * llama.cpp，难在哪"):
 *   y[m][n] = sum_kb dx[m][kb] * dw[n][kb] * I[m][n][kb],
 *   I = exact int32 dot of xq[m] and wq[n] over K-block kb (size kblock).
 * xq [M][K] int8, dx [M][K/kblock], wq [N][K] int8, dw [N][K/kblock],
 * y [M][N] fp32 (all device; xq, wq 16-byte aligned).  kblock 256, 32, or K:
 * one scale per row of each operand (dx [M][1], dw [N][1]: per-token
 * activations and per-output-row weights, the scaling an INT8 GEMM library
 * applies to its int32 result), y = dx[m] dw[n] I with I over the whole row.
 * K a multiple of kblock and of 64; QERR_INVALID_ARG for any other kblock. */
int qgemm_i8(const int8_t* xq, const float* dx, int32_t M, const int8_t* wq, const float* dw,
             int32_t N, int32_t K, int32_t kblock, float* y, void* stream);

/* Calibration for the GEMM's roofline (not part of the method): measures the
 * dense int8 matrix-core rate this device sustains, running only
 * v_mfma_i32_32x32x32_i8 (the GEMM's instruction) over four independent
 * accumulators, iters x 16 instructions per wave, blocks x 4 waves (launch
 * 2 blocks per compute unit for two waves per SIMD).  Each block's first
 * thread writes clocks[4 b .. 4 b + 3] = shader-cycle counter at start and end,
 * constant-rate reference counter at start and end (device, 8-byte aligned,
 * 4 x blocks entries, caller-owned; the reference rate is the device's wall
 * clock rate).  sink (device int32) is written only in a case that does not
 * occur, to keep the work live.  Time the call with events on the stream: the
 * rate is blocks x 4 x iters x 16 x 65536 ops over the elapsed time. */
int qcalib_mfma_i8(int32_t blocks, int32_t iters, uint64_t* clocks, int32_t* sink, void* stream);

/* Calibration for the GEMV's roofline (not part of the method): one streaming
 * read of buf [bytes] (device, 16-byte aligned, bytes a multiple of 16), every
 * byte read once with non-temporal 16-byte loads, four workgroups per compute
 * unit each reading one contiguous span, nothing written except sink (device
 * uint32), which is written
 * only in a case that practically never occurs, to keep the loads live.  Time
 * the call with events on the stream: bytes over the elapsed time is the
 * streaming-read rate this device sustains, the ceiling of a bandwidth-bound
 * decode GEMV ([P3] §1.2: bandwidth is the main bottleneck). */
int qcalib_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* QGEMV_H */
