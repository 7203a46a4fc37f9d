// internal.hpp — shared declarations of libqgemv's translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qgemv.h"

namespace qk {

// ---- format geometry ---------------------------------------------------------------
__host__ __device__ constexpr int32_t scale_block(int32_t fmt) {
  switch (fmt) {
    case QFMT_TERN_B3: return 256;
    case QFMT_INT2: return 32;
    case QFMT_SIGN1: return 128;
    case QFMT_INT4: return 32;
    case QFMT_TRELLIS2: return 64;
  }
  return 0;
}

// Scale storage: fp16 scales sit in tiles of 64 rows x G blocks, G =
// scale_group(fmt) (the blocks one GEMV segment spans: 1024 weights for 1-bit
// and ternary, 512 for 2-bit and trellis, 256 for 4-bit).  Tiles follow each
// other in row-major order over (row tile, block group); inside a tile the
// 64 rows' G scales are row-major.  A GEMV segment of a 64-row tile therefore
// reads one contiguous 128 G-byte run.  Slots past the last row or block are
// zero.
__host__ __device__ constexpr int32_t scale_group(int32_t fmt) {
  switch (fmt) {
    case QFMT_TERN_B3: return 4;
    case QFMT_INT2: return 16;
    case QFMT_SIGN1: return 8;
    case QFMT_INT4: return 8;
    case QFMT_TRELLIS2: return 8;
  }
  return 0;
}
__host__ __device__ inline int64_t scale_groups(int32_t fmt, int64_t cols) {
  const int64_t nsb = cols / scale_block(fmt);
  return (nsb + scale_group(fmt) - 1) / scale_group(fmt);
}
// Index of the scale of (row r, scale block b).
__host__ __device__ inline int64_t scale_index(int32_t fmt, int64_t cols, int64_t r, int64_t b) {
  const int64_t G = scale_group(fmt);
  return (((r >> 6) * scale_groups(fmt, cols) + b / G) * 64 + (r & 63)) * G + b % G;
}
__host__ __device__ inline int64_t scales_elems(int32_t fmt, int64_t rows, int64_t cols) {
  return (rows + 63) / 64 * scale_groups(fmt, cols) * 64 * scale_group(fmt);
}

// Lane exchange inside 16-lane groups: partner lane t ^ M.  M = 1, 2: DPP
// quad permutes; M = 4, 8: ds_swizzle in its bit mode (xor mask M).
template <int M>
__device__ __forceinline__ float xlane(float v) {
  const int b = __builtin_bit_cast(int, v);
  if constexpr (M == 1) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(b, 0xB1, 0xF, 0xF, false));
  else if constexpr (M == 2) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(b, 0x4E, 0xF, 0xF, false));
  else return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(b, 0x1F | (M << 10)));
}
template <int M>
__device__ __forceinline__ int xlane_i(int v) {
  return __builtin_bit_cast(int, xlane<M>(__builtin_bit_cast(float, v)));
}

// Packed bytes per row: bits per weight x cols / 8, ternary 52 bytes per 256.
__host__ __device__ inline int64_t packed_row_bytes(int32_t fmt, int64_t cols) {
  switch (fmt) {
    case QFMT_TERN_B3: return cols / 256 * 52;
    case QFMT_INT2: return cols / 4;
    case QFMT_SIGN1: return cols / 8;
    case QFMT_INT4: return cols / 2;
    case QFMT_TRELLIS2: return cols / 4;
  }
  return -1;
}

// fp64 -> IEEE fp16 bits, round to nearest even, from the double's fields.
__host__ __device__ inline uint16_t f64_to_f16_bits(double x) {
  const uint64_t bits = __builtin_bit_cast(uint64_t, x);
  const uint32_t sign = (uint32_t)(bits >> 48) & 0x8000u;
  const int ex = (int)((bits >> 52) & 0x7FF);
  const uint64_t frac = bits & 0xFFFFFFFFFFFFFull;
  if (ex == 0x7FF) return (uint16_t)(sign | 0x7C00u | (frac ? 0x200u : 0u));
  if (ex == 0) return (uint16_t)sign;  // double subnormals are far below fp16's range
  const int e = ex - 1023;
  const uint64_t m = frac | (1ull << 52);  // value = m * 2^(e - 52)
  int shift;      // low bits of m dropped
  uint32_t base;  // exponent field before rounding carries
  if (e >= -14) {
    if (e > 15) return (uint16_t)(sign | 0x7C00u);
    shift = 42;
    base = (uint32_t)(e + 14);  // biased exponent - 1; the implicit bit of n adds the 1
  } else {
    shift = 28 - e;  // subnormal quantum 2^-24
    base = 0;
    if (shift > 63) return (uint16_t)sign;
  }
  uint64_t n = m >> shift;
  const uint64_t rem = m & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (n & 1))) ++n;
  // normal: n in [1024, 2048] and base<<10 + n carries into the exponent by
  // itself; subnormal: bits = n (n = 1024 is the smallest normal).
  const uint32_t out = (base << 10) + (uint32_t)n;
  if (out >= 0x7C00u) return (uint16_t)(sign | 0x7C00u);
  return (uint16_t)(sign | out);
}

// ---- GEMV work description -------------------------------------------------------------
// One matrix of a grouped launch (or the single matrix of qgemv).  80 bytes.
struct alignas(16) GemvItem {
  const uint8_t* codes;
  const uint16_t* scales;
  const uint16_t* seeds;
  const int8_t* q;
  const float* d;
  const int32_t* qsum;
  float* y;
  int64_t row_bytes;
  int32_t fmt, rows, cols, pad;
};
static_assert(sizeof(GemvItem) == 80, "item layout");

struct alignas(8) GemvTile {
  uint32_t item;
  uint32_t row0;
};

// Plan blob: header, items, tiles, worker table (16-byte aligned sections).
// Tiles are grouped by format (format f owns tiles [fmt_begin[f],
// fmt_begin[f + 1]), f = 1..5); a run launches one kernel per format present,
// each compiled for that format alone.  Inside a format the tiles are dealt
// to n_workers lists of nearly equal total bytes (longest tile first, each to
// the list with the fewest bytes so far) and stored list by list, longest
// first inside a list: list w of format f is tiles [wb[w], wb[w + 1]) with
// wb = workers + f (n_workers + 1).  Workgroup g of a G-workgroup launch works
// through lists g, g + G, ...
struct alignas(16) PlanHeader {
  uint32_t magic;   // 'QGVP'
  uint32_t version;
  int32_t n_items;
  int32_t n_tiles;
  int32_t B;
  int32_t fmt_mask;  // bit f set if some item has format f
  int64_t items_off;
  int64_t tiles_off;
  int64_t total_bytes;
  int32_t fmt_begin[8];
  int32_t n_workers;
  int32_t pad_;
  int64_t workers_off;  // int32 [6][n_workers + 1]
};
static_assert(sizeof(PlanHeader) == 96, "plan header layout");
constexpr uint32_t kPlanVersion = 3;
// Lists per format: one per CU of a 256-CU part (one workgroup per CU).
constexpr int kPlanWorkers = 256;
constexpr uint32_t kPlanMagic = 0x50564751u;  // "QGVP"

// Codebook tables passed by value to the kernels that need them.
struct V8Table { int8_t v[256]; };
struct V16Table { uint16_t v[256]; };
// Host-side codebook (built once, thread-safe): V16, V8 and the gain V16[255]/127.
void trellis_tables(V16Table* v16, V8Table* v8, float* gain);

// Workgroups of `threads` threads of `kernel` the current device holds at once
// (compute units x resident workgroups per unit): the grid of a persistent
// launch.  Queried once per (kernel, device) and cached under a lock, so
// concurrent callers on any threads see a complete entry; 0 if a query fails
// or no workgroup fits.
int resident_workgroups(const void* kernel, int threads);

// ---- launchers (each returns a hipError_t) --------------------------------------------
hipError_t launch_act_quant(const float* x, int B, int K, int qblock, int8_t* q, float* d,
                            int32_t* qsum, hipStream_t s);
hipError_t launch_act_planes(const int8_t* q, int B, int K, uint32_t* planes, hipStream_t s);
hipError_t launch_act_quant_batch(const qact_job_t* jobs, int n, hipStream_t s);
hipError_t launch_hadamard_quant(const float* x, int B, int K, const uint32_t* sign_bits, int qblock,
                                 int8_t* q, float* d, int32_t* qsum, hipStream_t s);
hipError_t launch_quantize(int fmt, const float* w, int rows, int cols, uint8_t* codes,
                           int64_t row_bytes, uint16_t* scales, hipStream_t s);
hipError_t launch_pack(int fmt, const int8_t* levels, int rows, int cols, uint8_t* codes,
                       int64_t row_bytes, hipStream_t s);
hipError_t launch_scales_from_rows(int fmt, int rows, int cols, const uint16_t* rowmajor, uint16_t* scales,
                                  hipStream_t s);
hipError_t launch_scales_to_rows(int fmt, int rows, int cols, const uint16_t* scales, uint16_t* rowmajor,
                                hipStream_t s);
hipError_t launch_unpack_i8(const GemvItem& it, int8_t* wq, float* dw, hipStream_t s);
hipError_t launch_blockdots(const GemvItem& it, int32_t* out, hipStream_t s);
#define QK_DECL_NB(n)                                                    \
  hipError_t launch_gemv_b##n(const GemvItem& it, hipStream_t s);        \
  hipError_t launch_grouped_b##n(const PlanHeader& h, const void* plan, hipStream_t s);  /* all formats */
QK_DECL_NB(1)
QK_DECL_NB(2)
QK_DECL_NB(3)
QK_DECL_NB(4)
QK_DECL_NB(5)
QK_DECL_NB(6)
#undef QK_DECL_NB
// Matrix-core GEMV for batches of 16 TG - 15 .. 16 TG tokens (TG = 1..4).
#define QK_DECL_TG(n)                                                                  \
  hipError_t launch_gemv_mfma_tg##n(const GemvItem& it, int B, hipStream_t s);          \
  hipError_t launch_grouped_mfma_tg##n(const PlanHeader& h, const void* plan, hipStream_t s);
QK_DECL_TG(1)
QK_DECL_TG(2)
QK_DECL_TG(3)
QK_DECL_TG(4)
#undef QK_DECL_TG
// One token, the plan's ternary tiles, dot products on the matrix cores (gemv_tern1.hip).
hipError_t launch_grouped_tern1(const PlanHeader& h, const void* plan, hipStream_t s);
hipError_t launch_trellis_decode(const GemvItem& it, int oblock, int8_t* wq, float* dw, hipStream_t s);
// KV cache and decode attention (attn.hip).
int64_t attn_workspace_bytes(int n_kv, int group, int T);
hipError_t launch_kv_quant(int fmt, const float* x, int64_t rows, uint8_t* codes, uint16_t* scales, hipStream_t s);
hipError_t launch_attn_decode(int fmt, const float* q, int n_kv, int group, int heads_per_block, int T,
                              int64_t t_cap, const void* kc, const uint16_t* ks, const void* vc,
                              const uint16_t* vs, float* out, void* ws, hipStream_t s);
// Trellis encoder (encode.hip): workspace bytes and the launch sequence.
int64_t encode_workspace_bytes(int rows, int cols, int rows_per_pass);
hipError_t launch_trellis_encode(const float* w, int rows, int cols, const uint16_t* scales_in, uint8_t* codes,
                                 int64_t row_bytes, uint16_t* seeds, uint16_t* scales, float* cost,
                                 int rows_per_pass, void* ws, hipStream_t s);
hipError_t launch_mfma_peak(int blocks, int iters, uint64_t* clocks, int32_t* sink, hipStream_t s);
hipError_t launch_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_gemm(const int8_t* xq, const float* dx, int M, const int8_t* wq, const float* dw,
                       int N, int K, int kblock, float* y, hipStream_t s);
// One scale per row of each operand (gemm_rs.hip); wc = 128, 96, 80 or 64, the
// N extent of a wave's tile.
hipError_t launch_gemm_rs(const int8_t* xq, const float* dx, int M, const int8_t* wq, const float* dw,
                          int N, int K, int wc, float* y, hipStream_t s);

}  // namespace qk
