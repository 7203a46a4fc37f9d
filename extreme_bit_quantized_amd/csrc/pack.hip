// pack.hip — weight preparation on the GPU: quantize fp32 weights and pack
// them, pack integer codes, and unpack packed weights to int8 levels.
//
// The quantizers take their decisions in fp64 with sums in index order, one
// thread per scale block, so that the codes do not depend on launch shape.
#include <hip/hip_fp16.h>

#include "internal.hpp"

#pragma clang fp contract(off)

namespace qk {

__device__ __forceinline__ double f16_bits_to_f64(uint16_t h) {
  return (double)__half2float(__ushort_as_half(h));
}

// Ternary byte of five digits d0..d4 (digit 0 most significant): the base-3
// number b stored as ceil(256 b / 243).
__device__ __forceinline__ uint32_t tern_byte(const int (&t)[5]) {
  uint32_t b = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) b = b * 3 + (uint32_t)(t[i] + 1);
  return (b * 256 + 242) / 243;
}

// Writes one 256-weight ternary block (13 words) from trits tr[256].
template <typename Get>
__device__ __forceinline__ void write_tern_block(Get tr, uint32_t* out) {
  for (int m = 0; m < 13; ++m) {
    uint32_t word = 0;
    for (int p = 0; p < 4; ++p) {
      int t[5];
      for (int i = 0; i < 5; ++i) t[i] = m < 12 ? tr(20 * m + 4 * i + p) : (i < 4 ? tr(240 + 4 * i + p) : 0);
      word |= tern_byte(t) << (8 * p);
    }
    out[m] = word;
  }
}

// Bit offset of code k inside its 32-bit word: 1- and 2-bit codes nibble-lane
// (code 8j + n in nibble n at offset j * bits), 4-bit codes byte-lane (code
// 4j + b in byte b at offset 4j).
__device__ __forceinline__ int plane_bitpos(int k, int bits) {
  return bits == 4 ? 8 * (k & 3) + 4 * (k >> 2) : 4 * (k & 7) + (k >> 3) * bits;
}
// Plane word of `per_word` codes with `bits` bits: code k at plane_bitpos(k, bits).
template <typename Get>
__device__ __forceinline__ uint32_t plane_word(Get c, int bits) {
  const int per_word = 32 / bits;
  uint32_t w = 0;
  for (int k = 0; k < per_word; ++k) w |= ((uint32_t)c(k) & ((1u << bits) - 1)) << plane_bitpos(k, bits);
  return w;
}

// One thread per scale block.
__global__ __launch_bounds__(256) void k_quantize(int fmt, const float* __restrict__ w, int rows, int cols,
                                                  uint8_t* __restrict__ codes, int64_t row_bytes,
                                                  uint16_t* __restrict__ scales) {
  const int blk = scale_block(fmt);
  const int nb = cols / blk;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (int64_t)rows * nb) return;
  const int64_t row = id / nb;
  const int kb = (int)(id % nb);
  const float* wb = w + row * cols + (int64_t)kb * blk;
  uint8_t* rowp = codes + row * row_bytes;
  if (fmt == QFMT_SIGN1) {
    double sum = 0.0;
    for (int i = 0; i < 128; ++i) sum += fabs((double)wb[i]);
    uint32_t* out = (uint32_t*)(rowp + (int64_t)kb * 16);
    for (int wd = 0; wd < 4; ++wd) out[wd] = plane_word([&](int k) { return wb[32 * wd + k] >= 0.0f ? 1 : 0; }, 1);
    scales[scale_index(fmt, cols, row, kb)] = f64_to_f16_bits(sum / 128.0);
  } else if (fmt == QFMT_TERN_B3) {
    double sum = 0.0;
    for (int i = 0; i < 256; ++i) sum += fabs((double)wb[i]);
    const double sc = sum / 256.0 + 1e-8;
    auto tr = [&](int k) {
      double r = rint((double)wb[k] / sc);
      return (int)fmin(fmax(r, -1.0), 1.0);
    };
    write_tern_block(tr, (uint32_t*)(rowp + (int64_t)kb * 52));
    scales[scale_index(fmt, cols, row, kb)] = f64_to_f16_bits(sc);
  } else {  // INT2 / INT4: nearest of L half-integer levels, ties up
    const int L = fmt == QFMT_INT2 ? 4 : 16;
    const int bits = fmt == QFMT_INT2 ? 2 : 4;
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs((double)wb[i]));
    const uint16_t sh = f64_to_f16_bits(amax / ((L - 1) * 0.5));
    const double sc = f16_bits_to_f64(sh);
    auto code = [&](int k) {
      if (sc == 0.0) return L / 2;
      double f = floor((double)wb[k] / sc) + (double)(L / 2);
      return (int)fmin(fmax(f, 0.0), (double)(L - 1));
    };
    const int per_word = 32 / bits;
    uint32_t* out = (uint32_t*)(rowp + (int64_t)kb * (32 * bits / 8));
    for (int wd = 0; wd < 32 / per_word; ++wd) out[wd] = plane_word([&](int k) { return code(wd * per_word + k); }, bits);
    scales[scale_index(fmt, cols, row, kb)] = sh;
  }
}

// Tiled scale storage from row-major scales [rows][cols/block]: one thread per
// slot of the tiled array; slots past the last row or block get zero.  With
// rowmajor == nullptr only those padding slots are written.
__global__ __launch_bounds__(256) void k_scales_from_rows(int fmt, int rows, int cols,
                                                          const uint16_t* __restrict__ rowmajor,
                                                          uint16_t* __restrict__ scales) {
  const int64_t G = scale_group(fmt), ng = scale_groups(fmt, cols), nsb = cols / scale_block(fmt);
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= scales_elems(fmt, rows, cols)) return;
  const int64_t j = id % G, rr = (id / G) % 64, g = (id / (G * 64)) % ng, rt = id / (G * 64 * ng);
  const int64_t r = rt * 64 + rr, b = g * G + j;
  const bool real = r < rows && b < nsb;
  if (real && rowmajor) scales[id] = rowmajor[r * nsb + b];
  else if (!real) scales[id] = 0;
}

// Row-major scales [rows][cols/block] from the tiled storage.
__global__ __launch_bounds__(256) void k_scales_to_rows(int fmt, int rows, int cols,
                                                        const uint16_t* __restrict__ scales,
                                                        uint16_t* __restrict__ rowmajor) {
  const int64_t nsb = cols / scale_block(fmt);
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= rows * nsb) return;
  rowmajor[id] = scales[scale_index(fmt, cols, id / nsb, id % nsb)];
}

hipError_t launch_scales_from_rows(int fmt, int rows, int cols, const uint16_t* rowmajor, uint16_t* scales,
                                  hipStream_t s) {
  const int64_t n = scales_elems(fmt, rows, cols);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_scales_from_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, fmt, rows, cols,
                     rowmajor, scales);
  return hipGetLastError();
}

hipError_t launch_scales_to_rows(int fmt, int rows, int cols, const uint16_t* scales, uint16_t* rowmajor,
                                hipStream_t s) {
  const int64_t n = (int64_t)rows * (cols / scale_block(fmt));
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_scales_to_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, fmt, rows, cols,
                     scales, rowmajor);
  return hipGetLastError();
}

// Zero the row padding (bytes past the packed row inside the stride).
__global__ __launch_bounds__(256) void k_zero_pad(uint8_t* codes, int rows, int64_t packed, int64_t row_bytes) {
  const int64_t pad = row_bytes - packed;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (int64_t)rows * pad) return;
  codes[(id / pad) * row_bytes + packed + id % pad] = 0;
}

hipError_t zero_padding(uint8_t* codes, int rows, int cols, int fmt, int64_t row_bytes, hipStream_t s) {
  const int64_t packed = packed_row_bytes(fmt, cols);
  const int64_t n = (int64_t)rows * (row_bytes - packed);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_pad, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, codes, rows, packed, row_bytes);
  return hipGetLastError();
}

hipError_t launch_quantize(int fmt, const float* w, int rows, int cols, uint8_t* codes, int64_t row_bytes,
                           uint16_t* scales, hipStream_t s) {
  const int64_t n = (int64_t)rows * (cols / scale_block(fmt));
  hipLaunchKernelGGL(k_quantize, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, fmt, w, rows, cols, codes,
                     row_bytes, scales);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_scales_from_rows(fmt, rows, cols, nullptr, scales, s);  // zero the scale padding
  if (e != hipSuccess) return e;
  return zero_padding(codes, rows, cols, fmt, row_bytes, s);
}

// Pack integer codes: one thread per 32-bit output word (ternary: per block).
__global__ __launch_bounds__(256) void k_pack(int fmt, const int8_t* __restrict__ lv, int rows, int cols,
                                              uint8_t* __restrict__ codes, int64_t row_bytes) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row_units = fmt == QFMT_TERN_B3 ? cols / 256 : fmt == QFMT_TRELLIS2 ? cols / 16
                          : cols / (32 / (fmt == QFMT_INT2 ? 2 : fmt == QFMT_SIGN1 ? 1 : 4));
  if (id >= rows * row_units) return;
  const int64_t row = id / row_units;
  const int64_t u = id % row_units;
  const int8_t* r = lv + row * cols;
  uint8_t* rowp = codes + row * row_bytes;
  if (fmt == QFMT_TERN_B3) {
    const int8_t* b = r + u * 256;
    write_tern_block([&](int k) { return (int)b[k]; }, (uint32_t*)(rowp + u * 52));
  } else if (fmt == QFMT_TRELLIS2) {
    // 16 symbols -> 4 bytes, first symbol in the top bits of each byte
    const int8_t* c = r + u * 16;
    uint32_t w = 0;
    for (int g = 0; g < 4; ++g) {
      const uint32_t by = ((c[4 * g] & 3u) << 6) | ((c[4 * g + 1] & 3u) << 4) | ((c[4 * g + 2] & 3u) << 2) |
                          (c[4 * g + 3] & 3u);
      w |= by << (8 * g);
    }
    *(uint32_t*)(rowp + u * 4) = w;
  } else {
    const int bits = fmt == QFMT_INT2 ? 2 : fmt == QFMT_SIGN1 ? 1 : 4;
    const int per_word = 32 / bits;
    const int8_t* c = r + u * per_word;
    *(uint32_t*)(rowp + u * 4) = plane_word([&](int k) { return (int)c[k]; }, bits);
  }
}

hipError_t launch_pack(int fmt, const int8_t* levels, int rows, int cols, uint8_t* codes, int64_t row_bytes,
                       hipStream_t s) {
  const int64_t units = fmt == QFMT_TERN_B3 ? cols / 256 : fmt == QFMT_TRELLIS2 ? cols / 16
                      : cols / (32 / (fmt == QFMT_INT2 ? 2 : fmt == QFMT_SIGN1 ? 1 : 4));
  const int64_t n = (int64_t)rows * units;
  hipLaunchKernelGGL(k_pack, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, fmt, levels, rows, cols, codes,
                     row_bytes);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return zero_padding(codes, rows, cols, fmt, row_bytes, s);
}

// Unpack to int8 levels and per-32 fp32 factors: one thread per 32-block.
__global__ __launch_bounds__(256) void k_unpack_i8(GemvItem it, int8_t* __restrict__ wq, float* __restrict__ dw) {
  const int nkb = it.cols / 32;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (int64_t)it.rows * nkb) return;
  const int64_t row = id / nkb;
  const int kb = (int)(id % nkb);
  const uint8_t* rowp = it.codes + row * it.row_bytes;
  int8_t* out = wq + row * it.cols + (int64_t)kb * 32;
  const uint16_t sh = it.scales[scale_index(it.fmt, it.cols, row, (kb * 32) / scale_block(it.fmt))];
  const float s = __half2float(__ushort_as_half(sh));
  if (it.fmt == QFMT_TERN_B3) {
    // block of 256 = 13 words; act block kb covers words of 20 weights
    const int blk = kb / 8;
    const uint8_t* bb = rowp + (int64_t)blk * 52;
    for (int k = 0; k < 32; ++k) {
      const int kk = (kb % 8) * 32 + k;  // weight within the 256-block
      int word, p, dig;
      if (kk < 240) {
        word = kk / 20;
        p = kk % 4;
        dig = (kk % 20) / 4;
      } else {
        word = 12;
        p = kk % 4;
        dig = (kk - 240) / 4;
      }
      uint32_t r = bb[4 * word + p];
      uint32_t dgt = 0;
      for (int i = 0; i <= dig; ++i) {
        r *= 3;
        dgt = r >> 8;
        r &= 0xFF;
      }
      out[k] = (int8_t)((int)dgt - 1);
    }
    dw[id] = s;
  } else {
    const int bits = it.fmt == QFMT_INT2 ? 2 : it.fmt == QFMT_SIGN1 ? 1 : 4;
    const int per_word = 32 / bits;
    const uint32_t* words = (const uint32_t*)(rowp + (int64_t)kb * 32 * bits / 8);
    for (int k = 0; k < 32; ++k) {
      const uint32_t wv = words[k / per_word];
      const int kk = k % per_word;
      const int c = (int)((wv >> plane_bitpos(kk, bits)) & ((1u << bits) - 1));
      out[k] = (int8_t)(it.fmt == QFMT_INT2 ? 2 * c - 3 : it.fmt == QFMT_SIGN1 ? 2 * c - 1 : 2 * c - 15);
    }
    dw[id] = (it.fmt == QFMT_SIGN1) ? s : 0.5f * s;
  }
}

hipError_t launch_unpack_i8(const GemvItem& it, int8_t* wq, float* dw, hipStream_t s) {
  const int64_t n = (int64_t)it.rows * (it.cols / 32);
  hipLaunchKernelGGL(k_unpack_i8, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, it, wq, dw);
  return hipGetLastError();
}

}  // namespace qk
