// gemv_inst.hip — instantiates the GEMV kernels for one batch size.  Built once
// per batch size B = 1..6 with -DQGEMV_NB=B (separate objects, parallel build).
#include "gemv_impl.hpp"

#ifndef QGEMV_NB
#error "QGEMV_NB must be defined"
#endif

#define QK_CAT2(a, b) a##b
#define QK_CAT(a, b) QK_CAT2(a, b)

namespace qk {

namespace {
template <int NB, int ONLY>
hipError_t launch_grouped_variant(const PlanHeader& h, const void* plan, const V8Table& v8, float gain,
                                  hipStream_t s) {
  const int t0 = h.fmt_begin[ONLY], t1 = h.fmt_begin[ONLY + 1];
  if (t1 <= t0) return hipSuccess;
  constexpr int threads = 64 * grouped_wpg(NB, ONLY);
  // every CU filled to the kernel's occupancy (one workgroup per CU at the sizes chosen)
  const int grid = resident_workgroups((const void*)k_gemv_grouped<NB, ONLY>, threads);
  if (grid <= 0) return hipErrorInvalidDevice;
  hipLaunchKernelGGL((k_gemv_grouped<NB, ONLY>), dim3(grid), dim3(threads), 0, s, (const uint8_t*)plan, v8, gain);
  return hipGetLastError();
}
}  // namespace

hipError_t QK_CAT(launch_gemv_b, QGEMV_NB)(const GemvItem& it, hipStream_t s) {
  constexpr int NB = QGEMV_NB;
  V16Table v16;
  V8Table v8;
  float gain = 0.0f;
  if (it.fmt == QFMT_TRELLIS2) trellis_tables(&v16, &v8, &gain);
  const dim3 grid((it.rows + 63) / 64), block(256);
  switch (it.fmt) {
    case QFMT_SIGN1: hipLaunchKernelGGL((k_gemv<QFMT_SIGN1, NB, false>), grid, block, 0, s, it, v8, gain, nullptr); break;
    case QFMT_INT2: hipLaunchKernelGGL((k_gemv<QFMT_INT2, NB, false>), grid, block, 0, s, it, v8, gain, nullptr); break;
    case QFMT_INT4: hipLaunchKernelGGL((k_gemv<QFMT_INT4, NB, false>), grid, block, 0, s, it, v8, gain, nullptr); break;
    case QFMT_TERN_B3: hipLaunchKernelGGL((k_gemv<QFMT_TERN_B3, NB, false>), grid, block, 0, s, it, v8, gain, nullptr); break;
    case QFMT_TRELLIS2: hipLaunchKernelGGL((k_gemv<QFMT_TRELLIS2, NB, false>), grid, block, 0, s, it, v8, gain, nullptr); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t QK_CAT(launch_grouped_b, QGEMV_NB)(const PlanHeader& h, const void* plan, hipStream_t s) {
  constexpr int NB = QGEMV_NB;
  V16Table v16;
  V8Table v8;
  float gain = 0.0f;
  if (h.fmt_mask & (1 << QFMT_TRELLIS2)) trellis_tables(&v16, &v8, &gain);
  // one launch per format present, in stream order
  hipError_t e = hipSuccess;
  // ternary at one token: the matrix-core kernel of gemv_tern1.hip
  if (e == hipSuccess)
    e = NB == 1 ? launch_grouped_tern1(h, plan, s) : launch_grouped_variant<NB, QFMT_TERN_B3>(h, plan, v8, gain, s);
  if (e == hipSuccess) e = launch_grouped_variant<NB, QFMT_INT2>(h, plan, v8, gain, s);
  if (e == hipSuccess) e = launch_grouped_variant<NB, QFMT_SIGN1>(h, plan, v8, gain, s);
  if (e == hipSuccess) e = launch_grouped_variant<NB, QFMT_INT4>(h, plan, v8, gain, s);
  if (e == hipSuccess) e = launch_grouped_variant<NB, QFMT_TRELLIS2>(h, plan, v8, gain, s);
  return e;
}

#if QGEMV_NB == 1
hipError_t launch_blockdots(const GemvItem& it, int32_t* out, hipStream_t s) {
  V16Table v16;
  V8Table v8;
  float gain = 0.0f;
  if (it.fmt == QFMT_TRELLIS2) trellis_tables(&v16, &v8, &gain);
  const dim3 grid((it.rows + 63) / 64), block(256);
  switch (it.fmt) {
    case QFMT_SIGN1: hipLaunchKernelGGL((k_gemv<QFMT_SIGN1, 1, true>), grid, block, 0, s, it, v8, gain, out); break;
    case QFMT_INT2: hipLaunchKernelGGL((k_gemv<QFMT_INT2, 1, true>), grid, block, 0, s, it, v8, gain, out); break;
    case QFMT_INT4: hipLaunchKernelGGL((k_gemv<QFMT_INT4, 1, true>), grid, block, 0, s, it, v8, gain, out); break;
    case QFMT_TERN_B3: hipLaunchKernelGGL((k_gemv<QFMT_TERN_B3, 1, true>), grid, block, 0, s, it, v8, gain, out); break;
    case QFMT_TRELLIS2: hipLaunchKernelGGL((k_gemv<QFMT_TRELLIS2, 1, true>), grid, block, 0, s, it, v8, gain, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
#endif

}  // namespace qk
