// gemv_mfma_inst.hip — instantiates the matrix-core GEMV for one token-group
// count.  Built once per TG = 1..4 with -DQGEMV_TG=TG (batches 16 TG - 15 .. 16 TG).
#include "gemv_mfma.hpp"

#ifndef QGEMV_TG
#error "QGEMV_TG must be defined"
#endif

#define QK_CAT2(a, b) a##b
#define QK_CAT(a, b) QK_CAT2(a, b)

namespace qk {

namespace {
template <int TG, int ONLY>
hipError_t launch_grouped_mfma_variant(const PlanHeader& h, const void* plan, const V8Table& v8, float gain,
                                       hipStream_t s) {
  const int t0 = h.fmt_begin[ONLY], t1 = h.fmt_begin[ONLY + 1];
  if (t1 <= t0) return hipSuccess;
  constexpr int threads = 64 * mfma_wpg(TG, ONLY);
  const int grid = resident_workgroups((const void*)k_gemv_grouped_mfma<TG, ONLY>, threads);
  if (grid <= 0) return hipErrorInvalidDevice;
  hipLaunchKernelGGL((k_gemv_grouped_mfma<TG, ONLY>), dim3(grid), dim3(threads), 0, s, (const uint8_t*)plan, v8, gain);
  return hipGetLastError();
}
}  // namespace

hipError_t QK_CAT(launch_gemv_mfma_tg, QGEMV_TG)(const GemvItem& it, int B, hipStream_t s) {
  constexpr int TG = QGEMV_TG;
  V16Table v16;
  V8Table v8;
  float gain = 0.0f;
  if (it.fmt == QFMT_TRELLIS2) trellis_tables(&v16, &v8, &gain);
  const dim3 grid((it.rows + 63) / 64), block(256);
  switch (it.fmt) {
    case QFMT_SIGN1: hipLaunchKernelGGL((k_gemv_mfma<QFMT_SIGN1, TG>), grid, block, 0, s, it, B, v8, gain); break;
    case QFMT_INT2: hipLaunchKernelGGL((k_gemv_mfma<QFMT_INT2, TG>), grid, block, 0, s, it, B, v8, gain); break;
    case QFMT_INT4: hipLaunchKernelGGL((k_gemv_mfma<QFMT_INT4, TG>), grid, block, 0, s, it, B, v8, gain); break;
    case QFMT_TERN_B3: hipLaunchKernelGGL((k_gemv_mfma<QFMT_TERN_B3, TG>), grid, block, 0, s, it, B, v8, gain); break;
    case QFMT_TRELLIS2: hipLaunchKernelGGL((k_gemv_mfma<QFMT_TRELLIS2, TG>), grid, block, 0, s, it, B, v8, gain); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t QK_CAT(launch_grouped_mfma_tg, QGEMV_TG)(const PlanHeader& h, const void* plan, hipStream_t s) {
  constexpr int TG = QGEMV_TG;
  V16Table v16;
  V8Table v8;
  float gain = 0.0f;
  if (h.fmt_mask & (1 << QFMT_TRELLIS2)) trellis_tables(&v16, &v8, &gain);
  hipError_t e = hipSuccess;
  if (e == hipSuccess) e = launch_grouped_mfma_variant<TG, QFMT_TERN_B3>(h, plan, v8, gain, s);
  if (e == hipSuccess) e = launch_grouped_mfma_variant<TG, QFMT_INT2>(h, plan, v8, gain, s);
  if (e == hipSuccess) e = launch_grouped_mfma_variant<TG, QFMT_SIGN1>(h, plan, v8, gain, s);
  if (e == hipSuccess) e = launch_grouped_mfma_variant<TG, QFMT_INT4>(h, plan, v8, gain, s);
  if (e == hipSuccess) e = launch_grouped_mfma_variant<TG, QFMT_TRELLIS2>(h, plan, v8, gain, s);
  return e;
}

}  // namespace qk
