// api.hip — the C ABI of libqgemv: host-side validation, then dispatch.
// Every check runs before any HIP call, so rejected calls never touch the GPU.
#include <algorithm>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "internal.hpp"

using namespace qk;

namespace {

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
// The caller's stream for a launch.  Launch failures are read back with
// hipGetLastError right after each launch, and HIP keeps the last error of any
// earlier runtime call on the thread (the caller's own, or another library's)
// until it is read, so a stale one is cleared here first rather than reported
// as this call's failure.
inline hipStream_t S(void* s) {
  (void)hipGetLastError();
  return (hipStream_t)s;
}
// The HIP error behind the calling thread's last QERR_HIP (qhip_error_name).
thread_local hipError_t t_last_hip = hipSuccess;

inline int hip_rc(hipError_t e) {
  if (e == hipSuccess) return QERR_OK;
  t_last_hip = e;
  return QERR_HIP;
}

int check_weight(const qweight_t* w) {
  if (!w) return QERR_INVALID_ARG;
  const int32_t blk = scale_block(w->fmt);
  if (blk == 0) return QERR_UNSUPPORTED_FMT;
  if (w->rows < 0 || w->cols < 0) return QERR_INVALID_ARG;
  if (w->block != blk) return QERR_SHAPE;
  if (w->cols == 0 || w->cols % blk != 0 || w->cols % 32 != 0) return QERR_SHAPE;
  if (w->rows == 0) return QERR_OK;
  if (!w->codes || !w->scales) return QERR_INVALID_ARG;
  if (w->fmt == QFMT_TRELLIS2 && !w->seeds) return QERR_INVALID_ARG;
  const int64_t packed = packed_row_bytes(w->fmt, w->cols);
  if (w->row_bytes < packed || w->row_bytes % 16 != 0) return QERR_SHAPE;
  if (w->row_bytes >= ((int64_t)1 << 26)) return QERR_SHAPE;  // 64-row tile offsets fit 32 bits
  if (!aligned(w->codes, 16) || !aligned(w->scales, 16) || (w->seeds && !aligned(w->seeds, 2)))
    return QERR_ALIGNMENT;
  return QERR_OK;
}

// INT2 and SIGN1 read 4-bit activation planes instead of q.
inline bool uses_planes(int32_t fmt) { return fmt == QFMT_INT2 || fmt == QFMT_SIGN1; }

// it.q carries the planes (as bytes) for the formats that read them.
GemvItem make_item(const qweight_t* w, const int8_t* q, const uint32_t* planes, const float* d,
                   const int32_t* qsum, float* y) {
  GemvItem it{};
  it.codes = (const uint8_t*)w->codes;
  it.scales = w->scales;
  it.seeds = w->seeds;
  it.q = uses_planes(w->fmt) ? (const int8_t*)planes : q;
  it.d = d;
  it.qsum = qsum;
  it.y = y;
  it.row_bytes = w->row_bytes;
  it.fmt = w->fmt;
  it.rows = w->rows;
  it.cols = w->cols;
  return it;
}

int check_act(int32_t fmt, const int8_t* q, const uint32_t* planes, const float* d, const int32_t* qsum) {
  if (!d || !qsum) return QERR_INVALID_ARG;
  if (uses_planes(fmt)) {
    if (!planes) return QERR_INVALID_ARG;
    if (!aligned(planes, 32)) return QERR_ALIGNMENT;
  } else {
    if (!q) return QERR_INVALID_ARG;
    if (!aligned(q, 16)) return QERR_ALIGNMENT;
  }
  if (!aligned(d, 4) || !aligned(qsum, 4)) return QERR_ALIGNMENT;
  return QERR_OK;
}

int check_item(const qgemv_item_t& it, int32_t B) {
  int rc = check_weight(&it.w);
  if (rc) return rc;
  if (it.w.rows == 0) return QERR_OK;
  rc = check_act(it.w.fmt, it.q, it.planes, it.d, it.qsum);
  if (rc) return rc;
  if (!it.y) return QERR_INVALID_ARG;
  if (!aligned(it.y, 4)) return QERR_ALIGNMENT;
  (void)B;
  return QERR_OK;
}

using GemvLaunch = hipError_t (*)(const GemvItem&, hipStream_t);
using GroupedLaunch = hipError_t (*)(const PlanHeader&, const void*, hipStream_t);
const GemvLaunch kGemv[7] = {nullptr, launch_gemv_b1, launch_gemv_b2, launch_gemv_b3, launch_gemv_b4,
                             launch_gemv_b5, launch_gemv_b6};
const GroupedLaunch kGrouped[7] = {nullptr, launch_grouped_b1, launch_grouped_b2, launch_grouped_b3,
                                   launch_grouped_b4, launch_grouped_b5, launch_grouped_b6};
// Batches above kMaxDppBatch run on the matrix cores in groups of 16 tokens.
// Measured on 64-layer stacks: the lane-per-row dot4 kernels win up to 6 tokens
// in every format (2.16 ms against 2.34 ms for the 4-bit/ternary stack at 5
// tokens), the matrix cores from 7 (2.25 ms against 2.58 ms for the 1-bit stack
// at 8, 2.46 against 3.09 for the 2-bit one).
constexpr int kMaxDppBatch = 6;
constexpr int kMaxBatch = 64;
// Longest row the encoder takes (its choices use 4 KB per row and weight).
constexpr int32_t kMaxEncodeCols = 1 << 20;
using MfmaLaunch = hipError_t (*)(const GemvItem&, int, hipStream_t);
const MfmaLaunch kGemvMfma[5] = {nullptr, launch_gemv_mfma_tg1, launch_gemv_mfma_tg2, launch_gemv_mfma_tg3,
                                 launch_gemv_mfma_tg4};
const GroupedLaunch kGroupedMfma[5] = {nullptr, launch_grouped_mfma_tg1, launch_grouped_mfma_tg2,
                                       launch_grouped_mfma_tg3, launch_grouped_mfma_tg4};

hipError_t launch_gemv_any(const GemvItem& it, int B, hipStream_t s) {
  return B <= kMaxDppBatch ? kGemv[B](it, s) : kGemvMfma[(B + 15) / 16](it, B, s);
}
hipError_t launch_grouped_any(const PlanHeader& h, const void* plan, hipStream_t s) {
  return h.B <= kMaxDppBatch ? kGrouped[h.B](h, plan, s) : kGroupedMfma[(h.B + 15) / 16](h, plan, s);
}

int64_t align16(int64_t x) { return (x + 15) / 16 * 16; }

int64_t count_tiles(const qgemv_item_t* items, int32_t n) {
  int64_t t = 0;
  for (int32_t i = 0; i < n; ++i) t += (items[i].w.rows + 63) / 64;
  return t;
}

// Header of a plan built by qgemv_grouped_plan, or QERR_BUFFER.
int read_plan_header(const void* host_plan, PlanHeader* h) {
  std::memcpy(h, host_plan, sizeof(*h));
  if (h->magic != kPlanMagic || h->version != kPlanVersion || h->B < 1 || h->B > kMaxBatch || h->n_items < 1 ||
      h->n_tiles < 0 || h->n_workers != kPlanWorkers || h->total_bytes < (int64_t)sizeof(PlanHeader))
    return QERR_BUFFER;
  return QERR_OK;
}

// Plan storage of qgemv_grouped_run_static: a fixed device array, so that call
// allocates nothing.  In host code `scratch` names a host-side stand-in, not a
// device address; the device address comes from hipGetSymbolAddress, taken once
// per device with that device current, and only that address is used.
constexpr int64_t kStaticPlanBytes = QGEMV_STATIC_PLAN_BYTES;
__device__ __align__(256) uint8_t scratch[kStaticPlanBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (QERR_HIP if it cannot be had).
int static_plan_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QERR_OK;
}

}  // namespace

namespace qk {
int resident_workgroups(const void* kernel, int threads) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> cache;  // (kernel, device) -> workgroups
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(kernel, dev);
  const auto hit = cache.find(key);
  if (hit != cache.end()) return hit->second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) return 0;
  const int n = per_cu < 1 ? 0 : cus * per_cu;
  cache[key] = n;
  return n;
}
}  // namespace qk

extern "C" {

const char* qhip_error_name(void) { return hipGetErrorName(t_last_hip); }

const char* qstrerror(int err) {
  switch (err) {
    case QERR_OK: return "ok";
    case QERR_INVALID_ARG: return "invalid argument (null pointer, negative size or bad enum)";
    case QERR_UNSUPPORTED_FMT: return "unsupported weight format for this call";
    case QERR_SHAPE: return "shape violates the format's block rules";
    case QERR_ALIGNMENT: return "pointer or stride misaligned";
    case QERR_HIP: return "HIP launch or query failed";
    case QERR_BUFFER: return "caller buffer too small or corrupt";
    case QERR_TOO_LARGE: return "plan larger than the library's static plan storage (QGEMV_STATIC_PLAN_BYTES)";
  }
  return "unknown error";
}

int32_t qfmt_scale_block(int32_t fmt) { return scale_block(fmt); }

int64_t qfmt_packed_row_bytes(int32_t fmt, int32_t cols) {
  const int32_t blk = scale_block(fmt);
  if (blk == 0) return QERR_UNSUPPORTED_FMT;
  if (cols <= 0 || cols % blk != 0 || cols % 32 != 0) return QERR_SHAPE;
  return packed_row_bytes(fmt, cols);
}

int64_t qfmt_row_bytes(int32_t fmt, int32_t cols) {
  const int64_t b = qfmt_packed_row_bytes(fmt, cols);
  return b < 0 ? b : (b + 15) / 16 * 16;
}

int32_t qfmt_scale_group(int32_t fmt) { return scale_group(fmt); }

int64_t qfmt_scales_bytes(int32_t fmt, int32_t rows, int32_t cols) {
  const int32_t blk = scale_block(fmt);
  if (blk == 0) return QERR_UNSUPPORTED_FMT;
  if (rows < 0 || cols < 0) return QERR_INVALID_ARG;
  if (cols == 0 || cols % blk != 0 || cols % 32 != 0) return QERR_SHAPE;
  return 2 * scales_elems(fmt, rows, cols);
}

int qweight_check(const qweight_t* w) { return check_weight(w); }

int qweight_set_scales(const qweight_t* w, const uint16_t* rowmajor, void* stream) {
  const int rc = check_weight(w);
  if (rc) return rc;
  if (w->rows == 0) return QERR_OK;
  if (!rowmajor) return QERR_INVALID_ARG;
  if (!aligned(rowmajor, 2)) return QERR_ALIGNMENT;
  return hip_rc(launch_scales_from_rows(w->fmt, w->rows, w->cols, rowmajor, (uint16_t*)w->scales, S(stream)));
}

int qweight_get_scales(const qweight_t* w, uint16_t* rowmajor, void* stream) {
  const int rc = check_weight(w);
  if (rc) return rc;
  if (w->rows == 0) return QERR_OK;
  if (!rowmajor) return QERR_INVALID_ARG;
  if (!aligned(rowmajor, 2)) return QERR_ALIGNMENT;
  return hip_rc(launch_scales_to_rows(w->fmt, w->rows, w->cols, w->scales, rowmajor, S(stream)));
}

int qweight_quantize(int32_t fmt, const float* w, int32_t rows, int32_t cols, void* codes, int64_t row_bytes,
                     uint16_t* scales, void* stream) {
  if (fmt == QFMT_TRELLIS2) return QERR_UNSUPPORTED_FMT;
  qweight_t d{fmt, rows, cols, scale_block(fmt), codes, row_bytes, scales, nullptr};
  const int rc = check_weight(&d);
  if (rc) return rc;
  if (rows == 0) return QERR_OK;
  if (!w) return QERR_INVALID_ARG;
  if (!aligned(w, 4)) return QERR_ALIGNMENT;
  return hip_rc(launch_quantize(fmt, w, rows, cols, (uint8_t*)codes, row_bytes, scales, S(stream)));
}

int qweight_pack(int32_t fmt, const int8_t* levels, int32_t rows, int32_t cols, void* codes, int64_t row_bytes,
                 void* stream) {
  const int32_t blk = scale_block(fmt);
  if (blk == 0) return QERR_UNSUPPORTED_FMT;
  if (rows < 0 || cols < 0) return QERR_INVALID_ARG;
  if (cols == 0 || cols % blk != 0 || cols % 32 != 0) return QERR_SHAPE;
  if (rows == 0) return QERR_OK;
  if (!levels || !codes) return QERR_INVALID_ARG;
  if (row_bytes < packed_row_bytes(fmt, cols) || row_bytes % 16 != 0) return QERR_SHAPE;
  if (!aligned(codes, 16)) return QERR_ALIGNMENT;
  return hip_rc(launch_pack(fmt, levels, rows, cols, (uint8_t*)codes, row_bytes, S(stream)));
}

int qact_quant_i8(const float* x, int32_t B, int32_t K, int32_t qblock, int8_t* q, float* d, int32_t* qsum,
                  void* stream) {
  if (B < 0 || K < 0) return QERR_INVALID_ARG;
  if (qblock != 32 && qblock != 256) return QERR_INVALID_ARG;
  if (B == 0) return QERR_OK;
  if (K == 0 || K % qblock != 0) return QERR_SHAPE;
  if (!x || !q || !d || !qsum) return QERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(q, 4) || !aligned(d, 4) || !aligned(qsum, 4)) return QERR_ALIGNMENT;
  if ((int64_t)B * K >= ((int64_t)1 << 40)) return QERR_SHAPE;
  return hip_rc(launch_act_quant(x, B, K, qblock, q, d, qsum, S(stream)));
}

int qact_planes(const int8_t* q, int32_t B, int32_t K, uint32_t* planes, void* stream) {
  if (B < 0 || K < 0) return QERR_INVALID_ARG;
  if (B == 0) return QERR_OK;
  if (K == 0 || K % 32 != 0) return QERR_SHAPE;
  if (!q || !planes) return QERR_INVALID_ARG;
  if (!aligned(q, 4) || !aligned(planes, 32)) return QERR_ALIGNMENT;
  if ((int64_t)B * K >= ((int64_t)1 << 40)) return QERR_SHAPE;
  return hip_rc(launch_act_planes(q, B, K, planes, S(stream)));
}

int qact_quant_batch(const qact_job_t* jobs, int32_t n, void* stream) {
  if (n < 0 || n > QACT_BATCH_MAX) return QERR_INVALID_ARG;
  if (n == 0) return QERR_OK;
  if (!jobs) return QERR_INVALID_ARG;
  for (int j = 0; j < n; ++j) {
    const qact_job_t& J = jobs[j];
    if (J.B < 0 || J.K < 0) return QERR_INVALID_ARG;
    if (J.B == 0) continue;
    if (J.K == 0 || J.K % 32 != 0) return QERR_SHAPE;
    if (!J.x || !J.d || !J.qsum || (!J.q && !J.planes)) return QERR_INVALID_ARG;
    if (!aligned(J.x, 16) || !aligned(J.q, 4) || !aligned(J.planes, 32) || !aligned(J.d, 4) || !aligned(J.qsum, 4))
      return QERR_ALIGNMENT;
    if ((int64_t)J.B * J.K >= ((int64_t)1 << 36)) return QERR_SHAPE;
  }
  return hip_rc(launch_act_quant_batch(jobs, n, S(stream)));
}

int qact_hadamard_quant_i8(const float* x, int32_t B, int32_t K, const uint32_t* sign_bits, int32_t qblock,
                           int8_t* q, float* d, int32_t* qsum, void* stream) {
  if (B < 0 || K < 0) return QERR_INVALID_ARG;
  if (qblock != 32 && qblock != 256 && qblock != K) return QERR_INVALID_ARG;
  if (B == 0) return QERR_OK;
  if (K == 0 || K % 256 != 0) return QERR_SHAPE;
  if (qblock == K && K > 32768) return QERR_SHAPE;  // one scale per row: the row fits one workgroup
  if (!x || !q || !d || !qsum || !sign_bits) return QERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(q, 4) || !aligned(d, 4) || !aligned(qsum, 4) || !aligned(sign_bits, 4))
    return QERR_ALIGNMENT;
  if ((int64_t)B * (K / 256) >= ((int64_t)1 << 33)) return QERR_SHAPE;
  return hip_rc(launch_hadamard_quant(x, B, K, sign_bits, qblock, q, d, qsum, S(stream)));
}

int qgemv(const qweight_t* w, const int8_t* q, const uint32_t* planes, const float* d, const int32_t* qsum,
          int32_t B, float* y, void* stream) {
  int rc = check_weight(w);
  if (rc) return rc;
  if (B < 0 || B > kMaxBatch) return QERR_INVALID_ARG;
  if (B == 0 || w->rows == 0) return QERR_OK;
  rc = check_act(w->fmt, q, planes, d, qsum);
  if (rc) return rc;
  if (!y) return QERR_INVALID_ARG;
  if (!aligned(y, 4)) return QERR_ALIGNMENT;
  return hip_rc(launch_gemv_any(make_item(w, q, planes, d, qsum, y), B, S(stream)));
}

int qgemv_blockdots(const qweight_t* w, const int8_t* q, const uint32_t* planes, const int32_t* qsum, int32_t* out,
                    void* stream) {
  int rc = check_weight(w);
  if (rc) return rc;
  if (w->rows == 0) return QERR_OK;
  // the scale path is unused by the hook; pass qsum for d so no pointer is null
  rc = check_act(w->fmt, q, planes, (const float*)qsum, qsum);
  if (rc) return rc;
  if (!out) return QERR_INVALID_ARG;
  if (!aligned(out, 4)) return QERR_ALIGNMENT;
  return hip_rc(launch_blockdots(make_item(w, q, planes, (const float*)qsum, qsum, nullptr), out, S(stream)));
}

int64_t qgemv_grouped_plan_bytes(const qgemv_item_t* items, int32_t n, int32_t B) {
  if (!items || n <= 0 || B < 1 || B > kMaxBatch) return QERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) {
    const int rc = check_item(items[i], B);
    if (rc) return rc;
  }
  return align16(sizeof(PlanHeader)) + align16((int64_t)sizeof(GemvItem) * n) +
         align16((int64_t)sizeof(GemvTile) * count_tiles(items, n)) +
         align16((int64_t)sizeof(int32_t) * 6 * (kPlanWorkers + 1));
}

int qgemv_grouped_plan(const qgemv_item_t* items, int32_t n, int32_t B, void* host_plan, int64_t plan_bytes) {
  const int64_t need = qgemv_grouped_plan_bytes(items, n, B);
  if (need < 0) return (int)need;
  if (!host_plan) return QERR_INVALID_ARG;
  if (plan_bytes < need) return QERR_BUFFER;
  if (!aligned(host_plan, 16)) return QERR_ALIGNMENT;
  const int64_t ntiles = count_tiles(items, n);
  if (ntiles >= ((int64_t)1 << 31)) return QERR_SHAPE;
  uint8_t* base = (uint8_t*)host_plan;
  std::memset(base, 0, (size_t)need);
  PlanHeader h{};
  h.magic = kPlanMagic;
  h.version = kPlanVersion;
  h.n_items = n;
  h.n_tiles = (int32_t)ntiles;
  h.B = B;
  h.items_off = align16(sizeof(PlanHeader));
  h.tiles_off = h.items_off + align16((int64_t)sizeof(GemvItem) * n);
  h.workers_off = h.tiles_off + align16((int64_t)sizeof(GemvTile) * ntiles);
  h.n_workers = kPlanWorkers;
  h.total_bytes = need;
  GemvItem* it = (GemvItem*)(base + h.items_off);
  for (int32_t i = 0; i < n; ++i) {
    it[i] = make_item(&items[i].w, items[i].q, items[i].planes, items[i].d, items[i].qsum, items[i].y);
    if (items[i].w.rows > 0) h.fmt_mask |= 1 << items[i].w.fmt;
  }
  // Tiles: grouped by format; inside a format, dealt longest first to the
  // list with the fewest bytes so far (ties: the lowest list), stored list by
  // list.  Cost of a tile: its code and scale bytes.
  struct T { int64_t cost; uint32_t item, row0; };
  std::vector<std::vector<T>> q(6);
  for (int32_t i = 0; i < n; ++i) {
    const qweight_t& w = items[i].w;
    for (int32_t r = 0; r < w.rows; r += 64) {
      const int64_t rows = std::min(64, w.rows - r);
      const int64_t c = rows * (w.row_bytes + (int64_t)(w.cols / w.block) * 2);
      q[w.fmt].push_back({c, (uint32_t)i, (uint32_t)r});
    }
  }
  GemvTile* tiles = (GemvTile*)(base + h.tiles_off);
  int32_t* wb_all = (int32_t*)(base + h.workers_off);
  int64_t k = 0;
  for (int f = 1; f <= 5; ++f) {
    std::stable_sort(q[f].begin(), q[f].end(), [](const T& a, const T& b) { return a.cost > b.cost; });
    std::vector<std::vector<uint32_t>> lists(kPlanWorkers);
    std::vector<std::pair<int64_t, int>> heap;  // (bytes so far, list), a min-heap
    for (int w = 0; w < kPlanWorkers; ++w) heap.push_back({0, w});
    auto later = [](const std::pair<int64_t, int>& a, const std::pair<int64_t, int>& b) { return a > b; };
    for (size_t j = 0; j < q[f].size(); ++j) {
      std::pop_heap(heap.begin(), heap.end(), later);
      lists[heap.back().second].push_back((uint32_t)j);
      heap.back().first += q[f][j].cost;
      std::push_heap(heap.begin(), heap.end(), later);
    }
    h.fmt_begin[f] = (int32_t)k;
    int32_t* wb = wb_all + f * (kPlanWorkers + 1);
    for (int w = 0; w < kPlanWorkers; ++w) {
      wb[w] = (int32_t)k;
      for (uint32_t j : lists[w]) {
        tiles[k].item = q[f][j].item;
        tiles[k].row0 = q[f][j].row0;
        ++k;
      }
    }
    wb[kPlanWorkers] = (int32_t)k;
  }
  h.fmt_begin[6] = (int32_t)k;
  std::memcpy(base, &h, sizeof(h));
  return QERR_OK;
}

int qgemv_grouped_run(const void* host_plan, const void* dev_plan, void* stream) {
  if (!host_plan || !dev_plan) return QERR_INVALID_ARG;
  if (!aligned(host_plan, 16) || !aligned(dev_plan, 16)) return QERR_ALIGNMENT;
  PlanHeader h;
  if (read_plan_header(host_plan, &h)) return QERR_BUFFER;
  if (h.n_tiles == 0) return QERR_OK;
  return hip_rc(launch_grouped_any(h, dev_plan, S(stream)));
}

int qgemv_grouped_run_static(const void* host_plan, void* stream) {
  if (!host_plan) return QERR_INVALID_ARG;
  if (!aligned(host_plan, 16)) return QERR_ALIGNMENT;
  PlanHeader h;
  if (read_plan_header(host_plan, &h)) return QERR_BUFFER;
  if (h.total_bytes > kStaticPlanBytes) return QERR_TOO_LARGE;
  if (h.n_tiles == 0) return QERR_OK;
  void* dev_plan = nullptr;
  const int rc = static_plan_address(&dev_plan);
  if (rc) return rc;
  const hipStream_t st = S(stream);
  if (hipMemcpyAsync(dev_plan, host_plan, (size_t)h.total_bytes, hipMemcpyHostToDevice, st) != hipSuccess)
    return QERR_HIP;
  return hip_rc(launch_grouped_any(h, dev_plan, st));
}

int qtrellis_decode_i8(const qweight_t* w, int32_t oblock, int8_t* wq, float* dw, void* stream) {
  int rc = check_weight(w);
  if (rc) return rc;
  if (w->fmt != QFMT_TRELLIS2) return QERR_UNSUPPORTED_FMT;
  if (oblock != 32 && oblock != 256 && oblock != w->cols) return QERR_INVALID_ARG;
  if (w->cols % 256 != 0) return QERR_SHAPE;
  if (oblock == w->cols && w->cols > 32768) return QERR_SHAPE;  // one scale per row: the row fits one workgroup
  if (w->rows == 0) return QERR_OK;
  if (!wq || !dw) return QERR_INVALID_ARG;
  if (!aligned(wq, 4) || !aligned(dw, 4)) return QERR_ALIGNMENT;
  const GemvItem it = make_item(w, nullptr, nullptr, nullptr, nullptr, nullptr);
  return hip_rc(launch_trellis_decode(it, oblock, wq, dw, S(stream)));
}

int64_t qkv_row_bytes(int32_t fmt) {
  if (fmt == QKV_Q8) return QATTN_HEAD_DIM;
  if (fmt == QKV_Q4) return QATTN_HEAD_DIM / 2;
  return QERR_UNSUPPORTED_FMT;
}

int qkv_quant(int32_t fmt, const float* x, int64_t rows, void* codes, uint16_t* scales, void* stream) {
  if (fmt != QKV_Q8 && fmt != QKV_Q4) return QERR_UNSUPPORTED_FMT;
  if (rows < 0) return QERR_INVALID_ARG;
  if (rows == 0) return QERR_OK;
  if (!x || !codes || !scales) return QERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 2)) return QERR_ALIGNMENT;
  if (rows >= ((int64_t)1 << 40) / QATTN_HEAD_DIM) return QERR_SHAPE;
  return hip_rc(launch_kv_quant(fmt, x, rows, (uint8_t*)codes, scales, S(stream)));
}

int64_t qattn_decode_workspace_bytes(int32_t n_kv, int32_t group, int32_t T) {
  if (n_kv < 1 || group < 1 || group > 8 || T < 1) return QERR_INVALID_ARG;
  return attn_workspace_bytes(n_kv, group, T);
}

int qattn_decode(int32_t fmt, const float* q, int32_t n_kv, int32_t group, int32_t heads_per_block, int32_t T,
                 int64_t t_cap, const void* kcodes, const uint16_t* kscales, const void* vcodes,
                 const uint16_t* vscales, float* out, void* workspace, int64_t workspace_bytes, void* stream) {
  if (fmt != QKV_Q8 && fmt != QKV_Q4) return QERR_UNSUPPORTED_FMT;
  if (n_kv < 1 || group < 1 || group > 8 || (heads_per_block != 1 && heads_per_block != group))
    return QERR_INVALID_ARG;
  if (T < 1 || t_cap < T || n_kv > 65535 / group) return QERR_SHAPE;
  if (!q || !kcodes || !kscales || !vcodes || !vscales || !out || !workspace) return QERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(kcodes, 16) || !aligned(vcodes, 16) || !aligned(kscales, 16) ||
      !aligned(vscales, 16) || !aligned(out, 4) || !aligned(workspace, 16))
    return QERR_ALIGNMENT;
  if (workspace_bytes < attn_workspace_bytes(n_kv, group, T)) return QERR_BUFFER;
  return hip_rc(launch_attn_decode(fmt, q, n_kv, group, heads_per_block, T, t_cap, kcodes, kscales, vcodes, vscales,
                                   out, workspace, S(stream)));
}

int64_t qtrellis_encode_workspace_bytes(int32_t rows, int32_t cols, int32_t rows_per_pass) {
  if (rows < 1 || cols < 1 || rows_per_pass < 1) return QERR_INVALID_ARG;
  if (cols < 64 || cols % 64 != 0 || cols > kMaxEncodeCols) return QERR_SHAPE;
  return encode_workspace_bytes(rows, cols, rows_per_pass < rows ? rows_per_pass : rows);
}

int qtrellis_encode(const float* w, int32_t rows, int32_t cols, const uint16_t* scales_in, void* codes,
                    int64_t row_bytes, uint16_t* seeds, uint16_t* scales, float* cost, int32_t rows_per_pass,
                    void* workspace, int64_t workspace_bytes, void* stream) {
  if (rows < 0 || cols < 0 || rows_per_pass < 1) return QERR_INVALID_ARG;
  if (rows == 0) return QERR_OK;
  if (cols < 64 || cols % 64 != 0 || cols > kMaxEncodeCols) return QERR_SHAPE;
  if (!w || !codes || !seeds || !scales || !workspace) return QERR_INVALID_ARG;
  if (row_bytes < packed_row_bytes(QFMT_TRELLIS2, cols) || row_bytes % 16 != 0) return QERR_SHAPE;
  if (!aligned(w, 4) || !aligned(codes, 16) || !aligned(seeds, 2) || !aligned(scales, 16) ||
      !aligned(scales_in, 2) || !aligned(cost, 4) || !aligned(workspace, 256))
    return QERR_ALIGNMENT;
  const int32_t per = rows_per_pass < rows ? rows_per_pass : rows;
  if (workspace_bytes < encode_workspace_bytes(rows, cols, per)) return QERR_BUFFER;
  return hip_rc(launch_trellis_encode(w, rows, cols, scales_in, (uint8_t*)codes, row_bytes, seeds, scales, cost,
                                      per, workspace, S(stream)));
}

int qweight_unpack_i8(const qweight_t* w, int8_t* wq, float* dw, void* stream) {
  int rc = check_weight(w);
  if (rc) return rc;
  if (w->fmt == QFMT_TRELLIS2) return QERR_UNSUPPORTED_FMT;
  if (w->rows == 0) return QERR_OK;
  if (!wq || !dw) return QERR_INVALID_ARG;
  if (!aligned(dw, 4)) return QERR_ALIGNMENT;
  return hip_rc(launch_unpack_i8(make_item(w, nullptr, nullptr, nullptr, nullptr, nullptr), wq, dw, S(stream)));
}

int qgemm_i8(const int8_t* xq, const float* dx, int32_t M, const int8_t* wq, const float* dw, int32_t N, int32_t K,
             int32_t kblock, float* y, void* stream) {
  if (M < 0 || N < 0 || K < 0) return QERR_INVALID_ARG;
  if (kblock != 32 && kblock != 256 && kblock != K) return QERR_INVALID_ARG;
  if (M == 0 || N == 0) return QERR_OK;
  if (K == 0 || K % kblock != 0 || K % 64 != 0) return QERR_SHAPE;
  if (!xq || !dx || !wq || !dw || !y) return QERR_INVALID_ARG;
  if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(dx, 4) || !aligned(dw, 4) || !aligned(y, 4))
    return QERR_ALIGNMENT;
  return hip_rc(launch_gemm(xq, dx, M, wq, dw, N, K, kblock, y, S(stream)));
}

int qcalib_mfma_i8(int32_t blocks, int32_t iters, uint64_t* clocks, int32_t* sink, void* stream) {
  if (blocks < 0 || iters < 0) return QERR_INVALID_ARG;
  if (blocks == 0) return QERR_OK;
  if (!clocks || !sink) return QERR_INVALID_ARG;
  if (!aligned(clocks, 8) || !aligned(sink, 4)) return QERR_ALIGNMENT;
  return hip_rc(launch_mfma_peak(blocks, iters, clocks, sink, S(stream)));
}

int qcalib_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (bytes < 0) return QERR_INVALID_ARG;
  if (bytes == 0) return QERR_OK;
  if (!buf || !sink) return QERR_INVALID_ARG;
  if (bytes % 16 != 0) return QERR_SHAPE;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return QERR_ALIGNMENT;
  return hip_rc(launch_hbm_read(buf, bytes, sink, S(stream)));
}

}  // extern "C"
