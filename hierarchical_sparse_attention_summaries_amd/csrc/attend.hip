// Step 3 of HGA (abstract of "Hierarchical Global Attention (HGA)", arXiv
// 2606.30709): the exact-attention launch and its plan. The workgroup body
// (gather + online softmax + split merge) is in hga_attend_body.h.
#include <math.h>

#include "hga_attend_body.h"
#include "hga_device.h"
#include "hga_internal.h"

namespace hga {
namespace {

constexpr int kThreads = kAttendThreads;
constexpr int kMaxSplits = kAttendMaxSplits;

template <typename TKV, int D>
__global__ __launch_bounds__(kAttendThreads) void attend_kernel(AttendArgs a, int groups_per_wave,
                                                                int n_splits, int row_base) {
  attend_body<TKV, D>(a, groups_per_wave, n_splits, row_base, static_cast<int>(blockIdx.x));
}

template <typename TKV, int D>
hipError_t launch_t(const AttendArgs& a, const AttendPlan& plan, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(a.B) * a.Hq * a.Nq;
  // With splits, slices of at most kMaxCounters rows (one counter each) that
  // reuse the counters in stream order; without, one launch.
  const int64_t slice = plan.n_splits > 1 ? kMaxCounters : rows;
  for (int64_t base = 0; base < rows; base += slice) {
    const int64_t n = rows - base < slice ? rows - base : slice;
    hipLaunchKernelGGL((attend_kernel<TKV, D>), dim3(static_cast<unsigned>(n * plan.n_splits)),
                       dim3(kThreads), 0, stream, a, plan.groups_per_wave, plan.n_splits,
                       static_cast<int>(base));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

AttendPlan plan_attend(int64_t rows, int64_t D, int G, int k_g, int waves) {
  AttendPlan pl{};
  // Enough waves to keep every CU's memory pipe busy (each wave keeps two
  // groups in flight), no more: larger groups_per_wave means fewer partials
  // to merge and fewer workgroups bumping one arrival counter.
  const int64_t target_waves = 4 * static_cast<int64_t>(kPlanCus);
  int gpw = 1;
  while (gpw < 16 && rows * ((k_g + 2 * gpw - 1) / (2 * gpw)) >= target_waves) gpw *= 2;
  (void)G;
  // at most kMaxSplits workgroups (of `waves` waves) per row
  while ((k_g + gpw - 1) / gpw > kMaxSplits * waves) gpw *= 2;
  pl.groups_per_wave = gpw;
  const int waves_per_row = (k_g + gpw - 1) / gpw;
  pl.n_splits = (waves_per_row + waves - 1) / waves;
  pl.off_counters = 0;
  pl.off_partials = kZeroBytes;
  const size_t part = pl.n_splits > 1 ? static_cast<size_t>(rows) * pl.n_splits * (D + 2) * 4 : 0;
  pl.bytes = align_up(pl.off_partials + part, 256);
  return pl;
}

hipError_t launch_attend(const AttendArgs& a, int dtype, const AttendPlan& plan,
                         hipStream_t stream) {
  if (use_tile_attend(a, dtype)) return launch_attend_tiles(a, stream);
  if (dtype == kF32)
    return a.D == 64 ? launch_t<float, 64>(a, plan, stream) : launch_t<float, 128>(a, plan, stream);
  return a.D == 64 ? launch_t<uint16_t, 64>(a, plan, stream)
                   : launch_t<uint16_t, 128>(a, plan, stream);
}

}  // namespace hga
