// One decode step of HGA (abstract of "Hierarchical Global Attention (HGA)",
// arXiv 2606.30709) as a single launch: refresh the newest chunk summaries,
// route, attend.
//
// The grid is at most one workgroup per CU, all resident at once. Workgroups
// [0, R) first route: one per query row, refreshing the newest chunks of its
// sequence from K, scoring both levels on-chip and publishing the row's group
// ids with agent-coherent stores followed by a per-row ready flag. Then every
// workgroup [0, A) attends one (row, split) item: it waits (bounded) for its
// row's flag, reads the group ids coherently and gathers its share of the
// routed keys and values with 8 waves, one group per wave where the grid
// allows; the row's last workgroup clears the flag. So the attention spreads
// over every CU, the routing workgroups included once their row is done.
// Routing never waits, and every waiting workgroup is resident beside the
// routing it waits for. The step pays one launch instead of two.
#include "hga_attend_body.h"
#include "hga_route_row_launch.h"

namespace hga {
namespace {

using rowroute::kThreads;

template <typename T, int D, int E>
__global__ __launch_bounds__(kThreads) void decode_kernel(RouteArgs ra, AttendArgs aa,
                                                          int groups_per_wave, int n_splits,
                                                          int n_route, int n_attend,
                                                          unsigned* ready) {
  extern __shared__ float s_dyn[];
  const int bid = static_cast<int>(blockIdx.x);
  if (bid < n_route) rowroute::route_row_body<T, D, E, true, true, true>(ra, bid, s_dyn, ready);
  if (bid < n_attend)
    attend_body<T, D, true, rowroute::kWaves>(aa, groups_per_wave, n_splits, 0, bid, ready);
}

template <typename T, int D>
hipError_t launch_td(const RouteArgs& ra, const AttendArgs& aa, const AttendPlan& plan,
                     unsigned* ready, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(ra.B) * ra.Hq * ra.Nq;
  const int n_route = static_cast<int>(rowroute::route_row_grid(ra));
  const int n_attend = static_cast<int>(rows * plan.n_splits);
  const dim3 grid(static_cast<unsigned>(n_route > n_attend ? n_route : n_attend));
  const size_t lds = rowroute::route_row_lds_bytes(ra);
  const int gpw = plan.groups_per_wave, ns = plan.n_splits;
  switch (select_regs(ra)) {
#define HGA_DECODE_CASE(EV)                                                                 \
  case EV:                                                                                  \
    hipLaunchKernelGGL((decode_kernel<T, D, EV>), grid, dim3(kThreads), lds, stream, ra, aa, \
                       gpw, ns, n_route, n_attend, ready);                                  \
    break;
    HGA_DECODE_CASE(1)
    HGA_DECODE_CASE(2)
    HGA_DECODE_CASE(3)
    HGA_DECODE_CASE(4)
    HGA_DECODE_CASE(5)
    HGA_DECODE_CASE(6)
    HGA_DECODE_CASE(8)
    HGA_DECODE_CASE(16)
    HGA_DECODE_CASE(32)
    default:
      hipLaunchKernelGGL((decode_kernel<T, D, 64>), grid, dim3(kThreads), lds, stream, ra, aa,
                         gpw, ns, n_route, n_attend, ready);
      break;
#undef HGA_DECODE_CASE
  }
  return hipGetLastError();
}

}  // namespace

AttendPlan plan_decode_attend(int64_t rows, int64_t D, int k_g) {
  // The fewest groups per wave (8 waves per workgroup) that keep one
  // workgroup per (row, split) within one per CU.
  const int W = rowroute::kWaves;
  int gpw = 1;
  while (gpw < k_g &&
         (rows * ((k_g + W * gpw - 1) / (W * gpw)) > device_cu_count() ||
          (k_g + W * gpw - 1) / (W * gpw) > kAttendMaxSplits))
    gpw *= 2;
  AttendPlan pl{};
  pl.groups_per_wave = gpw;
  pl.n_splits = (k_g + W * gpw - 1) / (W * gpw);
  pl.off_counters = 0;
  pl.off_partials = kCounterBytes;
  const size_t part = pl.n_splits > 1 ? static_cast<size_t>(rows) * pl.n_splits * (D + 2) * 4 : 0;
  pl.bytes = (pl.off_partials + part + 255) / 256 * 256;
  return pl;
}

bool decode_step_one_launch(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t D, int G,
                            int k_g) {
  (void)G;
  const int64_t units = B * Hkv, rpu = (Hq / Hkv) * Nq, rows = B * Hq * Nq;
  const int64_t n_route = 8 * ((units + 7) / 8) * rpu;
  const AttendPlan plan = plan_decode_attend(rows, D, k_g);
  return n_route <= device_cu_count() && rows * plan.n_splits <= device_cu_count();
}

size_t decode_step_lds(int64_t D) {
  // attend_body's static LDS with 8 waves (bound)
  return static_cast<size_t>(2 * rowroute::kWaves + rowroute::kWaves * D +
                             kAttendMaxSplits * (D + 2)) * 4 + 64;
}

hipError_t launch_decode_step(const RouteArgs& ra, const AttendArgs& aa, const AttendPlan& plan,
                              int dtype, unsigned* ready, hipStream_t stream) {
  if (dtype == kF32)
    return ra.D == 64 ? launch_td<float, 64>(ra, aa, plan, ready, stream)
                      : launch_td<float, 128>(ra, aa, plan, ready, stream);
  return ra.D == 64 ? launch_td<uint16_t, 64>(ra, aa, plan, ready, stream)
                    : launch_td<uint16_t, 128>(ra, aa, plan, ready, stream);
}

}  // namespace hga
