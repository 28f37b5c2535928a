// One decode step of HGA (abstract of "Hierarchical Global Attention (HGA)",
// arXiv 2606.30709) as a single launch: refresh the newest chunk summaries,
// route, attend.
//
// The first workgroups of the grid route: one per query row, refreshing the
// newest chunks of its sequence from K, scoring both levels on-chip and
// publishing the row's group ids with agent-coherent stores followed by a
// per-row ready flag. The workgroups after them attend: each waits (bounded)
// for its row's flag, reads the group ids coherently and gathers its share of
// the routed keys and values; the row's last attention workgroup clears the
// flag. Workgroups start in index order on each XCD, so every routing
// workgroup is resident or done before any attention workgroup of its XCD
// occupies a slot: routing never waits, and attention only waits on it.
// Routing of one row overlaps the gathers of rows routed earlier, and the
// step pays one launch instead of two.
#include "hga_attend_body.h"
#include "hga_route_row_launch.h"

namespace hga {
namespace {

using rowroute::kThreads;

template <typename T, int D, int E>
__global__ __launch_bounds__(kThreads) void decode_kernel(RouteArgs ra, AttendArgs aa,
                                                          int groups_per_wave, int n_splits,
                                                          int n_route, unsigned* ready) {
  extern __shared__ float s_dyn[];
  const int bid = static_cast<int>(blockIdx.x);
  if (bid < n_route) {
    rowroute::route_row_body<T, D, E, true, true, true>(ra, bid, s_dyn, ready);
  } else {
    attend_body<T, D, true, rowroute::kWaves>(aa, groups_per_wave, n_splits, 0, bid - n_route,
                                              ready);
  }
}

template <typename T, int D>
hipError_t launch_td(const RouteArgs& ra, const AttendArgs& aa, const AttendPlan& plan,
                     unsigned* ready, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(ra.B) * ra.Hq * ra.Nq;
  const int n_route = static_cast<int>(rowroute::route_row_grid(ra));
  const dim3 grid(static_cast<unsigned>(n_route + rows * plan.n_splits));
  const size_t lds = rowroute::route_row_lds_bytes(ra);
  const int gpw = plan.groups_per_wave, ns = plan.n_splits;
  switch (select_regs(ra)) {
#define HGA_DECODE_CASE(EV)                                                                 \
  case EV:                                                                                  \
    hipLaunchKernelGGL((decode_kernel<T, D, EV>), grid, dim3(kThreads), lds, stream, ra, aa, \
                       gpw, ns, n_route, ready);                                            \
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
                         gpw, ns, n_route, ready);
      break;
#undef HGA_DECODE_CASE
  }
  return hipGetLastError();
}

}  // namespace

bool decode_step_one_launch(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t D, int G,
                            int k_g) {
  const int64_t units = B * Hkv, rpu = (Hq / Hkv) * Nq, rows = B * Hq * Nq;
  const int64_t n_route = 8 * ((units + 7) / 8) * rpu;
  const AttendPlan plan = plan_attend(rows, D, G, k_g, rowroute::kWaves);
  return n_route + rows * plan.n_splits <= device_cu_count();
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
