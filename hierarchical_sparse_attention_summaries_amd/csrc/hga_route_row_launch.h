// Launch of the one-workgroup-per-query-row route for one (dtype, D, refresh,
// form) combination; route_row.hip and route_row_fresh.hip instantiate it
// (without and with the summary refresh) so that the two compile in parallel.
#pragma once

#include "hga_route_row_body.h"

namespace hga {
namespace rowroute {

template <typename TQ, int D, int E, bool FRESH, bool BIG>
__global__ __launch_bounds__(kThreads) void route_row_kernel(RouteArgs a) {
  extern __shared__ float s_dyn[];
  route_row_body<TQ, D, E, FRESH, BIG>(a, static_cast<int>(blockIdx.x), s_dyn);
}

// Workgroups of the row route: rows of one (sequence, KV head) share an XCD,
// 8 units per round of XCDs.
inline int64_t route_row_grid(const RouteArgs& a) {
  const int64_t units = static_cast<int64_t>(a.B) * a.Hkv;
  const int64_t rpu = static_cast<int64_t>(a.Hq / a.Hkv) * a.Nq;
  return 8 * ((units + 7) / 8) * rpu;
}

template <typename TQ, int D, bool FRESH, bool BIG>
hipError_t launch_rows_t(const RouteArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(route_row_grid(a)));
  const size_t lds = route_row_lds_bytes(a);
  switch (select_regs(a)) {
#define HGA_ROW_CASE(EV)                                                                     \
  case EV:                                                                                   \
    hipLaunchKernelGGL((route_row_kernel<TQ, D, EV, FRESH, BIG>), grid, dim3(kThreads), lds, \
                       stream, a);                                                           \
    break;
    HGA_ROW_CASE(1)
    HGA_ROW_CASE(2)
    HGA_ROW_CASE(3)
    HGA_ROW_CASE(4)
    HGA_ROW_CASE(5)
    HGA_ROW_CASE(6)
    HGA_ROW_CASE(8)
    HGA_ROW_CASE(16)
    HGA_ROW_CASE(32)
#undef HGA_ROW_CASE
    default:
      hipLaunchKernelGGL((route_row_kernel<TQ, D, 64, FRESH, BIG>), grid, dim3(kThreads), lds,
                         stream, a);
      break;
  }
  return hipGetLastError();
}

template <bool FRESH>
hipError_t launch_rows(const RouteArgs& a, int dtype, hipStream_t stream) {
  // One workgroup per CU at most: the big form (more registers, fewer memory
  // round trips); else the lean form, two workgroups per CU.
  const bool big = route_row_grid(a) <= kPlanCus;
  if (dtype == kF32) {
    if (a.D == 64)
      return big ? launch_rows_t<float, 64, FRESH, true>(a, stream)
                 : launch_rows_t<float, 64, FRESH, false>(a, stream);
    return big ? launch_rows_t<float, 128, FRESH, true>(a, stream)
               : launch_rows_t<float, 128, FRESH, false>(a, stream);
  }
  if (a.D == 64)
    return big ? launch_rows_t<uint16_t, 64, FRESH, true>(a, stream)
               : launch_rows_t<uint16_t, 64, FRESH, false>(a, stream);
  return big ? launch_rows_t<uint16_t, 128, FRESH, true>(a, stream)
             : launch_rows_t<uint16_t, 128, FRESH, false>(a, stream);
}

}  // namespace rowroute

// Defined in route_row_fresh.hip.
hipError_t launch_route_rows_fresh(const RouteArgs& a, int dtype, hipStream_t stream);

}  // namespace hga
