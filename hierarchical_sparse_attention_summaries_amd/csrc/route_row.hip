// Step 2 of HGA (abstract of "Hierarchical Global Attention (HGA)", arXiv
// 2606.30709): the one-workgroup-per-query-row route and when it applies (the
// body is in hga_route_row_body.h; the refreshing launches are compiled in
// route_row_fresh.hip).
#include "hga_route_row_launch.h"

namespace hga {

using namespace rowroute;

bool use_row_route(int64_t B, int64_t Hq, int64_t Nq, int64_t T, int64_t D, int C, int G,
                   int k_c, int k_g, bool fresh, size_t extra_lds) {
  if (B * Hq * Nq > 1024) return false;
  if (fresh && (Nq > C || C / G > kFreshMaxGpc)) return false;
  const int64_t n_c = (T + C - 1) / C;
  const int64_t cap = std::min<int64_t>(int64_t(k_c) + 2, n_c);
  return route_row_lds_bytes(n_c, cap, C / G, k_c, k_g) + route_row_static_lds(D, fresh) +
             extra_lds <=
         kRowRouteMaxLds;
}

hipError_t launch_route_rows(const RouteArgs& a, int dtype, hipStream_t stream) {
  if (a.K) return launch_route_rows_fresh(a, dtype, stream);
  return launch_rows<false>(a, dtype, stream);
}

}  // namespace hga
