// Step 2 of HGA with the decode-step refresh of the newest chunks' summaries
// (abstract of "Hierarchical Global Attention (HGA)", arXiv 2606.30709): the
// refreshing launches of the one-workgroup-per-query-row route.
#include "hga_route_row_launch.h"

namespace hga {

hipError_t launch_route_rows_fresh(const RouteArgs& a, int dtype, hipStream_t stream) {
  return rowroute::launch_rows<true>(a, dtype, stream);
}

}  // namespace hga
