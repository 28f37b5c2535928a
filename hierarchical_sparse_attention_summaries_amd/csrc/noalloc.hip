// hga_decode_step_noalloc: hga_decode_step_ex for callers that cannot
// allocate device memory (code under graph capture, tight serving loops): the
// step's scratch comes from a fixed array in the library's own device memory
// instead of a caller workspace. Nothing here allocates.
#include <hip/hip_runtime.h>

#include <mutex>

#include "hga.h"
#include "hga_internal.h"

namespace {

// Largest scratch one call may use: the decode step's workspace (its 4 MiB
// zero region plus routing or attention plans), enough for 42 sequences at a
// 64K context with Qwen3-30B-A3B's 32 query heads. Each device the library runs on holds
// its own copy until the process ends.
constexpr size_t kScratchBytes = size_t{16} << 20;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];      // the array's device address on each device, once looked up
bool g_cleared[kMaxDevices];   // its zero region cleared (in stream order) on that device

}  // namespace

extern "C" int hga_decode_step_noalloc(const hga_shape* shape, const hga_kv_layout* layout,
                                       const void* Q, const void* K, const void* V,
                                       int32_t dtype, float* chunk_mean, float* group_mean,
                                       int32_t chunk, int32_t group, int32_t k_chunk,
                                       int32_t k_group, float scale, int32_t* chunk_idx,
                                       int32_t* group_idx, void* O, float* lse, int32_t reset,
                                       void* stream) {
  size_t need = 0;
  const int st = hga_decode_step_workspace_size(shape, chunk, group, k_chunk, k_group, &need);
  if (st != HGA_OK) return st;
  if (need > kScratchBytes) return HGA_ERR_WORKSPACE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HGA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    // The array's name is a host-side stand-in: its address on this device
    // comes from the runtime, once, with the device current.
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return HGA_ERR_HIP;
    g_ptr[dev] = p;
  }
  // The zero region is cleared before the first step on this device and
  // whenever the caller asks (after a step whose bounded wait gave up).
  const bool clear = !g_cleared[dev] || reset != 0;
  const int r = hga::decode_step_call(shape, layout, Q, K, V, dtype, chunk_mean, group_mean,
                                      chunk, group, k_chunk, k_group, scale, chunk_idx,
                                      group_idx, O, lse, g_ptr[dev], kScratchBytes, clear,
                                      stream);
  if (r == HGA_OK) g_cleared[dev] = true;
  return r;
}
