// Host-side argument checking of libhga, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the library's host code: every entry point is
// called with arguments it must reject before touching a device, and with
// size queries it must answer without one. Exits 0 when every status is the
// expected one; any sanitizer report aborts the run.
#include <stdint.h>
#include <stdio.h>

#include "hga.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: got %d, want %d\n", what, got, want);
    ++failures;
  }
}

int main() {
  // never dereferenced: every call below is rejected first
  void* fake = reinterpret_cast<void*>(uintptr_t{1} << 20);
  void* mis = reinterpret_cast<void*>((uintptr_t{1} << 20) + 4);
  float* ff = static_cast<float*>(fake);
  int32_t* fi = static_cast<int32_t*>(fake);
  hga_shape s{1, 32, 4, 1, 65536, 128};
  size_t n = 0, nr = 0, na = 0;

  expect(hga_abi_version(), HGA_ABI_VERSION, "abi version");
  expect(hga_workspace_zero_bytes() == (size_t{4} << 20), 1, "zero bytes");
  for (int st = -10; st <= 1; ++st) expect(hga_status_str(st) != nullptr, 1, "status text");

  int64_t nc = 0, ng = 0;
  expect(hga_summary_counts(65536, 256, 32, &nc, &ng), HGA_OK, "counts");
  expect(nc == 256 && ng == 2048, 1, "count values");
  expect(hga_summary_counts(100, 48, 32, nullptr, nullptr), HGA_ERR_PARAM, "chunk % group");
  expect(hga_summary_counts(0, 64, 16, nullptr, nullptr), HGA_ERR_SHAPE, "T = 0");

  expect(hga_build_summaries(nullptr, 1, 1, 4, 65536, 128, 256, 32, ff, ff, nullptr),
         HGA_ERR_NULL, "build null K");
  expect(hga_build_summaries(fake, 7, 1, 4, 65536, 128, 256, 32, ff, ff, nullptr),
         HGA_ERR_DTYPE, "build dtype");
  expect(hga_build_summaries(fake, 1, 1, 4, 65536, 96, 256, 32, ff, ff, nullptr),
         HGA_ERR_SHAPE, "build D");
  expect(hga_build_summaries(mis, 1, 1, 4, 65536, 128, 256, 32, ff, ff, nullptr),
         HGA_ERR_LAYOUT, "build misaligned");
  expect(hga_update_summaries(fake, 1, 1, 4, 1024, 128, 256, 32, 5, 5, ff, ff, nullptr),
         HGA_ERR_PARAM, "update empty range");
  expect(hga_update_summaries_ex(fake, 1, nullptr, 1, 4, 1024, 128, 256, 32, 0, ff, ff, nullptr),
         HGA_ERR_PARAM, "update newest 0");

  expect(hga_route_workspace_size(&s, 256, 32, 32, 64, &nr), HGA_OK, "route ws");
  expect(hga_route(&s, nullptr, 1, ff, ff, 256, 32, 32, 64, 0.f, fi, fi, fake, nr, nullptr),
         HGA_ERR_NULL, "route null Q");
  expect(hga_route(&s, fake, 1, ff, ff, 256, 32, 32, 64, 0.f, fi, fi, fake, nr - 1, nullptr),
         HGA_ERR_WORKSPACE, "route workspace");
  expect(hga_route(&s, fake, 1, ff, ff, 256, 32, -1, 64, 0.f, fi, fi, fake, nr, nullptr),
         HGA_ERR_PARAM, "route k_chunk");
  // each size within its own bound, their products past 64 bits
  const int64_t huge = (int64_t{1} << 31) - 1;
  hga_shape over{huge, huge, huge, 1, huge, 128};
  expect(hga_attend_workspace_size(&over, 32, 64, &n), HGA_ERR_SHAPE, "attend product");
  expect(hga_route_workspace_size(&over, 256, 32, 32, 64, &n), HGA_ERR_SHAPE, "route product");
  expect(hga_build_summaries(fake, 1, huge, huge, huge, 128, 256, 32, ff, ff, nullptr),
         HGA_ERR_SHAPE, "build product");
  hga_shape big = s;
  big.seq_len = int64_t{1} << 21;
  expect(hga_route_workspace_size(&big, 256, 32, 32, 64, &n), HGA_ERR_UNSUPPORTED, "route big");

  expect(hga_attend_workspace_size(&s, 32, 64, &na), HGA_OK, "attend ws");
  expect(hga_attend(&s, fake, nullptr, fake, 1, fi, 64, 32, 0.f, fake, nullptr, fake, na,
                    nullptr),
         HGA_ERR_NULL, "attend null K");
  expect(hga_attend(&s, fake, fake, fake, 1, fi, 64, 32, 0.f, mis, nullptr, fake, na, nullptr),
         HGA_ERR_LAYOUT, "attend misaligned O");

  hga_kv_layout bad_kind{7, 64, 128, 10, fi, nullptr};
  hga_kv_layout no_table{1, 64, 128, 10, nullptr, nullptr};
  expect(hga_build_summaries_ex(fake, 1, &bad_kind, 4, 2, 8192, 128, 256, 32, ff, ff, nullptr),
         HGA_ERR_PARAM, "layout kind");
  expect(hga_build_summaries_ex(fake, 1, &no_table, 4, 2, 8192, 128, 256, 32, ff, ff, nullptr),
         HGA_ERR_NULL, "layout table");

  expect(hga_decode_step_workspace_size(&s, 256, 32, 32, 64, &n), HGA_OK, "decode ws");
  expect(hga_decode_step_ex(&s, nullptr, fake, fake, fake, 1, ff, ff, 256, 32, 32, 64, 0.f, fi,
                            fi, fake, nullptr, fake, n - 1, nullptr),
         HGA_ERR_WORKSPACE, "decode workspace");
  expect(hga_decode_step_ex(&s, nullptr, fake, fake, fake, 9, ff, ff, 256, 32, 32, 64, 0.f, fi,
                            fi, fake, nullptr, fake, n, nullptr),
         HGA_ERR_DTYPE, "decode dtype");
  int32_t one = -1;
  expect(hga_decode_step_one_launch_cus(&s, 1, 256, 32, 32, 64, 256, &one), HGA_OK, "plan 256");
  expect(one, 1, "one launch on 256 CUs");
  expect(hga_decode_step_one_launch_cus(&s, 1, 256, 32, 32, 64, 31, &one), HGA_OK, "plan 31");
  expect(one, 0, "two launches on 31 CUs");
  expect(hga_decode_step_one_launch_cus(&s, 1, 256, 32, 32, 64, -1, &one), HGA_ERR_PARAM,
         "plan negative CUs");

  int64_t pages = 0;
  hga_shape h{4, 32, 4, 1, 262144, 128};
  expect(hga_attend_staged_sizes(&h, 32, 256, &pages, &n), HGA_OK, "staged sizes");
  expect(hga_attend_staged(&h, fake, fake, fake, 1, fi, 256, 32, 0.f, fake, nullptr, fake, fake,
                           pages - 1, fake, n, nullptr),
         HGA_ERR_PARAM, "staged pool");

  expect(hga_workspace_check(nullptr, size_t{4} << 20, nullptr), HGA_ERR_NULL, "check null");
  expect(hga_workspace_reset(fake, (size_t{4} << 20) - 1, nullptr), HGA_ERR_WORKSPACE,
         "reset small");
  hga_shape b43{43, 32, 4, 1, 65536, 128};
  expect(hga_decode_step_noalloc(&b43, nullptr, fake, fake, fake, 1, ff, ff, 256, 32, 32, 64,
                                 0.f, fi, fi, fake, nullptr, 0, nullptr),
         HGA_ERR_WORKSPACE, "noalloc too big");
  expect(hga_decode_step_noalloc(nullptr, nullptr, fake, fake, fake, 1, ff, ff, 256, 32, 32, 64,
                                 0.f, fi, fi, fake, nullptr, 0, nullptr),
         HGA_ERR_NULL, "noalloc null shape");

  if (failures == 0) printf("abi_errors: all checks passed\n");
  return failures == 0 ? 0 : 1;
}
