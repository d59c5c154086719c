/* A plain C caller of libfa.so: includes only include/fa.h, links the library and the HIP runtime,
 * and checks that malformed calls return the documented status before any device work (so it runs
 * without a GPU).  Built and run by tests/test_c_caller.py.  Exit status 0 means every check held. */
#include <math.h>
#include <stdio.h>
#include <stdint.h>

#include "fa.h"

static int failures = 0;

static void expect(const char* what, fa_status got, fa_status want) {
  if (got != want) {
    fprintf(stderr, "%s: got %d (%s), want %d\n", what, (int)got, fa_status_str(got), (int)want);
    ++failures;
  }
}

int main(void) {
  /* Stand-in device addresses: 256-byte aligned, never dereferenced (the checks fail first). */
  void* p = (void*)(uintptr_t)0x100000;
  float* f = (float*)p;
  void* mis = (void*)(uintptr_t)0x100008;

  expect("fa_fwd NULL q", fa_fwd(NULL, p, p, p, f, 1, 1, 64, 128, 1, 0.088f, NULL), FA_ERR_NULL);
  expect("fa_fwd B = 0", fa_fwd(p, p, p, p, f, 0, 1, 64, 128, 1, 0.088f, NULL), FA_ERR_SHAPE);
  expect("fa_fwd d = 80", fa_fwd(p, p, p, p, f, 1, 1, 64, 80, 1, 0.088f, NULL), FA_ERR_UNSUPPORTED);
  expect("fa_fwd scale nan", fa_fwd(p, p, p, p, f, 1, 1, 64, 128, 1, NAN, NULL), FA_ERR_UNSUPPORTED);
  expect("fa_fwd misaligned o", fa_fwd(p, p, p, mis, f, 1, 1, 64, 128, 1, 0.088f, NULL),
         FA_ERR_ALIGN);
  expect("fa_fwd_fp8 d = 512",
         fa_fwd_fp8(p, p, p, 1.f, 1.f, 1.f, p, f, 1, 1, 64, 512, 1, 0.0625f, NULL),
         FA_ERR_UNSUPPORTED);

  const size_t ws = fa_bwd_workspace_bytes(2, 3, 100, 128);
  if (ws != 2u * 3u * 100u * 4u + 256u - (2u * 3u * 100u * 4u) % 256u) {
    fprintf(stderr, "fa_bwd_workspace_bytes: %zu\n", ws);
    ++failures;
  }
  expect("fa_bwd workspace too small",
         fa_bwd(p, p, p, p, f, p, p, p, p, p, ws - 1, 2, 3, 100, 128, 1, 0.088f, NULL),
         FA_ERR_WORKSPACE);
  expect("fa_bwd_fp8 v_descale 0",
         fa_bwd_fp8(p, p, p, 1.f, 1.f, 0.f, p, f, p, p, p, p, p,
                    fa_bwd_fp8_workspace_bytes(1, 1, 64, 128), 1, 1, 64, 128, 1, 0.088f, NULL),
         FA_ERR_UNSUPPORTED);
  expect("fa_decode Nq = 33",
         fa_decode(p, p, p, p, f, p, (size_t)1 << 30, 1, 1, 33, 64, 128, 1, 0.088f, NULL),
         FA_ERR_SHAPE);
  if (fa_decode_workspace_bytes(1, 1, 1, 8, 80) != 0) {
    fprintf(stderr, "fa_decode_workspace_bytes accepted d = 80\n");
    ++failures;
  }
  const size_t fsplit = fa_fwd_split_workspace_bytes(1, 1, 16384, 128, 1);
  if (fsplit == 0 || fa_fwd_split_workspace_bytes(4, 32, 4096, 128, 1) != 0) {
    fprintf(stderr, "fa_fwd_split_workspace_bytes: %zu\n", fsplit);
    ++failures;
  }
  expect("fa_fwd_split workspace too small",
         fa_fwd_split(p, p, p, p, f, p, fsplit - 1, 1, 1, 16384, 128, 1, 0.088f, NULL),
         FA_ERR_WORKSPACE);
  expect("fa_fwd_fp8_split workspace NULL",
         fa_fwd_fp8_split(p, p, p, 1.f, 1.f, 1.f, p, f, NULL, 0, 1, 1, 16384, 128, 1, 0.088f, NULL),
         FA_ERR_WORKSPACE);
  const size_t bsplit = fa_bwd_split_workspace_bytes(1, 1, 16384, 128, 1);
  if (bsplit <= fa_bwd_workspace_bytes(1, 1, 16384, 128)) {
    fprintf(stderr, "fa_bwd_split_workspace_bytes: %zu\n", bsplit);
    ++failures;
  }
  expect("fa_bwd_split workspace too small",
         fa_bwd_split(p, p, p, p, f, p, p, p, p, p, bsplit - 1, 1, 1, 16384, 128, 1, 0.088f, NULL),
         FA_ERR_WORKSPACE);
  int cus = 0;
  expect("fa_device_info NULL clock", fa_device_info(0, &cus, NULL), FA_ERR_NULL);

  if (failures == 0) printf("abi_check: all checks passed\n");
  return failures == 0 ? 0 : 1;
}
