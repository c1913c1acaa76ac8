/* A plain C99 caller of the attention library's C ABI (include/fa.h).
 *
 * Built and run by the CPU test suite: it checks that the header is valid C
 * (no C++ constructs outside the extern "C" guard) and that the exported
 * functions can be called from C with the documented error behaviour.  Only
 * calls that fail argument validation, and the pure queries, are made: the
 * library checks every argument before any HIP call, so nothing here needs a
 * GPU.  Prints one line per check and exits non-zero on the first failure. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fa.h"

static int failures = 0;

static void expect(const char* what, fa_status got, fa_status want) {
  const int ok = got == want;
  printf("%s %s: got %s, want %s\n", ok ? "ok  " : "FAIL", what, fa_status_string(got),
         fa_status_string(want));
  if (!ok) ++failures;
}

int main(void) {
  /* Stand-in device addresses: 256-byte aligned, never dereferenced. */
  void* p = (void*)(uintptr_t)0x10000;
  float* pf = (float*)(uintptr_t)0x20000;
  void* odd = (void*)(uintptr_t)0x10002;
  const size_t bws = fa_bwd_workspace_bytes(2, 3, 100, 64);
  const size_t dws = fa_decode_workspace_bytes(2, 3, 128, 4);
  fa_status s;

  printf("version %s\n", fa_version());
  for (s = FA_OK; s <= FA_ERR_SCRATCH; s = (fa_status)(s + 1))
    if (fa_status_string(s) == NULL || strlen(fa_status_string(s)) == 0) {
      printf("FAIL status string %d\n", (int)s);
      ++failures;
    }
  if (bws == 0 || dws == 0) {
    printf("FAIL workspace sizes %zu %zu\n", bws, dws);
    ++failures;
  }

  expect("fwd null q", fa_fwd(NULL, p, p, p, pf, 1, 1, 16, 64, 0.125f, 1, FA_BF16, NULL),
         FA_ERR_NULL);
  expect("fwd d=96", fa_fwd(p, p, p, p, pf, 1, 1, 16, 96, 0.125f, 1, FA_BF16, NULL),
         FA_ERR_UNSUPPORTED);
  expect("fwd N=0", fa_fwd(p, p, p, p, pf, 1, 1, 0, 64, 0.125f, 0, FA_F16, NULL), FA_ERR_SHAPE);
  expect("fwd bad dtype", fa_fwd(p, p, p, p, pf, 1, 1, 16, 64, 0.125f, 0, (fa_dtype)7, NULL),
         FA_ERR_DTYPE);
  expect("fwd misaligned o", fa_fwd(p, p, p, odd, pf, 1, 1, 16, 64, 0.125f, 0, FA_F16, NULL),
         FA_ERR_ALIGN);
  expect("bwd small workspace",
         fa_bwd(p, p, p, p, pf, p, p, p, p, p, bws - 1, 2, 3, 100, 64, 0.125f, 1, FA_BF16, NULL),
         FA_ERR_WORKSPACE);
  expect("decode zero splits",
         fa_decode(p, p, p, p, pf, 2, 3, 50, 128, 0.1f, 0, p, dws, FA_BF16, NULL), FA_ERR_SPLITS);
  expect("decode too many splits",
         fa_decode(p, p, p, p, pf, 2, 3, 50, 128, 0.1f, FA_MAX_SPLITS + 1, p, dws, FA_BF16, NULL),
         FA_ERR_SPLITS);
  expect("fwd_ex heads not a multiple",
         fa_fwd_ex(p, p, p, p, pf, 1, 6, 4, 16, 64, 0.125f, 1, 0, FA_BF16, NULL), FA_ERR_SHAPE);
  expect("fwd_ex window without causal",
         fa_fwd_ex(p, p, p, p, pf, 1, 4, 2, 16, 64, 0.125f, 0, 8, FA_BF16, NULL),
         FA_ERR_UNSUPPORTED);
  expect("decode_varlen null lengths",
         fa_decode_varlen(p, p, p, NULL, p, pf, 2, 4, 2, 50, 128, 0.1f, 4,
                          p, fa_decode_workspace_bytes(2, 4, 128, 4), FA_BF16, NULL),
         FA_ERR_NULL);
  expect("decode_noalloc beyond the static scratch",
         fa_decode_noalloc(p, p, p, p, pf, 64, 64, 64, 50, 128, 0.1f, 32, FA_BF16, NULL),
         FA_ERR_SCRATCH);
  expect("decode_noalloc null q",
         fa_decode_noalloc(NULL, p, p, p, pf, 2, 4, 2, 50, 128, 0.1f, 4, FA_BF16, NULL),
         FA_ERR_NULL);
  printf("%d failure(s)\n", failures);
  return failures != 0;
}
