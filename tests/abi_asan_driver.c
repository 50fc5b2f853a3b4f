/*
 * Host-side driver for the sanitizer build of the library (AddressSanitizer +
 * UndefinedBehaviorSanitizer on the host code; no device code is built).
 *
 * It calls every entry point of include/bsgemm.h through its validation
 * paths with fake, never-dereferenced pointers and checks the documented
 * status codes; it enumerates the W4A16 selector over a grid of shapes and
 * checks the per-thread error message.  Calls that would pass validation
 * are made only where no GPU is visible (they must then stop at the device
 * check).  Exit status 0 means every check passed and no sanitizer fired.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "bsgemm.h"

static int failures = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);   \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

#define P ((void*)0x10000)    /* fake, 16-byte aligned */
#define MIS ((void*)0x10004)  /* fake, misaligned */

static int run(int fmt, int64_t m, int64_t n, int64_t k, void* a, void* sa, void* ta, void* b, void* sb,
               void* tb, void* c) {
  return bsgemm_run(fmt, m, n, k, a, sa, ta, b, sb, tb, c, NULL);
}

static void* other_thread(void* out) {
  *(const char**)out = bsgemm_last_error();
  return NULL;
}

extern int bsgemm_no_gpu_visible(void);

int main(int argc, char** argv) {
  const int no_gpu = argc > 1 && strcmp(argv[1], "--no-gpu") == 0;
  int s;

  CHECK(strcmp(bsgemm_status_string(BSGEMM_OK), "BSGEMM_OK") == 0);
  CHECK(strcmp(bsgemm_status_string(99), "unknown status") == 0);
  CHECK(bsgemm_version() == 600);

  /* bsgemm_run */
  CHECK(run(BSGEMM_NVFP4, 64, 64, 64, NULL, P, P, P, P, P, P) == BSGEMM_ERR_INVALID_ARG);
  CHECK(strstr(bsgemm_last_error(), "a is NULL") != NULL);
  CHECK(run(BSGEMM_NVFP4, -1, 64, 64, P, P, P, P, P, P, P) == BSGEMM_ERR_INVALID_ARG);
  CHECK(run(BSGEMM_NVFP4, 64, 64, 64, P, P, NULL, P, P, P, P) == BSGEMM_ERR_INVALID_ARG);
  CHECK(run(BSGEMM_NVFP4, 64, 64, 48, P, P, P, P, P, P, P) == BSGEMM_ERR_UNSUPPORTED);
  CHECK(run(9, 64, 64, 64, P, P, P, P, P, P, P) == BSGEMM_ERR_UNSUPPORTED);
  CHECK(run(BSGEMM_MXFP8, 64, 64, 64, P, P, P, P, P, P, P) == BSGEMM_ERR_UNSUPPORTED);
  CHECK(run(BSGEMM_MXFP8_EXACT, 64, 64, 64, P, P, P, P, P, P, P) == BSGEMM_ERR_UNSUPPORTED);
  CHECK(run(BSGEMM_MXFP4, 64, 64, 64, P, P, NULL, P, MIS, NULL, P) == BSGEMM_ERR_BAD_ALIGNMENT);
  CHECK(run(BSGEMM_NVFP4, 64, 64, 64, P, P, P, P, P, P, MIS) == BSGEMM_ERR_BAD_ALIGNMENT);
  CHECK(run(BSGEMM_NVFP4, 64, 64, (int64_t)1 << 22, P, P, P, P, P, P, P) == BSGEMM_ERR_RESOURCE);
  CHECK(run(BSGEMM_NVFP4, 0, 64, 48, NULL, NULL, P, P, P, P, NULL) == BSGEMM_ERR_UNSUPPORTED);

  /* quantizers */
  CHECK(bsgemm_quantize_nvfp4(4, 64, NULL, P, P, P, NULL) == BSGEMM_ERR_INVALID_ARG);
  CHECK(bsgemm_quantize_nvfp4(4, 64, P, P, P, NULL, NULL) == BSGEMM_ERR_INVALID_ARG);
  CHECK(bsgemm_quantize_nvfp4(4, 40, P, P, P, P, NULL) == BSGEMM_ERR_UNSUPPORTED);
  CHECK(bsgemm_quantize_nvfp4(4, 64, MIS, P, P, P, NULL) == BSGEMM_ERR_BAD_ALIGNMENT);
  CHECK(bsgemm_quantize_mxfp8(-1, 64, P, P, P, NULL) == BSGEMM_ERR_INVALID_ARG);
  CHECK(bsgemm_quantize_mxfp8(4, 16, P, P, P, NULL) == BSGEMM_ERR_UNSUPPORTED);
  CHECK(bsgemm_quantize_mxfp4(4, 64, P, P, MIS, NULL) == BSGEMM_ERR_BAD_ALIGNMENT);
  CHECK(bsgemm_quantize_mxfp4(4, 64, P, NULL, P, NULL) == BSGEMM_ERR_INVALID_ARG);

  /* grouped */
  CHECK(bsgemm_grouped_run(0, 64, 64, 64, P, P, P, P, P, P, NULL) == BSGEMM_ERR_INVALID_ARG);
  CHECK(bsgemm_grouped_run(2, 64, 64, 64, P, P, P, NULL, P, P, NULL) == BSGEMM_ERR_INVALID_ARG);
  CHECK(bsgemm_grouped_run(2, 64, 64, 33, P, P, P, P, P, P, NULL) == BSGEMM_ERR_UNSUPPORTED);
  CHECK(bsgemm_grouped_run(2, 64, 64, 64, P, P, P, P, MIS, P, NULL) == BSGEMM_ERR_BAD_ALIGNMENT);
  CHECK(bsgemm_grouped_run_ex(2, 64, 64, 64, 32, P, P, P, P, BSGEMM_W_BF16, P, NULL, NULL, NULL, NULL, P, NULL) ==
        BSGEMM_ERR_INVALID_ARG);
  CHECK(strstr(bsgemm_last_error(), "a_rows must equal m_total") != NULL);
  CHECK(bsgemm_grouped_run_ex(2, 64, 64, 64, 64, P, P, P, P, 7, P, NULL, NULL, NULL, NULL, P, NULL) ==
        BSGEMM_ERR_UNSUPPORTED);
  CHECK(bsgemm_grouped_run_ex(2, 64, 64, 64, 64, P, P, P, P, BSGEMM_W_F16, P, NULL, (void*)0x10002, NULL, NULL, P,
                              NULL) == BSGEMM_ERR_BAD_ALIGNMENT);
  CHECK(bsgemm_grouped_run_ex(2, 64, 64, 1024, (int64_t)1 << 26, P, P, P, P, BSGEMM_W_BF16, P, NULL, NULL, P, NULL,
                              P, NULL) == BSGEMM_ERR_RESOURCE);
  CHECK(bsgemm_grouped_kragged_run(2, 64, 64, 384, P, P, P, P, BSGEMM_W_BF16, P, P, NULL) == BSGEMM_ERR_UNSUPPORTED);
  CHECK(bsgemm_grouped_kragged_run(2, 64, 64, 512, P, P, P, (void*)0x10002, BSGEMM_W_BF16, P, P, NULL) ==
        BSGEMM_ERR_BAD_ALIGNMENT);
  CHECK(bsgemm_grouped_kragged_run(0, 64, 64, 512, P, P, P, P, BSGEMM_W_BF16, P, P, NULL) == BSGEMM_ERR_INVALID_ARG);

  /* W4A16: configurations, selector, forced path */
  const int ncfg = bsgemm_w4a16_num_configs();
  CHECK(ncfg == 34);
  for (int i = 0; i < ncfg; ++i) CHECK(bsgemm_w4a16_config_name(i) != NULL);
  CHECK(bsgemm_w4a16_config_name(ncfg) == NULL && bsgemm_w4a16_config_name(-1) == NULL);
  {
    const int64_t ns[] = {1, 64, 896, 1536, 4096, 4112, 14336, 65536, (int64_t)1 << 30};
    const int64_t ks[] = {32, 4096, 7168, 14336, (int64_t)1 << 21};
    long decisions = 0;
    for (unsigned a = 0; a < sizeof ns / sizeof ns[0]; ++a)
      for (unsigned b = 0; b < sizeof ks / sizeof ks[0]; ++b)
        for (int64_t m = 0; m < 300; ++m) {
          const int c = bsgemm_w4a16_select(m, ns[a], ks[b]);
          CHECK(c >= 0 && c < ncfg);
          ++decisions;
        }
    CHECK(decisions == 9 * 5 * 300);
    CHECK(bsgemm_w4a16_select(1 << 30, (int64_t)1 << 31, 4096) >= 0);
  }
  CHECK(bsgemm_w4a16_select(4, 64, 48) == -1 && bsgemm_w4a16_select(-1, 64, 64) == -1);
  CHECK(bsgemm_w4a16_run(1, 64, 64, NULL, P, P, P, P, NULL) == BSGEMM_ERR_INVALID_ARG);
  CHECK(bsgemm_w4a16_run(1, 64, 80, P, P, P, P, P, NULL) == BSGEMM_ERR_UNSUPPORTED);
  CHECK(bsgemm_w4a16_run(1, 64, 64, MIS, P, P, P, P, NULL) == BSGEMM_ERR_BAD_ALIGNMENT);
  CHECK(bsgemm_w4a16_run_config(99, 1, 64, 64, P, P, P, P, P, NULL) == BSGEMM_ERR_UNSUPPORTED);
  CHECK(bsgemm_w4a16_run_config(0, 70000, 64, 64, P, P, P, P, P, NULL) == BSGEMM_ERR_RESOURCE);
  CHECK(bsgemm_w4a16_run_config(33, 256, 64, 96, P, P, P, P, P, NULL) == BSGEMM_ERR_UNSUPPORTED);

  /* the error message is per thread */
  CHECK(run(BSGEMM_NVFP4, 64, 64, 64, NULL, P, P, P, P, P, P) == BSGEMM_ERR_INVALID_ARG);
  {
    const char* seen = "unset";
    pthread_t t;
    pthread_create(&t, NULL, other_thread, (void*)&seen);
    pthread_join(t, NULL);
    CHECK(seen != NULL && seen[0] == '\0');
    CHECK(strstr(bsgemm_last_error(), "a is NULL") != NULL);
  }

  /* calls that pass validation stop at the device check when no GPU is visible */
  if (no_gpu) {
    CHECK(run(BSGEMM_NVFP4, 64, 64, 64, P, P, P, P, P, P, P) == BSGEMM_ERR_DEVICE);
    CHECK(run(BSGEMM_MXFP8_EXACT, 64, 64, 64, P, P, NULL, P, P, NULL, P) == BSGEMM_ERR_DEVICE);
    CHECK(bsgemm_quantize_mxfp8(4, 64, P, P, P, NULL) == BSGEMM_ERR_DEVICE);
    CHECK(bsgemm_w4a16_run(1, 64, 64, P, P, P, P, P, NULL) == BSGEMM_ERR_DEVICE);
    s = bsgemm_grouped_run_ex(2, 64, 64, 64, 32, P, P, P, P, BSGEMM_W_F16, P, P, P, P, P, P, NULL);
    CHECK(s == BSGEMM_ERR_DEVICE);
  }
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("abi sanitizer driver: all checks passed\n");
  return 0;
}
