/* Host-side driver for the sanitizer build of the C ABI layer: every argument check, overflow
 * guard and NULL-handle path of include/vda.h that returns before any kernel is enqueued.  It
 * runs on a host with or without a GPU (with none, creating a valid plan fails with
 * VDA_ERROR_DEVICE, which exercises the plan's clean-up path).  Exit status 0 when every
 * call returned what the header documents. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "vda.h"

static int failures = 0;

static void expect(const char* what, vda_status got, vda_status want) {
  if (got != want) {
    fprintf(stderr, "%s: got %s, want %s\n", what, vda_status_string(got), vda_status_string(want));
    ++failures;
  }
}

static void create_case(const char* what, int64_t B, int64_t H, int64_t F, int64_t n, int64_t d, int64_t dv,
                        int64_t T, float lam, int dtype, vda_status want) {
  vda_plan_t plan = (vda_plan_t)(uintptr_t)0x1234;
  expect(what, vda_plan_create(B, H, F, n, d, dv, T, lam, (vda_dtype)dtype, &plan), want);
  if (plan != NULL) {
    fprintf(stderr, "%s: plan_out not cleared\n", what);
    ++failures;
  }
  /* the same shape through the entry point with no plan: the same checks, before any device call */
  vda_status nb = vda_forward_noalloc(B, H, F, n, d, dv, T, lam, (vda_dtype)dtype, NULL, NULL, NULL, NULL, NULL,
                                      NULL, NULL);
  expect(what, nb, want);
}

int main(void) {
  const int64_t big = (int64_t)1 << 40;
  create_case("d not supported", 1, 1, 1, 1, 48, 32, 0, 1.0f, 1, VDA_ERROR_NOT_SUPPORTED);
  create_case("dv not supported", 1, 1, 1, 1, 32, 256, 0, 1.0f, 1, VDA_ERROR_NOT_SUPPORTED);
  create_case("dtype", 1, 1, 1, 1, 32, 32, 0, 1.0f, 7, VDA_ERROR_NOT_SUPPORTED);
  create_case("negative B", -1, 1, 1, 1, 32, 32, 0, 1.0f, 1, VDA_ERROR_INVALID_VALUE);
  create_case("negative F", 1, 1, -2, 1, 32, 32, 0, 1.0f, 1, VDA_ERROR_INVALID_VALUE);
  create_case("negative T", 1, 1, 1, 1, 32, 32, -1, 1.0f, 1, VDA_ERROR_INVALID_VALUE);
  create_case("lambda 0", 1, 1, 1, 1, 32, 32, 0, 0.0f, 1, VDA_ERROR_INVALID_VALUE);
  create_case("lambda < 0", 1, 1, 1, 1, 32, 32, 0, -1.0f, 1, VDA_ERROR_INVALID_VALUE);
  create_case("lambda nan", 1, 1, 1, 1, 32, 32, 0, NAN, 1, VDA_ERROR_INVALID_VALUE);
  create_case("lambda inf", 1, 1, 1, 1, 32, 32, 0, INFINITY, 1, VDA_ERROR_INVALID_VALUE);
  create_case("B*H overflow", big, big, 1, 1, 32, 32, 0, 1.0f, 1, VDA_ERROR_INVALID_VALUE);
  create_case("B*H*(F+1) overflow", 1, big, big, 1, 32, 32, 0, 1.0f, 1, VDA_ERROR_INVALID_VALUE);
  create_case("F + 1 at the int64 limit", 1, 1, INT64_MAX, 1, 32, 32, 0, 1.0f, 1, VDA_ERROR_INVALID_VALUE);
  create_case("tokens overflow", 1, 1, (int64_t)1 << 40, (int64_t)1 << 23, 32, 32, 0, 1.0f, 1,
              VDA_ERROR_INVALID_VALUE);
  create_case("tokens * 128 overflow", 1, 1, (int64_t)1 << 36, (int64_t)1 << 23, 32, 32, 0, 1.0f, 1,
              VDA_ERROR_INVALID_VALUE);
  create_case("workspace frames above 2^30", 1, 1, ((int64_t)1 << 30), 1, 32, 32, 0, 1.0f, 1,
              VDA_ERROR_INVALID_VALUE);
  create_case("text tokens overflow", big, 1, 1, 1, 32, 32, (int64_t)1 << 23, 1.0f, 1, VDA_ERROR_INVALID_VALUE);
  create_case("frame too long", 1, 1, 1, (int64_t)1 << 24, 32, 32, 0, 1.0f, 1, VDA_ERROR_NOT_SUPPORTED);
  create_case("text too long", 1, 1, 1, 1, 32, 32, (int64_t)1 << 24, 1.0f, 1, VDA_ERROR_NOT_SUPPORTED);

  /* the entry point with no plan: a workspace above its fixed scratch, before any device call */
  expect("noalloc too large", vda_forward_noalloc(1, 4, 90, 4032, 128, 128, 256, 1.0f, VDA_DTYPE_BF16, NULL, NULL,
                                                  NULL, NULL, NULL, NULL, NULL),
         VDA_ERROR_TOO_LARGE);
  expect("noalloc empty", vda_forward_noalloc(1, 4, 0, 4032, 128, 128, 256, 1.0f, VDA_DTYPE_BF16, NULL, NULL, NULL,
                                              NULL, NULL, NULL, NULL),
         VDA_SUCCESS);

  /* NULL handles and out-pointers */
  expect("create NULL out", vda_plan_create(1, 1, 1, 1, 32, 32, 0, 1.0f, VDA_DTYPE_BF16, NULL),
         VDA_ERROR_INVALID_VALUE);
  expect("destroy NULL", vda_plan_destroy(NULL), VDA_SUCCESS);
  if (vda_plan_workspace_bytes(NULL) != 0) {
    fprintf(stderr, "workspace bytes of NULL\n");
    ++failures;
  }
  expect("forward NULL", vda_forward(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL), VDA_ERROR_INVALID_VALUE);
  expect("stages NULL", vda_forward_stages(NULL, 7, NULL, NULL, NULL, NULL, NULL, NULL, NULL),
         VDA_ERROR_INVALID_VALUE);
  expect("gated NULL", vda_forward_gated(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL),
         VDA_ERROR_INVALID_VALUE);
  expect("backward NULL", vda_backward(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL),
         VDA_ERROR_INVALID_VALUE);
  const void* p = NULL;
  expect("debug NULL", vda_debug_workspace(NULL, &p, NULL, NULL, NULL), VDA_ERROR_INVALID_VALUE);
  expect("timing NULL", vda_plan_enable_timing(NULL, 4), VDA_ERROR_INVALID_VALUE);
  int calls = 0;
  expect("timings NULL", vda_plan_timings(NULL, &calls, NULL, NULL, NULL), VDA_ERROR_INVALID_VALUE);
  expect("set chunk NULL", vda_plan_set_scan_chunk(NULL, 8), VDA_ERROR_INVALID_VALUE);
  expect("timed stages NULL", vda_plan_set_timed_stages(NULL, 4), VDA_ERROR_INVALID_VALUE);
  int64_t chunk = 0;
  expect("get chunk NULL", vda_plan_get_scan_chunk(NULL, &chunk), VDA_ERROR_INVALID_VALUE);

  /* status strings, including an unknown code */
  for (int s = 0; s <= 6; ++s)
    if (strncmp(vda_status_string((vda_status)s), "VDA_", 4) != 0) {
      fprintf(stderr, "status string %d\n", s);
      ++failures;
    }
  if (strcmp(vda_status_string((vda_status)99), "VDA_ERROR_UNKNOWN") != 0) {
    fprintf(stderr, "unknown status string\n");
    ++failures;
  }

  /* a valid shape: SUCCESS with a GPU, DEVICE without one; either way the plan is released */
  vda_plan_t plan = NULL;
  const vda_status st = vda_plan_create(1, 2, 3, 64, 32, 32, 4, 1.0f, VDA_DTYPE_BF16, &plan);
  if (st == VDA_SUCCESS) {
    expect("destroy", vda_plan_destroy(plan), VDA_SUCCESS);
  } else if (st != VDA_ERROR_DEVICE || plan != NULL) {
    fprintf(stderr, "valid plan: %s\n", vda_status_string(st));
    ++failures;
  }
  printf("abi_sanitize: %d failure(s)\n", failures);
  return failures == 0 ? 0 : 1;
}
