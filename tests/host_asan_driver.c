/* Host-side driver for the ASan build of libmscl (test infrastructure).
 * Exercises every C-ABI path that needs no GPU: argument validation for
 * every rank count (fake, never dereferenced device addresses), the
 * selector, error strings, and the channel calls on unknown handles.
 * Exit status 0 when every call returned the expected status. */
#include <stdint.h>
#include <stdio.h>

#include "mscl.h"

static int failures = 0;

static void expect(const char* what, mscl_status_t got, mscl_status_t want) {
  if (got != want) {
    fprintf(stderr, "%s: got %d (%s), want %d\n", what, got, mscl_last_error_string(), want);
    ++failures;
  }
}

#define FAKE(base, i) ((void*)(uintptr_t)((base) + (uintptr_t)(i) * 0x100000u))

int main(void) {
  const void* in[MSCL_MAX_RANKS];
  void* out[MSCL_MAX_RANKS];
  for (int s = -2; s < 12; ++s) (void)mscl_status_string(s);
  for (int R = 1; R <= MSCL_MAX_RANKS; ++R) {
    for (int r = 0; r < R; ++r) {
      in[r] = FAKE(0x10000000u, r);
      out[r] = FAKE(0x40000000u, r);
    }
    expect("count 0", mscl_allreduce(in, out, 0, MSCL_BFLOAT16, R, MSCL_ALGO_AUTO, 0), MSCL_SUCCESS);
    expect("bad dtype", mscl_allreduce(in, out, 64, (mscl_dtype_t)7, R, MSCL_ALGO_AUTO, 0), MSCL_ERR_INVALID_ARGUMENT);
    expect("bad algo", mscl_allreduce(in, out, 64, MSCL_FLOAT32, R, (mscl_algo_t)9, 0), MSCL_ERR_INVALID_ARGUMENT);
    expect("overflow", mscl_allreduce(in, out, SIZE_MAX / 2, MSCL_FLOAT32, R, MSCL_ALGO_AUTO, 0),
           MSCL_ERR_INVALID_ARGUMENT);
    void* saved = out[R - 1];
    out[R - 1] = (void*)((uintptr_t)saved + 4);
    expect("misaligned", mscl_allreduce(in, out, 64, MSCL_FLOAT32, R, MSCL_ALGO_AUTO, 0), MSCL_ERR_MISALIGNED);
    out[R - 1] = saved;
    if (R > 1) {
      saved = out[0];
      out[0] = (void*)in[R - 1];
      expect("output on another input", mscl_allreduce(in, out, 64, MSCL_FLOAT32, R, MSCL_ALGO_AUTO, 0),
             MSCL_ERR_INVALID_ARGUMENT);
      out[0] = out[1];
      expect("outputs overlap", mscl_allreduce(in, out, 64, MSCL_FLOAT32, R, MSCL_ALGO_AUTO, 0),
             MSCL_ERR_INVALID_ARGUMENT);
      out[0] = saved;
      expect("rs overlap", mscl_reduce_scatter(in, (void* const*)in, 64, MSCL_FLOAT32, R, 0),
             MSCL_ERR_INVALID_ARGUMENT);
      expect("ag overlap", mscl_allgather((const void* const*)out, out, 64, MSCL_FLOAT32, R, 0),
             MSCL_ERR_INVALID_ARGUMENT);
    }
    expect("rs count 0", mscl_reduce_scatter(in, out, 0, MSCL_FLOAT16, R, 0), MSCL_SUCCESS);
    expect("ag count 0", mscl_allgather(in, out, 0, MSCL_FLOAT16, R, 0), MSCL_SUCCESS);
    for (int k = 0; k < 40; ++k) {
      mscl_algo_t a;
      expect("select", mscl_select_algo((size_t)1 << k, MSCL_BFLOAT16, R, &a), MSCL_SUCCESS);
    }
  }
  expect("R 0", mscl_allreduce(in, out, 64, MSCL_FLOAT32, 0, MSCL_ALGO_AUTO, 0), MSCL_ERR_INVALID_ARGUMENT);
  expect("R 17", mscl_allreduce(in, out, 64, MSCL_FLOAT32, 17, MSCL_ALGO_AUTO, 0), MSCL_ERR_INVALID_ARGUMENT);
  expect("null arrays", mscl_allreduce(NULL, NULL, 64, MSCL_FLOAT32, 2, MSCL_ALGO_AUTO, 0), MSCL_ERR_INVALID_ARGUMENT);
  mscl_channel_t bogus = (mscl_channel_t)(uintptr_t)0x1234;
  uint64_t mism = 0;
  mscl_plan_t plan;
  expect("destroy", mscl_channel_destroy(bogus), MSCL_ERR_INVALID_ARGUMENT);
  expect("check", mscl_channel_check(bogus), MSCL_ERR_INVALID_ARGUMENT);
  expect("reset", mscl_channel_reset(bogus), MSCL_ERR_INVALID_ARGUMENT);
  expect("plan", mscl_channel_plan(bogus, 10, MSCL_FLOAT32, MSCL_ALGO_AUTO, 0, &plan), MSCL_ERR_INVALID_ARGUMENT);
  expect("faults", mscl_channel_set_fault_controls(bogus, 0, -1), MSCL_ERR_INVALID_ARGUMENT);
  expect("checks", mscl_channel_set_checks(bogus, 1, -1), MSCL_ERR_INVALID_ARGUMENT);
  expect("checks null", mscl_channel_set_checks(NULL, 0, -1), MSCL_ERR_INVALID_ARGUMENT);
  expect("selftest", mscl_channel_selftest(bogus, 1, &mism), MSCL_ERR_INVALID_ARGUMENT);
  mscl_channel_t h;
  expect("create R 0", mscl_channel_create(0, 0, &h), MSCL_ERR_INVALID_ARGUMENT);
  expect("create null", mscl_channel_create(2, 0, NULL), MSCL_ERR_INVALID_ARGUMENT);
  printf("%d failures, version %d\n", failures, mscl_version());
  return failures ? 1 : 0;
}
