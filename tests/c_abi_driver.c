/* A plain-C consumer of the library's C ABI: no Python, no torch, only the
 * HIP runtime for device memory and a stream.
 *
 *   c_abi_driver --version
 *       prints mscl_version() (no GPU needed)
 *   c_abi_driver R DTYPE COUNT ALGO IN_FILE OUT_FILE [inplace]
 *       reads R buffers of COUNT elements (raw, rank after rank) from
 *       IN_FILE, runs mscl_allreduce on device copies (three times in a row
 *       out of place, once in place) on a stream of its own, and writes the
 *       R outputs (raw, rank after rank) to OUT_FILE.
 *
 * Exit status: 0 success, 1 usage or file error, 2 HIP error, 3 library
 * error (the status and mscl_last_error_string() are printed).
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../include/mscl.h"

#define HIP_OK(call)                                                          \
  do {                                                                        \
    hipError_t e_ = (call);                                                   \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));             \
      return 2;                                                               \
    }                                                                         \
  } while (0)

#define MSCL_OK(call)                                                         \
  do {                                                                        \
    mscl_status_t s_ = (call);                                                \
    if (s_ != MSCL_SUCCESS) {                                                 \
      fprintf(stderr, "%s: %s (%s)\n", #call, mscl_status_string(s_),         \
              mscl_last_error_string());                                      \
      return 3;                                                               \
    }                                                                         \
  } while (0)

static int run(int R, int dtype, size_t count, int algo, const char* in_path, const char* out_path, int in_place) {
  const size_t esz = dtype == MSCL_FLOAT32 ? 4 : 2;
  const size_t bytes = count * esz;
  unsigned char* host = (unsigned char*)malloc(bytes * (size_t)R + 1);
  if (!host) return 1;
  FILE* f = fopen(in_path, "rb");
  if (!f || fread(host, 1, bytes * (size_t)R, f) != bytes * (size_t)R) {
    fprintf(stderr, "cannot read %zu bytes from %s\n", bytes * (size_t)R, in_path);
    if (f) fclose(f);
    free(host);
    return 1;
  }
  fclose(f);

  void* in[MSCL_MAX_RANKS] = {0};
  void* out[MSCL_MAX_RANKS] = {0};
  hipStream_t stream;
  HIP_OK(hipSetDevice(0));
  HIP_OK(hipStreamCreate(&stream));
  for (int r = 0; r < R; ++r) {
    HIP_OK(hipMalloc(&in[r], bytes ? bytes : 16));
    HIP_OK(hipMemcpy(in[r], host + (size_t)r * bytes, bytes, hipMemcpyHostToDevice));
    if (in_place) {
      out[r] = in[r];
    } else {
      HIP_OK(hipMalloc(&out[r], bytes ? bytes : 16));
      HIP_OK(hipMemset(out[r], 0xA5, bytes));
    }
  }

  mscl_channel_t ch;
  MSCL_OK(mscl_channel_create(R, 0, &ch));
  mscl_plan_t plan;
  MSCL_OK(mscl_channel_plan(ch, count, (mscl_dtype_t)dtype, (mscl_algo_t)algo, in_place, &plan));
  const int reps = in_place ? 1 : 3;
  for (int i = 0; i < reps; ++i)
    MSCL_OK(mscl_allreduce((const void* const*)in, (void* const*)out, count, (mscl_dtype_t)dtype, R,
                           (mscl_algo_t)algo, (void*)stream));
  HIP_OK(hipStreamSynchronize(stream));
  MSCL_OK(mscl_channel_check(ch));

  for (int r = 0; r < R; ++r) HIP_OK(hipMemcpy(host + (size_t)r * bytes, out[r], bytes, hipMemcpyDeviceToHost));
  f = fopen(out_path, "wb");
  if (!f || fwrite(host, 1, bytes * (size_t)R, f) != bytes * (size_t)R) {
    fprintf(stderr, "cannot write %s\n", out_path);
    if (f) fclose(f);
    free(host);
    return 1;
  }
  fclose(f);

  MSCL_OK(mscl_channel_destroy(ch));
  for (int r = 0; r < R; ++r) {
    HIP_OK(hipFree(in[r]));
    if (!in_place) HIP_OK(hipFree(out[r]));
  }
  HIP_OK(hipStreamDestroy(stream));
  free(host);
  printf("ok R=%d dtype=%d count=%zu algo=%d%s plan_algo=%d cached_puts=%d held_tiles=%d slices=%d "
         "tile_interleave=%d\n",
         R, dtype, count, algo, in_place ? " in place" : "", (int)plan.algo, plan.cached_puts, plan.held_tiles,
         plan.slices, plan.tile_interleave);
  return 0;
}

int main(int argc, char** argv) {
  if (argc == 2 && strcmp(argv[1], "--version") == 0) {
    printf("mscl version %d\n", mscl_version());
    return 0;
  }
  if (argc != 7 && argc != 8) {
    fprintf(stderr, "usage: %s --version | R DTYPE COUNT ALGO IN_FILE OUT_FILE [inplace]\n", argv[0]);
    return 1;
  }
  const int R = atoi(argv[1]);
  const int dtype = atoi(argv[2]);
  const size_t count = (size_t)strtoull(argv[3], NULL, 10);
  const int algo = atoi(argv[4]);
  const int in_place = argc == 8 && strcmp(argv[7], "inplace") == 0;
  if (R < 1 || R > MSCL_MAX_RANKS || dtype < 0 || dtype > 2) {
    fprintf(stderr, "bad R or dtype\n");
    return 1;
  }
  return run(R, dtype, count, algo, argv[5], argv[6], in_place);
}
