/*
 * Plain-C CPU oracle for the emulated-peer AllReduce — TEST INFRASTRUCTURE
 * ONLY (used by tests/ for full-size checks and by the benchmark's CPU
 * baseline leg).  It shares no code with the HIP library.
 *
 * Definition (same as oracle/allreduce.py, which is the authority and
 * against which this file is checked bit-for-bit):
 *   for each element i:
 *     a = f32(x_0[i]); for p = 1..R-1: a = a + f32(x_p[i])   (binary32, RNE)
 *     y[i] = RNE_dtype(a); every output r receives y.
 * The pages name AllReduce (MSCCL++ project summary, "Highlighted Details")
 * but fix no accumulation type, order or rounding; rank-order binary32
 * accumulation with a single final rounding is the reading taken.
 *
 * Threads only split the element range; each element is still reduced by one
 * thread in rank order, so the thread count cannot change any result.
 * Build with -O2 -fno-fast-math -ffp-contract=off (oracle/build.py): there is
 * nothing to contract, but the flags keep the compiler honest anyway.
 */
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

enum { ORC_FP32 = 0, ORC_FP16 = 1, ORC_BF16 = 2 };

static float f32_from_bits(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static uint32_t bits_from_f32(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return u;
}

/* binary16 -> binary32, exact, from the binary16 field layout:
 * sign(1) exponent(5, bias 15) fraction(10). */
static float f16_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h >> 15) << 31;
  uint32_t e = (h >> 10) & 0x1F;
  uint32_t f = h & 0x3FF;
  if (e == 0x1F) return f32_from_bits(sign | 0x7F800000u | (f << 13)); /* Inf/NaN */
  if (e != 0) return f32_from_bits(sign | ((e - 15 + 127) << 23) | (f << 13));
  if (f == 0) return f32_from_bits(sign); /* signed zero */
  /* subnormal: value = f * 2^-24; normalise f into 1.xxx form */
  int exp = -14;
  while ((f & 0x400) == 0) {
    f <<= 1;
    exp -= 1;
  }
  f &= 0x3FF;
  return f32_from_bits(sign | ((uint32_t)(exp + 127) << 23) | (f << 13));
}

/* Keep the top (24 - drop) bits of a significand, rounding the dropped bits
 * to nearest with ties to the even kept value.  drop must be in [1, 31]. */
static uint32_t rne_shift(uint32_t sig, int drop) {
  uint32_t kept = sig >> drop;
  uint32_t rest = sig & ((1u << drop) - 1u);
  uint32_t half = 1u << (drop - 1);
  if (rest > half || (rest == half && (kept & 1u))) kept += 1u;
  return kept;
}

/* binary32 -> binary16, round to nearest even, written from the definition:
 * the value |a| = sig * 2^(E-150) with sig the 24-bit significand.  A normal
 * binary16 keeps 11 significant bits; below 2^-14 the spacing is fixed at
 * 2^-24 (subnormals).  A carry out of the kept bits moves to the next binade;
 * anything that lands at or beyond 2^16 is infinity. */
uint16_t orc_f32_to_f16(float x) {
  uint32_t u = bits_from_f32(x);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000);
  uint32_t E = (u >> 23) & 0xFF;
  uint32_t m = u & 0x7FFFFF;
  if (E == 0xFF) {
    if (m == 0) return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | 0x7E00 | (m >> 13)); /* quiet NaN */
  }
  if (E == 0) return sign; /* binary32 subnormals are below 2^-126: +-0 */
  int e = (int)E - 127;    /* |a| in [2^e, 2^(e+1)) */
  uint32_t sig = m | 0x800000u;
  if (e > 15) return (uint16_t)(sign | 0x7C00);
  if (e >= -14) {
    uint32_t q = rne_shift(sig, 13); /* 11 bits, maybe 12 after a carry */
    if (q == 0x800u) {
      q = 0x400u;
      e += 1;
    }
    if (e > 15) return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | ((uint32_t)(e + 15) << 10) | (q & 0x3FF));
  }
  /* subnormal target: units of 2^-24; |a| = sig * 2^(e-23) = sig * 2^(e+1) units */
  int drop = -(e + 1); /* >= 14 */
  if (drop > 25) return sign; /* below half of 2^-24 */
  uint32_t q = rne_shift(sig, drop); /* may reach 0x400 = smallest normal */
  return (uint16_t)(sign | q);
}

/* binary32 -> bfloat16, round to nearest even.  bfloat16 is the top half of
 * a binary32 pattern; the low half decides the rounding.  A carry from the
 * kept fraction into the exponent is the correct next binade (and turns the
 * top binade into infinity).  NaNs are kept NaN and made quiet. */
uint16_t orc_f32_to_bf16(float x) {
  uint32_t u = bits_from_f32(x);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu) != 0)
    return (uint16_t)((u >> 16) | 0x0040);
  uint32_t hi = u >> 16;
  uint32_t lo = u & 0xFFFFu;
  if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1u;
  return (uint16_t)hi;
}

static float load_f32(const void* p, int dtype, size_t i) {
  if (dtype == ORC_FP32) return ((const float*)p)[i];
  uint16_t h = ((const uint16_t*)p)[i];
  if (dtype == ORC_FP16) return f16_to_f32(h);
  return f32_from_bits((uint32_t)h << 16);
}

struct orc_job {
  const void* const* inputs;
  void* const* outputs;
  size_t lo, hi;
  int dtype, nranks;
};

static void reduce_range(const struct orc_job* j) {
  for (size_t i = j->lo; i < j->hi; ++i) {
    float a = load_f32(j->inputs[0], j->dtype, i);
    for (int p = 1; p < j->nranks; ++p) a = a + load_f32(j->inputs[p], j->dtype, i);
    for (int r = 0; r < j->nranks; ++r) {
      if (j->dtype == ORC_FP32)
        ((float*)j->outputs[r])[i] = a;
      else if (j->dtype == ORC_FP16)
        ((uint16_t*)j->outputs[r])[i] = orc_f32_to_f16(a);
      else
        ((uint16_t*)j->outputs[r])[i] = orc_f32_to_bf16(a);
    }
  }
}

static void* reduce_thread(void* arg) {
  reduce_range((const struct orc_job*)arg);
  return NULL;
}

/* inputs/outputs: host arrays of nranks host pointers, count elements each.
 * Outputs must not alias inputs (the oracle reads every input element after
 * it may have written outputs for earlier elements only, so in-place is in
 * fact safe too, but the tests never rely on it).  Returns 0, or -1 on a bad
 * argument. */
int orc_allreduce(const void* const* inputs, void* const* outputs, size_t count, int dtype,
                  int nranks, int nthreads) {
  if (nranks < 1 || nranks > 64 || dtype < 0 || dtype > 2 || !inputs || !outputs) return -1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((size_t)nthreads > count) nthreads = count ? (int)count : 1;
  struct orc_job jobs[256];
  pthread_t tids[256];
  size_t per = (count + (size_t)nthreads - 1) / (size_t)nthreads;
  for (int t = 0; t < nthreads; ++t) {
    size_t lo = per * (size_t)t;
    size_t hi = lo + per;
    if (lo > count) lo = count;
    if (hi > count) hi = count;
    jobs[t] = (struct orc_job){inputs, outputs, lo, hi, dtype, nranks};
  }
  int started = 0;
  for (int t = 1; t < nthreads; ++t) {
    if (pthread_create(&tids[t], NULL, reduce_thread, &jobs[t]) != 0) break;
    started = t;
  }
  reduce_range(&jobs[0]);
  for (int t = started + 1; t < nthreads; ++t) reduce_range(&jobs[t]); /* threads that failed to start */
  for (int t = 1; t <= started; ++t) pthread_join(tids[t], NULL);
  return 0;
}

/* Element-wise conversions exposed for the pins. */
void orc_round_f16(const float* a, uint16_t* out, size_t n) {
  for (size_t i = 0; i < n; ++i) out[i] = orc_f32_to_f16(a[i]);
}
void orc_round_bf16(const float* a, uint16_t* out, size_t n) {
  for (size_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16(a[i]);
}
void orc_widen_f16(const uint16_t* h, float* out, size_t n) {
  for (size_t i = 0; i < n; ++i) out[i] = f16_to_f32(h[i]);
}
