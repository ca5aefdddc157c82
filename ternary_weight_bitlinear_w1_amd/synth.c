/* Seeded synthetic inputs for the BitLinear hot path (host only).
 *
 * This file draws random numbers and nothing else: it holds none of the
 * method's arithmetic, so the HIP path's tests and the CPU oracle can both take
 * their inputs from it.
 *
 * SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014) used as a counter-based generator: output i of the
 * stream with seed s is mix(s + (i + 1) * 0x9E3779B97F4A7C15) (mod 2^64).
 * Normal draws: Box-Muller in fp64 on outputs 2i and 2i+1,
 *   u1 = ((r0 >> 11) + 1) * 2^-53 in (0, 1],  u2 = (r1 >> 11) * 2^-53 in [0, 1),
 *   z  = sqrt(-2 ln u1) * cos(2 pi u2),        value = (float)(sigma * z).
 * Element i depends only on (seed, i), so the fill is split over threads
 * without changing any value.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>

#define SM_GOLDEN 0x9E3779B97F4A7C15ULL

static uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_u64(uint64_t seed, uint64_t i) { return sm_mix(seed + (i + 1) * SM_GOLDEN); }

void synth_raw_u64(uint64_t seed, uint64_t start, int64_t count, uint64_t *out) {
  for (int64_t i = 0; i < count; ++i) out[i] = synth_u64(seed, start + (uint64_t)i);
}

static float normal_at(uint64_t seed, uint64_t i, double sigma) {
  const double two_pi = 6.283185307179586476925286766559;
  uint64_t r0 = synth_u64(seed, 2 * i), r1 = synth_u64(seed, 2 * i + 1);
  double u1 = ((double)(r0 >> 11) + 1.0) * 0x1p-53;
  double u2 = (double)(r1 >> 11) * 0x1p-53;
  double z = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
  return (float)(sigma * z);
}

typedef struct {
  uint64_t seed, start;
  int64_t lo, hi;
  double sigma;
  float *out;
} fill_job;

static void *fill_run(void *p) {
  fill_job *j = (fill_job *)p;
  for (int64_t i = j->lo; i < j->hi; ++i) j->out[i] = normal_at(j->seed, j->start + (uint64_t)i, j->sigma);
  return 0;
}

/* out[i] = N(0, sigma^2) draw number start + i of stream `seed`, i < count. */
void synth_normal_f32(uint64_t seed, uint64_t start, int64_t count, double sigma, float *out, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  if (count < ((int64_t)1 << 16)) nthreads = 1;
  pthread_t th[64];
  fill_job jobs[64];
  int launched[64] = {0};
  int64_t per = (count + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    int64_t lo = per * t, hi = lo + per < count ? lo + per : count;
    if (lo > hi) lo = hi;
    jobs[t] = (fill_job){seed, start, lo, hi, sigma, out};
  }
  for (int t = 1; t < nthreads; ++t)
    launched[t] = pthread_create(&th[t], 0, fill_run, &jobs[t]) == 0;
  fill_run(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) {
    if (launched[t]) pthread_join(th[t], 0);
    else fill_run(&jobs[t]);
  }
}
