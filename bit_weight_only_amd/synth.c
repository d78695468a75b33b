/*
 * synth.c -- seeded synthetic inputs (no part of the layer's arithmetic).
 *
 * SplitMix64 (Steele, Lea and Flood, 2014): draw i of the stream seeded by
 * `seed` is mix(seed + (i + 1) * 0x9E3779B97F4A7C15), with the published
 * finaliser mix().  Normal e is Box-Muller on draws 2p and 2p+1, p = e / 2:
 *   u1 = ((d0 >> 11) + 1) * 2^-53,  u2 = (d1 >> 11) * 2^-53,
 *   z  = sqrt(-2 ln u1) * (e even ? cos(2 pi u2) : sin(2 pi u2)).
 * Counter based, so any slice of any stream is generated on its own and the
 * split over threads does not change a single value.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t seed, uint64_t i) {
  return mix(seed + (i + 1) * 0x9E3779B97F4A7C15ULL);
}

static inline double normal_at(uint64_t seed, uint64_t e) {
  const uint64_t p = e >> 1;
  const double u1 = ((double)(draw(seed, 2 * p) >> 11) + 1.0) * 0x1p-53;
  const double u2 = (double)(draw(seed, 2 * p + 1) >> 11) * 0x1p-53;
  const double rad = sqrt(-2.0 * log(u1));
  const double ang = 2.0 * 3.141592653589793 * u2; /* the double nearest pi */
  return (e & 1) ? rad * sin(ang) : rad * cos(ang);
}

static inline uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

enum { KIND_F64 = 0, KIND_F32_SCALED = 1, KIND_BF16 = 2, KIND_U64 = 3 };

typedef struct {
  int kind;
  uint64_t seed, offset;
  int64_t lo, hi;
  double scale;
  void *out;
} job_t;

static void run(const job_t *j) {
  for (int64_t i = j->lo; i < j->hi; ++i) {
    const uint64_t e = j->offset + (uint64_t)i;
    switch (j->kind) {
      case KIND_F64: ((double *)j->out)[i] = normal_at(j->seed, e); break;
      case KIND_F32_SCALED: ((float *)j->out)[i] = (float)(j->scale * normal_at(j->seed, e)); break;
      case KIND_BF16: ((uint16_t *)j->out)[i] = f32_to_bf16((float)normal_at(j->seed, e)); break;
      default: ((uint64_t *)j->out)[i] = draw(j->seed, e); break;
    }
  }
}

static void *thread_main(void *a) {
  run((const job_t *)a);
  return NULL;
}

/* kind: 0 = double normals, 1 = float(scale * normal), 2 = bf16 bits of
 * float(normal), 3 = raw 64-bit draws.  Elements offset .. offset+n-1. */
void synth_fill(int kind, uint64_t seed, uint64_t offset, int64_t n, double scale, void *out,
                int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 128) nthreads = 128;
  if (n < 65536) nthreads = 1;
  pthread_t th[128];
  job_t jobs[128];
  for (int t = 0; t < nthreads; ++t)
    jobs[t] = (job_t){kind, seed, offset, n * t / nthreads, n * (t + 1) / nthreads, scale, out};
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, thread_main, &jobs[t]);
  run(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
}
