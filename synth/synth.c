/*
 * synth.c — seeded, counter-based synthetic inputs for the MoE layer.
 *
 * Holds no arithmetic of the method itself: it draws numbers and encodes
 * them into the byte formats the layer consumes (binary32, bfloat16, OCP
 * E4M3). Both the HIP path and the CPU oracle read the bytes it writes.
 *
 * Counter-based stream: output j of seed s is splitmix64's mixing function
 * applied to s + (j+1) * 0x9E3779B97F4A7C15 (the SplitMix64 generator of
 * Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
 * OOPSLA 2014, as popularised by Vigna). Element i of a normal array uses
 * outputs 2i and 2i+1 through the Box-Muller transform, so any element can
 * be produced independently and threads split the index range freely.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t stream_at(uint64_t seed, uint64_t j) { return mix64(seed + (j + 1) * GOLDEN); }

uint64_t synth_u64(uint64_t seed, uint64_t j) { return stream_at(seed, j); }

static inline double normal_at(uint64_t seed, uint64_t i) {
  uint64_t r1 = stream_at(seed, 2 * i), r2 = stream_at(seed, 2 * i + 1);
  double u1 = ((double)(r1 >> 11) + 1.0) * 0x1.0p-53; /* (0, 1] */
  double u2 = (double)(r2 >> 11) * 0x1.0p-53;         /* [0, 1) */
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

/* binary32 -> bfloat16 bits, round to nearest even; NaN stays NaN. */
static inline uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/* binary32 -> OCP E4M3 (fn) byte, round to nearest even, saturating to
 * +-448 (the format has no infinity); NaN -> 0x7f. */
static inline uint8_t f32_to_e4m3(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint8_t sign = (uint8_t)((u >> 24) & 0x80);
  float a = fabsf(f);
  if (a != a) return 0x7f;
  if (a >= 464.0f) return sign | 0x7e; /* 464 is the midpoint above 448: saturate */
  /* exponent of the leading bit; normals of E4M3 have exponent -6..8 */
  int ex;
  frexpf(a, &ex);
  int lead = ex - 1;
  if (lead < -6) lead = -6; /* subnormal quantum 2^-9 */
  float q = ldexpf(1.0f, lead - 3);
  float r = rintf(a / q) * q; /* a/q exact; rintf is ties-to-even */
  if (r == 0.0f) return sign;
  if (r > 448.0f) return sign | 0x7e;
  int e2;
  float m = frexpf(r, &e2); /* r = m * 2^e2, m in [0.5,1) */
  int lead2 = e2 - 1;
  if (lead2 < -6) { /* subnormal: r = mant * 2^-9 */
    int mant = (int)ldexpf(r, 9);
    return sign | (uint8_t)mant;
  }
  int mant = (int)(ldexpf(m, 4)) - 8; /* m*16 in [8,16) */
  int eb = lead2 + 7;
  return sign | (uint8_t)((eb << 3) | mant);
}

typedef struct {
  int kind;
  uint64_t seed;
  int64_t begin, end;
  double mean, std;
  int lo, hi;
  void* out;
  const float* in;
  float scale;
} job_t;

enum { K_NORMAL_F32, K_NORMAL_BF16, K_INT_F32, K_INT_BF16, K_TO_BF16, K_TO_E4M3 };

static void* run_job(void* p) {
  job_t* j = (job_t*)p;
  for (int64_t i = j->begin; i < j->end; ++i) {
    switch (j->kind) {
      case K_NORMAL_F32:
        ((float*)j->out)[i] = (float)(j->mean + j->std * normal_at(j->seed, (uint64_t)i));
        break;
      case K_NORMAL_BF16:
        ((uint16_t*)j->out)[i] = f32_to_bf16((float)(j->mean + j->std * normal_at(j->seed, (uint64_t)i)));
        break;
      case K_INT_F32:
      case K_INT_BF16: {
        uint64_t span = (uint64_t)(j->hi - j->lo + 1);
        float v = (float)(j->lo + (int64_t)(stream_at(j->seed, (uint64_t)i) % span));
        if (j->kind == K_INT_F32)
          ((float*)j->out)[i] = v;
        else
          ((uint16_t*)j->out)[i] = f32_to_bf16(v);
        break;
      }
      case K_TO_BF16:
        ((uint16_t*)j->out)[i] = f32_to_bf16(j->in[i]);
        break;
      case K_TO_E4M3:
        ((uint8_t*)j->out)[i] = f32_to_e4m3(j->in[i] / j->scale);
        break;
    }
  }
  return NULL;
}

static void run_parallel(job_t proto, int64_t n, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  if (n < 65536) nthreads = 1;
  pthread_t th[64];
  int live[64] = {0};
  job_t jobs[64];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = proto;
    jobs[t].begin = n * t / nthreads;
    jobs[t].end = n * (t + 1) / nthreads;
  }
  for (int t = 1; t < nthreads; ++t) live[t] = pthread_create(&th[t], NULL, run_job, &jobs[t]) == 0;
  run_job(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) {
    if (live[t])
      pthread_join(th[t], NULL);
    else
      run_job(&jobs[t]); /* thread could not start: do its share here */
  }
}

void synth_normal_f32(uint64_t seed, int64_t n, double mean, double std, float* out, int nthreads) {
  job_t j = {K_NORMAL_F32, seed, 0, 0, mean, std, 0, 0, out, NULL, 1.0f};
  run_parallel(j, n, nthreads);
}

void synth_normal_bf16(uint64_t seed, int64_t n, double mean, double std, uint16_t* out, int nthreads) {
  job_t j = {K_NORMAL_BF16, seed, 0, 0, mean, std, 0, 0, out, NULL, 1.0f};
  run_parallel(j, n, nthreads);
}

void synth_int_f32(uint64_t seed, int64_t n, int lo, int hi, float* out, int nthreads) {
  job_t j = {K_INT_F32, seed, 0, 0, 0.0, 0.0, lo, hi, out, NULL, 1.0f};
  run_parallel(j, n, nthreads);
}

void synth_int_bf16(uint64_t seed, int64_t n, int lo, int hi, uint16_t* out, int nthreads) {
  job_t j = {K_INT_BF16, seed, 0, 0, 0.0, 0.0, lo, hi, out, NULL, 1.0f};
  run_parallel(j, n, nthreads);
}

void synth_f32_to_bf16(const float* in, int64_t n, uint16_t* out, int nthreads) {
  job_t j = {K_TO_BF16, 0, 0, 0, 0.0, 0.0, 0, 0, out, in, 1.0f};
  run_parallel(j, n, nthreads);
}

/* out[i] = E4M3(in[i] / scale) */
void synth_f32_to_e4m3(const float* in, int64_t n, float scale, uint8_t* out, int nthreads) {
  job_t j = {K_TO_E4M3, 0, 0, 0, 0.0, 0.0, 0, 0, out, in, scale};
  run_parallel(j, n, nthreads);
}

float synth_amax_f32(const float* in, int64_t n) {
  float m = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    float a = fabsf(in[i]);
    if (a > m) m = a;
  }
  return m;
}

/* Per token, K distinct experts drawn uniformly from E (a partial
 * Fisher-Yates shuffle driven by the stream), written in draw order.
 * This is a random routing assignment, not the router of the method. */
int synth_random_routing(uint64_t seed, int T, int E, int K, int32_t* idx) {
  if (E <= 0 || K <= 0 || K > E || E > 4096) return -1;
  int32_t perm[4096];
  uint64_t j = 0;
  for (int t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) perm[e] = e;
    for (int k = 0; k < K; ++k) {
      uint64_t r = stream_at(seed, j++);
      int pick = k + (int)(r % (uint64_t)(E - k));
      int32_t tmp = perm[k];
      perm[k] = perm[pick];
      perm[pick] = tmp;
      idx[(int64_t)t * K + k] = perm[k];
    }
  }
  return 0;
}
