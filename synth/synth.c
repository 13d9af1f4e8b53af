/*
 * Seeded, counter-based input generators for the compressed-attention
 * workloads.  This file holds no arithmetic of the attention method itself:
 * it only draws random numbers and formats them (fp32 / bf16 rounding, packed
 * 4-bit codes, exponent bytes).  Both the HIP path and the CPU oracle consume
 * the arrays written here.
 *
 * Generator: element i of stream s under seed S is the (i+1)-th output of
 * SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014) whose starting state is
 *     key(S, s) = mix64(S * GOLDEN ^ mix64(s + STREAM_SALT)),
 * i.e. draw(i) = mix64(key + (i + 1) * GOLDEN).  Any element can therefore be
 * regenerated on its own, in any order and on any number of threads.
 *
 * Normal variates: Box-Muller in fp64 on the pair (draw(2p), draw(2p+1)),
 * element 2p takes the cosine branch and 2p+1 the sine branch.  Uniforms are
 * ((x >> 11) + 0.5) * 2^-53, strictly inside (0, 1).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL
#define STREAM_SALT 0x632BE59BD9B4E019ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(seed * GOLDEN ^ mix64(stream + STREAM_SALT));
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN); }

static inline double unif(uint64_t x) { return ((double)(x >> 11) + 0.5) * 0x1.0p-53; }

/* uniform integer in [0, n) by the multiply-shift reduction of a 64-bit draw */
static inline uint32_t below(uint64_t x, uint32_t n) {
  return (uint32_t)(((unsigned __int128)x * n) >> 64);
}

static inline double normal_at(uint64_t key, uint64_t i) {
  uint64_t p = i >> 1;
  double u1 = unif(draw(key, 2 * p));
  double u2 = unif(draw(key, 2 * p + 1));
  double r = sqrt(-2.0 * log(u1));
  double a = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(a) : r * cos(a);
}

/* fp32 -> bf16 bits, round to nearest even (inputs here are always finite) */
static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* ---------------- threading ---------------- */
typedef struct {
  int kind;
  uint64_t key;
  uint64_t off, lo, hi;
  void* out;
  const uint8_t* codeset;
  int ncodes;
  int lo_e, hi_e;
  int bias;
} job_t;

enum { J_NORM_F32 = 0, J_NORM_BF16 = 1, J_CODES = 2, J_EXPBYTES = 3, J_POW2 = 4 };

static void* run_job(void* arg) {
  job_t* j = (job_t*)arg;
  switch (j->kind) {
    case J_NORM_F32: {
      float* o = (float*)j->out;
      for (uint64_t i = j->lo; i < j->hi; ++i) o[i] = (float)normal_at(j->key, j->off + i);
      break;
    }
    case J_NORM_BF16: {
      uint16_t* o = (uint16_t*)j->out;
      for (uint64_t i = j->lo; i < j->hi; ++i)
        o[i] = f32_to_bf16_rne((float)normal_at(j->key, j->off + i));
      break;
    }
    case J_CODES: { /* two 4-bit codes per byte: element 2b low nibble, 2b+1 high */
      uint8_t* o = (uint8_t*)j->out;
      for (uint64_t b = j->lo; b < j->hi; ++b) {
        uint64_t e = 2 * (j->off + b);
        uint8_t c0 = j->codeset[below(draw(j->key, e), (uint32_t)j->ncodes)];
        uint8_t c1 = j->codeset[below(draw(j->key, e + 1), (uint32_t)j->ncodes)];
        o[b] = (uint8_t)((c0 & 15) | ((c1 & 15) << 4));
      }
      break;
    }
    case J_EXPBYTES: { /* bias + uniform integer exponent in [lo_e, hi_e] */
      uint8_t* o = (uint8_t*)j->out;
      uint32_t span = (uint32_t)(j->hi_e - j->lo_e + 1);
      for (uint64_t i = j->lo; i < j->hi; ++i)
        o[i] = (uint8_t)(j->bias + j->lo_e + (int)below(draw(j->key, j->off + i), span));
      break;
    }
    case J_POW2: { /* 2^e with e uniform integer in [lo_e, hi_e] */
      float* o = (float*)j->out;
      uint32_t span = (uint32_t)(j->hi_e - j->lo_e + 1);
      for (uint64_t i = j->lo; i < j->hi; ++i)
        o[i] = ldexpf(1.0f, j->lo_e + (int)below(draw(j->key, j->off + i), span));
      break;
    }
  }
  return 0;
}

static void run_parallel(job_t proto, uint64_t n, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  if (n < 65536) nthreads = 1;
  pthread_t th[64];
  job_t jobs[64];
  uint64_t per = (n + (uint64_t)nthreads - 1) / (uint64_t)nthreads;
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = proto;
    jobs[t].lo = per * (uint64_t)t;
    jobs[t].hi = jobs[t].lo + per < n ? jobs[t].lo + per : n;
    if (jobs[t].lo >= jobs[t].hi) break;
    if (t == 0) continue;
    if (pthread_create(&th[t], 0, run_job, &jobs[t]) != 0) {
      run_job(&jobs[t]); /* fall back to this thread */
      jobs[t].kind = -1;
    }
    started = t;
  }
  if (n > 0) run_job(&jobs[0]);
  for (int t = 1; t <= started; ++t)
    if (jobs[t].kind >= 0) pthread_join(th[t], 0);
}

/* ---------------- exported API ---------------- */

uint64_t synth_raw_draw(uint64_t seed, uint64_t stream, uint64_t i) {
  return draw(stream_key(seed, stream), i);
}

double synth_normal_one(uint64_t seed, uint64_t stream, uint64_t i) {
  return normal_at(stream_key(seed, stream), i);
}

/* n normals of stream `stream`, elements [off, off+n), rounded once to fp32 */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t off, uint64_t n, float* out,
                      int nthreads) {
  job_t j = {J_NORM_F32, stream_key(seed, stream), off, 0, 0, out, 0, 0, 0, 0, 0};
  run_parallel(j, n, nthreads);
}

/* the same normals rounded to fp32 (RNE) and then to bf16 (RNE) */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t off, uint64_t n, uint16_t* out,
                       int nthreads) {
  job_t j = {J_NORM_BF16, stream_key(seed, stream), off, 0, 0, out, 0, 0, 0, 0, 0};
  run_parallel(j, n, nthreads);
}

/* n_bytes packed bytes = 2*n_bytes 4-bit codes, each uniform over codeset[0..ncodes) */
void synth_codes4(uint64_t seed, uint64_t stream, uint64_t off_bytes, uint64_t n_bytes,
                  const uint8_t* codeset, int ncodes, uint8_t* out, int nthreads) {
  job_t j = {J_CODES, stream_key(seed, stream), off_bytes, 0, 0, out, codeset, ncodes, 0, 0, 0};
  run_parallel(j, n_bytes, nthreads);
}

/* exponent bytes: bias + U{lo_e..hi_e} */
void synth_exp_bytes(uint64_t seed, uint64_t stream, uint64_t off, uint64_t n, int lo_e, int hi_e,
                     int bias, uint8_t* out, int nthreads) {
  job_t j = {J_EXPBYTES, stream_key(seed, stream), off, 0, 0, out, 0, 0, lo_e, hi_e, bias};
  run_parallel(j, n, nthreads);
}

/* powers of two 2^U{lo_e..hi_e} as fp32 */
void synth_pow2_f32(uint64_t seed, uint64_t stream, uint64_t off, uint64_t n, int lo_e, int hi_e,
                    float* out, int nthreads) {
  job_t j = {J_POW2, stream_key(seed, stream), off, 0, 0, out, 0, 0, lo_e, hi_e, 0};
  run_parallel(j, n, nthreads);
}

/* lengths floor(exp(U[ln lo, ln hi])) with values L % forbid_mod == 0 redrawn
 * (attempt a of sequence b uses element b*4096 + a of the stream) */
void synth_loguniform_lengths(uint64_t seed, uint64_t stream, int64_t n, double lo, double hi,
                              int64_t forbid_mod, int64_t* out) {
  uint64_t key = stream_key(seed, stream);
  for (int64_t b = 0; b < n; ++b) {
    int64_t L = 0;
    for (uint64_t a = 0; a < 4096; ++a) {
      double u = unif(draw(key, (uint64_t)b * 4096u + a));
      L = (int64_t)floor(exp(log(lo) + u * (log(hi) - log(lo))));
      if (L < (int64_t)lo) L = (int64_t)lo;
      if (L > (int64_t)hi) L = (int64_t)hi;
      if (forbid_mod <= 0 || L % forbid_mod != 0) break;
    }
    out[b] = L;
  }
}
