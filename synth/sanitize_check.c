/* Sanitizer driver for the input generator (synth.c).
 *
 * Calls every exported generator function on small ranges, with offsets,
 * one and several threads, so that a build of synth.c with AddressSanitizer
 * and UndefinedBehaviorSanitizer sees all of its code paths; it also checks
 * that results do not depend on the thread count or on the offset split.
 * Built and run by tests/test_sanitizers.py. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

uint64_t synth_raw_draw(uint64_t seed, uint64_t stream, uint64_t i);
double synth_normal_one(uint64_t seed, uint64_t stream, uint64_t i);
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t off, uint64_t n, float* out, int nthreads);
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t off, uint64_t n, uint16_t* out, int nthreads);
void synth_codes4(uint64_t seed, uint64_t stream, uint64_t off_bytes, uint64_t n_bytes, const uint8_t* codeset,
                  int ncodes, uint8_t* out, int nthreads);
void synth_exp_bytes(uint64_t seed, uint64_t stream, uint64_t off, uint64_t n, int lo_e, int hi_e, int bias,
                     uint8_t* out, int nthreads);
void synth_pow2_f32(uint64_t seed, uint64_t stream, uint64_t off, uint64_t n, int lo_e, int hi_e, float* out,
                    int nthreads);
void synth_loguniform_lengths(uint64_t seed, uint64_t stream, int64_t n, double lo, double hi, int64_t forbid_mod,
                              int64_t* out);

static int failures = 0;

static void same(const void* a, const void* b, size_t n, const char* what) {
  if (memcmp(a, b, n) != 0) {
    fprintf(stderr, "%s depends on the thread count or the split\n", what);
    ++failures;
  }
}

int main(void) {
  enum { N = 1000 };
  static float f1[N], f3[N], g[N];
  static uint16_t h1[N], h3[N];
  static uint8_t c1[N], c3[N], e1[N], e3[N];
  static int64_t L[64];
  const uint8_t codes[3] = {0x0, 0x1, 0x9};
  double acc = 0.0;
  for (uint64_t i = 0; i < 100; ++i) acc += (double)(synth_raw_draw(7, 3, i) >> 40) + synth_normal_one(7, 3, i);
  for (uint64_t n = 0; n <= N; n += N / 4) {
    synth_normal_f32(11, 1, 5, n, f1, 1);
    synth_normal_f32(11, 1, 5, n, f3, 3);
    same(f1, f3, n * sizeof(float), "synth_normal_f32");
    synth_normal_bf16(11, 1, 5, n, h1, 1);
    synth_normal_bf16(11, 1, 5, n, h3, 7);
    same(h1, h3, n * sizeof(uint16_t), "synth_normal_bf16");
    synth_codes4(11, 2, 9, n, codes, 3, c1, 1);
    synth_codes4(11, 2, 9, n, codes, 3, c3, 4);
    same(c1, c3, n, "synth_codes4");
    synth_exp_bytes(11, 4, 0, n, -2, 2, 127, e1, 1);
    synth_exp_bytes(11, 4, 0, n, -2, 2, 127, e3, 5);
    same(e1, e3, n, "synth_exp_bytes");
    synth_pow2_f32(11, 5, 0, n, -1, 1, f1, 1);
    synth_pow2_f32(11, 5, 0, n, -1, 1, f3, 2);
    same(f1, f3, n * sizeof(float), "synth_pow2_f32");
  }
  /* an element's value does not depend on how the range is split */
  synth_normal_f32(3, 1, 0, N, f1, 2);
  synth_normal_f32(3, 1, 0, N / 3, g, 1);
  synth_normal_f32(3, 1, N / 3, N - N / 3, g + N / 3, 3);
  same(f1, g, N * sizeof(float), "synth_normal_f32 split");
  synth_loguniform_lengths(5, 9, 64, 4096.0, 1048576.0, 4, L);
  synth_loguniform_lengths(5, 9, 0, 4096.0, 1048576.0, 0, L);
  for (int i = 0; i < 64; ++i) acc += (double)L[i];
  printf("sanitize_check: %d failures (checksum %g)\n", failures, acc);
  return failures == 0 ? 0 : 1;
}
