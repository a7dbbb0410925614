/*
 * Seeded synthetic bf16 operands for the AdaHOP GEMM workloads.
 *
 * This module only draws inputs. It holds none of the method's arithmetic
 * (no detection, rotation, quantization or product): both the GPU path and
 * the CPU oracle receive the bytes it writes.
 *
 * Generator (counter-based, so any element regenerates on its own):
 *   key(seed, stream) = splitmix64(splitmix64(seed) ^ stream * 0x9E3779B97F4A7C15)
 *   element e of a tensor: h1 = splitmix64(key + 2e), h2 = splitmix64(key + 2e + 1)
 *     u1 = ((h1 >> 11) + 1) * 2^-53 in (0, 1], u2 = (h2 >> 11) * 2^-53 in [0, 1)
 *     z  = sqrt(-2 ln u1) * cos(2 pi u2)          (Box-Muller, fp64)
 *     v  = z * sigma * (factor if e's row/column is a planted outlier line)
 *     stored as bf16: v -> fp32 (round to nearest) -> bf16 (round to nearest even)
 *   e = row * cols + col (the logical row-major index, independent of ld).
 * Planted outlier lines: a partial Fisher-Yates shuffle of [0, dim) driven by
 *   splitmix64(key(seed, 16 + stream) + i), first n entries, returned ascending.
 * splitmix64 is Steele, Lea and Flood's SplitMix64 finaliser (2014).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static inline uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t stream) {
  return splitmix64(splitmix64(seed) ^ (stream * 0x9E3779B97F4A7C15ull));
}

static int cmp_i64(const void* a, const void* b) {
  int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
  return (x > y) - (x < y);
}

/* n distinct line indices in [0, dim), ascending. Returns 0, or -1 on bad sizes. */
int synth_pick_lines(uint64_t seed, uint64_t stream, int64_t dim, int64_t n, int64_t* out) {
  if (dim < 0 || n < 0 || n > dim) return -1;
  if (n == 0) return 0;
  int64_t* perm = (int64_t*)malloc(sizeof(int64_t) * (size_t)dim);
  if (!perm) return -1;
  for (int64_t i = 0; i < dim; ++i) perm[i] = i;
  uint64_t key = synth_key(seed, 16 + stream);
  for (int64_t i = 0; i < n; ++i) {
    uint64_t r = splitmix64(key + (uint64_t)i);
    int64_t j = i + (int64_t)(r % (uint64_t)(dim - i));
    int64_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
  }
  memcpy(out, perm, sizeof(int64_t) * (size_t)n);
  free(perm);
  qsort(out, (size_t)n, sizeof(int64_t), cmp_i64);
  return 0;
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Fill out[r * ld + c] for r < rows, c < cols.
 * line_axis: 0 = planted lines are rows, 1 = columns, -1 = none.
 * lines: ascending indices of planted lines (nlines of them). */
int synth_fill_bf16(uint16_t* out, int64_t rows, int64_t cols, int64_t ld,
                    uint64_t seed, uint64_t stream, double sigma,
                    int line_axis, const int64_t* lines, int64_t nlines, double factor) {
  if (rows < 0 || cols < 0 || ld < cols || (nlines > 0 && !lines)) return -1;
  int64_t dim = line_axis == 0 ? rows : (line_axis == 1 ? cols : 0);
  unsigned char* planted = NULL;
  if (line_axis == 0 || line_axis == 1) {
    planted = (unsigned char*)calloc((size_t)(dim > 0 ? dim : 1), 1);
    if (!planted) return -1;
    for (int64_t i = 0; i < nlines; ++i) {
      if (lines[i] < 0 || lines[i] >= dim) { free(planted); return -1; }
      planted[lines[i]] = 1;
    }
  }
  const uint64_t key = synth_key(seed, stream);
  const double two_pi = 6.283185307179586476925286766559;
  const double inv53 = 1.0 / 9007199254740992.0;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t c = 0; c < cols; ++c) {
      uint64_t e = (uint64_t)r * (uint64_t)cols + (uint64_t)c;
      uint64_t h1 = splitmix64(key + 2 * e), h2 = splitmix64(key + 2 * e + 1);
      double u1 = (double)((h1 >> 11) + 1) * inv53;
      double u2 = (double)(h2 >> 11) * inv53;
      double z = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
      double s = sigma;
      if (planted && planted[line_axis == 0 ? r : c]) s *= factor;
      out[r * ld + c] = f32_to_bf16_rne((float)(z * s));
    }
  }
  free(planted);
  return 0;
}
