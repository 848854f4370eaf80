/*
 * Seeded synthetic inputs for the GPTQ layer quantizer: weights W and
 * calibration activations X.  Holds none of the quantizer's arithmetic.
 *
 * Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014) used in counter mode: the k-th 64-bit draw
 * of element i of a tensor is mix(key + (4*i + k + 1) * gamma), where mix is
 * SplitMix64's output finaliser and gamma its golden-ratio increment.  Every
 * element is a pure function of (seed, tensor id, element index), so any row
 * range or column subset can be regenerated on its own and gives the same
 * bytes as a whole-tensor pass.
 *
 * Distributions (all evaluated in double precision with the C library's
 * log/cos/sqrt, then rounded to float32 by the hardware cast):
 *   normal : Box-Muller, z = sqrt(-2 ln u1) * cos(2 pi u2)
 *   t4     : Student-t with 4 degrees of freedom, z / sqrt(c / 4) with
 *            c = -2 ln(u3 * u4), a chi-square(4) variate
 * u = (top 53 bits + 0.5) * 2^-53 lies strictly inside (0, 1).
 * bf16 values are the float32 value rounded to nearest-even in its top half.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SM_GAMMA 0x9e3779b97f4a7c15ULL

static inline uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t tensor) {
  return sm_mix(sm_mix(seed + SM_GAMMA) ^ sm_mix(tensor * SM_GAMMA + 0x632be59bd9b4e019ULL));
}

static inline uint64_t draw(uint64_t key, uint64_t idx, unsigned k) {
  return sm_mix(key + (idx * 4u + k + 1u) * SM_GAMMA);
}

static inline double u01(uint64_t z) { return ((double)(z >> 11) + 0.5) * 0x1.0p-53; }

static inline double sample(uint64_t key, uint64_t idx, int dist) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = u01(draw(key, idx, 0)), u2 = u01(draw(key, idx, 1));
  double z = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
  if (dist == 0) return z;
  double u3 = u01(draw(key, idx, 2)), u4 = u01(draw(key, idx, 3));
  double c = -2.0 * log(u3 * u4);
  return z / sqrt(c * 0.25);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  uint32_t lsb = (b >> 16) & 1u;
  return (uint16_t)((b + 0x7fffu + lsb) >> 16);
}

/* Raw 64-bit hashes h[c] = mix(key + (c+1)*gamma), c in [0, n): used to pick
   outlier channels (the k smallest) and per-layer bit widths. */
void synth_hash(uint64_t key, int64_t n, uint64_t* out) {
  for (int64_t c = 0; c < n; ++c) out[c] = sm_mix(key + (uint64_t)(c + 1) * SM_GAMMA);
}

/* Rows [r0, r0+nrows) of a [*, cols] tensor: value = sigma * colscale[c] * sample.
   colscale may be NULL.  out_f32 and/or out_bf16 may be NULL. */
void synth_rows(uint64_t key, int dist, double sigma, const double* colscale, int64_t r0,
                int64_t nrows, int64_t cols, float* out_f32, uint16_t* out_bf16) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; ++r) {
    for (int64_t c = 0; c < cols; ++c) {
      uint64_t idx = (uint64_t)(r0 + r) * (uint64_t)cols + (uint64_t)c;
      double v = sigma * sample(key, idx, dist);
      if (colscale) v *= colscale[c];
      float f = (float)v;
      if (out_f32) out_f32[r * cols + c] = f;
      if (out_bf16) out_bf16[r * cols + c] = f32_to_bf16_rne(f);
    }
  }
}

/* Selected columns of rows [0, nrows) of a [*, cols] tensor, written as
   out[r * ncol + k] for column sel[k]. */
void synth_columns(uint64_t key, int dist, double sigma, const double* colscale, int64_t nrows,
                   int64_t cols, const int64_t* sel, int64_t ncol, float* out_f32,
                   uint16_t* out_bf16) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; ++r) {
    for (int64_t k = 0; k < ncol; ++k) {
      int64_t c = sel[k];
      uint64_t idx = (uint64_t)r * (uint64_t)cols + (uint64_t)c;
      double v = sigma * sample(key, idx, dist);
      if (colscale) v *= colscale[c];
      float f = (float)v;
      if (out_f32) out_f32[r * ncol + k] = f;
      if (out_bf16) out_bf16[r * ncol + k] = f32_to_bf16_rne(f);
    }
  }
}
