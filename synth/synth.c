/*
 * synth.c - seeded, counter-based synthetic inputs for the sparse decode path.
 *
 * This file generates inputs only; it holds none of the selection or
 * attention arithmetic.  Both the CPU oracle and the GPU library consume the
 * bytes it writes, so they see identical inputs.
 *
 * Generator definition (stated so that it can be re-implemented anywhere):
 *   mix(z)      = SplitMix64 output function (Steele, Lea & Flood, 2014):
 *                 z ^= z>>30; z *= 0xBF58476D1CE4E5B9; z ^= z>>27;
 *                 z *= 0x94D049BB133111EB; z ^= z>>31
 *   base(s, t)  = mix(mix(s + GAMMA) ^ (t * 0xD1B54A32D192ED03))
 *   draw(b, i)  = mix(b + (i + 1) * GAMMA),  GAMMA = 0x9E3779B97F4A7C15
 *   u(b, i)     = ((draw(b, i) >> 11) + 0.5) * 2^-53          in (0, 1)
 *   normal pair j of stream b (Box-Muller, double precision):
 *                 r = sqrt(-2 ln u(b, 2j)), th = 2 pi u(b, 2j+1)
 *                 z[2j] = r cos th, z[2j+1] = r sin th
 * Value i of a stream depends only on (seed, tensor id, i), so the result
 * does not depend on the number of threads used to fill a buffer.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ULL;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBULL;
  z ^= z >> 31;
  return z;
}

static inline uint64_t stream_base(uint64_t seed, uint64_t tid) {
  return mix(mix(seed + GAMMA) ^ (tid * 0xD1B54A32D192ED03ULL));
}

static inline double unit_open(uint64_t b, uint64_t i) {
  uint64_t x = mix(b + (i + 1) * GAMMA);
  return ((double)(x >> 11) + 0.5) * 0x1p-53;
}

/* fp32 -> bf16 bits, round to nearest even (inputs are finite). */
static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* fp32 -> IEEE binary16 bits, round to nearest even (finite inputs,
 * overflow saturates to inf as IEEE prescribes). */
static uint16_t f32_to_f16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t sign = (u >> 16) & 0x8000u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x47800000u) { /* >= 65536: beyond the largest finite half after rounding */
    return (uint16_t)(sign | 0x7C00u);
  }
  if (a < 0x38800000u) { /* below 2^-14: half subnormal range (or zero) */
    /* value = a_float; half subnormal unit = 2^-24 */
    float af;
    memcpy(&af, &a, 4);
    float scaled = af * 16777216.0f; /* exact: multiply by 2^24 */
    /* round half to even */
    float fl = floorf(scaled);
    float frac = scaled - fl;
    uint32_t q = (uint32_t)fl;
    if (frac > 0.5f || (frac == 0.5f && (q & 1u))) q += 1u;
    return (uint16_t)(sign | q); /* q == 1024 yields the smallest normal, as required */
  }
  uint32_t exp = (a >> 23) - 127 + 15;
  uint32_t mant = a & 0x7FFFFFu;
  uint32_t h = (exp << 10) | (mant >> 13);
  uint32_t rem = mant & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u; /* carry may bump exponent: correct */
  return (uint16_t)(sign | h);
}

static inline float f16_bits_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t exp = (h >> 10) & 0x1Fu;
  uint32_t mant = h & 0x3FFu;
  float out;
  if (exp == 0) {
    out = (float)mant * 0x1p-24f;
    uint32_t u;
    memcpy(&u, &out, 4);
    u |= sign;
    memcpy(&out, &u, 4);
    return out;
  }
  uint32_t u = sign | ((exp == 31) ? (0xFFu << 23) : ((exp - 15 + 127) << 23)) | (mant << 13);
  memcpy(&out, &u, 4);
  return out;
}

/*
 * Fill n values of stream (seed, tid): x_i = mean + std * z_i, multiplied by
 * chan_scale[i % n_chan] when chan_scale is not NULL, rounded to fp32 and, for
 * out_dtype 1, further to bf16 (RNE).  out_dtype 0 writes float, 1 writes
 * bf16 bits (uint16).  'offset' shifts the stream index, so a tensor can be
 * filled in pieces.
 */
void synth_normal(uint64_t seed, uint64_t tid, uint64_t offset, uint64_t n, double mean,
                  double stdev, const float *chan_scale, uint64_t n_chan, int out_dtype,
                  void *out) {
  uint64_t b = stream_base(seed, tid);
  int64_t npairs_lo = (int64_t)(offset / 2);
  int64_t npairs_hi = (int64_t)((offset + n + 1) / 2);
#pragma omp parallel for schedule(static)
  for (int64_t j = npairs_lo; j < npairs_hi; ++j) {
    double u1 = unit_open(b, 2 * (uint64_t)j);
    double u2 = unit_open(b, 2 * (uint64_t)j + 1);
    double r = sqrt(-2.0 * log(u1));
    double th = 6.283185307179586476925286766559 * u2;
    double z[2] = {r * cos(th), r * sin(th)};
    for (int e = 0; e < 2; ++e) {
      uint64_t i = 2 * (uint64_t)j + (uint64_t)e;
      if (i < offset || i >= offset + n) continue;
      double x = mean + stdev * z[e];
      if (chan_scale) x *= (double)chan_scale[i % n_chan];
      float f = (float)x;
      uint64_t o = i - offset;
      if (out_dtype == 0) {
        ((float *)out)[o] = f;
      } else {
        ((uint16_t *)out)[o] = f32_to_bf16_rne(f);
      }
    }
  }
}

/* n uniform floats in [lo, hi): lo + (hi - lo) * u_i, rounded to fp32. */
void synth_uniform(uint64_t seed, uint64_t tid, uint64_t n, double lo, double hi, float *out) {
  uint64_t b = stream_base(seed, tid);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = (float)(lo + (hi - lo) * unit_open(b, (uint64_t)i));
}

/* n integers uniform in [lo, hi] (inclusive): lo + floor(u_i * (hi - lo + 1)). */
void synth_uniform_int(uint64_t seed, uint64_t tid, uint64_t n, int64_t lo, int64_t hi, int32_t *out) {
  uint64_t b = stream_base(seed, tid);
  double span = (double)(hi - lo + 1);
  for (uint64_t i = 0; i < n; ++i) {
    int64_t v = lo + (int64_t)floor(unit_open(b, i) * span);
    if (v > hi) v = hi;
    out[i] = (int32_t)v;
  }
}

/* Random permutation of 0..n-1 (Fisher-Yates, draw i picks the swap partner
 * for position n-1-i). */
void synth_permutation(uint64_t seed, uint64_t tid, uint64_t n, int32_t *out) {
  uint64_t b = stream_base(seed, tid);
  for (uint64_t i = 0; i < n; ++i) out[i] = (int32_t)i;
  for (uint64_t t = 0; n > 1 && t < n - 1; ++t) {
    uint64_t i = n - 1 - t;
    uint64_t j = (uint64_t)floor(unit_open(b, t) * (double)(i + 1));
    if (j > i) j = i;
    int32_t tmp = out[i];
    out[i] = out[j];
    out[j] = tmp;
  }
}

/*
 * Caller-side int8 KV cache format: rows of row_len fp32 values are
 * quantised symmetrically per row: scale = fp16_rne(amax / 127) (fp32
 * division), code = clamp(rint(x / scale_f32), -127, 127), where scale_f32 is
 * the stored half widened back to fp32.  A row of zeros gets scale 0 and
 * codes 0.
 */
void synth_quant_int8_rows(const float *x, uint64_t rows, int32_t row_len, int8_t *codes,
                           uint16_t *scale_f16) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < (int64_t)rows; ++r) {
    const float *xr = x + (uint64_t)r * (uint64_t)row_len;
    float amax = 0.0f;
    for (int32_t i = 0; i < row_len; ++i) {
      float a = fabsf(xr[i]);
      if (a > amax) amax = a;
    }
    uint16_t sh = f32_to_f16_rne(amax / 127.0f);
    float s = f16_bits_to_f32(sh);
    scale_f16[r] = sh;
    int8_t *cr = codes + (uint64_t)r * (uint64_t)row_len;
    for (int32_t i = 0; i < row_len; ++i) {
      if (s == 0.0f) {
        cr[i] = 0;
        continue;
      }
      float qv = rintf(xr[i] / s);
      if (qv > 127.0f) qv = 127.0f;
      if (qv < -127.0f) qv = -127.0f;
      cr[i] = (int8_t)qv;
    }
  }
}

/* Element-wise conversions used when the generator assembles tensors. */
void synth_f32_to_bf16(const float *x, uint64_t n, uint16_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = f32_to_bf16_rne(x[i]);
}

void synth_f32_to_f16(const float *x, uint64_t n, uint16_t *out) {
  for (uint64_t i = 0; i < n; ++i) out[i] = f32_to_f16_rne(x[i]);
}

void synth_f16_to_f32(const uint16_t *x, uint64_t n, float *out) {
  for (uint64_t i = 0; i < n; ++i) out[i] = f16_bits_to_f32(x[i]);
}

int synth_abi_version(void) { return 1; }
