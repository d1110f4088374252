/*
 * synth.c -- seeded, counter-based synthetic inputs for the DSA hot path.
 *
 * This file holds NO arithmetic of the method: it only draws numbers.  Both
 * the CPU oracle's inputs and the GPU library's inputs come from here (the GPU
 * receives uploaded copies), so the two sides always see identical bits.
 *
 * Generator: SplitMix64 (S. Vigna, public domain; the output function of
 * Java's SplittableRandom) used counter-style.  Stream (seed, id) has key
 *   key = mix(mix(seed) ^ id * 0xD1B54A32D192ED03)
 * and element i of the stream is mix(key + (i + 1) * 0x9E3779B97F4A7C15).
 * Any slice of any stream can therefore be produced on its own.
 *
 * Normals: Box-Muller (Box & Muller, 1958) in IEEE single precision (the
 * values are rounded to bf16 afterwards).  Elements 2j and 2j+1 share one
 * pair (u1, u2) built from draws 2j and 2j+1:
 *   u1 = (top 24 bits + 1) * 2^-24 in (0, 1],  u2 = top 24 bits * 2^-24,
 *   x_{2j} = sqrt(-2 ln u1) cos(2 pi u2),  x_{2j+1} = sqrt(-2 ln u1) sin(2 pi u2).
 * Uniform reals use the top 24 bits: lo + (hi - lo) * (bits * 2^-24).
 * Uniform integers in [lo, hi] use (top 32 bits * (hi - lo + 1)) >> 32.
 * Values are rounded double -> float (round-to-nearest-even) -> bf16
 * (round-to-nearest-even on the float's bits).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ULL
#define STREAM_MULT 0xD1B54A32D192ED03ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed) ^ (stream * STREAM_MULT));
}

uint64_t synth_draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN_GAMMA); }

static void box_muller(uint64_t key, uint64_t pair, float* c, float* sn) {
  float u1 = (float)((synth_draw(key, 2 * pair) >> 40) + 1) * 0x1p-24f;
  float u2 = (float)(synth_draw(key, 2 * pair + 1) >> 40) * 0x1p-24f;
  float r = sqrtf(-2.0f * logf(u1));
  float a = 6.28318530717958647692f * u2;
  *c = r * cosf(a);
  *sn = r * sinf(a);
}

static double normal_at(uint64_t key, uint64_t i) {
  float c, sn;
  box_muller(key, i >> 1, &c, &sn);
  return (i & 1) ? (double)sn : (double)c;
}

static double uniform_at(uint64_t key, uint64_t i, double lo, double hi) {
  return lo + (hi - lo) * ((double)(synth_draw(key, i) >> 40) * 0x1p-24);
}

static int64_t int_at(uint64_t key, uint64_t i, int64_t lo, int64_t hi) {
  uint64_t span = (uint64_t)(hi - lo + 1);
  return lo + (int64_t)(((synth_draw(key, i) >> 32) * span) >> 32);
}

static uint16_t float_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

uint16_t synth_bf16_from_double(double x) { return float_to_bf16_rne((float)x); }

/* out[i] = bf16(scale * N(0,1)[start + i]); pairs share one Box-Muller draw. */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t start, int64_t count,
                       double scale, uint16_t* out) {
  uint64_t key = synth_stream_key(seed, stream);
  if (count <= 0) return;
  int64_t head = (int64_t)(start & 1);       /* element start is an odd half-pair */
  if (head) {
    out[0] = float_to_bf16_rne((float)(scale * normal_at(key, start)));
  }
  int64_t npairs = (count - head) / 2;
  uint64_t pair0 = (start + (uint64_t)head) >> 1;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < npairs; ++j) {
    float c, sn;
    box_muller(key, pair0 + (uint64_t)j, &c, &sn);
    out[head + 2 * j] = float_to_bf16_rne((float)(scale * (double)c));
    out[head + 2 * j + 1] = float_to_bf16_rne((float)(scale * (double)sn));
  }
  int64_t done = head + 2 * npairs;
  if (done < count) out[done] = float_to_bf16_rne((float)(scale * normal_at(key, start + (uint64_t)done)));
}

/* out[i] = float(N(0,1)[start + i]) (double draw rounded to float) */
void synth_normal_f64(uint64_t seed, uint64_t stream, uint64_t start, int64_t count, double* out) {
  uint64_t key = synth_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = normal_at(key, start + (uint64_t)i);
}

/* out[i] = float(U[lo, hi)[start + i]) */
void synth_uniform_f32(uint64_t seed, uint64_t stream, uint64_t start, int64_t count, double lo,
                       double hi, float* out) {
  uint64_t key = synth_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = (float)uniform_at(key, start + (uint64_t)i, lo, hi);
}

/* out[i] = U[lo, hi)[start + i] in double */
void synth_uniform_f64(uint64_t seed, uint64_t stream, uint64_t start, int64_t count, double lo,
                       double hi, double* out) {
  uint64_t key = synth_stream_key(seed, stream);
  for (int64_t i = 0; i < count; ++i) out[i] = uniform_at(key, start + (uint64_t)i, lo, hi);
}

/* Uniform integers in [lo, hi], stored as bf16 bits (exact for |v| <= 256). */
void synth_int_bf16(uint64_t seed, uint64_t stream, uint64_t start, int64_t count, int64_t lo,
                    int64_t hi, uint16_t* out) {
  uint64_t key = synth_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i)
    out[i] = float_to_bf16_rne((float)int_at(key, start + (uint64_t)i, lo, hi));
}

/* Uniform integers in [lo, hi], stored as float32. */
void synth_int_f32(uint64_t seed, uint64_t stream, uint64_t start, int64_t count, int64_t lo,
                   int64_t hi, float* out) {
  uint64_t key = synth_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = (float)int_at(key, start + (uint64_t)i, lo, hi);
}

/*
 * Block-clustered keys for packed tokens [tok_begin, tok_begin + tok_count).
 * Token t of sequence b (local position s = t - cu[b]) gets, per channel c,
 *   x = N_noise[t * row_len + c] + mean_std * N_mean[(cu[b] + block*floor(s/block)) * row_len + c]
 * so every `block`-token frame of a sequence shares one mean vector.  If
 * (s mod block) < ts_count the token is a timestamp-like token and x is
 * multiplied by ts_scale.  out is bf16 [tok_count, row_len].
 */
void synth_clustered_bf16(uint64_t seed, uint64_t noise_stream, uint64_t mean_stream, int n_seq,
                          const int32_t* cu, int64_t row_len, int64_t block, double mean_std,
                          int64_t ts_count, double ts_scale, int64_t tok_begin, int64_t tok_count,
                          uint16_t* out) {
  uint64_t nkey = synth_stream_key(seed, noise_stream);
  uint64_t mkey = synth_stream_key(seed, mean_stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < tok_count; ++i) {
    int64_t t = tok_begin + i;
    int b = 0;
    while (b + 1 < n_seq && t >= cu[b + 1]) ++b;
    int64_t s = t - cu[b];
    int64_t base = ((int64_t)cu[b] + block * (s / block)) * row_len;
    double mul = (s % block) < ts_count ? ts_scale : 1.0;
    for (int64_t c = 0; c < row_len; ++c) {
      double x = normal_at(nkey, (uint64_t)(t * row_len + c)) +
                 mean_std * normal_at(mkey, (uint64_t)(base + c));
      out[i * row_len + c] = float_to_bf16_rne((float)(mul * x));
    }
  }
}
