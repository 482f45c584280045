/*
 * Seeded synthetic inputs for the latent-MoE layer: normal draws from a
 * counter-based generator, bf16 rounding, and the NVFP4-style two-level
 * quantiser that turns an fp32 weight matrix into e2m1 codes with E4M3
 * per-16 block scales and one fp32 scale per matrix.
 *
 * This file produces inputs only. It decodes no weights and computes no part
 * of the layer; both the CPU oracle and the HIP path consume its bytes.
 *
 * Random numbers: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
 * random numbers: as easy as 1, 2, 3", SC'11), turned into normals with the
 * Box-Muller transform. Element i of a stream (seed, tag, sub) is component
 * i % 4 of Philox(counter = {i/4 low, i/4 high, tag, sub}, key = seed).
 *
 * Formats (OCP Microscaling Formats v1.0 for e2m1, OCP 8-bit Floating Point
 * v1.0 for E4M3): rounding is to nearest, ties to even, saturating.
 *
 * Threads: plain pthreads (no OpenMP runtime, so the library can share a
 * process with torch's bundled one).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- Philox */

static inline void philox4x32_10(const uint32_t in[4], uint32_t seed_lo,
                                 uint32_t seed_hi, uint32_t out[4]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  uint32_t c0 = in[0], c1 = in[1], c2 = in[2], c3 = in[3];
  uint32_t k0 = seed_lo, k1 = seed_hi;
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += W0;
      k1 += W1;
    }
    uint64_t p0 = (uint64_t)M0 * c0;
    uint64_t p1 = (uint64_t)M1 * c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2],
                         uint32_t out[4]) {
  philox4x32_10(ctr, key[0], key[1], out);
}

/* Four standard normals from one Philox block (two Box-Muller pairs),
 * evaluated in single precision. */
static inline void normals4(uint64_t seed, uint32_t tag, uint32_t sub,
                            uint64_t block, float z[4]) {
  uint32_t ctr[4] = {(uint32_t)block, (uint32_t)(block >> 32), tag, sub};
  uint32_t r[4];
  philox4x32_10(ctr, (uint32_t)seed, (uint32_t)(seed >> 32), r);
  const float inv32 = 2.3283064365386963e-10f; /* 2^-32 */
  const float two_pi = 6.2831853071795865f;
  for (int p = 0; p < 2; ++p) {
    /* (r + 0.5) * 2^-32 computed in double so u0 is never 0 or 1 */
    float u0 = (float)(((double)r[2 * p] + 0.5) * (double)inv32);
    float u1 = (float)(((double)r[2 * p + 1] + 0.5) * (double)inv32);
    float rad = sqrtf(-2.0f * logf(u0));
    float sn, cs;
    sincosf(two_pi * u1, &sn, &cs);
    z[2 * p] = rad * cs;
    z[2 * p + 1] = rad * sn;
  }
}

static void fill_normal_f32(uint64_t seed, uint32_t tag, uint32_t sub,
                            float stddev, float *out, int64_t begin,
                            int64_t end) {
  float z[4];
  int64_t i = begin;
  while (i < end) {
    uint64_t block = (uint64_t)i >> 2;
    normals4(seed, tag, sub, block, z);
    int64_t stop = (int64_t)(block + 1) * 4;
    if (stop > end) stop = end;
    for (; i < stop; ++i) out[i - begin] = z[i & 3] * stddev;
  }
}

/* fp32 -> bf16 bits, round to nearest even (inputs are finite). */
static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------ quantiser */

/* E4M3 (fn variant: no infinities, S.1111.111 is NaN, max 448) encoding of a
 * finite v >= 0, round to nearest even, saturating at 448. */
static uint8_t e4m3_encode_rne(float v) {
  if (!(v > 0.0f)) return 0;
  if (v >= 448.0f) return 0x7E;
  if (v < 0.015625f) { /* below 2^-6: subnormals, spacing 2^-9 */
    float m = nearbyintf(v * 512.0f); /* exact scaling, ties to even */
    return (uint8_t)m; /* m == 8 is the smallest normal, code 0x08 */
  }
  int ex;
  float f = frexpf(v, &ex); /* v = f * 2^ex, f in [0.5, 1) */
  int e = ex - 1;           /* v = (2f) * 2^e, 2f in [1, 2) */
  float q = nearbyintf((2.0f * f - 1.0f) * 8.0f);
  int qi = (int)q;
  if (qi == 8) {
    qi = 0;
    e += 1;
  }
  int field = e + 7;
  if (field > 15 || (field == 15 && qi > 6)) return 0x7E;
  return (uint8_t)((field << 3) | qi);
}

/* Value of an E4M3 byte produced by e4m3_encode_rne (never NaN). Needed here
 * only to divide by the scale that was actually stored. */
static float e4m3_value(uint8_t b) {
  int e = (b >> 3) & 15, m = b & 7;
  float mag = (e == 0) ? ldexpf((float)m, -9) : ldexpf(1.0f + m / 8.0f, e - 7);
  return (b & 0x80) ? -mag : mag;
}

/* e2m1 code of v, round to nearest with ties to the even code, saturating at
 * +-6. Magnitudes of codes 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
static inline uint8_t e2m1_encode_rne(float v) {
  float a = fabsf(v);
  /* count of thresholds passed; strict/non-strict picks the even code at ties */
  uint8_t c = (uint8_t)((a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) +
                        (a > 2.5f) + (a >= 3.5f) + (a > 5.0f));
  if (v < 0.0f && c != 0) c |= 8;
  return c;
}

/* Quantise w[N][K] (K % 16 == 0). codes[N][K/2]: element 2j in the low
 * nibble, 2j+1 in the high nibble. scales[N][K/16]. *gscale = amax/(6*448),
 * or 1 when the matrix is all zero. */
void synth_quantize_fp4(const float *w, int64_t N, int64_t K, uint8_t *codes,
                        uint8_t *scales, float *gscale_out) {
  float amax = 0.0f;
  for (int64_t i = 0; i < N * K; ++i) {
    float a = fabsf(w[i]);
    if (a > amax) amax = a;
  }
  float gscale = (amax > 0.0f) ? amax / (6.0f * 448.0f) : 1.0f;
  *gscale_out = gscale;
  const int64_t nb = K / 16;
  for (int64_t n = 0; n < N; ++n) {
    const float *row = w + n * K;
    for (int64_t b = 0; b < nb; ++b) {
      const float *blk = row + b * 16;
      float bmax = 0.0f;
      for (int j = 0; j < 16; ++j) {
        float a = fabsf(blk[j]);
        if (a > bmax) bmax = a;
      }
      uint8_t s = e4m3_encode_rne(bmax / (6.0f * gscale));
      scales[n * nb + b] = s;
      float sv = e4m3_value(s);
      float denom = sv * gscale;
      uint8_t *cdst = codes + n * (K / 2) + b * 8;
      for (int j = 0; j < 8; ++j) {
        uint8_t lo = 0, hi = 0;
        if (sv > 0.0f) {
          lo = e2m1_encode_rne(blk[2 * j] / denom);
          hi = e2m1_encode_rne(blk[2 * j + 1] / denom);
        }
        cdst[j] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}

/* E1M1 (3-bit: sign, 1 exponent bit with bias 1, 1 mantissa bit; magnitudes
 * 0, 0.5, 1, 1.5): magnitude index = round-to-nearest-even of 2|v|, clamped
 * to 3. A zero magnitude is stored with sign 0. */
static inline uint8_t e1m1_encode_rne(float v) {
  float a = fabsf(v);
  uint8_t m = (uint8_t)((a > 0.25f) + (a >= 0.75f) + (a > 1.25f));
  return (uint8_t)(m ? m | ((v < 0.0f) << 2) : 0);
}

/* Quantise one [N][K] matrix to E1M1 codes with E4M3 per-16 block scales and
 * an fp32 matrix scale (the recipe of synth_quantize_fp4 with 1.5 as the
 * largest code magnitude). Codes: per row, K/32 chunks of 12 bytes, chunk c
 * holding elements 32c .. 32c+31 as three little-endian 32-bit words w0, w1,
 * w2. For g = 0, 1, 2, nibble p of w_g (bits 4p .. 4p+3) is element 8g + p as
 * an e2m1 code: sign at bit 3, exponent at bit 1, mantissa at bit 0; its
 * bit 2 (the e2m1 high exponent bit, always clear here) carries one bit of
 * element 24 + p instead: the mantissa in w0, the exponent in w1, the sign
 * in w2. */
void synth_quantize_e1m1(const float *w, int64_t N, int64_t K, uint8_t *codes,
                         uint8_t *scales, float *gscale_out) {
  float amax = 0.0f;
  for (int64_t i = 0; i < N * K; ++i) {
    float a = fabsf(w[i]);
    if (a > amax) amax = a;
  }
  float gscale = (amax > 0.0f) ? amax / (1.5f * 448.0f) : 1.0f;
  *gscale_out = gscale;
  const int64_t nb = K / 16;
  for (int64_t n = 0; n < N; ++n) {
    const float *row = w + n * K;
    for (int64_t c = 0; c < K / 32; ++c) {
      uint32_t word[3] = {0, 0, 0};
      for (int h = 0; h < 2; ++h) {
        const int64_t b = 2 * c + h;
        const float *blk = row + b * 16;
        float bmax = 0.0f;
        for (int j = 0; j < 16; ++j) {
          float a = fabsf(blk[j]);
          if (a > bmax) bmax = a;
        }
        uint8_t s = e4m3_encode_rne(bmax / (1.5f * gscale));
        scales[n * nb + b] = s;
        float denom = e4m3_value(s) * gscale;
        for (int j = 0; j < 16; ++j) {
          uint8_t q = denom > 0.0f ? e1m1_encode_rne(blk[j] / denom) : 0;
          const int i = 16 * h + j, grp = i / 8, pos = i % 8;
          const uint32_t m = q & 1, e = (q >> 1) & 1, sg = (q >> 2) & 1;
          if (grp < 3) {  /* nibble pos of word grp, as an e2m1 code (bit 2 clear) */
            word[grp] |= (m << (4 * pos)) | (e << (4 * pos + 1)) | (sg << (4 * pos + 3));
          } else {        /* bit 2 of nibble pos: mantissa in word 0, exponent 1, sign 2 */
            word[0] |= m << (4 * pos + 2);
            word[1] |= e << (4 * pos + 2);
            word[2] |= sg << (4 * pos + 2);
          }
        }
      }
      uint8_t *dst = codes + n * (K / 32) * 12 + c * 12;
      for (int w = 0; w < 3; ++w)
        for (int b = 0; b < 4; ++b) dst[4 * w + b] = (uint8_t)(word[w] >> (8 * b));
    }
  }
}

/* ------------------------------------------------------------- threading */

typedef struct {
  int kind; /* 0: f32 normals, 1: bf16 normals, 2: fp4 bank, 3: e1m1 bank */
  uint64_t seed;
  uint32_t tag;
  uint32_t sub;
  float stddev;
  void *out;
  int64_t n;
  /* bank */
  int32_t count;
  int64_t N, K;
  uint8_t *codes, *scales;
  float *gscales;
  /* partition */
  int nthreads;
  int tid;
} job_t;

static void *run_job(void *arg) {
  job_t *j = (job_t *)arg;
  if (j->kind == 0 || j->kind == 1) {
    int64_t per = (j->n + j->nthreads - 1) / j->nthreads;
    per = (per + 3) & ~(int64_t)3;
    int64_t begin = per * j->tid, end = begin + per;
    if (end > j->n) end = j->n;
    if (begin >= end) return NULL;
    if (j->kind == 0) {
      fill_normal_f32(j->seed, j->tag, j->sub, j->stddev,
                      (float *)j->out + begin, begin, end);
    } else {
      const int64_t chunk = 1 << 16;
      float *tmp = (float *)malloc(sizeof(float) * chunk);
      uint16_t *dst = (uint16_t *)j->out;
      for (int64_t s = begin; s < end; s += chunk) {
        int64_t e = s + chunk < end ? s + chunk : end;
        fill_normal_f32(j->seed, j->tag, j->sub, j->stddev, tmp, s, e);
        for (int64_t i = s; i < e; ++i) dst[i] = f32_to_bf16_rne(tmp[i - s]);
      }
      free(tmp);
    }
  } else {
    float *buf = (float *)malloc(sizeof(float) * j->N * j->K);
    for (int32_t m = j->tid; m < j->count; m += j->nthreads) {
      fill_normal_f32(j->seed, j->tag, (uint32_t)m, j->stddev, buf, 0,
                      j->N * j->K);
      if (j->kind == 2)
        synth_quantize_fp4(buf, j->N, j->K, j->codes + (int64_t)m * j->N * (j->K / 2),
                           j->scales + (int64_t)m * j->N * (j->K / 16), j->gscales + m);
      else
        synth_quantize_e1m1(buf, j->N, j->K, j->codes + (int64_t)m * j->N * (j->K / 32) * 12,
                            j->scales + (int64_t)m * j->N * (j->K / 16), j->gscales + m);
    }
    free(buf);
  }
  return NULL;
}

static void run_parallel(job_t proto, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  job_t jobs[256];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = proto;
    jobs[t].nthreads = nthreads;
    jobs[t].tid = t;
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, run_job, &jobs[t]);
  run_job(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* ---------------------------------------------------------------- C API */

void synth_normal_f32(uint64_t seed, uint32_t tag, uint32_t sub, float stddev,
                      float *out, int64_t n, int nthreads) {
  job_t j;
  memset(&j, 0, sizeof j);
  j.kind = 0; j.seed = seed; j.tag = tag; j.sub = sub; j.stddev = stddev;
  j.out = out; j.n = n;
  run_parallel(j, nthreads);
}

void synth_normal_bf16(uint64_t seed, uint32_t tag, uint32_t sub, float stddev,
                       uint16_t *out, int64_t n, int nthreads) {
  job_t j;
  memset(&j, 0, sizeof j);
  j.kind = 1; j.seed = seed; j.tag = tag; j.sub = sub; j.stddev = stddev;
  j.out = out; j.n = n;
  run_parallel(j, nthreads);
}

/* count matrices [N][K], matrix m drawn from stream (seed, tag, m). */
void synth_fp4_bank(uint64_t seed, uint32_t tag, int32_t count, int64_t N,
                    int64_t K, float stddev, uint8_t *codes, uint8_t *scales,
                    float *gscales, int nthreads) {
  job_t j;
  memset(&j, 0, sizeof j);
  j.kind = 2; j.seed = seed; j.tag = tag; j.stddev = stddev;
  j.count = count; j.N = N; j.K = K;
  j.codes = codes; j.scales = scales; j.gscales = gscales;
  if (nthreads > count) nthreads = count;
  run_parallel(j, nthreads);
}

void synth_e1m1_bank(uint64_t seed, uint32_t tag, int32_t count, int64_t N,
                     int64_t K, float stddev, uint8_t *codes, uint8_t *scales,
                     float *gscales, int nthreads) {
  job_t j;
  memset(&j, 0, sizeof j);
  j.kind = 3; j.seed = seed; j.tag = tag; j.stddev = stddev;
  j.count = count; j.N = N; j.K = K;
  j.codes = codes; j.scales = scales; j.gscales = gscales;
  if (nthreads > count) nthreads = count;
  run_parallel(j, nthreads);
}

void synth_f32_to_bf16(const float *in, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}
