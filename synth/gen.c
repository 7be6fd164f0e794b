/*
 * Seeded synthetic expert weights for the sparse MoE layer workloads.
 *
 * This is input generation only: it draws N(0, std) weights from a
 * counter-based generator and encodes them into the checkpoint formats the
 * FreeToken pages list for expert weights (page "FreeToken量子化：MoE推論の
 * セットアップガイド", the paragraph on supported precision formats; page
 * "VRAM高騰時代の救世主? ...", section "FreeTokenとは何か", the bullet on
 * MXFP4 / NVFP4 / FP8 / BF16).  Both the GPU library and the CPU oracle consume
 * the bytes written here; neither side's arithmetic lives in this file.
 *
 * Random numbers: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random
 * Numbers: As Easy as 1, 2, 3", SC'11), keyed by the 64-bit seed, with the
 * counter holding (element block, stream).  Each call of the bijection yields
 * four 32-bit words, turned into two pairs of uniforms in (0,1) and then into
 * four standard normals by the Box-Muller transform (computed in float).
 *
 * Encoders (OCP Microscaling Formats v1.0 for MXFP4; OCP OFP8 E4M3FN and the
 * two-level NVFP4 scheme for NVFP4):
 *   MXFP4: per 32 consecutive values along a row, shared exponent
 *          floor(log2(amax)) - 2 (E8M0 code 127 when the block is all zero),
 *          elements rounded to nearest-even on the E2M1 grid, saturating at 6.
 *   NVFP4: per-tensor multiplier g = amax / (6 * 448) (1 when amax is 0);
 *          per 16 values an E4M3 scale s = RNE(amax_block / (6 g)); elements
 *          E2M1(RNE, saturate)(v / (s g)); the dequantised weight is
 *          E2M1 * E4M3(s) * g.
 *   BF16:  round-to-nearest-even of the float32 draw.
 * The MXFP4 and BF16 encoders of one (seed, stream) see the same float draws.
 *
 * Packing: two E2M1 codes per byte, element 2i in the low nibble.
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------- Philox4x32-10 ---------------- */
static inline void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k0;
    uint32_t n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  philox4x32_10(c, key[0], key[1]);
  memcpy(out, c, sizeof c);
}

static inline float u01(uint32_t x) { return ((float)(x >> 8) + 0.5f) * (1.0f / 16777216.0f); }

/* Four normals for element block b of stream s (Box-Muller in float). */
static inline void normal4(uint64_t seed, uint64_t stream, uint64_t b, double z[4]) {
  uint32_t c[4] = {(uint32_t)b, (uint32_t)(b >> 32), (uint32_t)stream, (uint32_t)(stream >> 32)};
  philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  const float two_pi = 6.2831853071795864769f;
  for (int p = 0; p < 2; ++p) {
    float r = sqrtf(-2.0f * logf(u01(c[2 * p])));
    float sn, cs;
    sincosf(two_pi * u01(c[2 * p + 1]), &sn, &cs);
    z[2 * p] = (double)(r * cs);
    z[2 * p + 1] = (double)(r * sn);
  }
}

/* Element i of the stream, scaled by std, as float32. */
static void fill_normal(uint64_t seed, uint64_t stream, float std, float* out, int64_t n) {
  int64_t nb = (n + 3) / 4;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b) {
    double z[4];
    normal4(seed, stream, (uint64_t)b, z);
    for (int j = 0; j < 4; ++j) {
      int64_t i = b * 4 + j;
      if (i < n) out[i] = (float)(z[j] * (double)std);
    }
  }
}

void synth_normal_f32(uint64_t seed, uint64_t stream, float std, float* out, int64_t n) {
  fill_normal(seed, stream, std, out, n);
}

/* ---------------- encoders ---------------- */
static inline uint8_t e2m1_rne_sat(double v) {
  uint8_t sgn = signbit(v) ? 8 : 0;
  double a = fabs(v);
  uint8_t m;
  if (a <= 0.25) m = 0;
  else if (a < 0.75) m = 1;
  else if (a <= 1.25) m = 2;
  else if (a < 1.75) m = 3;
  else if (a <= 2.5) m = 4;
  else if (a < 3.5) m = 5;
  else if (a <= 5.0) m = 6;
  else m = 7;
  return sgn | m;
}

/* Positive value -> E4M3FN code, round to nearest even, saturate at 448. */
static uint8_t e4m3_rne_pos(double v) {
  if (!(v > 0)) return 0;
  if (v >= 448.0) return 0x7E;
  int e;
  frexp(v, &e);          /* v = f * 2^e, f in [0.5,1) */
  int ex = e - 1;        /* floor(log2 v) */
  if (ex < -6) {         /* subnormal grid: m * 2^-9 */
    double q = v * 512.0;
    double r = nearbyint(q); /* default rounding mode: nearest-even */
    int m = (int)r;
    if (m >= 8) return 0x08;
    return (uint8_t)m;
  }
  double frac = v / ldexp(1.0, ex); /* in [1,2) */
  double q = (frac - 1.0) * 8.0;
  int m = (int)nearbyint(q);
  if (m == 8) { m = 0; ex += 1; }
  int code = ((ex + 7) << 3) | m;
  if (code > 0x7E) code = 0x7E;
  return (uint8_t)code;
}

static double e4m3_pos_value(uint8_t c) {
  int e = (c >> 3) & 15, m = c & 7;
  if (e == 0) return ldexp((double)m / 8.0, -6);
  return ldexp(1.0 + (double)m / 8.0, e - 7);
}

static uint16_t bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t bias = 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)((u + bias) >> 16);
}

void synth_weight_bf16(uint64_t seed, uint64_t stream, float std, int rows, int cols, uint16_t* w) {
  int64_t n = (int64_t)rows * cols;
  float* tmp = (float*)malloc(sizeof(float) * (size_t)n);
  fill_normal(seed, stream, std, tmp, n);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) w[i] = bf16_rne(tmp[i]);
  free(tmp);
}

/* q: [rows, cols/2] packed codes; s: [rows, cols/32] E8M0 codes. cols % 32 == 0. */
void synth_weight_mxfp4(uint64_t seed, uint64_t stream, float std, int rows, int cols, uint8_t* q, uint8_t* s) {
  int64_t n = (int64_t)rows * cols;
  float* tmp = (float*)malloc(sizeof(float) * (size_t)n);
  fill_normal(seed, stream, std, tmp, n);
  int nbk = cols / 32;
#pragma omp parallel for schedule(static)
  for (int64_t rb = 0; rb < (int64_t)rows * nbk; ++rb) {
    int64_t r = rb / nbk, b = rb % nbk;
    const float* v = tmp + r * cols + b * 32;
    double amax = 0;
    for (int j = 0; j < 32; ++j) amax = fmax(amax, fabs((double)v[j]));
    int sexp;
    if (amax == 0) sexp = 0;
    else {
      int e;
      frexp(amax, &e);
      sexp = (e - 1) - 2;
      if (sexp < -127) sexp = -127;
      if (sexp > 127) sexp = 127;
    }
    s[r * nbk + b] = (uint8_t)(sexp + 127);
    uint8_t* qq = q + r * (cols / 2) + b * 16;
    for (int j = 0; j < 16; ++j) {
      uint8_t lo = e2m1_rne_sat(ldexp((double)v[2 * j], -sexp));
      uint8_t hi = e2m1_rne_sat(ldexp((double)v[2 * j + 1], -sexp));
      qq[j] = (uint8_t)(lo | (hi << 4));
    }
  }
  free(tmp);
}

/* q: [rows, cols/2]; s: [rows, cols/16] E4M3 codes; *g: dequant multiplier. cols % 16 == 0. */
void synth_weight_nvfp4(uint64_t seed, uint64_t stream, float std, int rows, int cols, uint8_t* q, uint8_t* s, float* g_out) {
  int64_t n = (int64_t)rows * cols;
  float* tmp = (float*)malloc(sizeof(float) * (size_t)n);
  fill_normal(seed, stream, std, tmp, n);
  double amax_t = 0;
  for (int64_t i = 0; i < n; ++i) amax_t = fmax(amax_t, fabs((double)tmp[i]));
  float g = (amax_t == 0) ? 1.0f : (float)(amax_t / (6.0 * 448.0));
  *g_out = g;
  int nbk = cols / 16;
#pragma omp parallel for schedule(static)
  for (int64_t rb = 0; rb < (int64_t)rows * nbk; ++rb) {
    int64_t r = rb / nbk, b = rb % nbk;
    const float* v = tmp + r * cols + b * 16;
    double amax = 0;
    for (int j = 0; j < 16; ++j) amax = fmax(amax, fabs((double)v[j]));
    uint8_t sc = e4m3_rne_pos(amax / (6.0 * (double)g));
    s[r * nbk + b] = sc;
    double denom = e4m3_pos_value(sc) * (double)g;
    uint8_t* qq = q + r * (cols / 2) + b * 8;
    for (int j = 0; j < 8; ++j) {
      uint8_t lo = 0, hi = 0;
      if (sc != 0) {
        lo = e2m1_rne_sat((double)v[2 * j] / denom);
        hi = e2m1_rne_sat((double)v[2 * j + 1] / denom);
      }
      qq[j] = (uint8_t)(lo | (hi << 4));
    }
  }
  free(tmp);
}

/* q: [rows, cols] E4M3FN codes of w / g (round to nearest even, saturating at
   448, sign from w); *g: the per-tensor dequant multiplier amax / 448 (1 if 0). */
void synth_weight_fp8(uint64_t seed, uint64_t stream, float std, int rows, int cols, uint8_t* q, float* g_out) {
  int64_t n = (int64_t)rows * cols;
  float* tmp = (float*)malloc(sizeof(float) * (size_t)n);
  fill_normal(seed, stream, std, tmp, n);
  double amax_t = 0;
  for (int64_t i = 0; i < n; ++i) amax_t = fmax(amax_t, fabs((double)tmp[i]));
  float g = (amax_t == 0) ? 1.0f : (float)(amax_t / 448.0);
  *g_out = g;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double v = (double)tmp[i] / (double)g;
    q[i] = (uint8_t)(e4m3_rne_pos(fabs(v)) | (v < 0 ? 0x80 : 0));
  }
  free(tmp);
}
