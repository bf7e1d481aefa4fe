/*
 * rmsq_oracle.c -- plain, slow, obviously correct CPU oracle (TEST INFRASTRUCTURE ONLY).
 *
 * What is computed, per token row t (sources cited in rmsq_oracle.h):
 *   1. residual add ([P1] "RMSNorm + quantization", fused-add variant; [P2] key source
 *      snippet, x and residual fed to the norm together): h = bf16(x + r), written back as the
 *      new residual.  Without a residual, h = x.
 *   2. RMSNorm ([P3] "Pattern matching structure": rms_norm(input, weight, epsilon)); the
 *      pages never print the formula, the textbook one is used:
 *      y = h / sqrt(mean(h^2) + eps) * w.
 *   3. quantization, one of ([P3] fused-op map and "Why this design"; [P2] "Motivation"):
 *      FP8 static per-tensor, FP8 dynamic per-token, FP8 dynamic per-token-group (64/128,
 *      row- or column-major scales, optional power-of-two E8M0 scales), FP4 e2m1 with
 *      16-element blocks, an e4m3 scale per block and a caller-supplied f32 global scale.
 *
 * Nothing here is blocked, fused or reordered: one row at a time, one element at a time,
 * index order, encoders by exhaustive nearest-value search over the decoded code values.
 */
#include "rmsq_oracle.h"

#include <float.h>
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ bit helpers */
static float u32_as_f32(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static uint32_t f32_as_u32(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

/* ------------------------------------------------------------------ bf16 */
/* bf16 is the upper half of a binary32 pattern. */
float orc_bf16_to_f32(uint16_t b) { return u32_as_f32((uint32_t)b << 16); }

/* Value of a bf16 pattern for rounding-distance purposes: infinity counts as 2^128, the
 * value one step beyond the largest finite bf16 (IEEE overflow rule). */
static double bf16_distance_value(uint16_t b) {
  if ((b & 0x7FFFu) == 0x7F80u) return ldexp(1.0, 128);
  return fabs((double)orc_bf16_to_f32(b));
}

/* Round to nearest bf16 by comparing the two bf16 neighbours of v; ties go to the one whose
 * significand is even (lowest bit 0).  NaN stays NaN (quiet), infinities stay infinite. */
uint16_t orc_f32_to_bf16(float v) {
  uint32_t u = f32_as_u32(v);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  if (isnan(v)) return (uint16_t)(sign | 0x7FC0u);
  if (isinf(v)) return (uint16_t)(sign | 0x7F80u);
  uint16_t lo = (uint16_t)((u >> 16) & 0x7FFFu); /* magnitude truncated toward zero */
  if (((uint32_t)lo << 16) == (u & 0x7FFFFFFFu)) return (uint16_t)(sign | lo); /* exact */
  uint16_t hi = (uint16_t)(lo + 1); /* next magnitude away from zero (may be infinity) */
  double a = fabs((double)v);
  double dlo = a - bf16_distance_value(lo);
  double dhi = bf16_distance_value(hi) - a;
  uint16_t pick;
  if (dlo < dhi) pick = lo;
  else if (dhi < dlo) pick = hi;
  else pick = (lo & 1u) ? hi : lo;
  return (uint16_t)(sign | pick);
}

/* ------------------------------------------------------------------ IEEE binary16 */
/* 1 sign bit, 5 exponent bits (bias 15), 10 mantissa bits; exponent field 0 is subnormal
 * (m * 2^-24); exponent field 31 is infinity (m = 0) or NaN.  Largest finite 65504. */
float orc_f16_to_f32(uint16_t b) {
  int s = (b >> 15) & 1, e = (b >> 10) & 0x1F, m = b & 0x3FF;
  double mag;
  if (e == 0x1F) return m ? NAN : (s ? -INFINITY : INFINITY);
  if (e == 0) mag = ldexp((double)m, -24);
  else mag = ldexp(1.0 + m / 1024.0, e - 15);
  return (float)(s ? -mag : mag);
}

/* Value of a binary16 magnitude code for rounding-distance purposes: infinity (0x7C00) counts
 * as 2^16, one step beyond the largest finite value (IEEE overflow rule). */
static double f16_distance_value(uint16_t code) {
  if (code >= 0x7C00u) return 65536.0;
  return (double)orc_f16_to_f32(code);
}

/* Nearest binary16 by comparing the two neighbours of |v|, found by bisection over the
 * magnitude codes (finite codes are ordered like their values); ties go to the even code. */
uint16_t orc_f32_to_f16(float v) {
  uint16_t sign = signbit(v) ? 0x8000u : 0x0000u;
  if (isnan(v)) return (uint16_t)(sign | 0x7E00u);
  double a = fabs((double)v);
  if (a >= 65536.0) return (uint16_t)(sign | 0x7C00u);
  uint16_t lo = 0, hi = 0x7C00u; /* decode(lo) <= a < value(hi) */
  while (hi - lo > 1) {
    uint16_t mid = (uint16_t)((lo + hi) / 2);
    if (f16_distance_value(mid) <= a) lo = mid;
    else hi = mid;
  }
  if (f16_distance_value(lo) == a) return (uint16_t)(sign | lo);
  double dlo = a - f16_distance_value(lo), dhi = f16_distance_value(hi) - a;
  uint16_t pick;
  if (dlo < dhi) pick = lo;
  else if (dhi < dlo) pick = hi;
  else pick = (lo & 1u) ? hi : lo;
  return (uint16_t)(sign | pick);
}

void orc_f32_to_f16_n(const float* v, uint16_t* b, int64_t n) {
  for (int64_t i = 0; i < n; ++i) b[i] = orc_f32_to_f16(v[i]);
}

/* ------------------------------------------------------------------ e4m3fn (OCP FP8) */
/* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is subnormal
 * (m * 2^-9); S.1111.111 is NaN; there is no infinity.  Largest finite magnitude 448. */
float orc_e4m3_decode(uint8_t c) {
  int s = (c >> 7) & 1, e = (c >> 3) & 0xF, m = c & 7;
  double mag;
  if (e == 0xF && m == 7) return NAN;
  if (e == 0) mag = ldexp((double)m, -9);
  else mag = ldexp(1.0 + m / 8.0, e - 7);
  return (float)(s ? -mag : mag);
}

/* Nearest of the 127 non-negative finite magnitudes (codes 0x00..0x7E), ties to the even
 * code; |v| >= 448 saturates to 448; the sign bit is copied from v (so -0 and negative
 * values that round to zero give 0x80); NaN gives 0x7F. */
uint8_t orc_e4m3_encode(float v) {
  if (isnan(v)) return 0x7F;
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  double a = fabs((double)v);
  if (a >= 448.0) return (uint8_t)(sign | 0x7E);
  int best = 0;
  double bestd = INFINITY;
  for (int k = 0; k <= 0x7E; ++k) {
    double d = fabs(a - (double)orc_e4m3_decode((uint8_t)k));
    if (d < bestd || (d == bestd && (k & 1) == 0)) {
      best = k;
      bestd = d;
    }
  }
  return (uint8_t)(sign | best);
}

/* ------------------------------------------------------------------ e2m1 (FP4) */
/* 1 sign bit (bit 3), 2 exponent bits (bias 1), 1 mantissa bit; exponent field 0 is
 * subnormal (m * 0.5).  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinity or NaN. */
float orc_e2m1_decode(uint8_t c) {
  int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + m / 2.0, e - 1);
  return (float)(s ? -mag : mag);
}

uint8_t orc_e2m1_encode(float v) {
  if (isnan(v)) return 0x7;
  uint8_t sign = signbit(v) ? 0x8 : 0x0;
  double a = fabs((double)v);
  if (a >= 6.0) return (uint8_t)(sign | 0x7);
  int best = 0;
  double bestd = INFINITY;
  for (int k = 0; k <= 7; ++k) {
    double d = fabs(a - (double)orc_e2m1_decode((uint8_t)k));
    if (d < bestd || (d == bestd && (k & 1) == 0)) {
      best = k;
      bestd = d;
    }
  }
  return (uint8_t)(sign | best);
}

/* ------------------------------------------------------------------ E8M0 */
/* E8M0 holds only a biased exponent: byte b means 2^(b-127).  A scale is rounded UP to
 * the next power of two so that no scaled element exceeds the FP8 range. */
int orc_e8m0_ceil_exp(float s) {
  for (int k = -127; k < 127; ++k)
    if (ldexp(1.0, k) >= (double)s) return k;
  return 127;
}

void orc_e4m3_encode_n(const float* v, uint8_t* c, int64_t n) {
  for (int64_t i = 0; i < n; ++i) c[i] = orc_e4m3_encode(v[i]);
}
void orc_e2m1_encode_n(const float* v, uint8_t* c, int64_t n) {
  for (int64_t i = 0; i < n; ++i) c[i] = orc_e2m1_encode(v[i]);
}
void orc_f32_to_bf16_n(const float* v, uint16_t* b, int64_t n) {
  for (int64_t i = 0; i < n; ++i) b[i] = orc_f32_to_bf16(v[i]);
}
void orc_e8m0_ceil_exp_n(const float* s, int32_t* k, int64_t n) {
  for (int64_t i = 0; i < n; ++i) k[i] = orc_e8m0_ceil_exp(s[i]);
}

/* ------------------------------------------------------------------ row steps */
static float in16_to_f32(uint16_t b, int f16) { return f16 ? orc_f16_to_f32(b) : orc_bf16_to_f32(b); }
static uint16_t f32_to_in16(float v, int f16) { return f16 ? orc_f32_to_f16(v) : orc_f32_to_bf16(v); }

void orc_residual_add_dt(const uint16_t* x, const uint16_t* r, uint16_t* h, int64_t n, int f16) {
  for (int64_t i = 0; i < n; ++i) {
    float sum = in16_to_f32(x[i], f16) + in16_to_f32(r[i], f16);
    h[i] = f32_to_in16(sum, f16);
  }
}

void orc_residual_add(const uint16_t* x, const uint16_t* r, uint16_t* h, int64_t n) {
  orc_residual_add_dt(x, r, h, n, 0);
}

float orc_inv_rms_dt(const uint16_t* h, int64_t n, float eps, int f16) {
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    double v = (double)in16_to_f32(h[i], f16);
    ss += v * v;
  }
  return (float)(1.0 / sqrt(ss / (double)n + (double)eps));
}

float orc_inv_rms(const uint16_t* h, int64_t n, float eps) { return orc_inv_rms_dt(h, n, eps, 0); }

void orc_normalize_dt(const uint16_t* h, const uint16_t* w, float inv, float* y, int64_t n,
                      int f16) {
  for (int64_t i = 0; i < n; ++i) {
    float t = in16_to_f32(h[i], f16) * inv;
    y[i] = t * in16_to_f32(w[i], f16);
  }
}

void orc_normalize(const uint16_t* h, const uint16_t* w, float inv, float* y, int64_t n) {
  orc_normalize_dt(h, w, inv, y, n, 0);
}

static float absmax(const float* y, int64_t n) {
  float a = 0.0f;
  for (int64_t i = 0; i < n; ++i)
    if (fabsf(y[i]) > a) a = fabsf(y[i]);
  return a;
}

/* ------------------------------------------------------------------ quantizers (one row) */
/* The value an element's code is encoded from: the element times the reciprocal scale (FP8)
 * or the block multiplier (FP4).  A zero element stays the zero it is, sign included, whatever
 * the multiplier: scaling zero gives zero, also where the multiplier has overflowed to infinity
 * (a scale below 1/FLT_MAX), where the literal product 0 * inf would be NaN. */
static float scaled(float y, float mul) { return (y == 0.0f) ? y : y * mul; }

static void quant_static(const float* y, int64_t H, float scale, uint8_t* q, float* pre) {
  float r = 1.0f / scale;
  for (int64_t i = 0; i < H; ++i) {
    float v = scaled(y[i], r);
    q[i] = orc_e4m3_encode(v);
    if (pre) pre[i] = v;
  }
}

/* Shared by the per-token (one group = the row) and per-group modes: the scale is the
 * group's absmax over the FP8 maximum 448; a zero scale gives zero codes. */
static float quant_group_fp8(const float* y, int64_t n, int e8m0, uint8_t* q, float* pre,
                             int* e8m0_byte) {
  float a = absmax(y, n);
  float s = a / 448.0f;
  float s_raw = s;
  if (e8m0) {
    int k = orc_e8m0_ceil_exp(s);
    s = ldexpf(1.0f, k);
    *e8m0_byte = k + 127;
  }
  if (s_raw == 0.0f) {
    for (int64_t i = 0; i < n; ++i) {
      q[i] = 0x00;
      if (pre) pre[i] = 0.0f;
    }
    return s;
  }
  float r = 1.0f / s;
  for (int64_t i = 0; i < n; ++i) {
    float v = scaled(y[i], r);
    q[i] = orc_e4m3_encode(v);
    if (pre) pre[i] = v;
  }
  return s;
}

/* FP4: block scale sf = e4m3(absmax * gs / 6), element multiplier m = gs / decode(sf). */
static void quant_fp4(const float* y, int64_t H, float gs, uint8_t* qrow, uint8_t* sfrow,
                      float* pre) {
  for (int64_t b = 0; b < H / 16; ++b) {
    const float* yb = y + b * 16;
    float a = absmax(yb, 16);
    uint8_t sf = orc_e4m3_encode((a * gs) / 6.0f);
    float d = orc_e4m3_decode(sf);
    sfrow[b] = sf;
    uint8_t codes[16];
    if (d > 0.0f) {
      float m = gs / d;
      for (int i = 0; i < 16; ++i) {
        float v = scaled(yb[i], m);
        codes[i] = orc_e2m1_encode(v);
        if (pre) pre[b * 16 + i] = v;
      }
    } else {
      for (int i = 0; i < 16; ++i) {
        codes[i] = 0;
        if (pre) pre[b * 16 + i] = 0.0f;
      }
    }
    for (int k = 0; k < 8; ++k)
      qrow[b * 8 + k] = (uint8_t)(codes[2 * k] | (codes[2 * k + 1] << 4));
  }
}

/* ------------------------------------------------------------------ one row's quantizer */
int orc_quantize_row(const float* y, int64_t H, int mode, float scale_in, int group_size,
                     unsigned flags, uint8_t* q, void* row_scales, float* pre) {
  if (mode == ORC_FP8_STATIC) {
    quant_static(y, H, scale_in, q, pre);
  } else if (mode == ORC_FP8_TOKEN) {
    int unused = 0;
    ((float*)row_scales)[0] = quant_group_fp8(y, H, 0, q, pre, &unused);
  } else if (mode == ORC_FP8_GROUP) {
    if ((group_size != 64 && group_size != 128) || H % group_size) return -1;
    int e8m0 = (flags & (ORC_SCALE_E8M0 | ORC_SCALE_E8M0_U8)) != 0;
    int64_t G = group_size;
    for (int64_t g = 0; g < H / G; ++g) {
      int byte = 0;
      float s = quant_group_fp8(y + g * G, G, e8m0, q + g * G, pre ? pre + g * G : NULL, &byte);
      if (flags & ORC_SCALE_E8M0_U8) ((uint8_t*)row_scales)[g] = (uint8_t)byte;
      else ((float*)row_scales)[g] = s;
    }
  } else if (mode == ORC_FP4_BLOCK16) {
    if (group_size != 16 || H % 16) return -1;
    quant_fp4(y, H, scale_in, q, (uint8_t*)row_scales, pre);
  } else {
    return -1;
  }
  return 0;
}

/* ------------------------------------------------------------------ whole operation */
int orc_fused(const uint16_t* x, const uint16_t* residual, const uint16_t* weight, float eps,
              int mode, float scale_in, uint8_t* out_q, void* out_scales, uint16_t* residual_out,
              int64_t T, int64_t H, int group_size, unsigned flags, int64_t scale_ld,
              float* pre_q) {
  if (T < 0 || H <= 0 || !x || !weight || !out_q) return -1;
  if ((residual == NULL) != (residual_out == NULL)) return -1;
  if (!(eps >= 0.0f) || isinf(eps)) return -1;
  if (scale_ld == 0) scale_ld = T;
  switch (mode) {
    case ORC_FP8_STATIC:
      break;
    case ORC_FP8_TOKEN:
      if (!out_scales) return -1;
      break;
    case ORC_FP8_GROUP:
      if (!out_scales || (group_size != 64 && group_size != 128) || H % group_size) return -1;
      if (scale_ld < T) return -1;
      break;
    case ORC_FP4_BLOCK16:
      if (!out_scales || group_size != 16 || H % 16) return -1;
      break;
    default:
      return -1;
  }

  uint16_t* h = (uint16_t*)malloc((size_t)H * sizeof(uint16_t));
  float* y = (float*)malloc((size_t)H * sizeof(float));
  float* sc = (float*)malloc((size_t)H * sizeof(float)); /* one row's scales */
  if (!h || !y || !sc) {
    free(h);
    free(y);
    free(sc);
    return -1;
  }

  const int f16 = (flags & ORC_INPUT_F16) != 0;
  for (int64_t t = 0; t < T; ++t) {
    if (residual) {
      orc_residual_add_dt(x + t * H, residual + t * H, h, H, f16);
      memcpy(residual_out + t * H, h, (size_t)H * sizeof(uint16_t));
    } else {
      memcpy(h, x + t * H, (size_t)H * sizeof(uint16_t));
    }
    float inv = orc_inv_rms_dt(h, H, eps, f16);
    orc_normalize_dt(h, weight, inv, y, H, f16);
    uint8_t* qrow = out_q + t * (mode == ORC_FP4_BLOCK16 ? H / 2 : H);
    orc_quantize_row(y, H, mode, scale_in, group_size, flags & ~(unsigned)ORC_INPUT_F16, qrow, sc,
                     pre_q ? pre_q + t * H : NULL);

    /* place this row's scales */
    if (mode == ORC_FP8_TOKEN) {
      ((float*)out_scales)[t] = sc[0];
    } else if (mode == ORC_FP8_GROUP) {
      int64_t ng = H / group_size;
      for (int64_t g = 0; g < ng; ++g) {
        int64_t idx = (flags & ORC_SCALE_COLMAJOR) ? g * scale_ld + t : t * ng + g;
        if (flags & ORC_SCALE_E8M0_U8) ((uint8_t*)out_scales)[idx] = ((uint8_t*)sc)[g];
        else ((float*)out_scales)[idx] = sc[g];
      }
    } else if (mode == ORC_FP4_BLOCK16) {
      memcpy((uint8_t*)out_scales + t * (H / 16), sc, (size_t)(H / 16));
    }
  }
  free(h);
  free(y);
  free(sc);
  return 0;
}

/* ------------------------------------------------------------------ FP4, batch global scale */
float orc_fp4_global_scale(float amax) {
  /* the largest e4m3 magnitude times the largest e2m1 magnitude, over the batch's absmax */
  const float gs = (448.0f * 6.0f) / amax;
  return (gs <= FLT_MAX) ? gs : FLT_MAX; /* amax == 0 (gs = inf) or tinier than 2688 / FLT_MAX */
}

int orc_fused_fp4_dynamic(const uint16_t* x, const uint16_t* residual, const uint16_t* weight,
                          float eps, uint8_t* out_q, uint8_t* out_scales, uint16_t* residual_out,
                          float* global_scale_out, int64_t T, int64_t H, unsigned flags,
                          float* pre_q) {
  if (T < 0 || H <= 0 || (H % 16) || !x || !weight || !out_q || !out_scales || !global_scale_out)
    return -1;
  if ((residual == NULL) != (residual_out == NULL)) return -1;
  if (!(eps >= 0.0f) || isinf(eps)) return -1;
  if (flags & ~(unsigned)ORC_INPUT_F16) return -1;
  const int f16 = (flags & ORC_INPUT_F16) != 0;
  uint16_t* h = (uint16_t*)malloc((size_t)H * sizeof(uint16_t));
  float* y = (float*)malloc((size_t)H * sizeof(float));
  if (!h || !y) {
    free(h);
    free(y);
    return -1;
  }
  /* pass 1: the largest |y| of the whole batch */
  float amax = 0.0f;
  for (int64_t t = 0; t < T; ++t) {
    if (residual) orc_residual_add_dt(x + t * H, residual + t * H, h, H, f16);
    else memcpy(h, x + t * H, (size_t)H * sizeof(uint16_t));
    orc_normalize_dt(h, weight, orc_inv_rms_dt(h, H, eps, f16), y, H, f16);
    for (int64_t i = 0; i < H; ++i) amax = fmaxf(amax, fabsf(y[i]));
  }
  free(h);
  free(y);
  const float gs = orc_fp4_global_scale(amax);
  *global_scale_out = gs;
  /* pass 2: the block-16 quantization with that global scale */
  return orc_fused(x, residual, weight, eps, ORC_FP4_BLOCK16, gs, out_q, out_scales, residual_out,
                   T, H, 16, flags, 0, pre_q);
}

/* ------------------------------------------------------------------ host twin of rmsq_fused */
int rmsq_ref_fused(const void* x, const void* residual, const void* weight, float eps, int mode,
                   const float* scale_in, void* out_q, void* out_scales, void* residual_out,
                   int64_t tokens, int64_t hidden, int group_size, unsigned flags,
                   int64_t scale_ld) {
  const int needs_scale = mode == ORC_FP8_STATIC || mode == ORC_FP4_BLOCK16;
  if (needs_scale && !scale_in) return -1;
  return orc_fused((const uint16_t*)x, (const uint16_t*)residual, (const uint16_t*)weight, eps,
                   mode, needs_scale ? *scale_in : 0.0f, (uint8_t*)out_q, out_scales,
                   (uint16_t*)residual_out, tokens, hidden, group_size, flags, scale_ld, NULL);
}

int orc_rms_norm_pad(const uint16_t* x, const uint16_t* residual, const uint16_t* weight,
                     float eps, uint16_t* out, uint16_t* residual_out, int64_t T, int64_t H,
                     int64_t out_ld, unsigned flags) {
  if (T < 0 || H <= 0 || out_ld < H || !x || !weight || !out) return -1;
  if (flags & ~(unsigned)ORC_INPUT_F16) return -1;
  const int f16 = (flags & ORC_INPUT_F16) != 0;
  if ((residual == NULL) != (residual_out == NULL)) return -1;
  if (!(eps >= 0.0f) || isinf(eps)) return -1;
  uint16_t* h = (uint16_t*)malloc((size_t)H * sizeof(uint16_t));
  float* y = (float*)malloc((size_t)H * sizeof(float));
  if (!h || !y) {
    free(h);
    free(y);
    return -1;
  }
  for (int64_t t = 0; t < T; ++t) {
    if (residual) {
      orc_residual_add_dt(x + t * H, residual + t * H, h, H, f16);
      memcpy(residual_out + t * H, h, (size_t)H * sizeof(uint16_t));
    } else {
      memcpy(h, x + t * H, (size_t)H * sizeof(uint16_t));
    }
    orc_normalize_dt(h, weight, orc_inv_rms_dt(h, H, eps, f16), y, H, f16);
    for (int64_t i = 0; i < out_ld; ++i) out[t * out_ld + i] = i < H ? f32_to_in16(y[i], f16) : 0;
  }
  free(h);
  free(y);
  return 0;
}

/* ------------------------------------------------------------------ QK-norm + RoPE */
void orc_rope_cache(float* cache, int64_t max_pos, int64_t D, double base) {
  for (int64_t p = 0; p < max_pos; ++p)
    for (int64_t i = 0; i < D / 2; ++i) {
      double theta = (double)p * pow(base, -2.0 * (double)i / (double)D);
      cache[p * D + i] = (float)cos(theta);
      cache[p * D + D / 2 + i] = (float)sin(theta);
    }
}

static void rotate_pair(float a, float b, float c, float s, float* out_a, float* out_b) {
  float ac = a * c, bs = b * s, bc = b * c, as = a * s;
  *out_a = ac - bs;
  *out_b = bc + as;
}

int orc_qk_norm_rope(uint16_t* qkv, const uint16_t* qw, const uint16_t* kw, const float* cache,
                     const int64_t* pos, float eps, int64_t T, int64_t Hq, int64_t Hkv,
                     int64_t D, int64_t max_pos, int neox, unsigned flags) {
  if (T < 0 || Hq < 0 || Hkv < 0 || D < 2 || (D % 2) || !qkv || !qw || !kw || !cache || !pos)
    return -1;
  if (flags & ~(unsigned)ORC_INPUT_F16) return -1;
  const int f16 = (flags & ORC_INPUT_F16) != 0;
  if (!(eps >= 0.0f) || isinf(eps)) return -1;
  float* y = (float*)malloc((size_t)D * sizeof(float));
  float* o = (float*)malloc((size_t)D * sizeof(float));
  if (!y || !o) {
    free(y);
    free(o);
    return -1;
  }
  const int64_t width = (Hq + 2 * Hkv) * D;
  for (int64_t t = 0; t < T; ++t) {
    if (pos[t] < 0 || pos[t] >= max_pos) continue;
    const float* cs = cache + pos[t] * D;
    for (int64_t hd = 0; hd < Hq + Hkv; ++hd) {
      uint16_t* head = qkv + t * width + hd * D;
      orc_normalize_dt(head, hd < Hq ? qw : kw, orc_inv_rms_dt(head, D, eps, f16), y, D, f16);
      for (int64_t i = 0; i < D / 2; ++i) {
        int64_t ia = neox ? i : 2 * i, ib = neox ? i + D / 2 : 2 * i + 1;
        rotate_pair(y[ia], y[ib], cs[i], cs[D / 2 + i], &o[ia], &o[ib]);
      }
      for (int64_t i = 0; i < D; ++i) head[i] = f32_to_in16(o[i], f16);
    }
  }
  free(y);
  free(o);
  return 0;
}

/* ------------------------------------------------------------------ SiLU+Mul -> quant */
static float silu_mul_values(double gd, double ud) { return (float)(gd * ud / (1.0 + exp(-gd))); }

float orc_silu_mul(uint16_t g, uint16_t u) {
  return silu_mul_values((double)orc_bf16_to_f32(g), (double)orc_bf16_to_f32(u));
}

void orc_silu_mul_row_dt(const uint16_t* x, int64_t I, float* a, int f16) {
  for (int64_t i = 0; i < I; ++i)
    a[i] = silu_mul_values((double)in16_to_f32(x[i], f16), (double)in16_to_f32(x[I + i], f16));
}

void orc_silu_mul_row(const uint16_t* x, int64_t I, float* a) { orc_silu_mul_row_dt(x, I, a, 0); }

int orc_silu_mul_quant(const uint16_t* x, int mode, float scale_in, uint8_t* out_q,
                       void* out_scales, int64_t T, int64_t I, int group_size, unsigned flags,
                       int64_t scale_ld, float* pre_q) {
  if (T < 0 || I <= 0 || !x || !out_q) return -1;
  if (scale_ld == 0) scale_ld = T;
  switch (mode) {
    case ORC_FP8_STATIC:
      break;
    case ORC_FP8_TOKEN:
      if (!out_scales) return -1;
      break;
    case ORC_FP8_GROUP:
      if (!out_scales || (group_size != 64 && group_size != 128) || I % group_size) return -1;
      if (scale_ld < T) return -1;
      break;
    case ORC_FP4_BLOCK16:
      if (!out_scales || group_size != 16 || I % 16) return -1;
      break;
    default:
      return -1;
  }
  float* a = (float*)malloc((size_t)I * sizeof(float));
  float* sc = (float*)malloc((size_t)I * sizeof(float));
  if (!a || !sc) {
    free(a);
    free(sc);
    return -1;
  }
  const int f16 = (flags & ORC_INPUT_F16) != 0;
  for (int64_t t = 0; t < T; ++t) {
    orc_silu_mul_row_dt(x + t * 2 * I, I, a, f16);
    uint8_t* qrow = out_q + t * (mode == ORC_FP4_BLOCK16 ? I / 2 : I);
    orc_quantize_row(a, I, mode, scale_in, group_size, flags & ~(unsigned)ORC_INPUT_F16, qrow, sc,
                     pre_q ? pre_q + t * I : NULL);
    if (mode == ORC_FP8_TOKEN) {
      ((float*)out_scales)[t] = sc[0];
    } else if (mode == ORC_FP8_GROUP) {
      int64_t ng = I / group_size;
      for (int64_t g = 0; g < ng; ++g) {
        int64_t idx = (flags & ORC_SCALE_COLMAJOR) ? g * scale_ld + t : t * ng + g;
        if (flags & ORC_SCALE_E8M0_U8) ((uint8_t*)out_scales)[idx] = ((uint8_t*)sc)[g];
        else ((float*)out_scales)[idx] = sc[g];
      }
    } else if (mode == ORC_FP4_BLOCK16) {
      memcpy((uint8_t*)out_scales + t * (I / 16), sc, (size_t)(I / 16));
    }
  }
  free(a);
  free(sc);
  return 0;
}
