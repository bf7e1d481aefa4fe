/* Drives every function of the CPU oracle (oracle/rmsq_oracle.h) over a spread of shapes,
 * modes and edge cases with exactly sized heap buffers, so that a build with AddressSanitizer
 * and UndefinedBehaviorSanitizer reports any out-of-bounds access, use of uninitialized
 * layout assumptions, overflow or invalid shift.  Test infrastructure only: compiled and run by
 * tests/test_oracle_sanitized.py with the host compiler; never part of the library.
 * Exit status 0 when every call returned what its contract says. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rmsq_oracle.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

static uint32_t next_u32(void) {  /* xorshift64*: test input generator only */
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (uint32_t)((g_state * 0x2545F4914F6CDD1Dull) >> 32);
}

static float next_unit(void) { return (float)(next_u32() >> 8) * (1.0f / 16777216.0f); }

static float next_normalish(float scale) {
  /* sum of uniforms: a bell-shaped value of mean 0 */
  float s = 0.0f;
  for (int i = 0; i < 4; ++i) s += next_unit() - 0.5f;
  return s * scale;
}

static void* xalloc(size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}

static uint16_t* bf16_array(int64_t n, float scale) {
  uint16_t* a = (uint16_t*)xalloc((size_t)n * sizeof(uint16_t));
  for (int64_t i = 0; i < n; ++i) a[i] = orc_f32_to_bf16(next_normalish(scale));
  return a;
}

static uint16_t* in16_array(int64_t n, float scale, int f16) {
  if (!f16) return bf16_array(n, scale);
  uint16_t* a = (uint16_t*)xalloc((size_t)n * sizeof(uint16_t));
  for (int64_t i = 0; i < n; ++i) a[i] = orc_f32_to_f16(next_normalish(scale));
  return a;
}

static int failures = 0;
#define EXPECT(cond, ...)                  \
  do {                                     \
    if (!(cond)) {                         \
      fprintf(stderr, __VA_ARGS__);        \
      fprintf(stderr, "\n");               \
      ++failures;                          \
    }                                      \
  } while (0)

static void formats(void) {
  for (int c = 0; c < 256; ++c) {
    const float v = orc_e4m3_decode((uint8_t)c);
    if (v == v) EXPECT(orc_e4m3_encode(v) == c || (v == 0.0f), "e4m3 round trip %d", c);
    (void)orc_e2m1_decode((uint8_t)c);
  }
  for (int i = 0; i < 200000; ++i) {
    uint32_t bits = next_u32();
    float f;
    memcpy(&f, &bits, 4);
    (void)orc_e4m3_encode(f);
    (void)orc_e2m1_encode(f);
    (void)orc_f32_to_bf16(f);
    if (f >= 0.0f) (void)orc_e8m0_ceil_exp(f);
    (void)orc_bf16_to_f32((uint16_t)bits);
    (void)orc_f32_to_f16(f);
    (void)orc_f16_to_f32((uint16_t)bits);
  }
  for (int64_t n = 0; n < 40; n += 7) {
    float* v = (float*)xalloc((size_t)n * 4);
    for (int64_t i = 0; i < n; ++i) v[i] = next_normalish(1000.0f);
    uint8_t* c = (uint8_t*)xalloc((size_t)n);
    uint16_t* b = (uint16_t*)xalloc((size_t)n * 2);
    int32_t* k = (int32_t*)xalloc((size_t)n * 4);
    orc_e4m3_encode_n(v, c, n);
    orc_e2m1_encode_n(v, c, n);
    orc_f32_to_bf16_n(v, b, n);
    for (int64_t i = 0; i < n; ++i) v[i] = fabsf(v[i]);
    orc_e8m0_ceil_exp_n(v, k, n);
    free(v);
    free(c);
    free(b);
    free(k);
  }
}

static size_t scale_bytes(int mode, int64_t T, int64_t H, int G, unsigned flags, int64_t ld) {
  switch (mode) {
    case ORC_FP8_TOKEN: return (size_t)T * 4;
    case ORC_FP8_GROUP: {
      const int64_t ng = H / G;
      const size_t el = (flags & ORC_SCALE_E8M0_U8) ? 1 : 4;
      return (size_t)((flags & ORC_SCALE_COLMAJOR) ? ng * ld : T * ng) * el;
    }
    case ORC_FP4_BLOCK16: return (size_t)T * (size_t)(H / 16);
    default: return 0;
  }
}

static void fused_case(int mode, int residual, int64_t T, int64_t H, int G, unsigned flags) {
  const int64_t ld = (flags & ORC_SCALE_COLMAJOR) ? T + 3 : 0;
  const int f16 = (flags & ORC_INPUT_F16) != 0;
  uint16_t* x = in16_array(T * H, 2.0f, f16);
  uint16_t* r = residual ? in16_array(T * H, 2.0f, f16) : NULL;
  uint16_t* w = in16_array(H, 0.5f, 0);
  for (int64_t i = 0; i < H; ++i) {
    const float wi = 1.0f + orc_bf16_to_f32(w[i]);
    w[i] = f16 ? orc_f32_to_f16(wi) : orc_f32_to_bf16(wi);
  }
  const size_t qb = mode == ORC_FP4_BLOCK16 ? (size_t)(T * H / 2) : (size_t)(T * H);
  uint8_t* q = (uint8_t*)xalloc(qb);
  const size_t sb = scale_bytes(mode, T, H, G, flags, ld);
  void* s = mode != ORC_FP8_STATIC ? xalloc(sb) : NULL;  /* required even when T == 0 */
  uint16_t* ro = residual ? (uint16_t*)xalloc((size_t)(T * H) * 2) : NULL;
  float* pre = (float*)xalloc((size_t)(T * H) * 4);
  const float sc = mode == ORC_FP4_BLOCK16 ? 500.0f : 0.01f;
  const int rc = orc_fused(x, r, w, 1e-6f, mode, sc, q, s, ro, T, H, G, flags, ld, pre);
  EXPECT(rc == 0, "orc_fused mode %d T %lld H %lld G %d flags %u -> %d", mode, (long long)T,
         (long long)H, G, flags, rc);
  /* the same row again through the row-level functions */
  if (T > 0 && rc == 0) {
    float* y = (float*)xalloc((size_t)H * 4);
    uint16_t* h = (uint16_t*)xalloc((size_t)H * 2);
    if (r) orc_residual_add_dt(x, r, h, H, f16);
    else memcpy(h, x, (size_t)H * 2);
    orc_normalize_dt(h, w, orc_inv_rms_dt(h, H, 1e-6f, f16), y, H, f16);
    uint8_t* q1 = (uint8_t*)xalloc(mode == ORC_FP4_BLOCK16 ? (size_t)H / 2 : (size_t)H);
    const size_t rsb = mode == ORC_FP8_TOKEN ? 4
                       : mode == ORC_FP8_GROUP ? (size_t)(H / G) * ((flags & ORC_SCALE_E8M0_U8) ? 1 : 4)
                       : mode == ORC_FP4_BLOCK16 ? (size_t)H / 16 : 0;
    void* s1 = rsb ? xalloc(rsb) : NULL;
    float* p1 = (float*)xalloc((size_t)H * 4);
    EXPECT(orc_quantize_row(y, H, mode, sc, G,
                            flags & ~(unsigned)(ORC_SCALE_COLMAJOR | ORC_INPUT_F16), q1, s1,
                            p1) == 0, "orc_quantize_row");
    EXPECT(memcmp(q1, q, mode == ORC_FP4_BLOCK16 ? (size_t)H / 2 : (size_t)H) == 0,
           "row 0 codes differ from orc_fused");
    free(y);
    free(h);
    free(q1);
    free(s1);
    free(p1);
  }
  free(x);
  free(r);
  free(w);
  free(q);
  free(s);
  free(ro);
  free(pre);
}

static void fused_all(void) {
  const int64_t Ts[] = {0, 1, 3, 17};
  const int64_t Hs[] = {64, 128, 384, 2048};
  for (int ti = 0; ti < 4; ++ti)
    for (int hi = 0; hi < 4; ++hi)
      for (int res = 0; res < 2; ++res) {
        const int64_t T = Ts[ti], H = Hs[hi];
        fused_case(ORC_FP8_STATIC, res, T, H, 0, 0);
        fused_case(ORC_FP8_TOKEN, res, T, H, 0, 0);
        fused_case(ORC_FP8_TOKEN, res, T, H, 0, ORC_INPUT_F16);
        fused_case(ORC_FP4_BLOCK16, res, T, H, 16, 0);
        fused_case(ORC_FP4_BLOCK16, res, T, H, 16, ORC_INPUT_F16);
        for (int G = 64; G <= 128; G *= 2) {
          if (H % G) continue;
          const unsigned fl[] = {0, ORC_SCALE_COLMAJOR, ORC_SCALE_E8M0,
                                 ORC_SCALE_E8M0 | ORC_SCALE_COLMAJOR, ORC_SCALE_E8M0_U8,
                                 ORC_SCALE_E8M0_U8 | ORC_SCALE_COLMAJOR};
          for (int f = 0; f < 6; ++f) fused_case(ORC_FP8_GROUP, res, T, H, G, fl[f]);
        }
      }
  /* invalid arguments come back as -1 without touching memory */
  uint16_t one = 0x3F80;
  uint8_t q = 0;
  EXPECT(orc_fused(&one, NULL, &one, 1e-6f, ORC_FP8_GROUP, 0.0f, &q, NULL, NULL, 1, 8, 0, 0, 0,
                   NULL) == -1, "group size 0 accepted");
  EXPECT(orc_fused(&one, NULL, &one, 1e-6f, 9, 0.0f, &q, NULL, NULL, 1, 8, 0, 0, 0, NULL) == -1,
         "mode 9 accepted");
}

static void pad_all(void) {
  const int64_t Hs[] = {8, 72, 2880};
  const int64_t pads[] = {0, 8, 128};
  for (int hi = 0; hi < 3; ++hi)
    for (int pi = 0; pi < 3; ++pi)
      for (int res = 0; res < 4; ++res) {
        const int f16 = res >> 1;
        const int64_t T = 5, H = Hs[hi], ld = H + pads[pi];
        uint16_t* x = in16_array(T * H, 1.0f, f16);
        uint16_t* r = (res & 1) ? in16_array(T * H, 1.0f, f16) : NULL;
        uint16_t* w = in16_array(H, 1.0f, f16);
        uint16_t* out = (uint16_t*)xalloc((size_t)(T * ld) * 2);
        uint16_t* ro = (res & 1) ? (uint16_t*)xalloc((size_t)(T * H) * 2) : NULL;
        EXPECT(orc_rms_norm_pad(x, r, w, 1e-5f, out, ro, T, H, ld, f16 ? ORC_INPUT_F16 : 0) == 0,
               "orc_rms_norm_pad");
        for (int64_t t = 0; t < T; ++t)
          for (int64_t i = H; i < ld; ++i) EXPECT(out[t * ld + i] == 0, "padding not zero");
        free(x);
        free(r);
        free(w);
        free(out);
        free(ro);
      }
}

static void rope_all(void) {
  const int64_t Ds[] = {2, 8, 64, 128, 256};
  for (int di = 0; di < 5; ++di)
    for (int variant = 0; variant < 4; ++variant) {
      const int neox = variant & 1, f16 = variant >> 1;
      const int64_t D = Ds[di], T = 9, Hq = 4, Hkv = 2, mp = 33;
      float* cache = (float*)xalloc((size_t)(mp * D) * 4);
      orc_rope_cache(cache, mp, D, 10000.0);
      uint16_t* qkv = in16_array(T * (Hq + 2 * Hkv) * D, 3.0f, f16);
      uint16_t* qw = in16_array(D, 1.0f, f16);
      uint16_t* kw = in16_array(D, 1.0f, f16);
      int64_t* pos = (int64_t*)xalloc((size_t)T * 8);
      for (int64_t t = 0; t < T; ++t) pos[t] = (int64_t)(next_u32() % 50) - 8;  /* some out of range */
      EXPECT(orc_qk_norm_rope(qkv, qw, kw, cache, pos, 1e-6f, T, Hq, Hkv, D, mp, neox,
                              f16 ? ORC_INPUT_F16 : 0) == 0,
             "orc_qk_norm_rope D %lld", (long long)D);
      free(cache);
      free(qkv);
      free(qw);
      free(kw);
      free(pos);
    }
  uint16_t h = 0;
  float c = 0.0f;
  int64_t p = 0;
  EXPECT(orc_qk_norm_rope(&h, &h, &h, &c, &p, 1e-6f, 1, 1, 1, 3, 1, 1, 0) == -1, "odd D accepted");
  EXPECT(orc_qk_norm_rope(&h, &h, &h, &c, &p, 1e-6f, 1, 1, 1, 2, 1, 1, 1u) == -1,
         "unknown flag accepted");
}

static void silu_all(void) {
  const int64_t Is[] = {16, 128, 1024};
  for (int ii = 0; ii < 3; ++ii) {
    const int64_t T = 6, I = Is[ii];
    uint16_t* x = bf16_array(T * 2 * I, 6.0f);
    float* a = (float*)xalloc((size_t)I * 4);
    orc_silu_mul_row(x, I, a);
    (void)orc_silu_mul(x[0], x[I]);
    free(a);
    for (int mode = 0; mode < 4; ++mode) {
      const int G = mode == ORC_FP8_GROUP ? 16 : (mode == ORC_FP4_BLOCK16 ? 16 : 0);
      if (mode == ORC_FP8_GROUP && I % 64) continue;
      const int Gm = mode == ORC_FP8_GROUP ? 64 : G;
      const size_t qb = mode == ORC_FP4_BLOCK16 ? (size_t)(T * I / 2) : (size_t)(T * I);
      uint8_t* q = (uint8_t*)xalloc(qb);
      const size_t sb = scale_bytes(mode, T, I, Gm, 0, 0);
      void* s = mode != ORC_FP8_STATIC ? xalloc(sb) : NULL;
      float* pre = (float*)xalloc((size_t)(T * I) * 4);
      EXPECT(orc_silu_mul_quant(x, mode, mode == ORC_FP4_BLOCK16 ? 300.0f : 0.05f, q, s, T, I,
                                Gm, 0, 0, pre) == 0,
             "orc_silu_mul_quant mode %d I %lld", mode, (long long)I);
      free(q);
      free(s);
      free(pre);
    }
    free(x);
  }
}

static void fp4_dynamic_all(void) {
  const int64_t Hs[] = {16, 48, 2048};
  for (int hi = 0; hi < 3; ++hi)
    for (int variant = 0; variant < 4; ++variant) {
      const int res = variant & 1, f16 = variant >> 1;
      const int64_t T = 7, H = Hs[hi];
      uint16_t* x = in16_array(T * H, 2.0f, f16);
      uint16_t* r = res ? in16_array(T * H, 2.0f, f16) : NULL;
      uint16_t* w = in16_array(H, 1.0f, f16);
      uint8_t* q = (uint8_t*)xalloc((size_t)(T * H / 2));
      uint8_t* sf = (uint8_t*)xalloc((size_t)(T * H / 16));
      uint16_t* ro = res ? (uint16_t*)xalloc((size_t)(T * H) * 2) : NULL;
      float* pre = (float*)xalloc((size_t)(T * H) * 4);
      float gs = 0.0f;
      EXPECT(orc_fused_fp4_dynamic(x, r, w, 1e-6f, q, sf, ro, &gs, T, H,
                                   f16 ? ORC_INPUT_F16 : 0, pre) == 0,
             "orc_fused_fp4_dynamic H %lld", (long long)H);
      EXPECT(gs > 0.0f, "global scale not positive");
      free(x);
      free(r);
      free(w);
      free(q);
      free(sf);
      free(ro);
      free(pre);
    }
  uint16_t h = 0;
  uint8_t b = 0;
  float g = 0.0f;
  EXPECT(orc_fused_fp4_dynamic(&h, NULL, &h, 1e-6f, &b, &b, NULL, &g, 1, 8, 0, NULL) == -1,
         "H not a multiple of 16 accepted");
  EXPECT(orc_fused_fp4_dynamic(&h, NULL, &h, 1e-6f, &b, &b, NULL, NULL, 1, 16, 0, NULL) == -1,
         "missing global scale output accepted");
}

int main(void) {
  formats();
  fused_all();
  fp4_dynamic_all();
  pad_all();
  rope_all();
  silu_all();
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("oracle sanitizer driver: all calls ok\n");
  return 0;
}
