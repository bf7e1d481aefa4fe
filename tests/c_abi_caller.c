/* A plain C caller of librmsq (test infrastructure): no Python, no torch.  It allocates device
 * buffers with the HIP runtime, runs entry points of include/rmsq.h on them and compares the
 * results with the oracle library's host twins (oracle/rmsq_oracle.h), which only a test may
 * link.  Inputs are synthetic (a xorshift generator and Box-Muller, rounded to bf16 by the
 * oracle's converter).
 *
 *   c_abi_caller validate   host-only checks: argument errors and status strings, no device
 *   c_abi_caller gpu        the device runs and their comparison with the oracle
 * Exit status 0 when every check passes. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rmsq.h"
#include "rmsq_oracle.h"

static int failures = 0;
#define CHECK(cond, ...)                 \
  do {                                   \
    if (!(cond)) {                       \
      fprintf(stderr, "FAIL: ");         \
      fprintf(stderr, __VA_ARGS__);      \
      fprintf(stderr, "\n");             \
      ++failures;                        \
    }                                    \
  } while (0)

#define HIP(call)                                                               \
  do {                                                                          \
    hipError_t e_ = (call);                                                     \
    if (e_ != hipSuccess) {                                                     \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, \
              __LINE__);                                                        \
      exit(2);                                                                  \
    }                                                                           \
  } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double next_uniform(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return ((double)(rng_state >> 11) + 0.5) / 9007199254740992.0;
}
static float next_normal(void) {
  const double u = next_uniform(), v = next_uniform();
  return (float)(sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v));
}
static uint16_t* bf16_array(size_t n, float scale, float offset) {
  uint16_t* a = (uint16_t*)malloc(n * sizeof(uint16_t));
  for (size_t i = 0; i < n; ++i) a[i] = orc_f32_to_bf16(offset + scale * next_normal());
  return a;
}

static void* to_device(const void* host, size_t bytes) {
  void* d = NULL;
  HIP(hipMalloc(&d, bytes ? bytes : 16));
  if (host && bytes) HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}
static void from_device(void* host, const void* dev, size_t bytes) {
  HIP(hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost));
}

/* codes may differ from the oracle only at rounding ties (the sum of squares is reduced in
 * another order); at most 1e-4 of them */
static void compare_codes(const char* what, const uint8_t* a, const uint8_t* b, size_t n) {
  size_t bad = 0;
  for (size_t i = 0; i < n; ++i) bad += a[i] != b[i];
  CHECK(bad * 10000 <= n, "%s: %zu of %zu codes differ", what, bad, n);
  printf("%s: %zu of %zu codes differ\n", what, bad, n);
}

static void fused_case(int mode, int residual, int64_t T, int64_t H, int G, unsigned flags,
                       int64_t ld, float scale_in) {
  const size_t act = (size_t)(T * H);
  uint16_t* x = bf16_array(act, 1.0f, 0.0f);
  uint16_t* r = residual ? bf16_array(act, 1.0f, 0.0f) : NULL;
  uint16_t* w = bf16_array((size_t)H, 0.25f, 1.0f);
  const size_t qbytes = mode == RMSQ_FP4_BLOCK16 ? act / 2 : act;
  size_t sbytes = 0;
  if (mode == RMSQ_FP8_TOKEN) sbytes = (size_t)T * 4;
  if (mode == RMSQ_FP8_GROUP) {
    const size_t el = (flags & RMSQ_SCALE_E8M0_U8) ? 1 : 4;
    sbytes = (flags & RMSQ_SCALE_COLMAJOR) ? (size_t)(H / G) * (size_t)ld * el
                                           : (size_t)(T * (H / G)) * el;
  }
  if (mode == RMSQ_FP4_BLOCK16) sbytes = (size_t)(T * (H / 16));
  uint8_t *q = calloc(qbytes, 1), *qr = calloc(qbytes, 1);
  uint8_t *s = calloc(sbytes + 1, 1), *sr = calloc(sbytes + 1, 1);
  uint16_t *ro = calloc(act, 2), *ror = calloc(act, 2);

  void *dx = to_device(x, act * 2), *dr = residual ? to_device(r, act * 2) : NULL;
  void *dw = to_device(w, (size_t)H * 2), *dq = to_device(NULL, qbytes);
  void *ds = sbytes ? to_device(NULL, sbytes) : NULL;
  void* dro = residual ? to_device(NULL, act * 2) : NULL;
  void* dsc = to_device(&scale_in, 4);
  const int needs_scale = mode == RMSQ_FP8_STATIC || mode == RMSQ_FP4_BLOCK16;
  if (ds) HIP(hipMemset(ds, 0, sbytes));  /* col-major padding columns stay zero */

  const int st = rmsq_fused(dx, dr, dw, 1e-6f, mode, needs_scale ? (const float*)dsc : NULL, dq,
                            ds, dro, T, H, G, flags, ld == T ? 0 : ld, NULL);
  CHECK(st == RMSQ_OK, "rmsq_fused mode %d: %s", mode, rmsq_status_string(st));
  HIP(hipDeviceSynchronize());
  from_device(q, dq, qbytes);
  if (ds) from_device(s, ds, sbytes);
  if (dro) from_device(ro, dro, act * 2);

  const int rs = rmsq_ref_fused(x, r, w, 1e-6f, mode, needs_scale ? &scale_in : NULL, qr,
                                sbytes ? (void*)sr : NULL, residual ? (void*)ror : NULL, T, H, G,
                                flags, ld == T ? 0 : ld);
  CHECK(rs == 0, "rmsq_ref_fused mode %d rejected the arguments", mode);
  char what[96];
  snprintf(what, sizeof what, "fused mode %d residual %d T %lld H %lld G %d flags %u", mode,
           residual, (long long)T, (long long)H, G, flags);
  compare_codes(what, q, qr, qbytes);
  CHECK(memcmp(s, sr, sbytes) == 0, "%s: scales differ", what);
  if (residual) CHECK(memcmp(ro, ror, act * 2) == 0, "%s: residual_out differs", what);

  HIP(hipFree(dx));
  if (dr) HIP(hipFree(dr));
  HIP(hipFree(dw));
  HIP(hipFree(dq));
  if (ds) HIP(hipFree(ds));
  if (dro) HIP(hipFree(dro));
  HIP(hipFree(dsc));
  free(x);
  free(r);
  free(w);
  free(q);
  free(qr);
  free(s);
  free(sr);
  free(ro);
  free(ror);
}

static void fp4_dynamic_case(int64_t T, int64_t H) {
  const size_t act = (size_t)(T * H);
  uint16_t *x = bf16_array(act, 1.0f, 0.0f), *r = bf16_array(act, 1.0f, 0.0f);
  uint16_t* w = bf16_array((size_t)H, 0.25f, 1.0f);
  uint8_t *q = calloc(act / 2, 1), *qr = calloc(act / 2, 1);
  uint8_t *s = calloc(act / 16, 1), *sr = calloc(act / 16, 1);
  uint16_t *ro = calloc(act, 2), *ror = calloc(act, 2);
  float gs = 0.0f, gsr = 0.0f;
  void *dx = to_device(x, act * 2), *dr = to_device(r, act * 2), *dw = to_device(w, H * 2);
  void *dq = to_device(NULL, act / 2), *ds = to_device(NULL, act / 16);
  void *dro = to_device(NULL, act * 2), *dg = to_device(NULL, 4);
  const int st = rmsq_fused_fp4_dynamic(dx, dr, dw, 1e-6f, dq, ds, dro, (float*)dg, T, H, 0, NULL);
  CHECK(st == RMSQ_OK, "rmsq_fused_fp4_dynamic: %s", rmsq_status_string(st));
  HIP(hipDeviceSynchronize());
  from_device(q, dq, act / 2);
  from_device(s, ds, act / 16);
  from_device(ro, dro, act * 2);
  from_device(&gs, dg, 4);
  CHECK(orc_fused_fp4_dynamic(x, r, w, 1e-6f, qr, sr, ror, &gsr, T, H, 0, NULL) == 0,
        "orc_fused_fp4_dynamic rejected the arguments");
  CHECK(memcmp(&gs, &gsr, 4) == 0, "batch global scale differs: %g vs %g", gs, gsr);
  compare_codes("fp4 with a batch global scale", q, qr, act / 2);
  CHECK(memcmp(s, sr, act / 16) == 0, "fp4 batch scale: block scales differ");
  CHECK(memcmp(ro, ror, act * 2) == 0, "fp4 batch scale: residual_out differs");
  hipFree(dx);
  hipFree(dr);
  hipFree(dw);
  hipFree(dq);
  hipFree(ds);
  hipFree(dro);
  hipFree(dg);
  free(x);
  free(r);
  free(w);
  free(q);
  free(qr);
  free(s);
  free(sr);
  free(ro);
  free(ror);
}

static void rope_case(int64_t T, int hq, int hkv, int D, int neox) {
  const int64_t width = (int64_t)(hq + 2 * hkv) * D, mp = 64;
  const size_t n = (size_t)(T * width);
  uint16_t* qkv = bf16_array(n, 1.0f, 0.0f);
  uint16_t* ref = malloc(n * 2);
  memcpy(ref, qkv, n * 2);
  uint16_t *qw = bf16_array((size_t)D, 0.25f, 1.0f), *kw = bf16_array((size_t)D, 0.25f, 1.0f);
  float* cache = malloc((size_t)(mp * D) * 4);
  orc_rope_cache(cache, mp, D, 1e6);
  int64_t* pos = malloc((size_t)T * 8);
  for (int64_t t = 0; t < T; ++t) pos[t] = (int64_t)(next_uniform() * (double)(mp + 4)) - 2;
  void *dq = to_device(qkv, n * 2), *dqw = to_device(qw, D * 2), *dkw = to_device(kw, D * 2);
  void *dc = to_device(cache, (size_t)(mp * D) * 4), *dp = to_device(pos, (size_t)T * 8);
  const int st = rmsq_qk_norm_rope(dq, dqw, dkw, (const float*)dc, (const int64_t*)dp, 1e-6f, T,
                                   hq, hkv, D, mp, neox, 0, NULL);
  CHECK(st == RMSQ_OK, "rmsq_qk_norm_rope: %s", rmsq_status_string(st));
  HIP(hipDeviceSynchronize());
  from_device(qkv, dq, n * 2);
  CHECK(orc_qk_norm_rope(ref, qw, kw, cache, pos, 1e-6f, T, hq, hkv, D, mp, neox, 0) == 0,
        "orc_qk_norm_rope rejected the arguments");
  CHECK(memcmp(qkv, ref, n * 2) == 0, "qk_norm_rope D %d neox %d: results differ", D, neox);
  printf("qk_norm_rope T %lld heads %d+%d D %d neox %d: %s\n", (long long)T, hq, hkv, D, neox,
         memcmp(qkv, ref, n * 2) == 0 ? "bit-exact" : "DIFFERENT");
  hipFree(dq);
  hipFree(dqw);
  hipFree(dkw);
  hipFree(dc);
  hipFree(dp);
  free(qkv);
  free(ref);
  free(qw);
  free(kw);
  free(cache);
  free(pos);
}

static void validate_only(void) {
  /* host-only: status codes through the C ABI, no pointer is dereferenced */
  const uintptr_t X = 0x10000000, R = 0x20000000, W = 0x30000000, Q = 0x40000000,
                  S = 0x50000000, RO = 0x60000000;
  CHECK(rmsq_abi_version() == RMSQ_ABI_VERSION, "ABI version %d", rmsq_abi_version());
  CHECK(rmsq_validate((void*)X, (void*)R, (void*)W, 1e-6f, RMSQ_FP8_TOKEN, NULL, (void*)Q,
                      (void*)S, (void*)RO, 4, 256, 0, 0, 0) == RMSQ_OK,
        "valid arguments refused");
  CHECK(rmsq_validate((void*)(X + 8), (void*)R, (void*)W, 1e-6f, RMSQ_FP8_TOKEN, NULL, (void*)Q,
                      (void*)S, (void*)RO, 4, 256, 0, 0, 0) == RMSQ_EALIGN,
        "misaligned x accepted");
  CHECK(rmsq_validate((void*)X, (void*)R, (void*)W, 1e-6f, RMSQ_FP8_TOKEN, NULL, (void*)X,
                      (void*)S, (void*)RO, 4, 256, 0, 0, 0) == RMSQ_EALIAS,
        "aliased output accepted");
  CHECK(rmsq_fused((void*)X, (void*)R, (void*)W, 0.0f, RMSQ_FP8_TOKEN, NULL, (void*)Q, (void*)S,
                   (void*)RO, 4, 256, 0, 0, 0, NULL) == RMSQ_EINVAL,
        "eps 0 accepted");
  CHECK(strlen(rmsq_status_string(RMSQ_EALIAS)) > 0, "empty status string");
  int64_t grid = 0;
  rmsq_launch l;
  CHECK(rmsq_query_launch(RMSQ_FP8_STATIC, 4096, 4096, 0, 0, &l, &grid) == RMSQ_OK &&
            l.threads_per_row == 256 && l.chunks_per_thread == 2 && grid == 4096,
        "default launch of 4096 x 4096");
}

int main(int argc, char** argv) {
  const int gpu = argc > 1 && strcmp(argv[1], "gpu") == 0;
  validate_only();
  if (gpu) {
    fused_case(RMSQ_FP8_TOKEN, 1, 37, 4096, 0, 0, 37, 0.0f);
    fused_case(RMSQ_FP8_STATIC, 0, 64, 2880, 0, 0, 64, 0.02f);
    fused_case(RMSQ_FP8_GROUP, 1, 21, 7168, 128, RMSQ_SCALE_COLMAJOR, 24, 0.0f);
    fused_case(RMSQ_FP8_GROUP, 1, 9, 5120, 64, RMSQ_SCALE_E8M0_U8, 9, 0.0f);
    fused_case(RMSQ_FP4_BLOCK16, 1, 33, 2048, 16, 0, 33, 300.0f);
    fp4_dynamic_case(40, 2048);
    rope_case(13, 32, 8, 128, 1);
    rope_case(5, 6, 2, 64, 0);
  }
  printf("%s: %d failure(s)\n", gpu ? "gpu" : "validate", failures);
  return failures ? 1 : 0;
}
