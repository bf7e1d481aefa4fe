/*
 * rmsq_oracle.h -- plain CPU oracle for fused (residual add ->) RMSNorm -> FP8/FP4 quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists to check the GPU library against the plain
 * definition of the operation.  Only the test suite, the package smoke check and the CPU-baseline
 * leg of the benchmark may load it; the product path never does.  It shares no code, header,
 * table or constant with the HIP library: every format is decoded here from its bit-field
 * definition and every encoder is a nearest-value search over those decoded values.
 *
 * Sources (cited by page and section; the pages never write the formulas, so the plain
 * textbook readings are used and listed in the design notes):
 *   [P1]  vLLM docs, "Fusion torch.compile passes", section "RMSNorm + quantization
 *         (fuse_norm_quant)": plain RMSNorm -> quant and fused-add RMSNorm -> quant, the latter
 *         updating the residual in place; FP8 static per-tensor, dynamic per-token and dynamic
 *         per-token-group (128/64) schemes.
 *   [P2]  prhub summary of vLLM PR #51925, "Motivation" and "Key source snippet": add-RMSNorm
 *         followed by NVFP4 quantization (block scales, then FP4 conversion, with a global
 *         activation scale supplied by the caller).
 *   [P3]  Blog "[vLLM] Compilation Fusion Passes", sections "Pattern matching structure"
 *         (rms_norm(input, weight, epsilon) -> quant, out-parameter result), the fused-op map
 *         (static per-tensor, dynamic per-token, per-block 128 keys, with and without fused add),
 *         "Type check" (input and weight share one dtype) and "Why this design" (E8M0 and
 *         column-major scale options).
 *
 * Precision: the sum of squares and the reciprocal RMS are taken in binary64; everything that
 * decides a quantized code (the normalized value, the scales, the scaled value fed to the
 * encoder) is binary32, the precision the GPU kernel takes those decisions in.
 * Build with -O2 -ffp-contract=off and without -ffast-math (no FMA contraction, no FTZ/DAZ).
 */
#ifndef RMSQ_ORACLE_H
#define RMSQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Quantization modes (the oracle's own numbering; the GPU library's header is independent). */
enum {
  ORC_FP8_STATIC = 0, /* per-tensor static scale: q = e4m3(y * (1/scale))            [P1][P3] */
  ORC_FP8_TOKEN = 1,  /* dynamic per-token: s = absmax(row)/448                       [P1][P3] */
  ORC_FP8_GROUP = 2,  /* dynamic per-token-group, G in {64,128}: s = absmax(group)/448 [P1][P3] */
  ORC_FP4_BLOCK16 = 3 /* e2m1 codes, 16-element blocks, e4m3 block scale, f32 global  [P2]     */
};
/* Flags for ORC_FP8_GROUP scales ([P3] "Why this design": E8M0 scales, column-major scales). */
enum {
  ORC_SCALE_COLMAJOR = 1u << 0, /* scales stored [H/G][scale_ld], element (t,g) at g*ld + t   */
  ORC_SCALE_E8M0 = 1u << 1,     /* scale rounded up to a power of two, stored as f32           */
  ORC_SCALE_E8M0_U8 = 1u << 2,  /* scale rounded up to a power of two, stored as its E8M0 byte */
  ORC_INPUT_F16 = 1u << 8       /* x, residual, weight, residual_out are IEEE binary16, not bf16 */
};

/* ---- formats (decoded from bit fields; encoders are nearest-value searches) ---- */
float orc_bf16_to_f32(uint16_t b);
uint16_t orc_f32_to_bf16(float v);  /* round to nearest, ties to even significand */
float orc_f16_to_f32(uint16_t b);    /* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa */
uint16_t orc_f32_to_f16(float v);    /* nearest binary16, ties to even, overflow to infinity */
void orc_f32_to_f16_n(const float* v, uint16_t* b, int64_t n);
float orc_e4m3_decode(uint8_t c);   /* OCP e4m3fn; 0x7F/0xFF decode to NaN */
uint8_t orc_e4m3_encode(float v);   /* nearest, ties -> even code, saturate at 448, NaN -> 0x7F */
float orc_e2m1_decode(uint8_t c);   /* low 4 bits used */
uint8_t orc_e2m1_encode(float v);   /* nearest, ties -> even code, saturate at 6, NaN -> 0x7 */
int orc_e8m0_ceil_exp(float s);     /* smallest k >= -127 with 2^k >= s (s >= 0), capped at 127 */

/* Array forms of the converters (for exhaustive checks from the test suite). */
void orc_e4m3_encode_n(const float* v, uint8_t* c, int64_t n);
void orc_e2m1_encode_n(const float* v, uint8_t* c, int64_t n);
void orc_f32_to_bf16_n(const float* v, uint16_t* b, int64_t n);
void orc_e8m0_ceil_exp_n(const float* s, int32_t* k, int64_t n);

/* ---- steps of one row ---- */
/* h = bf16(f32(x) + f32(r)) elementwise; residual_out takes h. */
void orc_residual_add(const uint16_t* x, const uint16_t* r, uint16_t* h, int64_t n);
/* The same three row steps for either 16-bit input type: f16 = 0 bf16, 1 IEEE binary16. */
void orc_residual_add_dt(const uint16_t* x, const uint16_t* r, uint16_t* h, int64_t n, int f16);
float orc_inv_rms_dt(const uint16_t* h, int64_t n, float eps, int f16);
void orc_normalize_dt(const uint16_t* h, const uint16_t* w, float inv, float* y, int64_t n,
                      int f16);
/* inv = 1 / sqrt(mean(h^2) + eps), sum in index order in binary64, result rounded to f32. */
float orc_inv_rms(const uint16_t* h, int64_t n, float eps);
/* y_i = (h_i * inv) * w_i, two binary32 products in that order. */
void orc_normalize(const uint16_t* h, const uint16_t* w, float inv, float* y, int64_t n);

/* Quantize one normalized row y[H] (the step after normalize).  row_scales receives this row's
 * scales contiguously: FP8_TOKEN 1 f32; FP8_GROUP H/G f32 (H/G bytes with E8M0_U8);
 * FP4 H/16 e4m3 bytes; FP8_STATIC none.  q gets H bytes (FP8) or H/2 packed bytes (FP4).
 * Returns 0, or -1 on an invalid mode/group size. */
int orc_quantize_row(const float* y, int64_t H, int mode, float scale_in, int group_size,
                     unsigned flags, uint8_t* q, void* row_scales, float* pre);

/* ---- the whole operation ----
 * x            [T,H] bf16 bits, row-major
 * residual     [T,H] bf16 bits or NULL (plain RMSNorm)
 * weight       [H]   bf16 bits
 * scale_in     FP8_STATIC: the dequant scale (q = y / scale); FP4: the global encode scale gs;
 *              otherwise ignored
 * out_q        FP8: [T,H] e4m3fn bytes; FP4: [T,H/2] bytes, element 2k in the low nibble
 * out_scales   FP8_TOKEN [T] f32; FP8_GROUP [T,H/G] or [H/G,scale_ld] f32 (u8 with E8M0_U8);
 *              FP4 [T,H/16] e4m3 bytes; FP8_STATIC: ignored (may be NULL)
 * residual_out [T,H] bf16 or NULL; must be non-NULL when residual is non-NULL
 * pre_q        optional [T,H] f32: the value each element's code was encoded from (diagnosis)
 * Returns 0 on success, -1 on an invalid argument. */
int orc_fused(const uint16_t* x, const uint16_t* residual, const uint16_t* weight, float eps,
              int mode, float scale_in, uint8_t* out_q, void* out_scales, uint16_t* residual_out,
              int64_t T, int64_t H, int group_size, unsigned flags, int64_t scale_ld,
              float* pre_q);

/* ---- FP4 block-16 with the global encode scale taken from the batch itself (the PR #51925
 * summary's test derives an NVFP4 global scale as 448 * 6 over a tensor's absmax; here the
 * tensor is the normalized batch y of every row). ----
 * orc_fp4_global_scale: (448 * 6) / amax in f32, or FLT_MAX when that exceeds FLT_MAX (amax
 * zero or below 2688 / FLT_MAX).
 * orc_fused_fp4_dynamic: amax = max |y| over all T rows (y exactly as in orc_fused), gs from
 * it, written to *global_scale_out, then orc_fused(ORC_FP4_BLOCK16, scale_in = gs).  flags: 0 or
 * ORC_INPUT_F16.  Returns 0, or -1 on an invalid argument. */
float orc_fp4_global_scale(float amax);
int orc_fused_fp4_dynamic(const uint16_t* x, const uint16_t* residual, const uint16_t* weight,
                          float eps, uint8_t* out_q, uint8_t* out_scales, uint16_t* residual_out,
                          float* global_scale_out, int64_t T, int64_t H, unsigned flags,
                          float* pre_q);

/* The whole operation with the argument list of the GPU library's fused entry point, on host
 * buffers and without a stream: the oracle's counterpart of that call, so that a caller can run
 * both sides of a parity check with one set of arguments.  scale_in points at one f32 (FP8
 * static dequant scale, FP4 global scale) or is NULL for the dynamic modes.  Same behaviour and
 * return value as orc_fused (no pre_q output). */
int rmsq_ref_fused(const void* x, const void* residual, const void* weight, float eps, int mode,
                   const float* scale_in, void* out_q, void* out_scales, void* residual_out,
                   int64_t tokens, int64_t hidden, int group_size, unsigned flags,
                   int64_t scale_ld);

/* ---- residual add + RMSNorm -> padded 16-bit output (vLLM docs "Fusion torch.compile passes",
 * section "RMSNorm + padding (fuse_act_padding)": the residual add and RMSNorm fused with the
 * padding of the hidden dimension to the multiple a downstream GEMM needs; hidden size 2880).
 * out [T, out_ld]: out[t, i] = y_i rounded to the input type (nearest even) for i < H (y as in
 * orc_fused), 0 for H <= i < out_ld.  residual_out as in orc_fused.  flags: 0 (bf16) or
 * ORC_INPUT_F16 (x, residual, weight, residual_out and out IEEE binary16; binary16 rounding
 * overflows to infinity).  Returns 0, or -1 on an invalid argument. */
int orc_rms_norm_pad(const uint16_t* x, const uint16_t* residual, const uint16_t* weight,
                     float eps, uint16_t* out, uint16_t* residual_out, int64_t T, int64_t H,
                     int64_t out_ld, unsigned flags);

/* ---- QK-norm + RoPE (vLLM docs "Fusion torch.compile passes", section "QK Norm + RoPE":
 * for models with per-head Q/K normalization, the per-head RMSNorm of q and k fused with the
 * rotary embedding that follows, on the packed qkv tensor). ----
 * cache [max_pos, D] f32: cache[p, i] = cos(p * base^(-2i/D)), cache[p, D/2 + i] = sin(...),
 * i < D/2, evaluated in binary64 and rounded once to f32. */
void orc_rope_cache(float* cache, int64_t max_pos, int64_t D, double base);
/* qkv [T, (Hq + 2 Hkv) * D] bf16, rewritten in place: for each q head (weight qw [D]) and each
 * k head (weight kw [D]) of token t with 0 <= pos[t] < max_pos:
 *   y = rmsnorm(head) exactly as orc_normalize after orc_inv_rms over the D values,
 *   NeoX (neox != 0): pairs (i, i + D/2); GPT-J: pairs (2i, 2i + 1); with c, s the cache's
 *   cos and sin of the pair's frequency i at position pos[t]:
 *     out_a = a*c - b*s,  out_b = b*c + a*s   (each product rounded to f32, then the sum)
 *   written back rounded to bf16.  v heads and out-of-range tokens are left unchanged.
 * flags: 0, or ORC_INPUT_F16: qkv, qw and kw are IEEE binary16 and the result is rounded to
 * binary16 (nearest even, overflow to infinity).
 * Returns 0, or -1 on an invalid argument (D even, D >= 2). */
int orc_qk_norm_rope(uint16_t* qkv, const uint16_t* qw, const uint16_t* kw, const float* cache,
                     const int64_t* pos, float eps, int64_t T, int64_t Hq, int64_t Hkv,
                     int64_t D, int64_t max_pos, int neox, unsigned flags);

/* ---- SiLU+Mul -> quantization (vLLM docs "Fusion torch.compile passes", section "SiLU+Mul +
 * quantization (fuse_act_quant)": the gated up-projection activation silu_and_mul fused with the
 * quantization that follows; FP8 static per-tensor, FP8 dynamic per-group 128/64, FP4). ----
 * A row of x is [2I] bf16: the gate g = x[0:I], the up projection u = x[I:2I].
 * a_i = silu(g_i) * u_i = g_i * u_i / (1 + exp(-g_i)), evaluated in binary64 and rounded once to
 * f32; a is then quantized exactly like the normalized row of orc_fused. */
float orc_silu_mul(uint16_t g, uint16_t u);
void orc_silu_mul_row(const uint16_t* x, int64_t I, float* a);
/* The same for either 16-bit input type (f16 = 1: IEEE binary16). */
void orc_silu_mul_row_dt(const uint16_t* x, int64_t I, float* a, int f16);
/* x [T, 2I] bf16 (IEEE binary16 with ORC_INPUT_F16 in flags); out_q FP8 [T, I] / FP4 [T, I/2];
 * out_scales laid out as in orc_fused with H = I.  Returns 0, or -1 on an invalid argument. */
int orc_silu_mul_quant(const uint16_t* x, int mode, float scale_in, uint8_t* out_q,
                       void* out_scales, int64_t T, int64_t I, int group_size, unsigned flags,
                       int64_t scale_ld, float* pre_q);

#ifdef __cplusplus
}
#endif
#endif
