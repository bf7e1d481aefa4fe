/*
 * rmsq.h -- C ABI of librmsq: fused (residual add ->) RMSNorm -> FP8 / FP4 quantization on
 * AMD MI355X (gfx950).
 *
 * The operation, per token row t of a row-major [T, H] bf16 activation (sources: vLLM docs
 * "Fusion torch.compile passes", section "RMSNorm + quantization (fuse_norm_quant)"; blog
 * "[vLLM] Compilation Fusion Passes", sections "Pattern matching structure", the fused-op map
 * and "Why this design"; prhub summary of vLLM PR #51925, "Motivation" and "Key source
 * snippet"):
 *
 *   h      = bf16(x + residual)          fused-add form; h is written back as the new residual
 *          = x                           plain form (residual == NULL)
 *   inv    = 1 / sqrt(sum(h^2)/H + eps)  sum and root in binary64, inv rounded to binary32
 *   y      = (h * inv) * weight          binary32, never stored
 *   codes  = quantize(y)                 FP8 e4m3fn (OCP, max 448) or FP4 e2m1 (max 6), round to
 *                                        nearest even, saturating
 *
 * Quantization modes (the pages' quant keys: static per-tensor, dynamic per-token, dynamic
 * per-token-group 128/64; NVFP4-style block-16):
 *   RMSQ_FP8_STATIC   q = e4m3(y * (1/scale)); scale = *scale_in, the dequant scale
 *   RMSQ_FP8_TOKEN    s_t = absmax(y_t)/448 (f32), q = e4m3(y * (1/s_t)); s_t = 0 gives 0 codes
 *   RMSQ_FP8_GROUP    per group of G in {64,128}: s = absmax/448, optionally rounded up to a
 *                     power of two (E8M0); a zero group (absmax/448 == 0) gives 0 codes
 *   RMSQ_FP4_BLOCK16  per 16-element block: sf = e4m3(absmax * gs / 6), d = decode(sf),
 *                     q = e2m1(y * (gs / d)), 0 codes when d == 0; gs = *scale_in, the global
 *                     encode scale (dequant: value = e2m1 * d / gs)
 * In every mode a zero element (y = +0 or -0) gives the zero code of its sign, also where the
 * reciprocal scale 1/s or the FP4 multiplier gs/d overflows to infinity (a scale below
 * 1/FLT_MAX); every other element times an infinite multiplier saturates.
 *
 * Ownership and threading: the caller owns every buffer.  The library never allocates, frees
 * or synchronizes; work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and all
 * pointers except where noted are DEVICE pointers.  Argument errors are returned synchronously
 * before anything is enqueued.  No C++ exception crosses this boundary.  Calls are thread-safe.
 * Library state: one process-wide table remembers, per HIP device index below 64, whether that
 * device is a gfx950 (read with hipGetDeviceProperties by the first call that launches on it;
 * devices at index 64 and above are queried on every call).  Nothing else is kept between calls.
 */
#ifndef RMSQ_H
#define RMSQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define RMSQ_API __attribute__((visibility("default")))
#else
#define RMSQ_API
#endif

/* 5: rmsq_convert accepts RMSQ_CVT_E4M3_IN_RANGE;
 * 4: rmsq_query_launch takes the call's flags in place of a residual flag it never used;
 * 3: rmsq_rms_norm_pad_query_launch takes the call's flags (the default shape depends on the
 *    activation type); 2: the padding and QK-norm + RoPE entry points take flags. */
#define RMSQ_ABI_VERSION 5
#define RMSQ_MAX_HIDDEN 65536 /* largest H one workgroup keeps in registers */

/* ---- status codes ---- */
enum {
  RMSQ_OK = 0,
  RMSQ_EINVAL = -1,       /* bad size, null pointer, bad group size, eps <= 0, ld < T, ... */
  RMSQ_EALIGN = -2,       /* a pointer is not aligned as documented below */
  RMSQ_EALIAS = -3,       /* an output overlaps an input or another output */
  RMSQ_EUNSUPPORTED = -4, /* flag not valid for the mode, or the device is not gfx950 */
  RMSQ_ELAUNCH = -5,      /* the kernel launch was refused by the HIP runtime */
  RMSQ_EDEVICE = -6       /* no current HIP device could be queried */
};

/* ---- quantization modes ---- */
typedef enum {
  RMSQ_FP8_STATIC = 0,
  RMSQ_FP8_TOKEN = 1,
  RMSQ_FP8_GROUP = 2,
  RMSQ_FP4_BLOCK16 = 3
} rmsq_mode;

/* ---- scale-layout flags, RMSQ_FP8_GROUP only (blog "Why this design": E8M0 scales and
 *      column-major scales) ---- */
enum {
  RMSQ_SCALE_COLMAJOR = 1u << 0, /* scales stored [H/G][scale_ld]: element (t,g) at g*ld + t */
  RMSQ_SCALE_E8M0 = 1u << 1,     /* scale rounded up to 2^ceil(log2 s), stored as f32        */
  RMSQ_SCALE_E8M0_U8 = 1u << 2   /* same rounding, stored as the E8M0 byte (exponent + 127)  */
};

/* ---- activation type flag: any mode of rmsq_fused and rmsq_silu_mul_quant, and
 *      rmsq_rms_norm_pad and rmsq_qk_norm_rope (docs "Fusion torch.compile passes" and the
 *      blog's type check: x and the weight share the model's activation dtype) ---- */
enum {
  RMSQ_INPUT_F16 = 1u << 8 /* x, residual, weight, residual_out are IEEE binary16, not bf16 */
};

/*
 * rmsq_fused -- one launch of the fused kernel family.
 *
 *  x            [T,H] bf16 (binary16 with RMSQ_INPUT_F16), row stride H, 16-byte aligned.
 *               Read only; must not overlap any output.
 *  residual     [T,H] same type, 16-byte aligned, or NULL for plain RMSNorm (vLLM rms_norm ->
 *               quant); non-NULL selects the fused-add form (fused_add_rms_norm -> quant).
 *  weight       [H] same type as x, 16-byte aligned (the blog's "Type check" rejects mixed
 *               input/weight dtypes: bf16, or binary16 for all three with RMSQ_INPUT_F16).
 *  eps          finite, > 0 (the pages' patterns use 1e-5 and 1e-6).
 *  mode         rmsq_mode.
 *  scale_in     device f32, 4-byte aligned: FP8_STATIC the per-tensor dequant scale (positive,
 *               finite); FP4_BLOCK16 the global encode scale gs (positive, finite); must be
 *               NULL for FP8_TOKEN and FP8_GROUP.
 *  out_q        FP8: [T,H] e4m3fn bytes, 8-byte aligned.  FP4: [T,H/2] bytes, 4-byte aligned,
 *               element 2k in the low nibble of byte k.
 *  out_scales   FP8_STATIC: must be NULL.  FP8_TOKEN: [T] f32.  FP8_GROUP: [T,H/G] f32
 *               row-major, or [H/G, scale_ld] f32 with RMSQ_SCALE_COLMAJOR, or bytes with
 *               RMSQ_SCALE_E8M0_U8.  FP4_BLOCK16: [T,H/16] e4m3 bytes, row-major.  f32 scales
 *               need 4-byte alignment.  Column-major padding (columns T..ld-1) is not written.
 *  residual_out [T,H] same type as x, 16-byte aligned; receives h = x + residual rounded to
 *               that type (nearest even; binary16 overflows to infinity).  Non-NULL iff
 *               residual is; may equal residual exactly (in-place update, as vLLM's fused_add_rms_norm
 *               does), must not otherwise overlap anything.
 *  tokens       T >= 0; T == 0 is a successful no-op (pointers are then not checked).
 *  hidden       H: 8 <= H <= RMSQ_MAX_HIDDEN, H % 8 == 0, and H % group_size == 0.
 *  group_size   FP8_GROUP: 64 or 128.  FP4_BLOCK16: 16.  Otherwise 0.
 *  flags        RMSQ_SCALE_* for FP8_GROUP (E8M0 and E8M0_U8 are exclusive), plus
 *               RMSQ_INPUT_F16 in any mode; 0 otherwise.
 *  scale_ld     FP8_GROUP with RMSQ_SCALE_COLMAJOR: leading dimension >= T (0 means T).
 *               Otherwise 0.
 *  stream       hipStream_t to enqueue on.
 * Returns RMSQ_OK or a negative status (see rmsq_status_string).
 */
RMSQ_API int rmsq_fused(const void* x, const void* residual, const void* weight, float eps,
                        int mode, const float* scale_in, void* out_q, void* out_scales,
                        void* residual_out, int64_t tokens, int64_t hidden, int group_size,
                        unsigned flags, int64_t scale_ld, void* stream);

/* Host-only argument check of rmsq_fused: returns exactly the status rmsq_fused would return
 * for these arguments before it touches the device (RMSQ_OK when they are valid).  Makes no HIP
 * call and dereferences no pointer. */
RMSQ_API int rmsq_validate(const void* x, const void* residual, const void* weight, float eps,
                           int mode, const float* scale_in, const void* out_q,
                           const void* out_scales, const void* residual_out, int64_t tokens,
                           int64_t hidden, int group_size, unsigned flags, int64_t scale_ld);

/*
 * Launch shape of the kernel family: one row of H elements is spread over threads_per_row
 * threads (a multiple of 64, <= 1024), each holding chunks_per_thread 16-byte chunks (1 to 8)
 * of the row in registers; rows_per_block rows share one workgroup
 * (rows_per_block * threads_per_row <= 1024).  threads_per_row * chunks_per_thread * 8 >= H.
 * options: RMSQ_LAUNCH_* bits.
 */
enum {
  /* By default workgroup b takes row block b, so the workgroups in flight touch one compact
   * window of each array (best for HBM page locality).  With this bit each of the 8 XCDs takes
   * a contiguous range of row blocks instead (rmsq_block_to_rowblock). */
  RMSQ_LAUNCH_XCD_RANGES = 1,
  /* rmsq_silu_mul_quant only, and not with per-token scaling (which needs a whole row per
   * workgroup): each row is cut into tiles of threads_per_row x chunks_per_thread chunks
   * (chunks_per_thread 1, 2 or 4) and each workgroup takes one tile (rows_per_block must be 1).
   * Results are identical to whole-row launches. */
  RMSQ_LAUNCH_ROW_TILES = 2
};
typedef struct rmsq_launch {
  int32_t threads_per_row;
  int32_t chunks_per_thread;
  int32_t rows_per_block;
  int32_t options; /* RMSQ_LAUNCH_* bits; other bits must be 0 */
} rmsq_launch;

/* rmsq_fused with an explicit launch shape (for tuning sweeps); launch == NULL behaves as
 * rmsq_fused.  Results are identical for every valid shape. */
RMSQ_API int rmsq_fused_with_launch(const void* x, const void* residual, const void* weight,
                                    float eps, int mode, const float* scale_in, void* out_q,
                                    void* out_scales, void* residual_out, int64_t tokens,
                                    int64_t hidden, int group_size, unsigned flags,
                                    int64_t scale_ld, const rmsq_launch* launch, void* stream);

/* rmsq_fused_with_launch for measurement: the kernel is dispatched with hipExtLaunchKernel so
 * that start_event and stop_event (hipEvent_t created by the caller, either may be NULL) are
 * stamped by the dispatch itself at the kernel's start and end; their elapsed time is the
 * kernel's own duration, without the queue gaps between back-to-back launches. */
RMSQ_API int rmsq_fused_timed(const void* x, const void* residual, const void* weight, float eps,
                              int mode, const float* scale_in, void* out_q, void* out_scales,
                              void* residual_out, int64_t tokens, int64_t hidden, int group_size,
                              unsigned flags, int64_t scale_ld, const rmsq_launch* launch,
                              void* start_event, void* stop_event, void* stream);

/*
 * rmsq_fused_fp4_dynamic -- (residual add ->) RMSNorm -> FP4 block-16 with the global encode scale
 * taken from the batch itself (prhub summary of vLLM PR #51925: NVFP4 output with block scales and
 * a global scale; its test derives a global scale as 448 * 6 over a tensor's absmax -- here the
 * tensor is the normalized batch):
 *
 *   amax = max |y| over all T rows (y exactly as in rmsq_fused)
 *   gs   = (448 * 6) / amax in f32, or FLT_MAX where that is not finite (an all-zero batch)
 *   then exactly RMSQ_FP4_BLOCK16 with that gs.
 *
 *  x, residual, weight, eps, residual_out, tokens, hidden
 *               as for rmsq_fused; hidden % 16 == 0.
 *  out_q, out_scales
 *               as for rmsq_fused in RMSQ_FP4_BLOCK16.  out_q also holds the row pass's
 *               per-workgroup maxima (f32, at most its first 4T bytes) between the launches; its
 *               final contents are the codes.
 *  global_scale device f32, 4-byte aligned, written with gs (the dequantization needs it: value =
 *               e2m1 * decode(sf) / gs).  Must not overlap any other argument.  Also the word
 *               through which the launches hand gs over (cleared to 0 first).
 *  flags        0 (bf16) or RMSQ_INPUT_F16; any other bit is RMSQ_EUNSUPPORTED.
 * The global scale depends on every row, so the work is two launches on `stream`: (1) the
 * residual add and normalization, writing the new residual and each workgroup's largest |y|
 * (and clearing global_scale); (2) the block quantization, which normalizes the new residual (or
 * x) again.  Launch 2's first workgroup reduces the maxima to gs and stores it to global_scale;
 * the other workgroups load their rows meanwhile and then wait for a non-zero global_scale (a
 * bounded wait, ~0.1 s: the first workgroup is dispatched before them and does not wait on
 * anything; should a wait ever run out, global_scale is left NaN, so every value dequantized
 * with it is NaN rather than silently wrong).
 * No workgroup writes out_q, where the maxima are, before gs exists.  Where that workgroup could
 * not reduce the maxima in one round of loads (more than eight per thread: very large T, or a
 * caller's shape with one row per workgroup), a one-workgroup reduction launch runs between the
 * two instead.  The second read of the normalized input (2H bytes per token) is the price of the
 * batch scale.  Returns RMSQ_OK or a negative status.
 */
RMSQ_API int rmsq_fused_fp4_dynamic(const void* x, const void* residual, const void* weight,
                                    float eps, void* out_q, void* out_scales, void* residual_out,
                                    float* global_scale, int64_t tokens, int64_t hidden,
                                    unsigned flags, void* stream);

/* rmsq_fused_fp4_dynamic with an explicit launch shape for the row pass, and for the block pass
 * where it normalizes again (NULL: the default, as rmsq_fused but with up to 16 rows to a
 * workgroup) and optional dispatch-stamped events: start_event is stamped by the first launch,
 * stop_event by the last (NULL: none). */
RMSQ_API int rmsq_fused_fp4_dynamic_ex(const void* x, const void* residual, const void* weight,
                                       float eps, void* out_q, void* out_scales,
                                       void* residual_out, float* global_scale, int64_t tokens,
                                       int64_t hidden, unsigned flags, const rmsq_launch* launch,
                                       void* start_event, void* stop_event, void* stream);

/* Host-only argument check of rmsq_fused_fp4_dynamic (no HIP call, no dereference). */
RMSQ_API int rmsq_fused_fp4_dynamic_validate(const void* x, const void* residual,
                                             const void* weight, float eps, const void* out_q,
                                             const void* out_scales, const void* residual_out,
                                             const float* global_scale, int64_t tokens,
                                             int64_t hidden, unsigned flags);

/*
 * rmsq_rms_norm_pad -- (residual add ->) RMSNorm -> 16-bit output in a padded row layout, in one
 * launch (vLLM docs "Fusion torch.compile passes", section "RMSNorm + padding
 * (fuse_act_padding)": the residual add and RMSNorm fused with padding the hidden dimension --
 * 2880 for the model named there -- to the multiple a downstream GEMM needs).
 *
 *  x, residual, weight, eps, residual_out, tokens, hidden
 *               exactly as for rmsq_fused (residual NULL: plain RMSNorm).
 *  out          [T, out_ld], the type of x, 16-byte aligned: out[t, i] = y_i rounded to that
 *               type (nearest even; binary16 overflows to infinity) for i < H and 0 for
 *               H <= i < out_ld.  Must not overlap any input or residual_out.
 *  out_ld       the padded row length: H <= out_ld <= RMSQ_MAX_HIDDEN, out_ld % 8 == 0.
 *  flags        0 (bf16) or RMSQ_INPUT_F16 (x, residual, weight, residual_out and out are IEEE
 *               binary16); any other bit is RMSQ_EUNSUPPORTED.
 * Returns RMSQ_OK or a negative status.
 */
RMSQ_API int rmsq_rms_norm_pad(const void* x, const void* residual, const void* weight,
                               float eps, void* out, void* residual_out, int64_t tokens,
                               int64_t hidden, int64_t out_ld, unsigned flags, void* stream);

/* rmsq_rms_norm_pad with an explicit launch shape (NULL: the default, see
 * rmsq_rms_norm_pad_query_launch; a shape must cover out_ld) and optional dispatch-stamped
 * events. */
RMSQ_API int rmsq_rms_norm_pad_ex(const void* x, const void* residual, const void* weight,
                                  float eps, void* out, void* residual_out, int64_t tokens,
                                  int64_t hidden, int64_t out_ld, unsigned flags,
                                  const rmsq_launch* launch, void* start_event, void* stop_event,
                                  void* stream);

/* Host-only argument check of rmsq_rms_norm_pad (no HIP call, no dereference). */
RMSQ_API int rmsq_rms_norm_pad_validate(const void* x, const void* residual, const void* weight,
                                        float eps, const void* out, const void* residual_out,
                                        int64_t tokens, int64_t hidden, int64_t out_ld,
                                        unsigned flags);

/*
 * rmsq_silu_mul_quant -- SiLU+Mul -> quantization in one launch (vLLM docs "Fusion
 * torch.compile passes", section "SiLU+Mul + quantization (fuse_act_quant)": the gated
 * up-projection activation fused with the quantization that follows, so the full-precision
 * activation is never written).
 *
 *  x            [T, 2I] bf16 (IEEE binary16 with RMSQ_INPUT_F16 in flags), 16-byte aligned: row
 *               t is the gate g = x[t, 0:I] followed by the up projection u = x[t, I:2I].  Read
 *               only.
 *  a            = silu(g) * u = g / (1 + exp(-g)) * u, in f32 (within a few ulp of the exactly
 *               rounded value: expf and the hardware reciprocal), never stored.
 *  mode, scale_in, out_q, out_scales, group_size, flags, scale_ld
 *               exactly as for rmsq_fused, with I in place of H (codes FP8 [T, I] or FP4
 *               [T, I/2]; scales over the I values of a row).
 *  tokens       T >= 0 (0 is a no-op); inter = I: 8 <= I <= RMSQ_MAX_HIDDEN, I % 8 == 0,
 *               I % group_size == 0.
 * Outputs must not overlap x, scale_in or each other.  Returns RMSQ_OK or a negative status.
 */
RMSQ_API int rmsq_silu_mul_quant(const void* x, int mode, const float* scale_in, void* out_q,
                                 void* out_scales, int64_t tokens, int64_t inter, int group_size,
                                 unsigned flags, int64_t scale_ld, void* stream);

/* rmsq_silu_mul_quant with an explicit launch shape (NULL: the default, chosen from I as for
 * rmsq_fused) and optional dispatch-stamped events (as rmsq_fused_timed; NULL: none). */
RMSQ_API int rmsq_silu_mul_quant_ex(const void* x, int mode, const float* scale_in, void* out_q,
                                    void* out_scales, int64_t tokens, int64_t inter,
                                    int group_size, unsigned flags, int64_t scale_ld,
                                    const rmsq_launch* launch, void* start_event,
                                    void* stop_event, void* stream);

/* Host-only argument check of rmsq_silu_mul_quant (no HIP call, no dereference). */
RMSQ_API int rmsq_silu_mul_quant_validate(const void* x, int mode, const float* scale_in,
                                          const void* out_q, const void* out_scales,
                                          int64_t tokens, int64_t inter, int group_size,
                                          unsigned flags, int64_t scale_ld);

/*
 * rmsq_qk_norm_rope -- per-head RMSNorm of the q and k heads followed by the rotary position
 * embedding, in place, in one launch (vLLM docs "Fusion torch.compile passes", section "QK Norm
 * + RoPE": for models that normalize Q and K per head, the split of the packed qkv tensor, the
 * two RMSNorms and the rotary embedding become one kernel).
 *
 *  qkv          [T, (Hq + 2 Hkv) * D] bf16 (IEEE binary16 with RMSQ_INPUT_F16), 16-byte
 *               aligned, row t = Hq q heads, Hkv k heads, Hkv v heads of D elements each.
 *               Rewritten in place: every q head h becomes rope(rmsnorm(h) * q_weight), every k
 *               head rope(rmsnorm(h) * k_weight), rounded once from f32 to the type of qkv
 *               (nearest even; binary16 overflows to infinity); v heads are not touched.
 *  rmsnorm      y_i = (h_i * inv) * w_i in f32, inv = 1/sqrt(sum h_i^2 / D + eps) from a
 *               binary64 sum, rounded to f32 (as rmsq_fused, over one head of D elements).
 *  q_weight, k_weight
 *               [D], the type of qkv, 16-byte aligned, read only.
 *  cos_sin_cache
 *               [max_position, D] f32, 16-byte aligned: row p = cos(p * f_i) for i < D/2, then
 *               sin(p * f_i); the caller builds it (any base).  Read only.
 *  positions    [T] int64, 8-byte aligned: token t uses cache row positions[t].  A token whose
 *               position lies outside [0, max_position) is left entirely unchanged.
 *  is_neox      nonzero: element i pairs with i + D/2 (half split); zero: 2i pairs with 2i + 1
 *               (interleaved).  Pair (a, b) with frequency j becomes (a c - b s, b c + a s),
 *               each product rounded to f32 before the sum.
 *  tokens       T >= 0 (0 is a no-op); num_q_heads Hq >= 1, num_kv_heads Hkv >= 1,
 *               (Hq + 2 Hkv) * D <= 2^20; head_dim D in {64, 128, 256}; max_position >= 1.
 *  flags        0 (bf16) or RMSQ_INPUT_F16 (qkv and both weights IEEE binary16); any other bit
 *               is RMSQ_EUNSUPPORTED.
 * qkv must not overlap the other arguments.  Returns RMSQ_OK or a negative status.
 */
RMSQ_API int rmsq_qk_norm_rope(void* qkv, const void* q_weight, const void* k_weight,
                               const float* cos_sin_cache, const int64_t* positions, float eps,
                               int64_t tokens, int num_q_heads, int num_kv_heads, int head_dim,
                               int64_t max_position, int is_neox, unsigned flags, void* stream);

/* rmsq_qk_norm_rope with an explicit launch shape and optional dispatch-stamped events (as
 * rmsq_fused_timed; NULL: none).  A head is held by D/16 lanes (16 elements each); a lane group
 * serves heads_per_lane heads (1 to 6) and a workgroup heads_per_block heads of one token, a
 * multiple of heads_per_lane, with (heads_per_block / heads_per_lane) * D/16 <= 1024 threads.
 * Both 0: the default shape. */
RMSQ_API int rmsq_qk_norm_rope_ex(void* qkv, const void* q_weight, const void* k_weight,
                                  const float* cos_sin_cache, const int64_t* positions,
                                  float eps, int64_t tokens, int num_q_heads, int num_kv_heads,
                                  int head_dim, int64_t max_position, int is_neox,
                                  unsigned flags, int heads_per_block, int heads_per_lane,
                                  void* start_event, void* stop_event, void* stream);

/* Host-only argument check of rmsq_qk_norm_rope (no HIP call, no dereference). */
RMSQ_API int rmsq_qk_norm_rope_validate(const void* qkv, const void* q_weight,
                                        const void* k_weight, const float* cos_sin_cache,
                                        const int64_t* positions, float eps, int64_t tokens,
                                        int num_q_heads, int num_kv_heads, int head_dim,
                                        int64_t max_position, unsigned flags);

/* The default launch shape of rmsq_qk_norm_rope (heads per workgroup, heads per lane group) and
 * its grid size (tokens times the workgroups per token).  Host only; makes no HIP call.
 * Returns RMSQ_OK or RMSQ_EINVAL. */
RMSQ_API int rmsq_qk_norm_rope_query_launch(int64_t tokens, int num_q_heads, int num_kv_heads,
                                            int head_dim, int* heads_per_block,
                                            int* heads_per_lane, int64_t* grid);

/* The launch shape rmsq_fused picks for (mode, T, H, group_size, flags) and its grid size
 * (number of workgroups).  The arguments are checked as rmsq_fused checks them (flags:
 * RMSQ_SCALE_* for FP8_GROUP, RMSQ_INPUT_F16 in any mode).  The shape depends on T, H and
 * whether the mode is RMSQ_FP8_TOKEN (whose row-wide reduction takes one wave per row for
 * batches of 1024+ rows of 1536 or 2048 elements); it is the same with and without a residual
 * and for either activation type.  rmsq_fused_fp4_dynamic's default row pass takes the
 * per-token shape, with as many rows per workgroup as its block pass needs.  Host only; makes no
 * HIP call.  Returns RMSQ_OK, RMSQ_EINVAL or RMSQ_EUNSUPPORTED (a flag the mode does not take). */
RMSQ_API int rmsq_query_launch(int mode, int64_t tokens, int64_t hidden, int group_size,
                               unsigned flags, rmsq_launch* launch, int64_t* grid);

/* The launch shape rmsq_rms_norm_pad picks for (T, H, out_ld, flags) and its grid size: flags
 * as passed to rmsq_rms_norm_pad (0 or RMSQ_INPUT_F16; the default shape depends on the
 * activation type).  Host only; makes no HIP call.  Returns RMSQ_OK or RMSQ_EINVAL. */
RMSQ_API int rmsq_rms_norm_pad_query_launch(int64_t tokens, int64_t hidden, int64_t out_ld,
                                            unsigned flags, rmsq_launch* launch,
                                            int64_t* grid);

/* The launch shape rmsq_silu_mul_quant picks for (mode, T, I, group_size) and its grid size:
 * row tiles of 64 threads x 2 chunks (RMSQ_LAUNCH_ROW_TILES) for FP4 block-16, whole rows as
 * rmsq_query_launch's per-H default otherwise.  Host only; makes no HIP call.  Returns RMSQ_OK
 * or RMSQ_EINVAL. */
RMSQ_API int rmsq_silu_mul_query_launch(int mode, int64_t tokens, int64_t inter, int group_size,
                                        rmsq_launch* launch, int64_t* grid);

/* Which block of rows workgroup `block` of a `grid`-workgroup launch processes.  Workgroups are
 * dispatched round-robin over the MI355X's 8 accelerator dies (XCDs); this map hands each die
 * a contiguous range of row blocks.  Host copy of the device mapping, for tests. */
RMSQ_API int64_t rmsq_block_to_rowblock(int64_t block, int64_t grid);

/* Diagnostic: run the kernels' own converters over n f32 values (device pointers).
 *  RMSQ_CVT_E4M3  out: n bytes, saturating e4m3fn (the static and per-token schemes'
 *                 conversion, and the FP4 block scales')
 *  RMSQ_CVT_E4M3_IN_RANGE
 *                 out: n bytes, e4m3fn without the clamp (the per-group scheme's conversion,
 *                 whose inputs stay within 448 (1 + 2^-20)): the saturating code for
 *                 |v| <= 464, the NaN code of v's sign above that
 *  RMSQ_CVT_E2M1  out: n/2 bytes, element 2k in the low nibble (the FP4 epilogue's conversion);
 *                 n must be a multiple of 8
 *  RMSQ_CVT_BF16  out: n uint16 bf16 patterns (the residual-add rounding)
 *  RMSQ_CVT_INV_SQRT
 *                 out: n f32, the kernels' inverse RMS of m = in[i] widened to binary64, i.e.
 *                 (float)(1.0 / sqrt(m)) with binary64 root and quotient (m > 0 assumed)
 *  n must be a multiple of 8; in/out 16-byte aligned.  Used to pin gfx950's conversion
 *  instructions, and the inverse-RMS sequence, against the reference definitions. */
enum {
  RMSQ_CVT_E4M3 = 0,
  RMSQ_CVT_E2M1 = 1,
  RMSQ_CVT_BF16 = 2,
  RMSQ_CVT_INV_SQRT = 3,
  RMSQ_CVT_E4M3_IN_RANGE = 4
};
RMSQ_API int rmsq_convert(int format, const float* in, void* out, int64_t n, void* stream);

/* Human-readable text for a status code (static storage). */
RMSQ_API const char* rmsq_status_string(int status);

/* RMSQ_ABI_VERSION of the loaded library. */
RMSQ_API int rmsq_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* RMSQ_H */
