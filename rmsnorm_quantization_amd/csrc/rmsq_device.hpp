// rmsq_device.hpp -- gfx950 device helpers for the fused RMSNorm + quantization kernels:
// bf16 unpack/pack, hardware FP8 (OCP e4m3fn) / FP4 (e2m1) conversion, DPP group reductions.
//
// Formats (the pages name FP8 e4m3 and NVFP4-style e2m1 outputs -- vLLM docs "Fusion
// torch.compile passes", "RMSNorm + quantization"; PR #51925 summary, "Motivation" -- but not
// their bit layouts; the OCP definitions are used): e4m3fn saturates at 448, e2m1 at 6, both
// round to nearest even.  The FP8 converter is fed values already clamped to the format's
// range, so its saturation never depends on the instruction's overflow behaviour; the FP4
// converter saturates by itself (e2m1 has no infinity or NaN code: every finite or infinite
// magnitude from 6 up gives +-6, pinned against the oracle by the converter tests).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rmsq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kFp8Max = 448.0f;
constexpr float kFp4Max = 6.0f;

// ---- addressing --------------------------------------------------------------------------
// A row pointer plus a 32-bit byte offset.  The address stays (row base, uniform over the wave)
// + (32-bit lane offset), which the global load and store instructions take directly with the
// base in scalar registers: no 64-bit address is built per lane and access.  Every offset the
// kernels form this way is below 2^22 (at most a row of 2^20 16-bit elements).
template <class T>
__device__ __forceinline__ T* boff(T* p, uint32_t bytes) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(p) + bytes);
}
template <class T>
__device__ __forceinline__ const T* boff(const T* p, uint32_t bytes) {
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(p) + bytes);
}

// ---- bf16 ------------------------------------------------------------------------------
// A dword holds two bf16 values, element 2j in the low half.  bf16 is the upper half of an
// f32 pattern, so widening is a shift or a mask.
__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// Round two f32 to bf16 (nearest even; v_cvt_pk_bf16_f32), a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// ---- IEEE binary16 ----------------------------------------------------------------------
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float f16_lo(uint32_t d) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(d & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t d) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(d >> 16));
}

// Round two f32 to binary16 (nearest even, overflow to infinity), a in the low half.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  f16x2 r = __builtin_convertvector((f32x2){a, b}, f16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// The 16-bit activation type of a launch: DT 0 = bf16, 1 = IEEE binary16.
template <int DT>
__device__ __forceinline__ float in_lo(uint32_t d) {
  if constexpr (DT == 1) return f16_lo(d);
  else return bf16_lo(d);
}
template <int DT>
__device__ __forceinline__ float in_hi(uint32_t d) {
  if constexpr (DT == 1) return f16_hi(d);
  else return bf16_hi(d);
}
template <int DT>
__device__ __forceinline__ uint32_t pack_in(float a, float b) {
  if constexpr (DT == 1) return pack_f16x2(a, b);
  else return pack_bf16x2(a, b);
}

// ---- FP8 e4m3fn --------------------------------------------------------------------------
__device__ __forceinline__ float clamp_sym(float v, float m) {
  return __builtin_amdgcn_fmed3f(v, -m, m);
}

// Four f32 -> four e4m3fn bytes, element 0 in the lowest byte (v_cvt_pk_fp8_f32).
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_sym(a, kFp8Max), clamp_sym(b, kFp8Max), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_sym(c, kFp8Max), clamp_sym(d, kFp8Max), w, true);
  return (uint32_t)w;
}

// Four f32 of magnitude at most 464 -> four e4m3fn bytes, with no clamp.  The conversion rounds
// the magnitude to nearest even: everything up to 464, the midpoint between 448 and the step
// above it (whose pattern is the NaN code), gives 448, and only larger magnitudes give NaN
// (checked on the device; pinned against the oracle's saturating encoder over |v| <= 464 by the
// converter test).  The per-group scheme meets that bound by construction: with s = RN(m/448)
// and r = RN(1/s) finite, any |y| <= m gives |y * r| <= 448 (1 + 2^-20), also where s is
// subnormal (then s >= 2^-128 and its relative error is at most 2^-21); E8M0 scales give at most
// 448.  (Per-token scaling would too, but its widest rows have no register to spare for the
// different zero-safe step below, and its headline shape hides the clamp behind memory.)
__device__ __forceinline__ uint32_t fp8x4_in_range(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// One f32 -> one e4m3fn byte.
__device__ __forceinline__ uint32_t fp8x1(float a) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp_sym(a, kFp8Max), 0.0f, 0, false) & 0xFFu;
}

// e4m3fn byte -> f32 (exact; v_cvt_f32_fp8).
__device__ __forceinline__ float fp8_decode(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// ---- scaled values ---------------------------------------------------------------------------
// True in every lane when p holds in some lane of the wave: a wave-uniform value, so a branch on
// it is a scalar branch.  Must run with all lanes of the wave active.
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// A multiplier that is not a finite binary32 value: a reciprocal scale (or an FP4 block
// multiplier) that overflowed to infinity.
__device__ __forceinline__ bool not_finite(float m) { return !(fabsf(m) <= __FLT_MAX__); }

// The codes are encoded from y * m, where m is a reciprocal scale (or an FP4 block multiplier)
// that overflows to infinity for a scale below 1/FLT_MAX.  There a non-zero y gives an infinity,
// which saturates, but a zero y gives NaN, while scaling a zero gives that zero.  In such a lane,
// (y * 2^64) * 2^100 takes the place of y * m: a zero stays the zero it is, sign included, and every
// non-zero finite y ends at least 2^15 in magnitude (or infinite), past the largest code of either
// format -- the same codes, with no select per element.  zero_safe rewrites y and m that way
// where `inf` holds; callers evaluate the condition once per row or per chunk.
__device__ __forceinline__ void zero_safe(float (&y)[8], float& m, bool inf) {
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = inf ? y[e] * 0x1p64f : y[e];
  m = inf ? 0x1p100f : m;
}

// The same codes for the unclamped FP8 conversion (fp8x4_in_range), whose input must stay
// within 464: where `inf` holds, a zero y stays itself, any other y becomes +-448 (what it
// would saturate to), and m becomes 1.  Runs only in waves that meet an infinite multiplier.
__device__ __forceinline__ void zero_safe_in_range(float (&y)[8], float& m, bool inf) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    y[e] = (inf && y[e] != 0.0f) ? __builtin_copysignf(kFp8Max, y[e]) : y[e];
  m = inf ? 1.0f : m;
}

// ---- FP4 e2m1 ----------------------------------------------------------------------------
// Eight f32 -> eight e2m1 nibbles in one dword, element 2k in the low nibble of byte k
// (v_cvt_scalef32_pk_fp4_f32 with a unit scale, so the instruction's scale does nothing; it
// rounds to nearest even and saturates to +-6 without a clamp).
__device__ __forceinline__ uint32_t fp4x8(const float* v) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
  return w;
}

// ---- per-group scale ------------------------------------------------------------------------
// absmax / 448 exactly as IEEE division rounds it: m * RN(1/448) corrected once by its FMA
// residual equals the correctly rounded quotient for every m >= 2^-120 (checked exhaustively
// over all binary32 m on the host); below that the quotient is subnormal and may differ, so a
// wave holding such an m takes the IEEE division (a uniform branch).  m == 0 gives 0 either way.
// Must run with all lanes of the wave active.
__device__ __forceinline__ float div448(float m) {
  constexpr float kInv448 = 1.0f / 448.0f;
  const float q0 = m * kInv448;
  float s = fmaf(fmaf(-q0, 448.0f, m), kInv448, q0);
  if (wave_any(m > 0.0f && m < 0x1p-120f)) {
    asm volatile("");  // keeps the division in its branch (not computed for every wave)
    s = m / 448.0f;
  }
  return s;
}

// ---- E8M0 ---------------------------------------------------------------------------------
// Round a non-negative f32 scale up to the next power of two 2^k, k in [-127, 127], from its
// bit pattern: a normal s with a non-zero mantissa moves up one binade; s == 0 and the
// subnormals at or below 2^-127 give 2^-127 (E8M0 byte 0).  Returns the E8M0 byte (k + 127)
// and the power of two as f32 in *p2.
__device__ __forceinline__ uint32_t e8m0_ceil(float s, float* p2) {
  const uint32_t b = __float_as_uint(s);
  const uint32_t e = b >> 23, m = b & 0x7FFFFFu;
  uint32_t byte;
  if (e == 0) byte = (m > 0x400000u) ? 1u : 0u;  // subnormal: 2^-126 or 2^-127
  else byte = e + (m != 0u ? 1u : 0u);
  if (byte > 254u) byte = 254u;
  *p2 = byte == 0u ? __uint_as_float(0x00400000u) : __uint_as_float(byte << 23);
  return byte;
}

// ---- inverse RMS ----------------------------------------------------------------------------
// (float)(1.0 / sqrt(m)): the binary32 rounding of the correctly rounded binary64 quotient of one
// by the correctly rounded binary64 root, as the plain definition of the inverse RMS computes it,
// without that definition's two long binary64 sequences in the common case.  The hardware
// estimate (v_rsq_f64, within 2^-24 relative on gfx950 over 2^24 sampled m) is refined by two
// Newton steps y <- y + (y/2)(1 - m y^2), which leave y within a few binary64 ulps of 1/sqrt(m)
// from any estimate better than 2^-12; the definition's value lies within two ulps of 1/sqrt(m)
// as well.  Rounding to binary32 is monotonic, so when
// y(1 - 2^-40) and y(1 + 2^-40) round to the same binary32 value every value between them does,
// the definition's included; then inv_sqrt_window stores it and returns true.  Otherwise (about
// one value in 2^16, and NaN or infinite m) the caller runs the definition's own sequence.
__device__ __forceinline__ bool inv_sqrt_window(double m, float* out) {
  double y = __builtin_amdgcn_rsq(m);
#pragma unroll
  for (int i = 0; i < 2; ++i) y = fma(0.5 * y, fma(-m, y * y, 1.0), y);
  const float lo = (float)(y * (1.0 - 0x1p-40)), hi = (float)(y * (1.0 + 0x1p-40));
  *out = lo;
  return lo == hi;
}

__device__ __forceinline__ float inv_sqrt_f32(double m) {
  float v;
  if (inv_sqrt_window(m, &v)) return v;
  return (float)(1.0 / sqrt(m));
}

// The inverse RMS of a row from its binary64 sum of squares: (float)(1 / sqrt(ss/H + eps)) with
// the quotient, sum, root and reciprocal in binary64, as the plain definition computes it.  For
// a power-of-two H the mean is an exact scaling by 2^-k.  Otherwise ss * RN(1/H) (inv_h, from the
// host) stands in for the quotient: it lies within 2^-51 (relative) of it, which moves 1/sqrt by
// about 2^-52, far inside the 2^-40 window of inv_sqrt_window, so the window decides the rounding
// exactly as it would for the quotient itself; where the window straddles a binary32 rounding
// boundary, the quotient and the definition's own sequence run.  The branch on H is uniform.
__device__ __forceinline__ float inv_rms(double ss, int64_t H, double inv_h, float eps) {
  const bool pow2 = (H & (H - 1)) == 0;
  const double mean =
      pow2 ? ldexp(ss, -__builtin_ctzll((unsigned long long)H)) : ss * inv_h;
  float v;
  if (inv_sqrt_window(mean + (double)eps, &v)) return v;
  const double exact = pow2 ? mean : ss / (double)H;
  return (float)(1.0 / sqrt(exact + (double)eps));
}

// ---- cross-lane reductions ---------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Max over aligned groups of LANES consecutive lanes (2, 4, 8 or 16: one DPP row at most) of
// non-negative values (absolute values: no NaN, no negative zero); every lane of a group ends with
// the group's max.  Non-negative binary32 values order like their bit patterns as unsigned
// integers, so the integer max takes its DPP operand directly (no move, no canonicalization).
// Must run with all lanes of the wave active.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int LANES>
__device__ __forceinline__ float group_max(float v) {
  static_assert(LANES == 1 || LANES == 2 || LANES == 4 || LANES == 8 || LANES == 16, "lanes");
  uint32_t u = __float_as_uint(v);
  if (LANES >= 2) u = max(u, dpp_u32<0xB1>(u));   // quad_perm [1,0,3,2]: lane ^ 1
  if (LANES >= 4) u = max(u, dpp_u32<0x4E>(u));   // quad_perm [2,3,0,1]: lane ^ 2
  if (LANES >= 8) u = max(u, dpp_u32<0x141>(u));  // row_half_mirror: other quad of the 8
  if (LANES >= 16) u = max(u, dpp_u32<0x140>(u)); // row_mirror: other half of the 16
  return __uint_as_float(u);
}

template <int CTRL>
__device__ __forceinline__ double dpp(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo =
      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ double readlane(double v, int lane) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Sum / max over the 64 lanes of a wave, the same value in every lane.  Within each 16-lane
// DPP row a butterfly (lane^1, lane^2, other quad, other half) leaves the row total in every
// lane -- both partners of a step add the same two numbers and IEEE addition is commutative,
// so the lanes agree bit for bit; the four row totals are then read as scalars and combined
// in one fixed order.  Must run with all lanes of the wave active.
__device__ __forceinline__ double wave_sum(double v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  return (readlane(v, 0) + readlane(v, 16)) + (readlane(v, 32) + readlane(v, 48));
}
// (non-negative values, as group_max)
__device__ __forceinline__ float wave_max(float v) {
  v = group_max<16>(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float e = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, e));
}

// ---- XCD-aware block order -------------------------------------------------------------
// Workgroups are handed to the 8 XCDs round-robin (workgroup b runs on XCD b % 8).  Giving
// XCD x the contiguous range of row blocks [x*q + min(x,r), ...) keeps neighbouring rows in
// one L2, where the partial-line writes of small per-row scales merge.
constexpr uint32_t kNumXcd = 8;
__host__ __device__ __forceinline__ uint32_t rowblock_of(uint32_t b, uint32_t n) {
  const uint32_t x = b % kNumXcd, i = b / kNumXcd;
  const uint32_t q = n / kNumXcd, r = n % kNumXcd;
  return x * q + (x < r ? x : r) + i;
}

}  // namespace rmsq
