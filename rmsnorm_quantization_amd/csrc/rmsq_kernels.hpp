// rmsq_kernels.hpp -- the gfx950 kernels of librmsq: the fused (residual add ->) RMSNorm ->
// FP8 / FP4 quantization kernel family and the converter diagnostic kernel.
//
// Operation (vLLM docs "Fusion torch.compile passes", section "RMSNorm + quantization
// (fuse_norm_quant)"; blog "[vLLM] Compilation Fusion Passes", "Pattern matching structure",
// fused-op map, "Why this design"; PR #51925 summary, "Motivation"): per token row,
// h = bf16(x + residual) (written back as the residual), y = h / sqrt(mean(h^2) + eps) * w,
// then FP8 static / per-token / per-group or FP4 block-16 quantization of y.  The fusion's
// point is that y never reaches memory: HBM sees x, residual and weight once and the codes,
// scales and new residual once.
//
// Kernel shape (MI355X-first, not taken from any of the pages' kernels):
//   * a row of H bf16 is split into 16-byte chunks of 8 elements; chunk c of a row lives on
//     thread (c mod threads_per_row) of the row's waves, in registers, for the whole kernel, so
//     every input byte is loaded exactly once (128-bit non-temporal loads);
//     the row's base address is wave-uniform (scalar registers) and each lane adds a 32-bit
//     byte offset;
//   * sum of squares in binary64 (exact products of bf16 values), DPP butterfly within the
//     wave, LDS only across the waves of one row; inv_rms rounded once to f32 (inv_sqrt_f32);
//   * per-group (64/128) and per-block (16) absmax: a group is 8 / 16 consecutive lanes (2 for
//     an FP4 block), reduced with DPP row operations -- no LDS, no barrier;
//   * hardware conversions: v_cvt_pk_bf16_f32, v_cvt_pk_fp8_f32 (OCP e4m3fn on gfx950),
//     v_cvt_scalef32_pk_fp4_f32 (unit scale), v_cvt_f32_fp8; the FP4 block scale and element
//     multiplier are exact quotients formed without a division sequence per chunk;
//   * no MFMA: there is no contraction here, the op is HBM-bandwidth bound.
#pragma once

#include "rmsq_device.hpp"
#include "rmsq.h"

namespace rmsq {

constexpr int kMaxWavesPerBlock = 16;
// Internal mode of fused_kernel: the normalized row rounded to the 16-bit input type and written
// with a padded row stride (ld), the padding columns zero.  Not a quantization scheme, so not in
// rmsq_mode.
constexpr int kModePad = 4;
// Internal mode of fused_kernel: no codes, only the workgroup's largest |y| (f32, over all its
// rows) to scales[blockIdx.x] -- the first pass of FP4 with the global scale taken from the batch.
constexpr int kModeRowAmax = 5;
// Internal mode of fused_kernel: FP4 block-16 as the block pass of FP4 with the global scale
// taken from the batch -- the inverse RMS read from the row pass's staging (inv_rows) rather than
// recomputed where the row pass left it, and the global scale either read (scale_in) or derived by
// workgroup 0 from the row pass's maxima and waited for by the others (amax_parts).  Its own
// instantiations, so that plain FP4 carries none of it.
constexpr int kModeFp4Batch = 6;

struct KArgs {
  const uint16_t* x;
  const uint16_t* res;
  const uint16_t* w;
  uint16_t* res_out;
  uint8_t* q;
  void* scales;
  const float* scale_in;
  int64_t T;
  int64_t H;
  int64_t ld;
  double inv_h;   // RN(1/H) in binary64 (inv_rms)
  float eps;
  uint32_t flags;
  int32_t tpr;    // threads per row (multiple of 64)
  int32_t rpb;    // rows per block
  uint32_t nblk;  // workgroups in the grid
  int32_t xcd_ranges;  // XCD-contiguous row-block ranges instead of launch order
  // FP4 with a batch global scale: row t's inverse RMS as f32 at inv_rows + t * inv_stride
  // (the first bytes of that row's block scales), written by the row-absmax pass and read by
  // the block pass instead of normalizing again; null otherwise
  uint8_t* inv_rows;
  int64_t inv_stride;
  // FP4 with a batch global scale, the block pass (scale_in null): the row pass's n_parts
  // workgroup maxima, and the global scale's word.  Workgroup 0 reduces the maxima and publishes
  // gs = (448 * 6) / amax there; the other workgroups wait for it (batch_scale_*).  In the row
  // pass (kModeRowAmax) gs_out, if set, is cleared to 0, the "not yet published" value.
  const float* amax_parts;
  int64_t n_parts;
  float* gs_out;
};

// The FP4 global scale of a batch from its largest |y| (PR #51925 summary: NVFP4 with block
// scales and a global scale; its test derives a global scale as 448 * 6 over a tensor's absmax):
// (448 * 6) / amax by IEEE division, or FLT_MAX where that is not finite (amax == 0).  Always a
// positive normal value (amax <= FLT_MAX), so 0 can mark a global scale not yet published.
__device__ __forceinline__ float batch_fp4_scale(float amax) {
  const float g = (kFp8Max * kFp4Max) / amax;
  return (g <= __FLT_MAX__) ? g : __FLT_MAX__;
}

// Workgroup 0 of the block pass: the largest of the n row-pass maxima (every thread takes every
// blockDim-th one, eight loads in flight per round; the host keeps n within one round), then
// gs, published to *gs_out -- an agent-scope compare-and-swap from 0, so that a NaN left there by
// a wait that ran out (batch_scale_await) stays -- and returned to every thread.  Workgroup 0 is
// the first one dispatched, so it is resident whatever the others do while they wait.  Must be
// called by every thread of the workgroup.
__device__ float batch_scale_publish(const float* parts, int64_t n, float* gs_out, float* s_red) {
  constexpr int kLoads = 8;
  const int64_t stride = blockDim.x;
  float m = 0.0f;
  for (int64_t base = threadIdx.x; base < n; base += kLoads * stride) {
    float v[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int64_t i = base + u * stride;
      v[u] = (i < n) ? parts[i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kLoads; ++u) m = fmaxf(m, v[u]);
  }
  m = wave_max(m);
  const int nw = (int)(blockDim.x >> 6);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = 0.0f;
  for (int i = 0; i < nw; ++i) m = fmaxf(m, s_red[i]);
  const float gs = batch_fp4_scale(m);
  if (threadIdx.x == 0) {
    uint32_t expected = 0u;
    __hip_atomic_compare_exchange_strong(reinterpret_cast<uint32_t*>(gs_out), &expected,
                                         __float_as_uint(gs), __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
  }
  return gs;
}

// The other workgroups of the block pass: `seen` is an agent-scope load of *gs_out issued with the
// row's loads; while it still reads 0, poll (sleeping between polls) until workgroup 0 has
// published.  The wait is bounded (2^20 polls, about 0.1 s) so that every wave ends.  A wave
// whose wait runs out -- which workgroup 0, resident and waiting on nothing, does not let happen
// -- swaps a NaN into *gs_out unless the scale arrived meanwhile, and workgroup 0 publishes only
// over a 0: the call's global scale then reads NaN, and so does every value dequantized with it,
// instead of codes made with no scale passing for valid ones.
__device__ __forceinline__ float batch_scale_await(float seen, float* gs_out) {
  float g = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(seen)));
  for (int it = 0; g == 0.0f && it < (1 << 20); ++it) {
    __builtin_amdgcn_s_sleep(4);
    const float r = __hip_atomic_load(gs_out, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    g = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(r)));
  }
  if (g == 0.0f) {  // uniform; never taken while workgroup 0 runs
    uint32_t cur = 0u;
    __hip_atomic_compare_exchange_strong(reinterpret_cast<uint32_t*>(gs_out), &cur, 0x7FC00000u,
                                         __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    g = __uint_as_float(__builtin_amdgcn_readfirstlane(cur == 0u ? 0x7FC00000u : cur));
  }
  return g;
}

// One element of y = (h * inv) * w from the packed 16-bit chunk dwords (DT: 0 bf16, 1 binary16).
template <int DT = 0>
__device__ __forceinline__ float y_of(const u32x4& h, const u32x4& w, int e, float inv) {
  const uint32_t hd = h[e >> 1], wd = w[e >> 1];
  const float hf = (e & 1) ? in_hi<DT>(hd) : in_lo<DT>(hd);
  const float wf = (e & 1) ? in_hi<DT>(wd) : in_lo<DT>(wd);
  return (hf * inv) * wf;
}

// Where and how one row's quantized values go.
struct RowOut {
  uint8_t* q;       // codes: FP8 [T, n] bytes, FP4 [T, n/2] bytes
  void* scales;     // per-token [T] f32, per-group [T, n/G] or [n/G, ld], FP4 [T, n/16] bytes
  int64_t row;      // token index
  bool row_ok;      // row < T
  size_t obase;     // row * n: the row's element offset in the outputs
  int64_t n;        // values per row
  int64_t ld;       // column-major scale leading dimension
  uint32_t flags;   // RMSQ_SCALE_*
  uint32_t lr;      // thread within the row
  int tpr, wpr, rib, tid;
};

// Quantize and store one row held as VPT 8-element chunks per thread; Y(k, e) is the f32 value of
// element e of the thread's chunk k (chunk index lr + k * tpr).  One of the four schemes
// (vLLM docs "Fusion torch.compile passes": FP8 static per-tensor, dynamic per-token, dynamic
// per-token-group 128/64; PR #51925 summary: FP4 with block scales and a global scale):
//   static     q = e4m3(y * (1/scale))
//   per-token  s = absmax(row)/448, q = e4m3(y * (1/s)); s == 0 gives 0 codes
//   per-group  s = absmax(group)/448 (E8M0: rounded up to a power of two), same rule
//   FP4        sf = e4m3(absmax(block16) * gs / 6), q = e2m1(y * (gs / decode(sf)))
// A zero element gives the zero code of its own sign in every scheme, also where the reciprocal
// scale or the FP4 multiplier has overflowed to infinity (zero_safe).
// DT (the 16-bit output type of the padded mode only): 0 bf16, 1 IEEE binary16.
// FP4_BATCH: the FP4 epilogue takes all of the lane's chunks at once (up to 4) rather than one at
// a time.
template <int MODE, int VPT, int GS, int DT = 0, bool FP4_BATCH = true, class YF>
__device__ __forceinline__ void quantize_store(const YF& Y, const bool (&ok)[VPT], const RowOut& o,
                                               float scale_val, float* s_mx) {
  if constexpr (MODE == RMSQ_FP8_STATIC) {
    float r = 1.0f / scale_val;
    const bool inf = wave_any(not_finite(r));  // uniform: one scale per launch
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = Y(k, e);
      if (inf) zero_safe(v, r, true);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= r;
      const u32x2 qc = {fp8x4(v[0], v[1], v[2], v[3]), fp8x4(v[4], v[5], v[6], v[7])};
      if (ok[k]) {
        const uint32_t c = o.lr + (uint32_t)(k * o.tpr);
        __builtin_nontemporal_store(qc, boff(reinterpret_cast<u32x2*>(o.q + o.obase), c << 3));
      }
    }
  } else if constexpr (MODE == RMSQ_FP8_TOKEN) {
    float mx = 0.0f;
#pragma unroll
    for (int k = 0; k < VPT; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(Y(k, e)));
    mx = wave_max(mx);
    if (o.wpr > 1) {  // uniform over the block
      if ((o.tid & 63) == 0) s_mx[o.tid >> 6] = mx;
      __syncthreads();
      mx = 0.0f;
      for (int i = 0; i < o.wpr; ++i) mx = fmaxf(mx, s_mx[o.rib * o.wpr + i]);
    }
    const float s = mx / kFp8Max;
    if (o.lr == 0 && o.row_ok) static_cast<float*>(o.scales)[o.row] = s;
    const bool zero = (s == 0.0f);
    float r = zero ? 0.0f : 1.0f / s;
    const bool inf = wave_any(not_finite(r));  // uniform: one scale per row
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = Y(k, e);
      if (inf) zero_safe(v, r, true);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= r;
      u32x2 qc = {fp8x4(v[0], v[1], v[2], v[3]), fp8x4(v[4], v[5], v[6], v[7])};
      if (zero) qc = (u32x2){0u, 0u};
      if (ok[k]) {
        const uint32_t c = o.lr + (uint32_t)(k * o.tpr);
        __builtin_nontemporal_store(qc, boff(reinterpret_cast<u32x2*>(o.q + o.obase), c << 3));
      }
    }
  } else if constexpr (MODE == RMSQ_FP8_GROUP) {
    constexpr int L = GS / 8;  // lanes per group
    const bool e8 = (o.flags & (RMSQ_SCALE_E8M0 | RMSQ_SCALE_E8M0_U8)) != 0;
    const bool u8 = (o.flags & RMSQ_SCALE_E8M0_U8) != 0;
    const bool col = (o.flags & RMSQ_SCALE_COLMAJOR) != 0;
    // Chunks in phases as for FP4 below (scales, codes, stores), up to four at a time: the
    // chunks' reciprocal chains interleave and no divergent scale store separates them.
    constexpr int KB = VPT <= 4 ? VPT : 1;
    float y[VPT][8], s[VPT], r[VPT];
    uint32_t byte[VPT];
    bool zero[VPT];
#pragma unroll
    for (int k0 = 0; k0 < VPT; k0 += KB) {
#pragma unroll
      for (int k = k0; k < k0 + KB; ++k) {  // scales
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          y[k][e] = Y(k, e);
          m = fmaxf(m, fabsf(y[k][e]));
        }
        m = group_max<L>(m);
        s[k] = div448(m);
        zero[k] = (s[k] == 0.0f);  // before the E8M0 rounding turns it into 2^-127
        byte[k] = 0;
        if (e8) {  // uniform: a power of two 2^(byte-127), whose reciprocal is exact
          byte[k] = e8m0_ceil(s[k], &s[k]);
          r[k] = __builtin_amdgcn_ldexpf(1.0f, 127 - (int)byte[k]);
        } else {
          r[k] = 1.0f / s[k];
        }
      }
      u32x2 qc[VPT];
#pragma unroll
      for (int k = k0; k < k0 + KB; ++k) {  // codes; a zero scale (zero group) gives zero codes
        const bool inf = !zero[k] && not_finite(r[k]);
        if (wave_any(inf)) zero_safe_in_range(y[k], r[k], inf);  // uniform over the wave
        const float rk = r[k];
        qc[k] = (u32x2){fp8x4_in_range(y[k][0] * rk, y[k][1] * rk, y[k][2] * rk, y[k][3] * rk),
                        fp8x4_in_range(y[k][4] * rk, y[k][5] * rk, y[k][6] * rk, y[k][7] * rk)};
        if (zero[k]) qc[k] = (u32x2){0u, 0u};
      }
#pragma unroll
      for (int k = k0; k < k0 + KB; ++k) {  // stores
        const uint32_t c = o.lr + (uint32_t)(k * o.tpr);
        if (ok[k]) {
          __builtin_nontemporal_store(qc[k], boff(reinterpret_cast<u32x2*>(o.q + o.obase), c << 3));
          if ((o.lr % L) == 0) {
            const int64_t g = c / L;
            const int64_t idx = col ? g * o.ld + o.row : o.row * (o.n / GS) + g;
            if (u8) static_cast<uint8_t*>(o.scales)[idx] = (uint8_t)byte[k];
            else static_cast<float*>(o.scales)[idx] = s[k];
          }
        }
      }
    }
  } else if constexpr (MODE == kModeRowAmax) {
    float mx = 0.0f;
#pragma unroll
    for (int k = 0; k < VPT; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(Y(k, e)));
    mx = wave_max(mx);
    // One value per workgroup: the largest |y| over all its rows (rows past T hold zeros), at
    // scales[blockIdx.x].  Only the batch's maximum is needed, and fewer values make its
    // reduction short enough for the block pass's first workgroup.
    const int nw = (int)(blockDim.x >> 6);
    if (nw > 1) {  // uniform over the block
      if ((o.tid & 63) == 0) s_mx[o.tid >> 6] = mx;
      __syncthreads();
      mx = 0.0f;
      for (int i = 0; i < nw; ++i) mx = fmaxf(mx, s_mx[i]);
    }
    if (o.tid == 0) static_cast<float*>(o.scales)[blockIdx.x] = mx;
  } else if constexpr (MODE == kModePad) {
    // 16-bit row of n values at a stride of ld elements; chunks n/8 .. ld/8-1 are zero padding.
    // The launch covers ld/8 chunks per row (ok[] marks the chunks below n).
    const uint32_t nchp = (uint32_t)(o.ld >> 3);
    u32x4* orow = reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(o.q) + o.obase);
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const uint32_t c = o.lr + (uint32_t)(k * o.tpr);
      u32x4 v = (u32x4){0u, 0u, 0u, 0u};
      if (ok[k]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = pack_in<DT>(Y(k, 2 * j), Y(k, 2 * j + 1));
      }
      if (o.row_ok && c < nchp) __builtin_nontemporal_store(v, boff(orow, c << 4));
    }
  } else {  // RMSQ_FP4_BLOCK16
    const float gs = scale_val;
    // Both divisions of the scheme, exactly as IEEE division rounds them, without a division
    // sequence per chunk:
    //  * (a * gs) / 6: p * RN(1/6) corrected once by its FMA residual is the correctly rounded
    //    quotient for every binary32 p (checked exhaustively over [1, 4), both binades of the
    //    quotient; powers of two carry it to every p whose quotient can give a non-zero e4m3
    //    code).  An infinite p is replaced by FLT_MAX, which encodes to the same saturated code.
    //  * gs / decode(sf): decode(sf) = (1 + j/8) * 2^e, so the quotient is (gs / (1 + j/8)) * 2^-e,
    //    and scaling a binary32 value by a power of two is exact for normal results and
    //    overflows exactly when the quotient does.  Lane i of each wave holds gs / (1 + (i mod 8)/8)
    //    (one IEEE division per lane) and a chunk fetches its j with ds_bpermute.  When |gs| is
    //    below 2^-100 a quotient could be subnormal, and the IEEE division runs instead (the
    //    branch is uniform: gs is one value per launch).
    const bool by_table = fabsf(gs) >= 0x1p-100f;
    const float g_tab = gs / (1.0f + (float)(o.tid & 7) * 0.125f);
    constexpr float kSixth = 1.0f / 6.0f;
    // Chunks are taken KB at a time, in phases -- block scales, table exchanges, codes, stores --
    // so that nothing divergent separates one chunk's arithmetic from the next within a batch
    // and the batch's exchanges are in flight together.  Measured on MI355X: all chunks at once
    // is faster for one-wave rows (3-4 chunks per lane: 4096 x 2048 at 64 x 4 11.4 -> 11.3 us)
    // and for SiLU+Mul (4096 x 14336: 51.3 -> 47.4-48.9 us); the norm's rows of two chunks per
    // lane take them one at a time (16384 x 2048 at 128 x 2: 34.6 against 35.6 us; 4096 x 2048,
    // now 128 x 2 by default: 10.76 us either way).
    constexpr int KB = (FP4_BATCH && VPT <= 4) ? VPT : 1;  // more would spill registers
    float y[VPT][8], d[VPT], g[VPT];
    uint32_t sf[VPT], qc[VPT];
#pragma unroll
    for (int k0 = 0; k0 < VPT; k0 += KB) {
#pragma unroll
      for (int k = k0; k < k0 + KB; ++k) {  // block scales
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          y[k][e] = Y(k, e);
          m = fmaxf(m, fabsf(y[k][e]));
        }
        m = group_max<2>(m);  // a 16-element block is two neighbouring lanes
        const float p = fminf(m * gs, __FLT_MAX__);
        const float q0 = p * kSixth;
        sf[k] = fp8x1(fmaf(fmaf(-q0, 6.0f, p), kSixth, q0));
        d[k] = fp8_decode(sf[k]);
      }
#pragma unroll
      for (int k = k0; k < k0 + KB; ++k)  // every lane takes part, before any branch
        g[k] = __int_as_float(__builtin_amdgcn_ds_bpermute(
            (int)(((__float_as_uint(d[k]) >> 20) & 7u) << 2), __float_as_int(g_tab)));
#pragma unroll
      for (int k = k0; k < k0 + KB; ++k) {  // codes
        const bool live = d[k] > 0.0f;  // a zero block scale gives zero codes
        float mul = by_table ? __builtin_amdgcn_ldexpf(
                                   g[k], 127 - (int)((__float_as_uint(d[k]) >> 23) & 0xFFu))
                             : gs / d[k];
        const bool inf = live && not_finite(mul);
        if (wave_any(inf)) zero_safe(y[k], mul, inf);  // uniform over the wave
#pragma unroll
        for (int e = 0; e < 8; ++e) y[k][e] *= mul;
        qc[k] = live ? fp4x8(y[k]) : 0u;
      }
#pragma unroll
      for (int k = k0; k < k0 + KB; ++k) {  // stores
        const uint32_t c = o.lr + (uint32_t)(k * o.tpr);
        if (ok[k]) {
          *boff(reinterpret_cast<uint32_t*>(o.q + o.obase / 2), c << 2) = qc[k];
          if ((c & 1) == 0) static_cast<uint8_t*>(o.scales)[o.obase / 16 + c / 2] = (uint8_t)sf[k];
        }
      }
    }
  }
}

// EXACT: the launch covers every chunk of every row with no remainder (threads_per_row x
// chunks_per_thread x 8 == H and T a multiple of rows_per_block), so no load or store needs a
// predicate; otherwise out-of-range chunks and rows are masked.
// DT: the activation type of x, the residual, the weight and the new residual (0 bf16,
// 1 IEEE binary16); everything after the residual sum is f32 either way.
template <int MODE, bool RES, int VPT, int GS, bool EXACT, int DT>
__global__ void __launch_bounds__(1024) fused_kernel(KArgs a) {
  __shared__ double s_ss[kMaxWavesPerBlock];
  __shared__ float s_mx[kMaxWavesPerBlock];

  const int tid = threadIdx.x;
  const int tpr = a.tpr;
  const int wpr = tpr >> 6;  // waves per row
  // Row bookkeeping is wave-uniform (scalar registers): a row spans whole waves, so the wave
  // index decides the row within the block, and row base addresses stay scalar.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rib = (a.rpb == 1) ? 0 : wave / wpr;  // row within the block
  const uint32_t lr = (uint32_t)(tid - rib * tpr);  // thread within the row
  const uint32_t rb = a.xcd_ranges ? rowblock_of(blockIdx.x, a.nblk) : blockIdx.x;
  const int64_t row = (int64_t)rb * a.rpb + rib;
  const bool row_ok = EXACT || row < a.T;
  const int nch = (int)(a.H >> 3);
  const size_t base = (size_t)(row_ok ? row : 0) * (size_t)a.H;  // element offset of the row
  const u32x4* xrow = reinterpret_cast<const u32x4*>(a.x + base);
  const u32x4* rrow = reinterpret_cast<const u32x4*>(a.res + base);
  const u32x4* wrow = reinterpret_cast<const u32x4*>(a.w);

  // The per-tensor scale is fetched first, with the row: fetched later it would cost every
  // workgroup a second memory round trip after the reduction.
  float scale_val = 0.0f;
  if constexpr (MODE == RMSQ_FP8_STATIC || MODE == RMSQ_FP4_BLOCK16) scale_val = a.scale_in[0];
  if constexpr (MODE == kModeFp4Batch) {
    if (a.amax_parts == nullptr) {  // uniform: a launch either has the scale or derives it
      scale_val = a.scale_in[0];
    } else if (blockIdx.x == 0) {  // s_mx: not otherwise used by the FP4 epilogue
      scale_val = batch_scale_publish(a.amax_parts, a.n_parts, a.gs_out, s_mx);
    }
  }
  if constexpr (MODE == kModeRowAmax) {
    if (a.gs_out != nullptr && blockIdx.x == 0 && tid == 0) *a.gs_out = 0.0f;
  }

  // ---- load: x (+ residual) first, then the weight (an L2 hit), each byte once ----
  u32x4 hv[VPT], wv[VPT], rv[VPT];
  bool ok[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const uint32_t c = lr + (uint32_t)(k * tpr);
    ok[k] = EXACT || (row_ok && c < (uint32_t)nch);
    hv[k] = (u32x4){0u, 0u, 0u, 0u};
    rv[k] = (u32x4){0u, 0u, 0u, 0u};
    if constexpr (DT == 1 || (MODE == RMSQ_FP8_TOKEN && VPT >= 7)) {
      // binary16: a masked chunk loads chunk 0 of the row (always present; row 0 for a row
      // past T) and discards it.  Without a branch around the loads the binary16 instantiations
      // stay within their register budget at many chunks per lane (with it, 6-8 chunks spill);
      // bf16 keeps the branch, which measured faster for it, except for the per-token scheme at
      // 7-8 chunks per lane (rows beyond 57344 elements), which needs the registers.
      const uint32_t cs = ok[k] ? c : 0u;
      const u32x4 xl = __builtin_nontemporal_load(boff(xrow, cs << 4));
      hv[k] = ok[k] ? xl : hv[k];
      if constexpr (RES) {
        const u32x4 rl = __builtin_nontemporal_load(boff(rrow, cs << 4));
        rv[k] = ok[k] ? rl : rv[k];
      }
    } else if (ok[k]) {
      hv[k] = __builtin_nontemporal_load(boff(xrow, c << 4));
      if (RES) rv[k] = __builtin_nontemporal_load(boff(rrow, c << 4));
    }
  }
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const uint32_t c = lr + (uint32_t)(k * tpr);
    wv[k] = (u32x4){0u, 0u, 0u, 0u};
    if constexpr (DT == 1) {
      const u32x4 wl = *boff(wrow, (ok[k] ? c : 0u) << 4);
      wv[k] = ok[k] ? wl : wv[k];
    } else if (ok[k]) {
      wv[k] = *boff(wrow, c << 4);
    }
  }

  // The published global scale, loaded behind the row (used only by the epilogue).
  float gs_seen = 0.0f;
  if constexpr (MODE == kModeFp4Batch) {
    if (a.amax_parts != nullptr && blockIdx.x != 0)
      gs_seen = __hip_atomic_load(a.gs_out, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- residual add: h = round16(x + r), written back as the new residual ----
  if constexpr (RES) {
    u32x4* orow = reinterpret_cast<u32x4*>(a.res_out + base);
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      u32x4 h;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        h[j] = pack_in<DT>(in_lo<DT>(hv[k][j]) + in_lo<DT>(rv[k][j]),
                           in_hi<DT>(hv[k][j]) + in_hi<DT>(rv[k][j]));
      hv[k] = h;
      if (ok[k]) __builtin_nontemporal_store(h, boff(orow, (lr + (uint32_t)(k * tpr)) << 4));
    }
  }

  float inv;
  if (MODE == kModeFp4Batch && a.inv_rows != nullptr) {
    // the block pass of FP4 with a batch scale (one wave per row, uniform branch): the row
    // pass's inverse RMS, staged in this row's own block-scale bytes; every store of this wave
    // depends on it, so the load completes before the wave overwrites those bytes
    inv = *reinterpret_cast<const float*>(a.inv_rows +
                                          (size_t)(row_ok ? row : 0) * (size_t)a.inv_stride);
  } else {
    // ---- sum of squares (binary64; two chains, the products are exact) -> inv_rms ----
    double ss0 = 0.0, ss1 = 0.0;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const double lo = (double)in_lo<DT>(hv[k][j]);
        const double hi = (double)in_hi<DT>(hv[k][j]);
        ss0 = fma(lo, lo, ss0);
        ss1 = fma(hi, hi, ss1);
      }
    }
    double ss = wave_sum(ss0 + ss1);
    if (wpr > 1) {  // uniform over the block
      if ((tid & 63) == 0) s_ss[tid >> 6] = ss;
      __syncthreads();
      ss = 0.0;
      for (int i = 0; i < wpr; ++i) ss += s_ss[rib * wpr + i];
    }
    inv = inv_rms(ss, a.H, a.inv_h, a.eps);
  }
  if constexpr (MODE == kModeRowAmax) {  // stage it for the block pass
    if (a.inv_rows != nullptr && lr == 0 && row_ok)
      *reinterpret_cast<float*>(a.inv_rows + (size_t)row * (size_t)a.inv_stride) = inv;
  }

  // ---- quantize ----
  RowOut o;
  o.q = a.q;
  o.scales = a.scales;
  o.row = row;
  o.row_ok = row_ok;
  o.obase = (MODE == kModePad) ? (size_t)(row_ok ? row : 0) * (size_t)a.ld : base;
  o.n = a.H;
  o.ld = a.ld;
  o.flags = a.flags;
  o.lr = lr;
  o.tpr = tpr;
  o.wpr = wpr;
  o.rib = rib;
  o.tid = tid;
  if constexpr (MODE == kModeFp4Batch) {
    if (a.amax_parts != nullptr && blockIdx.x != 0) scale_val = batch_scale_await(gs_seen, a.gs_out);
  }
  constexpr int QMODE = (MODE == kModeFp4Batch) ? RMSQ_FP4_BLOCK16 : MODE;
  quantize_store<QMODE, VPT, GS, DT, (VPT >= 3)>(
      [&](int k, int e) { return y_of<DT>(hv[k], wv[k], e, inv); }, ok, o, scale_val, s_mx);
}

// ------------------------------------------------------------------ FP4 global scale of a batch
// The middle launch of FP4 with the global scale taken from the batch (PR #51925 summary: NVFP4
// with block scales and a global scale; its test derives a global scale as 448 * 6 over a
// tensor's absmax), where the block pass's first workgroup cannot reduce the row pass's maxima
// in one round of loads: one workgroup reduces the T maxima to the batch's largest |y| and
// writes gs (batch_fp4_scale).  The kernel (fp4_global_scale_kernel) is defined in
// table_misc.hip.
struct GArgs {
  const float* row_amax;  // [T], non-negative
  float* gs;              // [1]
  int64_t T;
};

// ------------------------------------------------------------------ SiLU+Mul -> quantization
// vLLM docs "Fusion torch.compile passes", section "SiLU+Mul + quantization (fuse_act_quant)":
// the gated up-projection activation silu_and_mul fused with the quantization that follows, so
// the f32 activation never reaches memory.  Row t of x is [2I] 16-bit values (DT 0 bf16, 1 IEEE
// binary16): gate g = x[t, 0:I], up u = x[t, I:2I]; a = silu(g) * u = g / (1 + exp(-g)) * u in
// f32, then quantize_store.
struct AArgs {
  const uint16_t* x;
  uint8_t* q;
  void* scales;
  const float* scale_in;
  int64_t T;
  int64_t I;
  int64_t ld;
  uint32_t flags;
  int32_t tpr;
  int32_t rpb;
  uint32_t nblk;
  int32_t xcd_ranges;
  uint32_t tiles;  // row-tiled launch: tiles per row
};

// exp(x) for x <= 0 in f32, within ~2 ulp: 2^(x log2 e) on the hardware exp2 (v_exp_f32), with
// the rounding error of the product x * log2(e) -- recovered exactly by an FMA, plus the part of
// log2(e) that f32 cannot hold -- applied as the first-order factor 1 + r ln 2.  For x <= 0 the
// result lies in [0, 1], so no overflow handling is needed; below about -103 it is 0.
__device__ __forceinline__ float exp_nonpositive(float x) {
  constexpr float kLog2e = 1.44269502162933349609375f;    // log2(e) rounded to f32
  constexpr float kLog2eLo = 1.925963033500011e-08f;      // log2(e) - kLog2e
  constexpr float kLn2 = 0.693147180559945309f;
  const float p = x * kLog2e;
  const float r = fmaf(x, kLog2eLo, fmaf(x, kLog2e, -p));
  const float e0 = __builtin_amdgcn_exp2f(p);
  return fmaf(e0, r * kLn2, e0);
}

// silu(g) * u in f32, within a few ulp of the exactly rounded value: with e = exp(-|g|),
// silu(g) = g / (1 + e) for g >= 0 and g * e / (1 + e) for g < 0 (nothing overflows; very
// negative gates give the tiny activations they should), the reciprocal on the hardware
// v_rcp_f32 (1 ulp).
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = exp_nonpositive(-fabsf(g));
  const float num = g >= 0.0f ? g : g * e;
  return (num * __builtin_amdgcn_rcpf(1.0f + e)) * u;
}

template <int MODE, int VPT, int GS, bool EXACT, int DT>
__global__ void __launch_bounds__(1024) silu_mul_kernel(AArgs a) {
  __shared__ float s_mx[kMaxWavesPerBlock];

  const int tid = threadIdx.x;
  const int tpr = a.tpr;
  const int wpr = tpr >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rib = (a.rpb == 1) ? 0 : wave / wpr;
  const uint32_t lr = (uint32_t)(tid - rib * tpr);
  const uint32_t rb = a.xcd_ranges ? rowblock_of(blockIdx.x, a.nblk) : blockIdx.x;
  const int64_t row = (int64_t)rb * a.rpb + rib;
  const bool row_ok = EXACT || row < a.T;
  const int nch = (int)(a.I >> 3);
  const size_t obase = (size_t)(row_ok ? row : 0) * (size_t)a.I;
  const u32x4* grow = reinterpret_cast<const u32x4*>(a.x + 2 * obase);
  const u32x4* urow = reinterpret_cast<const u32x4*>(a.x + 2 * obase + a.I);

  float scale_val = 0.0f;
  if constexpr (MODE == RMSQ_FP8_STATIC || MODE == RMSQ_FP4_BLOCK16) scale_val = a.scale_in[0];

  u32x4 gv[VPT], uv[VPT];
  bool ok[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const uint32_t c = lr + (uint32_t)(k * tpr);
    ok[k] = EXACT || (row_ok && c < (uint32_t)nch);
    gv[k] = (u32x4){0u, 0u, 0u, 0u};
    uv[k] = (u32x4){0u, 0u, 0u, 0u};
    if constexpr (DT == 1) {  // binary16: branch-free masked loads, as in fused_kernel
      const uint32_t cs = ok[k] ? c : 0u;
      const u32x4 gl = __builtin_nontemporal_load(boff(grow, cs << 4));
      const u32x4 ul = __builtin_nontemporal_load(boff(urow, cs << 4));
      gv[k] = ok[k] ? gl : gv[k];
      uv[k] = ok[k] ? ul : uv[k];
    } else if (ok[k]) {
      gv[k] = __builtin_nontemporal_load(boff(grow, c << 4));
      uv[k] = __builtin_nontemporal_load(boff(urow, c << 4));
    }
  }
  float act[VPT][8];
#pragma unroll
  for (int k = 0; k < VPT; ++k)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      act[k][2 * j] = silu_mul(in_lo<DT>(gv[k][j]), in_lo<DT>(uv[k][j]));
      act[k][2 * j + 1] = silu_mul(in_hi<DT>(gv[k][j]), in_hi<DT>(uv[k][j]));
    }

  RowOut o;
  o.q = a.q;
  o.scales = a.scales;
  o.row = row;
  o.row_ok = row_ok;
  o.obase = obase;
  o.n = a.I;
  o.ld = a.ld;
  o.flags = a.flags;
  o.lr = lr;
  o.tpr = tpr;
  o.wpr = wpr;
  o.rib = rib;
  o.tid = tid;
  quantize_store<MODE, VPT, GS>([&](int k, int e) { return act[k][e]; }, ok, o, scale_val, s_mx);
}

// Row-tiled SiLU+Mul -> quantization for the schemes that need no row-wide reduction (static,
// per-group, FP4): workgroup b takes tile (b mod tiles) of row (b / tiles), a tile being
// threads x VPT chunks, so consecutive workgroups cover consecutive stretches of a row and a
// long row does not become one very wide workgroup.  Tiles hold whole groups (threads is a
// multiple of 64, a group at most 16 chunks).
template <int MODE, int VPT, int GS, bool EXACT, int DT>
__global__ void __launch_bounds__(1024) silu_mul_tile_kernel(AArgs a) {
  static_assert(MODE != RMSQ_FP8_TOKEN, "per-token scaling needs whole rows");
  const int tid = threadIdx.x;
  const int tpr = a.tpr;  // threads per tile
  const uint32_t row32 = blockIdx.x / a.tiles;
  const uint32_t tile = blockIdx.x - row32 * a.tiles;
  const int64_t row = row32;
  const int nch = (int)(a.I >> 3);
  const uint32_t lr = tile * (uint32_t)(tpr * VPT) + (uint32_t)tid;  // first chunk of this thread
  const size_t obase = (size_t)row * (size_t)a.I;
  const u32x4* grow = reinterpret_cast<const u32x4*>(a.x + 2 * obase);
  const u32x4* urow = reinterpret_cast<const u32x4*>(a.x + 2 * obase + a.I);

  float scale_val = 0.0f;
  if constexpr (MODE == RMSQ_FP8_STATIC || MODE == RMSQ_FP4_BLOCK16) scale_val = a.scale_in[0];

  u32x4 gv[VPT], uv[VPT];
  bool ok[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const uint32_t c = lr + (uint32_t)(k * tpr);
    ok[k] = EXACT || c < (uint32_t)nch;
    gv[k] = (u32x4){0u, 0u, 0u, 0u};
    uv[k] = (u32x4){0u, 0u, 0u, 0u};
    if constexpr (DT == 1) {  // binary16: branch-free masked loads, as in fused_kernel
      const uint32_t cs = ok[k] ? c : 0u;
      const u32x4 gl = __builtin_nontemporal_load(boff(grow, cs << 4));
      const u32x4 ul = __builtin_nontemporal_load(boff(urow, cs << 4));
      gv[k] = ok[k] ? gl : gv[k];
      uv[k] = ok[k] ? ul : uv[k];
    } else if (ok[k]) {
      gv[k] = __builtin_nontemporal_load(boff(grow, c << 4));
      uv[k] = __builtin_nontemporal_load(boff(urow, c << 4));
    }
  }
  float act[VPT][8];
#pragma unroll
  for (int k = 0; k < VPT; ++k)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      act[k][2 * j] = silu_mul(in_lo<DT>(gv[k][j]), in_lo<DT>(uv[k][j]));
      act[k][2 * j + 1] = silu_mul(in_hi<DT>(gv[k][j]), in_hi<DT>(uv[k][j]));
    }

  RowOut o;
  o.q = a.q;
  o.scales = a.scales;
  o.row = row;
  o.row_ok = true;
  o.obase = obase;
  o.n = a.I;
  o.ld = a.ld;
  o.flags = a.flags;
  o.lr = lr;
  o.tpr = tpr;
  o.wpr = 1;
  o.rib = 0;
  o.tid = tid;
  quantize_store<MODE, VPT, GS>([&](int k, int e) { return act[k][e]; }, ok, o, scale_val,
                                nullptr);
}

// ------------------------------------------------------------------ QK-norm + RoPE
// vLLM docs "Fusion torch.compile passes", section "QK Norm + RoPE": for models with per-head
// Q/K normalization, each q and k head of the packed qkv tensor is RMS-normalized (q and k with
// their own weights) and rotated by the rotary embedding, in place, in one pass.
//
// Layout on the lanes: a head of D elements is held by L = D/16 consecutive lanes; lane c holds
// the two 8-element chunks c and c + L, i.e. elements 8c..8c+7 of the first half of the head and
// the same offsets of the second half.  Every NeoX pair (i, i + D/2) and every interleaved pair
// (2i, 2i+1) is then inside one lane, so the rotation needs no cross-lane traffic; only the sum
// of squares is reduced over the L lanes.  A workgroup serves hpb heads of one token with
// hpb / HPT lane groups; group g takes heads g, g + groups, ... (HPT of them), so each load
// instruction of a wave reads whole 128-byte lines and every lane has 2*HPT chunks in flight.
struct RArgs {
  uint16_t* qkv;           // [T, (Hq + 2 Hkv) * D] 16-bit, q and k heads rewritten in place
  const uint16_t* qw;      // [D]
  const uint16_t* kw;      // [D]
  const float* cache;      // [max_pos, D]: cos | sin
  const int64_t* pos;      // [T]
  int64_t T;
  int64_t max_pos;
  float eps;
  int32_t hq;              // q heads
  int32_t nh;              // q + k heads (the ones rewritten)
  int32_t width;           // (Hq + 2 Hkv) * D
  int32_t hpb;             // heads per workgroup
  int32_t groups;          // lane groups per workgroup (hpb / HPT)
  uint32_t nhb;            // workgroups per token
};

template <int L>
__device__ __forceinline__ double group_sum(double v) {
  // Sum over aligned groups of L lanes (2 to 16, within one DPP row); every lane of a group
  // gets the sum.  Must run with all lanes of the group active.
  v += dpp<0xB1>(v);                   // lane ^ 1
  if (L >= 4) v += dpp<0x4E>(v);       // lane ^ 2
  if (L >= 8) v += dpp<0x141>(v);      // the other quad of the 8
  if (L >= 16) v += dpp<0x140>(v);     // the other half of the 16
  return v;
}

// DT: the 16-bit type of qkv and the weights (0 bf16, 1 IEEE binary16); the arithmetic is f32
// (binary64 sum of squares) either way and the result is rounded back to DT.
template <int D, bool NEOX, int HPT, int DT>
__global__ void __launch_bounds__(1024) qk_norm_rope_kernel(RArgs a) {
  constexpr int L = D / 16;   // lanes per head
  constexpr int CH = D / 8;   // 16-byte chunks per head
  const uint32_t t = blockIdx.x / a.nhb;
  const uint32_t hb = blockIdx.x - t * a.nhb;
  const int64_t p = a.pos[t];
  if (p < 0 || p >= a.max_pos) return;  // out-of-range position: the token is left unchanged
  const int tid = threadIdx.x;
  const int c = tid % L;
  const int h0 = (int)hb * a.hpb + tid / L;
  u32x4* row = reinterpret_cast<u32x4*>(a.qkv + (size_t)t * (size_t)a.width);

  // every load first: the heads' chunks, both weights, this lane's cos/sin
  u32x4 xv[HPT][2];
#pragma unroll
  for (int k = 0; k < HPT; ++k) {
    const int h = h0 + k * a.groups;
    xv[k][0] = xv[k][1] = (u32x4){0u, 0u, 0u, 0u};
    if (h < a.nh) {
      xv[k][0] = __builtin_nontemporal_load(row + h * CH + c);
      xv[k][1] = __builtin_nontemporal_load(row + h * CH + c + L);
    }
  }
  const u32x4* qw = reinterpret_cast<const u32x4*>(a.qw);
  const u32x4* kw = reinterpret_cast<const u32x4*>(a.kw);
  const u32x4 wq0 = qw[c], wq1 = qw[c + L], wk0 = kw[c], wk1 = kw[c + L];
  const float* cs = a.cache + (size_t)p * D;
  float cv[16], sv[16];
  if constexpr (NEOX) {
    // elements 8c+e and D/2+8c+e form pair j = 8c+e
    const f32x4* cp = reinterpret_cast<const f32x4*>(cs + 8 * c);
    const f32x4* sp = reinterpret_cast<const f32x4*>(cs + D / 2 + 8 * c);
    const f32x4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      cv[e] = c0[e]; cv[4 + e] = c1[e];
      sv[e] = s0[e]; sv[4 + e] = s1[e];
    }
  } else {
    // chunk c holds pairs j = 4c..4c+3, chunk c+L pairs j = D/4+4c..D/4+4c+3
    const f32x4 c0 = *reinterpret_cast<const f32x4*>(cs + 4 * c);
    const f32x4 c1 = *reinterpret_cast<const f32x4*>(cs + D / 4 + 4 * c);
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(cs + D / 2 + 4 * c);
    const f32x4 s1 = *reinterpret_cast<const f32x4*>(cs + D / 2 + D / 4 + 4 * c);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      cv[m] = c0[m]; cv[4 + m] = c1[m];
      sv[m] = s0[m]; sv[4 + m] = s1[m];
    }
  }

#pragma unroll
  for (int k = 0; k < HPT; ++k) {
    const int h = h0 + k * a.groups;
    double ss0 = 0.0, ss1 = 0.0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const double lo = (double)in_lo<DT>(xv[k][hh][j]);
        const double hi = (double)in_hi<DT>(xv[k][hh][j]);
        ss0 = fma(lo, lo, ss0);
        ss1 = fma(hi, hi, ss1);
      }
    }
    const double ss = group_sum<L>(ss0 + ss1);
    // D is a power of two: ss * (1/D) is exact, the same value as the quotient ss / D
    const float inv = inv_sqrt_f32(ss * (1.0 / D) + (double)a.eps);
    const bool isq = h < a.hq;
    const u32x4 w0 = isq ? wq0 : wk0, w1 = isq ? wq1 : wk1;
    float y0[8], y1[8], o0[8], o1[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      y0[e] = y_of<DT>(xv[k][0], w0, e, inv);
      y1[e] = y_of<DT>(xv[k][1], w1, e, inv);
    }
    if constexpr (NEOX) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ac = y0[e] * cv[e], bs = y1[e] * sv[e];
        const float bc = y1[e] * cv[e], as = y0[e] * sv[e];
        o0[e] = ac - bs;
        o1[e] = bc + as;
      }
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        {
          const float ac = y0[2 * m] * cv[m], bs = y0[2 * m + 1] * sv[m];
          const float bc = y0[2 * m + 1] * cv[m], as = y0[2 * m] * sv[m];
          o0[2 * m] = ac - bs;
          o0[2 * m + 1] = bc + as;
        }
        {
          const float ac = y1[2 * m] * cv[4 + m], bs = y1[2 * m + 1] * sv[4 + m];
          const float bc = y1[2 * m + 1] * cv[4 + m], as = y1[2 * m] * sv[4 + m];
          o1[2 * m] = ac - bs;
          o1[2 * m + 1] = bc + as;
        }
      }
    }
    if (h < a.nh) {
      __builtin_nontemporal_store(
          (u32x4){pack_in<DT>(o0[0], o0[1]), pack_in<DT>(o0[2], o0[3]),
                  pack_in<DT>(o0[4], o0[5]), pack_in<DT>(o0[6], o0[7])},
          row + h * CH + c);
      __builtin_nontemporal_store(
          (u32x4){pack_in<DT>(o1[0], o1[1]), pack_in<DT>(o1[2], o1[3]),
                  pack_in<DT>(o1[4], o1[5]), pack_in<DT>(o1[6], o1[7])},
          row + h * CH + c + L);
    }
  }
}

}  // namespace rmsq
