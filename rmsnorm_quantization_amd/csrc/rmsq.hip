// rmsq.hip -- fused (residual add ->) RMSNorm -> FP8 / FP4 quantization for MI355X (gfx950),
// and the C ABI declared in include/rmsq.h.
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
//     lane (c mod threads_per_row) of the row's waves, in registers, for the whole kernel, so
//     every input byte is loaded exactly once (128-bit non-temporal loads);
//   * sum of squares in binary64 (exact products of bf16 values), butterfly within the wave,
//     LDS only across the waves of one row; inv_rms rounded once to f32;
//   * per-group (64/128) and per-block (16) absmax: a group is 8 / 16 consecutive lanes (2 for
//     an FP4 block), reduced with DPP row operations -- no LDS, no barrier;
//   * hardware conversions: v_cvt_pk_bf16_f32, v_cvt_pk_fp8_f32 (OCP e4m3fn on gfx950),
//     v_cvt_scalef32_pk_fp4_f32 (unit scale), v_cvt_f32_fp8;
//   * no MFMA: there is no contraction here, the op is HBM-bandwidth bound.
#include "rmsq_device.hpp"

#include <atomic>
#include <cmath>
#include <cstring>

#include "rmsq.h"

namespace rmsq {

constexpr int kMaxWavesPerBlock = 16;

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
  float eps;
  uint32_t flags;
  int32_t tpr;    // threads per row (multiple of 64)
  int32_t rpb;    // rows per block
  uint32_t nblk;  // workgroups in the grid
};

// One element of y = (h * inv) * w from the packed bf16 chunk dwords.
__device__ __forceinline__ float y_of(const u32x4& h, const u32x4& w, int e, float inv) {
  const uint32_t hd = h[e >> 1], wd = w[e >> 1];
  const float hf = (e & 1) ? bf16_hi(hd) : bf16_lo(hd);
  const float wf = (e & 1) ? bf16_hi(wd) : bf16_lo(wd);
  return (hf * inv) * wf;
}

template <int MODE, bool RES, int VPT, int GS>
__global__ void __launch_bounds__(1024) fused_kernel(KArgs a) {
  __shared__ double s_ss[kMaxWavesPerBlock];
  __shared__ float s_mx[kMaxWavesPerBlock];

  const int tid = threadIdx.x;
  const int tpr = a.tpr;
  const int rib = tid / tpr;       // row within the block
  const int lr = tid - rib * tpr;  // thread within the row
  const int wpr = tpr >> 6;        // waves per row
  const int64_t row = (int64_t)rowblock_of(blockIdx.x, a.nblk) * a.rpb + rib;
  const bool row_ok = row < a.T;
  const int64_t nch = a.H >> 3;
  const size_t base = (size_t)(row_ok ? row : 0) * (size_t)a.H;  // element offset of the row

  // ---- load: x (+ residual) and weight chunks, each byte once ----
  u32x4 hv[VPT], wv[VPT], rv[VPT];
  bool ok[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int64_t c = lr + (int64_t)k * tpr;
    ok[k] = row_ok && c < nch;
    hv[k] = (u32x4){0u, 0u, 0u, 0u};
    wv[k] = (u32x4){0u, 0u, 0u, 0u};
    rv[k] = (u32x4){0u, 0u, 0u, 0u};
    if (ok[k]) {
      hv[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.x + base) + c);
      if (RES) rv[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.res + base) + c);
      wv[k] = reinterpret_cast<const u32x4*>(a.w)[c];
    }
  }

  // ---- residual add: h = bf16(x + r), written back as the new residual ----
  if constexpr (RES) {
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      u32x4 h;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        h[j] = pack_bf16x2(bf16_lo(hv[k][j]) + bf16_lo(rv[k][j]),
                           bf16_hi(hv[k][j]) + bf16_hi(rv[k][j]));
      hv[k] = h;
      if (ok[k]) {
        const int64_t c = lr + (int64_t)k * tpr;
        __builtin_nontemporal_store(h, reinterpret_cast<u32x4*>(a.res_out + base) + c);
      }
    }
  }

  // ---- sum of squares (binary64) -> inv_rms ----
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double lo = (double)bf16_lo(hv[k][j]);
      const double hi = (double)bf16_hi(hv[k][j]);
      ss = fma(lo, lo, ss);
      ss = fma(hi, hi, ss);
    }
  }
  ss = wave_sum(ss);
  if (wpr > 1) {  // uniform over the block
    if ((tid & 63) == 0) s_ss[tid >> 6] = ss;
    __syncthreads();
    ss = 0.0;
    for (int i = 0; i < wpr; ++i) ss += s_ss[rib * wpr + i];
  }
  const float inv = (float)(1.0 / sqrt(ss / (double)a.H + (double)a.eps));

  // ---- quantize ----
  if constexpr (MODE == RMSQ_FP8_STATIC) {
    const float r = 1.0f / a.scale_in[0];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = y_of(hv[k], wv[k], e, inv) * r;
      const u32x2 qc = {fp8x4(v[0], v[1], v[2], v[3]), fp8x4(v[4], v[5], v[6], v[7])};
      if (ok[k]) {
        const int64_t c = lr + (int64_t)k * tpr;
        __builtin_nontemporal_store(qc, reinterpret_cast<u32x2*>(a.q + base) + c);
      }
    }
  } else if constexpr (MODE == RMSQ_FP8_TOKEN) {
    float mx = 0.0f;
#pragma unroll
    for (int k = 0; k < VPT; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(y_of(hv[k], wv[k], e, inv)));
    mx = wave_max(mx);
    if (wpr > 1) {
      if ((tid & 63) == 0) s_mx[tid >> 6] = mx;
      __syncthreads();
      mx = 0.0f;
      for (int i = 0; i < wpr; ++i) mx = fmaxf(mx, s_mx[rib * wpr + i]);
    }
    const float s = mx / kFp8Max;
    if (lr == 0 && row_ok) static_cast<float*>(a.scales)[row] = s;
    const bool zero = (s == 0.0f);
    const float r = zero ? 0.0f : 1.0f / s;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = y_of(hv[k], wv[k], e, inv) * r;
      u32x2 qc = {fp8x4(v[0], v[1], v[2], v[3]), fp8x4(v[4], v[5], v[6], v[7])};
      if (zero) qc = (u32x2){0u, 0u};
      if (ok[k]) {
        const int64_t c = lr + (int64_t)k * tpr;
        __builtin_nontemporal_store(qc, reinterpret_cast<u32x2*>(a.q + base) + c);
      }
    }
  } else if constexpr (MODE == RMSQ_FP8_GROUP) {
    constexpr int L = GS / 8;  // lanes per group
    const bool e8 = (a.flags & (RMSQ_SCALE_E8M0 | RMSQ_SCALE_E8M0_U8)) != 0;
    const bool u8 = (a.flags & RMSQ_SCALE_E8M0_U8) != 0;
    const bool col = (a.flags & RMSQ_SCALE_COLMAJOR) != 0;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int64_t c = lr + (int64_t)k * tpr;
      float y[8];
      float m = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y[e] = y_of(hv[k], wv[k], e, inv);
        m = fmaxf(m, fabsf(y[e]));
      }
      m = group_max<L>(m);
      float s = m / kFp8Max;
      const bool zero = (s == 0.0f);
      uint32_t byte = 0;
      if (e8) byte = e8m0_ceil(s, &s);
      const float r = 1.0f / s;
      u32x2 qc = {fp8x4(y[0] * r, y[1] * r, y[2] * r, y[3] * r),
                  fp8x4(y[4] * r, y[5] * r, y[6] * r, y[7] * r)};
      if (zero) qc = (u32x2){0u, 0u};
      if (ok[k]) {
        __builtin_nontemporal_store(qc, reinterpret_cast<u32x2*>(a.q + base) + c);
        if ((lr % L) == 0) {
          const int64_t g = c / L;
          const int64_t idx = col ? g * a.ld + row : row * (a.H / GS) + g;
          if (u8) static_cast<uint8_t*>(a.scales)[idx] = (uint8_t)byte;
          else static_cast<float*>(a.scales)[idx] = s;
        }
      }
    }
  } else {  // RMSQ_FP4_BLOCK16
    const float gs = a.scale_in[0];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int64_t c = lr + (int64_t)k * tpr;
      float y[8];
      float m = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y[e] = y_of(hv[k], wv[k], e, inv);
        m = fmaxf(m, fabsf(y[e]));
      }
      m = group_max<2>(m);  // a 16-element block is two neighbouring lanes
      const uint32_t sf = fp8x1((m * gs) / 6.0f);
      const float d = fp8_decode(sf);
      uint32_t qc = 0u;
      if (d > 0.0f) {
        const float mul = gs / d;
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] *= mul;
        qc = fp4x8(y);
      }
      if (ok[k]) {
        reinterpret_cast<uint32_t*>(a.q + base / 2)[c] = qc;
        if ((c & 1) == 0) static_cast<uint8_t*>(a.scales)[base / 16 + c / 2] = (uint8_t)sf;
      }
    }
  }
}

// The kernels' own converters over a flat f32 array, 8 elements per thread.
__global__ void __launch_bounds__(256) convert_kernel(int fmt, const float* in, void* out,
                                                      int64_t nchunks) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= nchunks) return;
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = in[c * 8 + e];
  if (fmt == RMSQ_CVT_E4M3) {
    reinterpret_cast<u32x2*>(out)[c] =
        (u32x2){fp8x4(v[0], v[1], v[2], v[3]), fp8x4(v[4], v[5], v[6], v[7])};
  } else if (fmt == RMSQ_CVT_E2M1) {
    reinterpret_cast<uint32_t*>(out)[c] = fp4x8(v);
  } else {
    reinterpret_cast<u32x4*>(out)[c] = (u32x4){pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                               pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
  }
}

// ------------------------------------------------------------------ kernel table
template <int MODE, bool RES, int GS>
const void* pick_vpt(int vpt) {
  switch (vpt) {
    case 1: return reinterpret_cast<const void*>(&fused_kernel<MODE, RES, 1, GS>);
    case 2: return reinterpret_cast<const void*>(&fused_kernel<MODE, RES, 2, GS>);
    case 4: return reinterpret_cast<const void*>(&fused_kernel<MODE, RES, 4, GS>);
    case 8: return reinterpret_cast<const void*>(&fused_kernel<MODE, RES, 8, GS>);
    default: return nullptr;
  }
}

template <bool RES>
const void* pick_kernel(int mode, int gs, int vpt) {
  switch (mode) {
    case RMSQ_FP8_STATIC: return pick_vpt<RMSQ_FP8_STATIC, RES, 0>(vpt);
    case RMSQ_FP8_TOKEN: return pick_vpt<RMSQ_FP8_TOKEN, RES, 0>(vpt);
    case RMSQ_FP8_GROUP:
      return gs == 64 ? pick_vpt<RMSQ_FP8_GROUP, RES, 64>(vpt)
                      : pick_vpt<RMSQ_FP8_GROUP, RES, 128>(vpt);
    case RMSQ_FP4_BLOCK16: return pick_vpt<RMSQ_FP4_BLOCK16, RES, 16>(vpt);
    default: return nullptr;
  }
}

// ------------------------------------------------------------------ host side
bool valid_launch(const rmsq_launch& l, int64_t H) {
  if (l.reserved != 0) return false;
  if (l.threads_per_row < 64 || l.threads_per_row > 1024 || (l.threads_per_row % 64) != 0)
    return false;
  if (l.chunks_per_thread != 1 && l.chunks_per_thread != 2 && l.chunks_per_thread != 4 &&
      l.chunks_per_thread != 8)
    return false;
  if (l.rows_per_block < 1 || (int64_t)l.rows_per_block * l.threads_per_row > 1024) return false;
  if ((int64_t)l.threads_per_row * l.chunks_per_thread * 8 < H) return false;
  return true;
}

// Default launch shape.  One wave per row while the row fits in 4 chunks per lane (H <= 2048);
// beyond that two chunks per lane and as many waves as the row needs (H = 4096: 4 waves,
// 8192: 8 waves), four chunks per lane past 16384.  Short rows are packed several to a
// workgroup so a workgroup has at least 256 threads.
rmsq_launch default_launch(int64_t H) {
  rmsq_launch l{64, 1, 1, 0};
  const int64_t nch = H / 8;
  if (nch <= 256) {
    l.threads_per_row = 64;
    l.chunks_per_thread = nch <= 64 ? 1 : (nch <= 128 ? 2 : 4);
  } else {
    int vpt = nch <= 2048 ? 2 : (nch <= 4096 ? 4 : 8);
    int64_t t = (nch + vpt - 1) / vpt;
    l.threads_per_row = (int32_t)((t + 63) / 64 * 64);
    l.chunks_per_thread = vpt;
  }
  l.rows_per_block = l.threads_per_row >= 256 ? 1 : 256 / l.threads_per_row;
  return l;
}

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }
Span span(const void* p, size_t bytes) {
  const uintptr_t u = reinterpret_cast<uintptr_t>(p);
  return Span{u, u + bytes};
}
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

std::atomic<int> g_arch[64];  // per device: 0 unknown, 1 gfx950, 2 other

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return RMSQ_EDEVICE;
  int st = dev < 64 ? g_arch[dev].load(std::memory_order_relaxed) : 0;
  if (st == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return RMSQ_EDEVICE;
    st = std::strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    if (dev < 64) g_arch[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? RMSQ_OK : RMSQ_EUNSUPPORTED;
}

// Validation of the scalar arguments (no pointer is touched).
int check_scalars(int64_t T, int64_t H, float eps, int mode, int gs, unsigned flags,
                  int64_t ld) {
  if (T < 0 || H < 8 || H > RMSQ_MAX_HIDDEN || (H % 8) != 0) return RMSQ_EINVAL;
  if (!(eps > 0.0f) || !std::isfinite(eps)) return RMSQ_EINVAL;
  if (T > 0x7FFFFFFFLL) return RMSQ_EINVAL;
  switch (mode) {
    case RMSQ_FP8_STATIC:
    case RMSQ_FP8_TOKEN:
      if (gs != 0) return RMSQ_EINVAL;
      if (flags != 0) return RMSQ_EUNSUPPORTED;
      if (ld != 0) return RMSQ_EINVAL;
      break;
    case RMSQ_FP8_GROUP: {
      if (gs != 64 && gs != 128) return RMSQ_EINVAL;
      if ((H % gs) != 0) return RMSQ_EINVAL;
      const unsigned known = RMSQ_SCALE_COLMAJOR | RMSQ_SCALE_E8M0 | RMSQ_SCALE_E8M0_U8;
      if ((flags & ~known) != 0) return RMSQ_EUNSUPPORTED;
      if ((flags & RMSQ_SCALE_E8M0) && (flags & RMSQ_SCALE_E8M0_U8)) return RMSQ_EUNSUPPORTED;
      if (flags & RMSQ_SCALE_COLMAJOR) {
        if (ld != 0 && ld < T) return RMSQ_EINVAL;
      } else if (ld != 0) {
        return RMSQ_EINVAL;
      }
      break;
    }
    case RMSQ_FP4_BLOCK16:
      if (gs != 16 || (H % 16) != 0) return RMSQ_EINVAL;
      if (flags != 0) return RMSQ_EUNSUPPORTED;
      if (ld != 0) return RMSQ_EINVAL;
      break;
    default:
      return RMSQ_EINVAL;
  }
  return RMSQ_OK;
}

int check_pointers(const void* x, const void* res, const void* w, int mode, const float* scale_in,
                   const void* q, const void* scales, const void* res_out, int64_t T, int64_t H,
                   int gs, unsigned flags, int64_t ld) {
  if (!x || !w || !q) return RMSQ_EINVAL;
  if ((res == nullptr) != (res_out == nullptr)) return RMSQ_EINVAL;
  const bool needs_scale_in = (mode == RMSQ_FP8_STATIC || mode == RMSQ_FP4_BLOCK16);
  if (needs_scale_in != (scale_in != nullptr)) return RMSQ_EINVAL;
  const bool has_scales = (mode != RMSQ_FP8_STATIC);
  if (has_scales != (scales != nullptr)) return RMSQ_EINVAL;

  // alignment
  if (!aligned(x, 16) || !aligned(w, 16)) return RMSQ_EALIGN;
  if (res && (!aligned(res, 16) || !aligned(res_out, 16))) return RMSQ_EALIGN;
  if (!aligned(q, mode == RMSQ_FP4_BLOCK16 ? 4 : 8)) return RMSQ_EALIGN;
  if (scale_in && !aligned(scale_in, 4)) return RMSQ_EALIGN;
  const bool f32_scales = (mode == RMSQ_FP8_TOKEN) ||
                          (mode == RMSQ_FP8_GROUP && !(flags & RMSQ_SCALE_E8M0_U8));
  if (f32_scales && !aligned(scales, 4)) return RMSQ_EALIGN;

  // aliasing: outputs must not overlap inputs or each other; residual_out may be residual
  const size_t act = (size_t)T * (size_t)H * 2;
  const size_t qbytes = mode == RMSQ_FP4_BLOCK16 ? (size_t)T * (size_t)H / 2 : (size_t)T * H;
  size_t sbytes = 0;
  if (mode == RMSQ_FP8_TOKEN) sbytes = (size_t)T * 4;
  if (mode == RMSQ_FP8_GROUP) {
    const size_t ng = (size_t)(H / gs), el = (flags & RMSQ_SCALE_E8M0_U8) ? 1 : 4;
    sbytes = (flags & RMSQ_SCALE_COLMAJOR) ? ((ng - 1) * (size_t)(ld ? ld : T) + (size_t)T) * el
                                           : (size_t)T * ng * el;
  }
  if (mode == RMSQ_FP4_BLOCK16) sbytes = (size_t)T * (size_t)(H / 16);
  const Span sx = span(x, act), sw = span(w, (size_t)H * 2), sq = span(q, qbytes);
  const Span ss = span(scales, sbytes), si = span(scale_in, scale_in ? 4 : 0);
  Span outs[3] = {sq, ss, Span{0, 0}};
  int nout = scales ? 2 : 1;
  if (res_out) outs[nout++] = span(res_out, act);
  for (int i = 0; i < nout; ++i) {
    if (overlap(outs[i], sx) || overlap(outs[i], sw) || overlap(outs[i], si)) return RMSQ_EALIAS;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return RMSQ_EALIAS;
  }
  if (res) {
    const Span sr = span(res, act);
    if (overlap(sq, sr) || (scales && overlap(ss, sr))) return RMSQ_EALIAS;
    if (res_out != res && overlap(span(res_out, act), sr)) return RMSQ_EALIAS;
  }
  return RMSQ_OK;
}

int validate(const void* x, const void* res, const void* w, float eps, int mode,
             const float* scale_in, const void* q, const void* scales, const void* res_out,
             int64_t T, int64_t H, int gs, unsigned flags, int64_t ld) {
  const int st = check_scalars(T, H, eps, mode, gs, flags, ld);
  if (st != RMSQ_OK || T == 0) return st;
  return check_pointers(x, res, w, mode, scale_in, q, scales, res_out, T, H, gs, flags, ld);
}

int fused_impl(const void* x, const void* res, const void* w, float eps, int mode,
               const float* scale_in, void* q, void* scales, void* res_out, int64_t T, int64_t H,
               int gs, unsigned flags, int64_t ld, const rmsq_launch* launch, void* stream) {
  int st = validate(x, res, w, eps, mode, scale_in, q, scales, res_out, T, H, gs, flags, ld);
  if (st != RMSQ_OK) return st;
  const rmsq_launch l = launch ? *launch : default_launch(H);
  if (!valid_launch(l, H)) return RMSQ_EINVAL;
  if (T == 0) return RMSQ_OK;
  st = check_device();
  if (st != RMSQ_OK) return st;

  const void* fn = res ? pick_kernel<true>(mode, gs, l.chunks_per_thread)
                       : pick_kernel<false>(mode, gs, l.chunks_per_thread);
  if (!fn) return RMSQ_EINVAL;
  const int64_t nblk = (T + l.rows_per_block - 1) / l.rows_per_block;
  KArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.res = static_cast<const uint16_t*>(res);
  a.w = static_cast<const uint16_t*>(w);
  a.res_out = static_cast<uint16_t*>(res_out);
  a.q = static_cast<uint8_t*>(q);
  a.scales = scales;
  a.scale_in = scale_in;
  a.T = T;
  a.H = H;
  a.ld = (flags & RMSQ_SCALE_COLMAJOR) ? (ld ? ld : T) : 0;
  a.eps = eps;
  a.flags = flags;
  a.tpr = l.threads_per_row;
  a.rpb = l.rows_per_block;
  a.nblk = (uint32_t)nblk;
  void* args[] = {&a};
  const hipError_t e =
      hipLaunchKernel(fn, dim3((uint32_t)nblk), dim3((uint32_t)(l.threads_per_row * l.rows_per_block)),
                      args, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RMSQ_OK : RMSQ_ELAUNCH;
}

}  // namespace rmsq

using namespace rmsq;

extern "C" {

int rmsq_fused(const void* x, const void* residual, const void* weight, float eps, int mode,
               const float* scale_in, void* out_q, void* out_scales, void* residual_out,
               int64_t tokens, int64_t hidden, int group_size, unsigned flags, int64_t scale_ld,
               void* stream) {
  return fused_impl(x, residual, weight, eps, mode, scale_in, out_q, out_scales, residual_out,
                    tokens, hidden, group_size, flags, scale_ld, nullptr, stream);
}

int rmsq_fused_with_launch(const void* x, const void* residual, const void* weight, float eps,
                           int mode, const float* scale_in, void* out_q, void* out_scales,
                           void* residual_out, int64_t tokens, int64_t hidden, int group_size,
                           unsigned flags, int64_t scale_ld, const rmsq_launch* launch,
                           void* stream) {
  return fused_impl(x, residual, weight, eps, mode, scale_in, out_q, out_scales, residual_out,
                    tokens, hidden, group_size, flags, scale_ld, launch, stream);
}

int rmsq_validate(const void* x, const void* residual, const void* weight, float eps, int mode,
                  const float* scale_in, const void* out_q, const void* out_scales,
                  const void* residual_out, int64_t tokens, int64_t hidden, int group_size,
                  unsigned flags, int64_t scale_ld) {
  return validate(x, residual, weight, eps, mode, scale_in, out_q, out_scales, residual_out,
                  tokens, hidden, group_size, flags, scale_ld);
}

int rmsq_query_launch(int mode, int64_t tokens, int64_t hidden, int group_size,
                      int has_residual, rmsq_launch* launch, int64_t* grid) {
  (void)has_residual;
  if (!launch) return RMSQ_EINVAL;
  const unsigned flags = 0;
  const int st = check_scalars(tokens, hidden, 1e-6f, mode, group_size, flags, 0);
  if (st != RMSQ_OK) return st;
  *launch = default_launch(hidden);
  if (grid) *grid = (tokens + launch->rows_per_block - 1) / launch->rows_per_block;
  return RMSQ_OK;
}

int64_t rmsq_block_to_rowblock(int64_t block, int64_t grid) {
  if (grid <= 0 || grid > 0xFFFFFFFFLL || block < 0 || block >= grid) return -1;
  return (int64_t)rowblock_of((uint32_t)block, (uint32_t)grid);
}

int rmsq_convert(int format, const float* in, void* out, int64_t n, void* stream) {
  if (format != RMSQ_CVT_E4M3 && format != RMSQ_CVT_E2M1 && format != RMSQ_CVT_BF16)
    return RMSQ_EINVAL;
  if (n < 0 || (n % 8) != 0) return RMSQ_EINVAL;
  if (n == 0) return RMSQ_OK;
  if (!in || !out) return RMSQ_EINVAL;
  if (!aligned(in, 16) || !aligned(out, 16)) return RMSQ_EALIGN;
  const size_t ob = format == RMSQ_CVT_E4M3 ? (size_t)n : format == RMSQ_CVT_E2M1 ? n / 2 : n * 2;
  if (overlap(span(in, (size_t)n * 4), span(out, ob))) return RMSQ_EALIAS;
  const int st = check_device();
  if (st != RMSQ_OK) return st;
  const int64_t nch = n / 8;
  const int64_t blocks = (nch + 255) / 256;
  if (blocks > 0x7FFFFFFFLL) return RMSQ_EINVAL;
  int fmt = format;
  void* args[] = {&fmt, &in, &out, const_cast<int64_t*>(&nch)};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&convert_kernel),
                                       dim3((uint32_t)blocks), dim3(256), args, 0,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RMSQ_OK : RMSQ_ELAUNCH;
}

const char* rmsq_status_string(int status) {
  switch (status) {
    case RMSQ_OK: return "ok";
    case RMSQ_EINVAL: return "invalid argument";
    case RMSQ_EALIGN: return "misaligned pointer";
    case RMSQ_EALIAS: return "output overlaps an input or another output";
    case RMSQ_EUNSUPPORTED: return "unsupported flag/mode combination or device (gfx950 only)";
    case RMSQ_ELAUNCH: return "kernel launch failed";
    case RMSQ_EDEVICE: return "no HIP device";
    default: return "unknown status";
  }
}

int rmsq_abi_version(void) { return RMSQ_ABI_VERSION; }

}  // extern "C"
