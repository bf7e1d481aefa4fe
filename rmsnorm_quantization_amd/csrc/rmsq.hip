// rmsq.hip -- host side of librmsq: argument validation, launch-shape heuristics, kernel
// dispatch and the C ABI declared in include/rmsq.h.  The kernels are in rmsq_kernels.hpp; their
// instantiations live in the table_*.hip units (compiled in parallel), reached through
// rmsq_kernel_table.hpp.
#include <hip/hip_ext.h>

#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>

#include "rmsq_kernel_table.hpp"

namespace rmsq {

// ------------------------------------------------------------------ host side
bool valid_launch(const rmsq_launch& l, int64_t H) {
  if ((l.options & ~RMSQ_LAUNCH_XCD_RANGES) != 0) return false;
  if (l.threads_per_row < 64 || l.threads_per_row > 1024 || (l.threads_per_row % 64) != 0)
    return false;
  if (l.chunks_per_thread < 1 || l.chunks_per_thread > 8) return false;
  if (l.rows_per_block < 1 || (int64_t)l.rows_per_block * l.threads_per_row > 1024) return false;
  if ((int64_t)l.threads_per_row * l.chunks_per_thread * 8 < H) return false;
  return true;
}

// Default launch shape, from sweeps on MI355X.  Rows of at most 128 chunks (H <= 1024) take one
// wave each, four rows to a workgroup.  Longer rows take the chunks-per-thread count in 2..8
// that leaves the fewest idle lanes with at most 1024 threads per row, fewer chunks per thread
// on a tie: H = 2048 / 4096 / 5120 / 7168 / 8192 / 16384 give 128 / 256 / 320 / 448 / 512 /
// 1024 threads x 2 chunks, all exact fits (no predicated loads).  Exact fits measured 2-3%
// faster than 256 threads with idle lanes.
rmsq_launch default_launch(int64_t H) {
  rmsq_launch l{64, 1, 1, 0};
  const int64_t nch = H / 8;
  if (nch <= 128) {
    l.chunks_per_thread = (int32_t)((nch + 63) / 64);
    l.rows_per_block = 4;
    return l;
  }
  int64_t best_waste = -1;
  for (int vpt = 2; vpt <= 8; ++vpt) {
    const int64_t tpr = ((nch + vpt - 1) / vpt + 63) / 64 * 64;
    if (tpr > 1024) continue;
    const int64_t waste = tpr * vpt - nch;
    if (best_waste < 0 || waste < best_waste) {
      best_waste = waste;
      l.threads_per_row = (int32_t)tpr;
      l.chunks_per_thread = vpt;
    }
  }
  return l;
}

// Default shape of the quantizing launch for a batch of T rows.  For the schemes whose epilogue
// ends in one row-wide reduction (per-token scaling, and the row pass of FP4 with a batch scale:
// `row_reduction`), a batch that is in flight all at once (at least 1024 rows and at most 2^20
// chunks, so every wave is resident from the start) whose rows fill two to four whole waves'
// worth of single chunks (H = 1536 or 2048) takes one wave per row with 3-4 chunks per lane: such
// a wave reduces its row with DPP alone, no LDS exchange and no barrier.  Measured on MI355X
// (median of 300 dispatch-stamped launches, two alternations), 64 x 4 against 128 x 2 at H = 2048:
// per-token 4.36-4.40 against 4.68-5.16 us at 1024 rows, 11.52 against 11.60 us at 4096; the
// batch-scale FP4 step 8.84 against 9.03 us at 1024 rows.  The other schemes keep default_launch
// (128 x 2 there), which the same sweep found as fast or faster now that their epilogues work in
// phases: per-group-128 4.56-4.64 against 4.96 us at 1024 rows and 11.64 against 12.20-12.24 us
// at 4096, FP4 block-16 10.76-10.84 against 11.12-11.16 us at 4096, static within 1%.  Rows of
// 8 chunks per lane (H = 4096) measured 6% slower at 2048 rows than 256 x 2 and keep
// default_launch, as do larger batches.
rmsq_launch default_fused_launch(int64_t T, int64_t H, bool row_reduction) {
  const int64_t nch = H / 8;
  if (row_reduction && nch > 128 && nch <= 256 && (nch % 64) == 0 && T >= 1024 &&
      T * nch <= (int64_t(1) << 20))
    return rmsq_launch{64, (int32_t)(nch / 64), 1, 0};
  return default_launch(H);
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

// Per device index below 64: 0 unknown, 1 gfx950, 2 other (the library's only state, stated in
// rmsq.h); filled by the first call that launches on the device.
std::atomic<int> g_arch[64];

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

// ---- validation shared by both ops: the quantization outputs ----------------------------
// Scalar arguments of a quantization of T rows of n values (no pointer is touched).
int check_quant_scalars(int64_t T, int64_t n, int mode, int gs, unsigned flags, int64_t ld) {
  if (T < 0 || T > 0x7FFFFFFFLL) return RMSQ_EINVAL;
  if (n < 8 || n > RMSQ_MAX_HIDDEN || (n % 8) != 0) return RMSQ_EINVAL;
  switch (mode) {
    case RMSQ_FP8_STATIC:
    case RMSQ_FP8_TOKEN:
      if (gs != 0) return RMSQ_EINVAL;
      if (flags != 0) return RMSQ_EUNSUPPORTED;
      if (ld != 0) return RMSQ_EINVAL;
      break;
    case RMSQ_FP8_GROUP: {
      if (gs != 64 && gs != 128) return RMSQ_EINVAL;
      if ((n % gs) != 0) return RMSQ_EINVAL;
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
      if (gs != 16 || (n % 16) != 0) return RMSQ_EINVAL;
      if (flags != 0) return RMSQ_EUNSUPPORTED;
      if (ld != 0) return RMSQ_EINVAL;
      break;
    default:
      return RMSQ_EINVAL;
  }
  return RMSQ_OK;
}

// Presence, alignment and byte extents of the quantization outputs (and the per-tensor scale
// input); outputs[0..*nout) receives the output extents, in_scale the scale_in extent.
int check_quant_outputs(int mode, const float* scale_in, const void* q, const void* scales,
                        int64_t T, int64_t n, int gs, unsigned flags, int64_t ld, Span* outputs,
                        int* nout, Span* in_scale) {
  if (!q) return RMSQ_EINVAL;
  const bool needs_scale_in = (mode == RMSQ_FP8_STATIC || mode == RMSQ_FP4_BLOCK16);
  if (needs_scale_in != (scale_in != nullptr)) return RMSQ_EINVAL;
  const bool has_scales = (mode != RMSQ_FP8_STATIC);
  if (has_scales != (scales != nullptr)) return RMSQ_EINVAL;
  if (!aligned(q, mode == RMSQ_FP4_BLOCK16 ? 4 : 8)) return RMSQ_EALIGN;
  if (scale_in && !aligned(scale_in, 4)) return RMSQ_EALIGN;
  const bool f32_scales = (mode == RMSQ_FP8_TOKEN) ||
                          (mode == RMSQ_FP8_GROUP && !(flags & RMSQ_SCALE_E8M0_U8));
  if (f32_scales && !aligned(scales, 4)) return RMSQ_EALIGN;
  const size_t qbytes = mode == RMSQ_FP4_BLOCK16 ? (size_t)T * (size_t)n / 2 : (size_t)T * n;
  size_t sbytes = 0;
  if (mode == RMSQ_FP8_TOKEN) sbytes = (size_t)T * 4;
  if (mode == RMSQ_FP8_GROUP) {
    const size_t ng = (size_t)(n / gs), el = (flags & RMSQ_SCALE_E8M0_U8) ? 1 : 4;
    sbytes = (flags & RMSQ_SCALE_COLMAJOR) ? ((ng - 1) * (size_t)(ld ? ld : T) + (size_t)T) * el
                                           : (size_t)T * ng * el;
  }
  if (mode == RMSQ_FP4_BLOCK16) sbytes = (size_t)T * (size_t)(n / 16);
  outputs[0] = span(q, qbytes);
  *nout = 1;
  if (scales) outputs[(*nout)++] = span(scales, sbytes);
  *in_scale = span(scale_in, scale_in ? 4 : 0);
  return RMSQ_OK;
}

// Outputs must not overlap one another or any input span.
int check_aliasing(const Span* outs, int nout, const Span* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlap(outs[i], ins[j])) return RMSQ_EALIAS;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return RMSQ_EALIAS;
  }
  return RMSQ_OK;
}

int launch_kernel(const void* fn, int64_t nblk, int threads, void* argstruct, void* stream,
                  void* start_event, void* stop_event) {
  // the dispatch packet's grid is counted in work-items, a 32-bit quantity
  if (nblk <= 0 || nblk * (int64_t)threads > 0xFFFFFFFFLL) return RMSQ_EINVAL;
  void* args[] = {argstruct};
  const dim3 grid((uint32_t)nblk), block((uint32_t)threads);
  hipError_t e;
  if (start_event || stop_event)
    e = hipExtLaunchKernel(fn, grid, block, args, 0, static_cast<hipStream_t>(stream),
                           static_cast<hipEvent_t>(start_event),
                           static_cast<hipEvent_t>(stop_event), 0);
  else
    e = hipLaunchKernel(fn, grid, block, args, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RMSQ_OK : RMSQ_ELAUNCH;
}

bool exact_fit(const rmsq_launch& l, int64_t T, int64_t n) {
  return (int64_t)l.threads_per_row * l.chunks_per_thread * 8 == n && (T % l.rows_per_block) == 0;
}

// ---- fused (residual add ->) RMSNorm -> quantization ---------------------------------------
int validate(const void* x, const void* res, const void* w, float eps, int mode,
             const float* scale_in, const void* q, const void* scales, const void* res_out,
             int64_t T, int64_t H, int gs, unsigned flags, int64_t ld) {
  flags &= ~(unsigned)RMSQ_INPUT_F16;  // the activation type; the rest describes the scales
  int st = check_quant_scalars(T, H, mode, gs, flags, ld);
  if (st != RMSQ_OK) return st;
  if (!(eps > 0.0f) || !std::isfinite(eps)) return RMSQ_EINVAL;
  if (T == 0) return RMSQ_OK;
  if (!x || !w) return RMSQ_EINVAL;
  if ((res == nullptr) != (res_out == nullptr)) return RMSQ_EINVAL;
  Span outs[3], sin;
  int nout = 0;
  st = check_quant_outputs(mode, scale_in, q, scales, T, H, gs, flags, ld, outs, &nout, &sin);
  if (st != RMSQ_OK) return st;
  if (!aligned(x, 16) || !aligned(w, 16)) return RMSQ_EALIGN;
  if (res && (!aligned(res, 16) || !aligned(res_out, 16))) return RMSQ_EALIGN;
  const size_t act = (size_t)T * (size_t)H * 2;
  const Span ins[3] = {span(x, act), span(w, (size_t)H * 2), sin};
  // residual_out may be the residual itself (in-place update) but must not otherwise overlap
  // it; it is an output like the others with respect to x, weight and scale_in
  if (res_out) outs[nout++] = span(res_out, act);
  st = check_aliasing(outs, nout, ins, 3);
  if (st != RMSQ_OK) return st;
  if (res) {
    const Span sr = span(res, act);
    for (int i = 0; i < nout - 1; ++i)
      if (overlap(outs[i], sr)) return RMSQ_EALIAS;
    if (res_out != res && overlap(span(res_out, act), sr)) return RMSQ_EALIAS;
  }
  return RMSQ_OK;
}

int fused_impl(const void* x, const void* res, const void* w, float eps, int mode,
               const float* scale_in, void* q, void* scales, void* res_out, int64_t T, int64_t H,
               int gs, unsigned flags, int64_t ld, const rmsq_launch* launch, void* stream,
               void* start_event = nullptr, void* stop_event = nullptr) {
  int st = validate(x, res, w, eps, mode, scale_in, q, scales, res_out, T, H, gs, flags, ld);
  if (st != RMSQ_OK) return st;
  const rmsq_launch l = launch ? *launch : default_fused_launch(T, H, mode == RMSQ_FP8_TOKEN);
  if (!valid_launch(l, H)) return RMSQ_EINVAL;
  if (T == 0) return RMSQ_OK;
  st = check_device();
  if (st != RMSQ_OK) return st;
  const bool exact = exact_fit(l, T, H);
  const void* fn = (flags & RMSQ_INPUT_F16)
                       ? fused_kernel_f16(mode, res != nullptr, gs, l.chunks_per_thread, exact)
                       : fused_kernel_bf16(mode, res != nullptr, gs, l.chunks_per_thread, exact);
  if (!fn) return RMSQ_EINVAL;
  const int64_t nblk = (T + l.rows_per_block - 1) / l.rows_per_block;
  KArgs a{};
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
  a.inv_h = 1.0 / (double)H;
  a.flags = flags;
  a.tpr = l.threads_per_row;
  a.rpb = l.rows_per_block;
  a.nblk = (uint32_t)nblk;
  a.xcd_ranges = (l.options & RMSQ_LAUNCH_XCD_RANGES) ? 1 : 0;
  return launch_kernel(fn, nblk, l.threads_per_row * l.rows_per_block, &a, stream, start_event,
                       stop_event);
}

// ---- FP4 block-16 with the global scale taken from the batch --------------------------------
// Everything the static FP4 call checks, with global_scale in the place of scale_in; as an output
// it must not overlap x, the residual or the weight either.
int validate_fp4_dynamic(const void* x, const void* res, const void* w, float eps, const void* q,
                         const void* scales, const void* res_out, const float* global_scale,
                         int64_t T, int64_t H, unsigned flags) {
  if ((flags & ~(unsigned)RMSQ_INPUT_F16) != 0) return RMSQ_EUNSUPPORTED;
  int st = validate(x, res, w, eps, RMSQ_FP4_BLOCK16, global_scale, q, scales, res_out, T, H, 16,
                    flags, 0);
  if (st != RMSQ_OK || T == 0) return st;
  const size_t act = (size_t)T * (size_t)H * 2;
  const Span g = span(global_scale, 4);
  if (overlap(g, span(x, act)) || overlap(g, span(w, (size_t)H * 2)) ||
      (res && overlap(g, span(res, act))))
    return RMSQ_EALIAS;
  return RMSQ_OK;
}

// Two launches: (1) residual add + RMSNorm, each workgroup's largest |y| staged as f32 at the
// start of out_q, global_scale cleared to 0; (2) the FP4 block-16 kernel without a residual on
// the normalized input (the new residual, or x), whose workgroup 0 reduces the maxima to gs and
// hands it to the others through global_scale.  Where that workgroup cannot reduce them in one
// round, a one-workgroup reduction runs between the two instead and launch 2 reads gs.  Launch
// 2 must see launch 1's y.  Where a row's block scales can hold an f32 (H % 64 == 0,
// out_scales 4-byte aligned) and a row fits one wave (H <= 4096), launch 1 also stages each
// row's inverse RMS there and launch 2 runs one wave per row and reads it: only that wave later
// writes those bytes.  Otherwise both launches use the same threads and chunks per row, so that
// both reduce each row's squares in the same order.
// Rows per workgroup of the block pass of FP4 with a batch global scale: raised from the
// default shape's up to 16 (within 1024 threads) while the grid keeps at least 256 workgroups,
// so a batch in flight all at once still spreads over every CU.  Its workgroup 0 reduces the row
// pass's maxima, eight loads per thread in one round: 16 one-wave rows take up to 8192.
int32_t batch_rows_per_block(const rmsq_launch& l, int64_t T) {
  for (int32_t r = 16; r > l.rows_per_block; r /= 2)
    if ((int64_t)r * l.threads_per_row <= 1024 && T >= 256 * (int64_t)r) return r;
  return l.rows_per_block;
}

// Rows per workgroup of the row pass when the caller gives no shape: the default shape's, raised
// only as far as it takes for its per-workgroup maxima to fit that one round (`cap` of them).
// More rows per workgroup measured slower for this pass (4096 x 2048, graph replay per step:
// 18.2-18.5 us with one, 19.1-19.3 us with 16; 16384 x 2048: 54.1-54.5 us with two or four,
// 58.0 us with 16, 55.4 us with one, which leaves too many maxima and takes the middle launch).
int32_t row_pass_rows_per_block(const rmsq_launch& l, int64_t T, int64_t cap) {
  int32_t r = l.rows_per_block;
  while ((T + r - 1) / r > cap && (int64_t)(2 * r) * l.threads_per_row <= 1024) r *= 2;
  return r;
}

int fp4_dynamic_impl(const void* x, const void* res, const void* w, float eps, void* q,
                     void* scales, void* res_out, float* global_scale, int64_t T, int64_t H,
                     unsigned flags, const rmsq_launch* launch, void* start_event,
                     void* stop_event, void* stream) {
  int st = validate_fp4_dynamic(x, res, w, eps, q, scales, res_out, global_scale, T, H, flags);
  if (st != RMSQ_OK) return st;
  rmsq_launch l = launch ? *launch : default_fused_launch(T, H, true);
  if (!valid_launch(l, H)) return RMSQ_EINVAL;
  if (T == 0) return RMSQ_OK;
  st = check_device();
  if (st != RMSQ_OK) return st;
  const bool stage = (H % 64) == 0 && H <= 4096 && aligned(scales, 4);
  // pass 3's shape: one wave per row where it reads the staged inverse RMS; otherwise the row
  // pass's threads and chunks, so that both passes sum each row's squares in the same order
  // (rows per workgroup do not enter that order)
  rmsq_launch l3 = l;
  if (stage) {
    l3 = default_launch(H);  // one wave per row (several rows per workgroup for H <= 1024)
    if (l3.threads_per_row != 64) l3 = rmsq_launch{64, (int32_t)((H / 8 + 63) / 64), 1, 0};
  }
  if (stage || !launch) l3.rows_per_block = batch_rows_per_block(l3, T);
  if (!launch)
    l.rows_per_block =
        row_pass_rows_per_block(l, T, 8 * (int64_t)l3.threads_per_row * l3.rows_per_block);
  const bool exact = exact_fit(l, T, H), f16 = (flags & RMSQ_INPUT_F16) != 0;
  const int vpt = l.chunks_per_thread;
  // The row pass leaves one maximum per workgroup.  When the block pass's first workgroup can
  // reduce them in one round (eight loads per thread), it derives and publishes gs itself while
  // the other workgroups load their rows, and there is no middle launch; otherwise the
  // one-workgroup reduction runs between the passes.
  const int64_t nblk = (T + l.rows_per_block - 1) / l.rows_per_block;
  const bool fold = nblk <= 8 * (int64_t)l3.threads_per_row * l3.rows_per_block;
  const bool exact3 = exact_fit(l3, T, H);
  const void* pass1 = f16 ? amax_kernel_f16(res != nullptr, vpt, exact)
                          : amax_kernel_bf16(res != nullptr, vpt, exact);
  const void* pass3 = f16 ? batch_fp4_kernel_f16(l3.chunks_per_thread, exact3)
                          : batch_fp4_kernel_bf16(l3.chunks_per_thread, exact3);
  if (!pass1 || !pass3) return RMSQ_EINVAL;
  const int threads = l.threads_per_row * l.rows_per_block;
  KArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.res = static_cast<const uint16_t*>(res);
  a.w = static_cast<const uint16_t*>(w);
  a.res_out = static_cast<uint16_t*>(res_out);
  a.q = nullptr;
  a.scales = q;  // the workgroup maxima, [nblk] f32 at the start of out_q
  a.scale_in = nullptr;
  a.T = T;
  a.H = H;
  a.ld = 0;
  a.eps = eps;
  a.inv_h = 1.0 / (double)H;
  a.flags = 0;
  a.tpr = l.threads_per_row;
  a.rpb = l.rows_per_block;
  a.nblk = (uint32_t)nblk;
  a.xcd_ranges = (l.options & RMSQ_LAUNCH_XCD_RANGES) ? 1 : 0;
  a.inv_rows = stage ? static_cast<uint8_t*>(scales) : nullptr;
  a.inv_stride = H / 16;
  a.gs_out = fold ? global_scale : nullptr;  // cleared to 0: not yet published
  st = launch_kernel(pass1, nblk, threads, &a, stream, start_event, nullptr);
  if (st != RMSQ_OK) return st;
  if (!fold) {
    GArgs g;
    g.row_amax = static_cast<const float*>(q);
    g.gs = global_scale;
    g.T = nblk;
    st = launch_kernel(fp4_global_scale_kernel_ptr(), 1, 1024, &g, stream, nullptr, nullptr);
    if (st != RMSQ_OK) return st;
  }
  KArgs b = a;
  b.x = res ? static_cast<const uint16_t*>(res_out) : static_cast<const uint16_t*>(x);
  b.res = nullptr;
  b.res_out = nullptr;
  b.q = static_cast<uint8_t*>(q);
  b.scales = scales;
  b.scale_in = fold ? nullptr : global_scale;
  b.amax_parts = fold ? static_cast<const float*>(q) : nullptr;
  b.n_parts = fold ? nblk : 0;
  b.gs_out = fold ? global_scale : nullptr;
  b.tpr = l3.threads_per_row;
  b.rpb = l3.rows_per_block;
  const int64_t nblk3 = (T + l3.rows_per_block - 1) / l3.rows_per_block;
  b.nblk = (uint32_t)nblk3;
  b.xcd_ranges = (l3.options & RMSQ_LAUNCH_XCD_RANGES) ? 1 : 0;
  return launch_kernel(pass3, nblk3, l3.threads_per_row * l3.rows_per_block, &b, stream, nullptr,
                       stop_event);
}

// ---- residual add + RMSNorm -> padded 16-bit output ------------------------------------------
int validate_pad(const void* x, const void* res, const void* w, float eps, const void* out,
                 const void* res_out, int64_t T, int64_t H, int64_t out_ld, unsigned flags) {
  if ((flags & ~(unsigned)RMSQ_INPUT_F16) != 0) return RMSQ_EUNSUPPORTED;
  if (T < 0 || T > 0x7FFFFFFFLL) return RMSQ_EINVAL;
  if (H < 8 || H > RMSQ_MAX_HIDDEN || (H % 8) != 0) return RMSQ_EINVAL;
  if (out_ld < H || out_ld > RMSQ_MAX_HIDDEN || (out_ld % 8) != 0) return RMSQ_EINVAL;
  if (!(eps > 0.0f) || !std::isfinite(eps)) return RMSQ_EINVAL;
  if (T == 0) return RMSQ_OK;
  if (!x || !w || !out) return RMSQ_EINVAL;
  if ((res == nullptr) != (res_out == nullptr)) return RMSQ_EINVAL;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(out, 16)) return RMSQ_EALIGN;
  if (res && (!aligned(res, 16) || !aligned(res_out, 16))) return RMSQ_EALIGN;
  const size_t act = (size_t)T * (size_t)H * 2;
  Span outs[2] = {span(out, (size_t)T * (size_t)out_ld * 2), Span{0, 0}};
  int nout = 1;
  if (res_out) outs[nout++] = span(res_out, act);
  const Span ins[2] = {span(x, act), span(w, (size_t)H * 2)};
  int st = check_aliasing(outs, nout, ins, 2);
  if (st != RMSQ_OK) return st;
  if (res) {
    const Span sr = span(res, act);
    if (overlap(outs[0], sr)) return RMSQ_EALIAS;
    if (res_out != res && overlap(span(res_out, act), sr)) return RMSQ_EALIAS;
  }
  return RMSQ_OK;
}

// Default shape of the padded-output launch: one wave per row with up to 8 chunks per lane when
// the padded row fits (ld <= 4096: 64 threads x ceil(ld/512) chunks), else the quantizing
// kernel's rule.  Measured on MI355X for 2880 -> 3072 (4096 rows): 17.1 us against 18.3 us
// for 192 threads x 2 chunks; equal at 4000 -> 4096; better at 2000 -> 2048.
//
// Binary16 activations take the one-wave shape only up to 6 chunks per lane (4096 rows,
// 2880 -> 3072: 17.6 us at 64 x 6 against 18.0 us at 192 x 2; 4000 -> 4096: 24.4 us at 64 x 8
// against 23.9 us at 256 x 2); longer binary16 rows take the quantizing kernel's rule.
rmsq_launch default_pad_launch(int64_t ld, unsigned flags) {
  const int64_t nch = ld / 8;
  const int64_t max_chunks = (flags & RMSQ_INPUT_F16) ? 6 : 8;
  if (nch > 128 && (nch + 63) / 64 <= max_chunks)
    return rmsq_launch{64, (int32_t)((nch + 63) / 64), 1, 0};
  return default_launch(ld);
}

int pad_impl(const void* x, const void* res, const void* w, float eps, void* out, void* res_out,
             int64_t T, int64_t H, int64_t out_ld, unsigned flags, const rmsq_launch* launch,
             void* start_event, void* stop_event, void* stream) {
  int st = validate_pad(x, res, w, eps, out, res_out, T, H, out_ld, flags);
  if (st != RMSQ_OK) return st;
  const rmsq_launch l = launch ? *launch : default_pad_launch(out_ld, flags);
  if (!valid_launch(l, out_ld)) return RMSQ_EINVAL;  // the launch covers the padded row
  if (T == 0) return RMSQ_OK;
  st = check_device();
  if (st != RMSQ_OK) return st;
  const void* fn = (flags & RMSQ_INPUT_F16) ? pad_kernel_f16(res != nullptr, l.chunks_per_thread)
                                            : pad_kernel_bf16(res != nullptr, l.chunks_per_thread);
  if (!fn) return RMSQ_EINVAL;
  const int64_t nblk = (T + l.rows_per_block - 1) / l.rows_per_block;
  KArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.res = static_cast<const uint16_t*>(res);
  a.w = static_cast<const uint16_t*>(w);
  a.res_out = static_cast<uint16_t*>(res_out);
  a.q = static_cast<uint8_t*>(out);
  a.scales = nullptr;
  a.scale_in = nullptr;
  a.T = T;
  a.H = H;
  a.ld = out_ld;
  a.eps = eps;
  a.inv_h = 1.0 / (double)H;
  a.flags = 0;
  a.tpr = l.threads_per_row;
  a.rpb = l.rows_per_block;
  a.nblk = (uint32_t)nblk;
  a.xcd_ranges = (l.options & RMSQ_LAUNCH_XCD_RANGES) ? 1 : 0;
  return launch_kernel(fn, nblk, l.threads_per_row * l.rows_per_block, &a, stream, start_event,
                       stop_event);
}

// ---- SiLU+Mul -> quantization --------------------------------------------------------------
int validate_act(const void* x, int mode, const float* scale_in, const void* q,
                 const void* scales, int64_t T, int64_t I, int gs, unsigned flags, int64_t ld) {
  flags &= ~(unsigned)RMSQ_INPUT_F16;  // the activation type; the rest describes the scales
  int st = check_quant_scalars(T, I, mode, gs, flags, ld);
  if (st != RMSQ_OK || T == 0) return st;
  if (!x) return RMSQ_EINVAL;
  Span outs[2], sin;
  int nout = 0;
  st = check_quant_outputs(mode, scale_in, q, scales, T, I, gs, flags, ld, outs, &nout, &sin);
  if (st != RMSQ_OK) return st;
  if (!aligned(x, 16)) return RMSQ_EALIGN;
  const Span ins[2] = {span(x, (size_t)T * (size_t)I * 4), sin};
  return check_aliasing(outs, nout, ins, 2);
}

// Default SiLU+Mul launch: whole rows per workgroup, shaped as for rmsq_fused.  On MI355X at
// I = 14336 this beat every row-tiled shape (64-1024 threads x 1-4 chunks) by 3-10%.
// Default shape of SiLU+Mul -> quantization.  FP4 block-16 takes row tiles of one wave x 2 chunks
// (each workgroup 1024 elements of one row); whole rows with default_launch otherwise.  Measured
// on MI355X (median of 200 dispatch-stamped launches, two runs), FP4 at I = 14336: 46.2-46.3
// against 47.1-47.6 us at 4096 tokens, 172.4-173.2 against 178.6-179.1 us at 16384, 5.24-5.36
// against 5.48 us at 256, 13.84-13.92 against 13.76-13.96 us at 1024; I = 11008 at 4096 tokens
// 37.6-37.8 us.  Static and per-group scales keep whole rows, 3-8% faster at 16384 tokens than
// any tile (per-group 181.9 against 187.1-191.7 us, static 176.9-177.4 against 192.5-199.1 us).
rmsq_launch default_act_launch(int mode, int64_t T, int64_t I) {
  if (mode == RMSQ_FP4_BLOCK16) {
    const rmsq_launch tiles{64, 2, 1, RMSQ_LAUNCH_ROW_TILES};
    if (T * ((I / 8 + 127) / 128) <= 0x7FFFFFFFLL) return tiles;
  }
  return default_launch(I);
}

bool valid_act_launch(const rmsq_launch& l, int mode, int64_t I) {
  if (!(l.options & RMSQ_LAUNCH_ROW_TILES)) return valid_launch(l, I);
  if (l.options != RMSQ_LAUNCH_ROW_TILES || mode == RMSQ_FP8_TOKEN) return false;
  if (l.threads_per_row < 64 || l.threads_per_row > 1024 || (l.threads_per_row % 64) != 0)
    return false;
  if (l.chunks_per_thread != 1 && l.chunks_per_thread != 2 && l.chunks_per_thread != 4)
    return false;
  return l.rows_per_block == 1;
}

int act_impl(const void* x, int mode, const float* scale_in, void* q, void* scales, int64_t T,
             int64_t I, int gs, unsigned flags, int64_t ld, const rmsq_launch* launch,
             void* start_event, void* stop_event, void* stream) {
  int st = validate_act(x, mode, scale_in, q, scales, T, I, gs, flags, ld);
  if (st != RMSQ_OK) return st;
  const rmsq_launch l = launch ? *launch : default_act_launch(mode, T, I);
  if (!valid_act_launch(l, mode, I)) return RMSQ_EINVAL;
  if (T == 0) return RMSQ_OK;
  st = check_device();
  if (st != RMSQ_OK) return st;
  const bool tiled = (l.options & RMSQ_LAUNCH_ROW_TILES) != 0;
  const int64_t tile = (int64_t)l.threads_per_row * l.chunks_per_thread;
  const int64_t tiles = (I / 8 + tile - 1) / tile;
  const void* fn;
  int64_t nblk;
  const bool f16 = (flags & RMSQ_INPUT_F16) != 0;
  if (tiled) {
    if (T * tiles > 0x7FFFFFFFLL) return RMSQ_EINVAL;
    fn = f16 ? act_kernel_f16(true, (I / 8) % tile == 0, mode, gs, l.chunks_per_thread)
             : act_kernel_bf16(true, (I / 8) % tile == 0, mode, gs, l.chunks_per_thread);
    nblk = T * tiles;
  } else {
    fn = f16 ? act_kernel_f16(false, exact_fit(l, T, I), mode, gs, l.chunks_per_thread)
             : act_kernel_bf16(false, exact_fit(l, T, I), mode, gs, l.chunks_per_thread);
    nblk = (T + l.rows_per_block - 1) / l.rows_per_block;
  }
  if (!fn) return RMSQ_EINVAL;
  AArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.q = static_cast<uint8_t*>(q);
  a.scales = scales;
  a.scale_in = scale_in;
  a.T = T;
  a.I = I;
  a.ld = (flags & RMSQ_SCALE_COLMAJOR) ? (ld ? ld : T) : 0;
  a.flags = flags;
  a.tpr = l.threads_per_row;
  a.rpb = l.rows_per_block;
  a.nblk = (uint32_t)nblk;
  a.xcd_ranges = (l.options & RMSQ_LAUNCH_XCD_RANGES) ? 1 : 0;
  a.tiles = (uint32_t)tiles;
  return launch_kernel(fn, nblk, l.threads_per_row * l.rows_per_block, &a, stream, start_event,
                       stop_event);
}

// ---- QK-norm + RoPE ------------------------------------------------------------------------
constexpr int64_t kMaxQkvWidth = 1 << 20;  // elements of one token's qkv row

bool valid_rope_hpl(int hpl) { return hpl >= 1 && hpl <= 6; }

int validate_rope(const void* qkv, const void* qw, const void* kw, const float* cache,
                  const int64_t* pos, float eps, int64_t T, int hq, int hkv, int D,
                  int64_t max_pos, unsigned flags) {
  if ((flags & ~(unsigned)RMSQ_INPUT_F16) != 0) return RMSQ_EUNSUPPORTED;
  if (T < 0 || T > 0x7FFFFFFFLL) return RMSQ_EINVAL;
  if (D != 64 && D != 128 && D != 256) return RMSQ_EINVAL;
  if (hq < 1 || hkv < 1 || (int64_t)(hq + 2LL * hkv) * D > kMaxQkvWidth) return RMSQ_EINVAL;
  if (max_pos < 1) return RMSQ_EINVAL;
  if (!(eps > 0.0f) || !std::isfinite(eps)) return RMSQ_EINVAL;
  if (T == 0) return RMSQ_OK;
  if (!qkv || !qw || !kw || !cache || !pos) return RMSQ_EINVAL;
  if (!aligned(qkv, 16) || !aligned(qw, 16) || !aligned(kw, 16) || !aligned(cache, 16) ||
      !aligned(pos, 8))
    return RMSQ_EALIGN;
  const Span out = span(qkv, (size_t)T * (size_t)(hq + 2 * hkv) * (size_t)D * 2);
  const Span ins[4] = {span(qw, (size_t)D * 2), span(kw, (size_t)D * 2),
                       span(cache, (size_t)max_pos * (size_t)D * 4), span(pos, (size_t)T * 8)};
  return check_aliasing(&out, 1, ins, 4);
}

// Default shape: heads per lane group (hpl) and heads per workgroup (hpb, a multiple of hpl).
//
// A shape is judged by the lane-head slots it wastes per token (idle heads, partly filled
// waves) and by how many "rounds" its grid takes: waves / (what the chip holds at once, from
// the kernel's register use).  Measured on MI355X (40 heads of 128, T = 256 ... 16384):
//  * while one head per lane still fits in one round, it wins (more, shorter waves: T <= 1024);
//  * else the most heads per lane that still fits in one round (T = 2048, 4096: 5 per lane,
//    one 64-thread workgroup per token, 15.9 us at 4096 against 17.2-18.4 for the others);
//  * past one round, 2 heads per lane in single-wave workgroups (T = 8192: 29.2 us against
//    31.7 for 5 per lane; T = 16384: 55.4 against 60.5).
// Waves per SIMD by heads per lane (VGPRs 57 / 76 / 86 / 96 / 104 / 116 of 512), the same for
// every head size since a lane always holds 16 elements of a head.
constexpr int kRopeWavesPerSimd[7] = {0, 8, 6, 5, 5, 4, 4};
constexpr int64_t kSimds = 256 * 4;  // MI355X: 256 CUs x 4 SIMDs

void default_rope_shape(int64_t T, int nh, int D, int* hpl_out, int* hpb_out) {
  const int L = D / 16;
  struct Cand {
    int hpl, hpb;
    int64_t waste, wpb, dist;
    bool fits;
  };
  Cand cs[6 * 1024];
  int n = 0;
  int64_t least = -1;
  for (int hpl = 1; hpl <= 6; ++hpl) {
    if (hpl > nh) continue;
    for (int g = 1; g * L <= 1024; ++g) {
      const int hpb = g * hpl;
      if (hpb - hpl >= nh) break;                        // a lane group with no head at all
      if ((g * L) % 64 != 0 && hpb < nh) continue;       // whole waves, or all of a token's heads
      Cand c;
      c.hpl = hpl;
      c.hpb = hpb;
      const int64_t nhb = (nh + hpb - 1) / hpb;
      c.wpb = ((int64_t)g * L + 63) / 64;
      // lane-head slots of one token's workgroups minus the ones its heads fill
      c.waste = nhb * c.wpb * 64 * hpl - (int64_t)nh * L;
      c.dist = std::llabs((int64_t)g * L - 256);
      c.fits = T * nhb * c.wpb <= kSimds * kRopeWavesPerSimd[hpl];
      cs[n++] = c;
      if (least < 0 || c.waste < least) least = c.waste;
    }
  }
  // the pick: (a) one head per lane if it fits in one round; (b) else the most heads per lane
  // that fits in one round; both among the shapes of least waste, closest to 256 threads;
  // (c) else two heads per lane, least waste among those, then single-wave workgroups
  int best = -1;
  auto take = [&](int k, bool by_wpb) {
    if (best < 0) { best = k; return; }
    const Cand &c = cs[k], &b = cs[best];
    if (c.waste != b.waste) { if (c.waste < b.waste) best = k; return; }
    if (by_wpb && c.wpb != b.wpb) { if (c.wpb < b.wpb) best = k; return; }
    if (c.dist < b.dist) best = k;
  };
  for (int k = 0; k < n; ++k)
    if (cs[k].hpl == 1 && cs[k].waste == least && cs[k].fits) take(k, false);
  if (best < 0) {
    int top = 0;
    for (int k = 0; k < n; ++k)
      if (cs[k].waste == least && cs[k].fits && cs[k].hpl > top) top = cs[k].hpl;
    for (int k = 0; k < n; ++k)
      if (top && cs[k].hpl == top && cs[k].waste == least && cs[k].fits) take(k, false);
  }
  if (best < 0)
    for (int k = 0; k < n; ++k)
      if (cs[k].hpl == 2) take(k, true);
  if (best < 0)  // a single head: one head per lane
    for (int k = 0; k < n; ++k)
      if (cs[k].hpl == 1) take(k, false);
  *hpl_out = cs[best].hpl;
  *hpb_out = cs[best].hpb;
}

int rope_impl(void* qkv, const void* qw, const void* kw, const float* cache, const int64_t* pos,
              float eps, int64_t T, int hq, int hkv, int D, int64_t max_pos, int neox,
              unsigned flags, int heads_per_block, int heads_per_lane, void* start_event,
              void* stop_event, void* stream) {
  int st = validate_rope(qkv, qw, kw, cache, pos, eps, T, hq, hkv, D, max_pos, flags);
  if (st != RMSQ_OK) return st;
  const int nh = hq + hkv;
  int hpl = heads_per_lane, hpb = heads_per_block;
  if (hpl < 0 || hpb < 0 || (hpl == 0) != (hpb == 0)) return RMSQ_EINVAL;
  if (hpl == 0) default_rope_shape(T, nh, D, &hpl, &hpb);
  if (!valid_rope_hpl(hpl) || hpb % hpl != 0 || (int64_t)(hpb / hpl) * (D / 16) > 1024)
    return RMSQ_EINVAL;
  if (T == 0) return RMSQ_OK;
  st = check_device();
  if (st != RMSQ_OK) return st;
  const void* fn = (flags & RMSQ_INPUT_F16) ? rope_kernel_f16(D, neox != 0, hpl)
                                            : rope_kernel_bf16(D, neox != 0, hpl);
  if (!fn) return RMSQ_EINVAL;
  const int64_t nhb = (nh + hpb - 1) / hpb;
  RArgs a;
  a.qkv = static_cast<uint16_t*>(qkv);
  a.qw = static_cast<const uint16_t*>(qw);
  a.kw = static_cast<const uint16_t*>(kw);
  a.cache = cache;
  a.pos = pos;
  a.T = T;
  a.max_pos = max_pos;
  a.eps = eps;
  a.hq = hq;
  a.nh = nh;
  a.width = (hq + 2 * hkv) * D;
  a.hpb = hpb;
  a.groups = hpb / hpl;
  a.nhb = (uint32_t)nhb;
  return launch_kernel(fn, T * nhb, (hpb / hpl) * (D / 16), &a, stream, start_event, stop_event);
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

int rmsq_fused_timed(const void* x, const void* residual, const void* weight, float eps, int mode,
                     const float* scale_in, void* out_q, void* out_scales, void* residual_out,
                     int64_t tokens, int64_t hidden, int group_size, unsigned flags,
                     int64_t scale_ld, const rmsq_launch* launch, void* start_event,
                     void* stop_event, void* stream) {
  return fused_impl(x, residual, weight, eps, mode, scale_in, out_q, out_scales, residual_out,
                    tokens, hidden, group_size, flags, scale_ld, launch, stream, start_event,
                    stop_event);
}

int rmsq_validate(const void* x, const void* residual, const void* weight, float eps, int mode,
                  const float* scale_in, const void* out_q, const void* out_scales,
                  const void* residual_out, int64_t tokens, int64_t hidden, int group_size,
                  unsigned flags, int64_t scale_ld) {
  return validate(x, residual, weight, eps, mode, scale_in, out_q, out_scales, residual_out,
                  tokens, hidden, group_size, flags, scale_ld);
}

int rmsq_fused_fp4_dynamic(const void* x, const void* residual, const void* weight, float eps,
                           void* out_q, void* out_scales, void* residual_out, float* global_scale,
                           int64_t tokens, int64_t hidden, unsigned flags, void* stream) {
  return fp4_dynamic_impl(x, residual, weight, eps, out_q, out_scales, residual_out, global_scale,
                          tokens, hidden, flags, nullptr, nullptr, nullptr, stream);
}

int rmsq_fused_fp4_dynamic_ex(const void* x, const void* residual, const void* weight, float eps,
                              void* out_q, void* out_scales, void* residual_out,
                              float* global_scale, int64_t tokens, int64_t hidden, unsigned flags,
                              const rmsq_launch* launch, void* start_event, void* stop_event,
                              void* stream) {
  return fp4_dynamic_impl(x, residual, weight, eps, out_q, out_scales, residual_out, global_scale,
                          tokens, hidden, flags, launch, start_event, stop_event, stream);
}

int rmsq_fused_fp4_dynamic_validate(const void* x, const void* residual, const void* weight,
                                    float eps, const void* out_q, const void* out_scales,
                                    const void* residual_out, const float* global_scale,
                                    int64_t tokens, int64_t hidden, unsigned flags) {
  return validate_fp4_dynamic(x, residual, weight, eps, out_q, out_scales, residual_out,
                              global_scale, tokens, hidden, flags);
}

int rmsq_rms_norm_pad(const void* x, const void* residual, const void* weight, float eps,
                      void* out, void* residual_out, int64_t tokens, int64_t hidden,
                      int64_t out_ld, unsigned flags, void* stream) {
  return pad_impl(x, residual, weight, eps, out, residual_out, tokens, hidden, out_ld, flags,
                  nullptr, nullptr, nullptr, stream);
}

int rmsq_rms_norm_pad_ex(const void* x, const void* residual, const void* weight, float eps,
                         void* out, void* residual_out, int64_t tokens, int64_t hidden,
                         int64_t out_ld, unsigned flags, const rmsq_launch* launch,
                         void* start_event, void* stop_event, void* stream) {
  return pad_impl(x, residual, weight, eps, out, residual_out, tokens, hidden, out_ld, flags,
                  launch, start_event, stop_event, stream);
}

int rmsq_rms_norm_pad_validate(const void* x, const void* residual, const void* weight, float eps,
                               const void* out, const void* residual_out, int64_t tokens,
                               int64_t hidden, int64_t out_ld, unsigned flags) {
  return validate_pad(x, residual, weight, eps, out, residual_out, tokens, hidden, out_ld,
                      flags);
}

int rmsq_silu_mul_quant(const void* x, int mode, const float* scale_in, void* out_q,
                        void* out_scales, int64_t tokens, int64_t inter, int group_size,
                        unsigned flags, int64_t scale_ld, void* stream) {
  return act_impl(x, mode, scale_in, out_q, out_scales, tokens, inter, group_size, flags,
                  scale_ld, nullptr, nullptr, nullptr, stream);
}

int rmsq_silu_mul_quant_ex(const void* x, int mode, const float* scale_in, void* out_q,
                           void* out_scales, int64_t tokens, int64_t inter, int group_size,
                           unsigned flags, int64_t scale_ld, const rmsq_launch* launch,
                           void* start_event, void* stop_event, void* stream) {
  return act_impl(x, mode, scale_in, out_q, out_scales, tokens, inter, group_size, flags,
                  scale_ld, launch, start_event, stop_event, stream);
}

int rmsq_silu_mul_quant_validate(const void* x, int mode, const float* scale_in,
                                 const void* out_q, const void* out_scales, int64_t tokens,
                                 int64_t inter, int group_size, unsigned flags,
                                 int64_t scale_ld) {
  return validate_act(x, mode, scale_in, out_q, out_scales, tokens, inter, group_size, flags,
                      scale_ld);
}

int rmsq_query_launch(int mode, int64_t tokens, int64_t hidden, int group_size, unsigned flags,
                      rmsq_launch* launch, int64_t* grid) {
  if (!launch) return RMSQ_EINVAL;
  // the activation type; the rest describes the scales, as in rmsq_fused
  const int st = check_quant_scalars(tokens, hidden, mode, group_size,
                                     flags & ~(unsigned)RMSQ_INPUT_F16, 0);
  if (st != RMSQ_OK) return st;
  *launch = default_fused_launch(tokens, hidden, mode == RMSQ_FP8_TOKEN);
  if (grid) *grid = (tokens + launch->rows_per_block - 1) / launch->rows_per_block;
  return RMSQ_OK;
}

int rmsq_rms_norm_pad_query_launch(int64_t tokens, int64_t hidden, int64_t out_ld,
                                   unsigned flags, rmsq_launch* launch, int64_t* grid) {
  if (tokens < 0 || hidden < 8 || (hidden % 8) != 0 || out_ld < hidden ||
      out_ld > RMSQ_MAX_HIDDEN || (out_ld % 8) != 0 || (flags & ~(unsigned)RMSQ_INPUT_F16) != 0)
    return RMSQ_EINVAL;
  const rmsq_launch l = rmsq::default_pad_launch(out_ld, flags);
  if (launch) *launch = l;
  if (grid) *grid = (tokens + l.rows_per_block - 1) / l.rows_per_block;
  return RMSQ_OK;
}

int rmsq_silu_mul_query_launch(int mode, int64_t tokens, int64_t inter, int group_size,
                               rmsq_launch* launch, int64_t* grid) {
  if (!launch) return RMSQ_EINVAL;
  const int st = check_quant_scalars(tokens, inter, mode, group_size, 0, 0);
  if (st != RMSQ_OK) return st;
  *launch = default_act_launch(mode, tokens, inter);
  if (grid) {
    if (launch->options & RMSQ_LAUNCH_ROW_TILES) {
      const int64_t tile = (int64_t)launch->threads_per_row * launch->chunks_per_thread;
      *grid = tokens * ((inter / 8 + tile - 1) / tile);
    } else {
      *grid = (tokens + launch->rows_per_block - 1) / launch->rows_per_block;
    }
  }
  return RMSQ_OK;
}

int rmsq_qk_norm_rope(void* qkv, const void* q_weight, const void* k_weight,
                      const float* cos_sin_cache, const int64_t* positions, float eps,
                      int64_t tokens, int num_q_heads, int num_kv_heads, int head_dim,
                      int64_t max_position, int is_neox, unsigned flags, void* stream) {
  return rope_impl(qkv, q_weight, k_weight, cos_sin_cache, positions, eps, tokens, num_q_heads,
                   num_kv_heads, head_dim, max_position, is_neox, flags, 0, 0, nullptr, nullptr,
                   stream);
}

int rmsq_qk_norm_rope_ex(void* qkv, const void* q_weight, const void* k_weight,
                         const float* cos_sin_cache, const int64_t* positions, float eps,
                         int64_t tokens, int num_q_heads, int num_kv_heads, int head_dim,
                         int64_t max_position, int is_neox, unsigned flags,
                         int heads_per_block, int heads_per_lane, void* start_event,
                         void* stop_event, void* stream) {
  return rope_impl(qkv, q_weight, k_weight, cos_sin_cache, positions, eps, tokens, num_q_heads,
                   num_kv_heads, head_dim, max_position, is_neox, flags, heads_per_block,
                   heads_per_lane, start_event, stop_event, stream);
}

int rmsq_qk_norm_rope_validate(const void* qkv, const void* q_weight, const void* k_weight,
                               const float* cos_sin_cache, const int64_t* positions, float eps,
                               int64_t tokens, int num_q_heads, int num_kv_heads, int head_dim,
                               int64_t max_position, unsigned flags) {
  return validate_rope(qkv, q_weight, k_weight, cos_sin_cache, positions, eps, tokens,
                       num_q_heads, num_kv_heads, head_dim, max_position, flags);
}

int rmsq_qk_norm_rope_query_launch(int64_t tokens, int num_q_heads, int num_kv_heads,
                                   int head_dim, int* heads_per_block, int* heads_per_lane,
                                   int64_t* grid) {
  if (tokens < 0 || num_q_heads < 1 || num_kv_heads < 1) return RMSQ_EINVAL;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return RMSQ_EINVAL;
  const int nh = num_q_heads + num_kv_heads;
  int hpl = 1, hpb = 1;
  rmsq::default_rope_shape(tokens, nh, head_dim, &hpl, &hpb);
  if (heads_per_block) *heads_per_block = hpb;
  if (heads_per_lane) *heads_per_lane = hpl;
  if (grid) *grid = tokens * ((nh + hpb - 1) / hpb);
  return RMSQ_OK;
}

int64_t rmsq_block_to_rowblock(int64_t block, int64_t grid) {
  if (grid <= 0 || grid > 0xFFFFFFFFLL || block < 0 || block >= grid) return -1;
  return (int64_t)rowblock_of((uint32_t)block, (uint32_t)grid);
}

int rmsq_convert(int format, const float* in, void* out, int64_t n, void* stream) {
  if (format != RMSQ_CVT_E4M3 && format != RMSQ_CVT_E2M1 && format != RMSQ_CVT_BF16 &&
      format != RMSQ_CVT_INV_SQRT && format != RMSQ_CVT_E4M3_IN_RANGE)
    return RMSQ_EINVAL;
  if (n < 0 || (n % 8) != 0) return RMSQ_EINVAL;
  if (n == 0) return RMSQ_OK;
  if (!in || !out) return RMSQ_EINVAL;
  if (!aligned(in, 16) || !aligned(out, 16)) return RMSQ_EALIGN;
  const size_t ob = (format == RMSQ_CVT_E4M3 || format == RMSQ_CVT_E4M3_IN_RANGE) ? (size_t)n
                    : format == RMSQ_CVT_E2M1 ? (size_t)n / 2
                    : format == RMSQ_CVT_BF16 ? (size_t)n * 2
                                              : (size_t)n * 4;
  if (overlap(span(in, (size_t)n * 4), span(out, ob))) return RMSQ_EALIAS;
  const int st = check_device();
  if (st != RMSQ_OK) return st;
  const int64_t nch = n / 8;
  const int64_t blocks = (nch + 255) / 256;
  if (blocks > 0x7FFFFFFFLL) return RMSQ_EINVAL;
  int fmt = format;
  void* args[] = {&fmt, &in, &out, const_cast<int64_t*>(&nch)};
  const hipError_t e = hipLaunchKernel(convert_kernel_ptr(),
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
