// rmsq_kernel_table.hpp -- the kernel instantiations librmsq launches, one lookup per family.
// Each returns the host-side handle of the kernel to pass to hipLaunchKernel, or nullptr for a
// combination that does not exist.  Defined in the table_*.hip units, so that the many template
// instantiations compile in parallel.
#pragma once

#include "rmsq_kernels.hpp"

namespace rmsq {

// fused (residual add ->) RMSNorm -> quantization, bf16 or IEEE binary16 activations
const void* fused_kernel_bf16(int mode, bool res, int gs, int vpt, bool exact);
const void* fused_kernel_f16(int mode, bool res, int gs, int vpt, bool exact);
// (residual add ->) RMSNorm -> each workgroup's largest |y| (first pass of FP4 with a batch
// scale)
const void* amax_kernel_bf16(bool res, int vpt, bool exact);
const void* amax_kernel_f16(bool res, int vpt, bool exact);
// the block pass of FP4 with a batch scale (no residual: it reads the new residual or x)
const void* batch_fp4_kernel_bf16(int vpt, bool exact);
const void* batch_fp4_kernel_f16(int vpt, bool exact);
// (residual add ->) RMSNorm -> padded 16-bit output (launches always masked)
const void* pad_kernel_bf16(bool res, int vpt);
const void* pad_kernel_f16(bool res, int vpt);
// SiLU+Mul -> quantization, whole rows or row tiles
const void* act_kernel_bf16(bool tiled, bool exact, int mode, int gs, int vpt);
const void* act_kernel_f16(bool tiled, bool exact, int mode, int gs, int vpt);
// QK-norm + RoPE
const void* rope_kernel_bf16(int D, bool neox, int hpl);
const void* rope_kernel_f16(int D, bool neox, int hpl);
// the diagnostic converters
const void* convert_kernel_ptr();
// the one-workgroup reduction of the row pass's maxima to the FP4 global scale
const void* fp4_global_scale_kernel_ptr();

// The fused_kernel instantiation for (mode, residual, chunks per thread, group, exact, type);
// each table unit instantiates the pickers for one 16-bit type.
template <int MODE, bool RES, int GS, bool EXACT, int DT>
const void* pick_vpt(int vpt) {
  switch (vpt) {
    case 1: return reinterpret_cast<const void*>(&fused_kernel<MODE, RES, 1, GS, EXACT, DT>);
    case 2: return reinterpret_cast<const void*>(&fused_kernel<MODE, RES, 2, GS, EXACT, DT>);
    case 3: return reinterpret_cast<const void*>(&fused_kernel<MODE, RES, 3, GS, EXACT, DT>);
    case 4: return reinterpret_cast<const void*>(&fused_kernel<MODE, RES, 4, GS, EXACT, DT>);
    case 5: return reinterpret_cast<const void*>(&fused_kernel<MODE, RES, 5, GS, EXACT, DT>);
    case 6: return reinterpret_cast<const void*>(&fused_kernel<MODE, RES, 6, GS, EXACT, DT>);
    case 7: return reinterpret_cast<const void*>(&fused_kernel<MODE, RES, 7, GS, EXACT, DT>);
    case 8: return reinterpret_cast<const void*>(&fused_kernel<MODE, RES, 8, GS, EXACT, DT>);
    default: return nullptr;
  }
}

template <bool RES, bool EXACT, int DT>
const void* pick_mode(int mode, int gs, int vpt) {
  switch (mode) {
    case RMSQ_FP8_STATIC: return pick_vpt<RMSQ_FP8_STATIC, RES, 0, EXACT, DT>(vpt);
    case RMSQ_FP8_TOKEN: return pick_vpt<RMSQ_FP8_TOKEN, RES, 0, EXACT, DT>(vpt);
    case RMSQ_FP8_GROUP:
      return gs == 64 ? pick_vpt<RMSQ_FP8_GROUP, RES, 64, EXACT, DT>(vpt)
                      : pick_vpt<RMSQ_FP8_GROUP, RES, 128, EXACT, DT>(vpt);
    case RMSQ_FP4_BLOCK16: return pick_vpt<RMSQ_FP4_BLOCK16, RES, 16, EXACT, DT>(vpt);
    default: return nullptr;
  }
}

template <int DT>
const void* pick_kernel_dt(int mode, bool res, int gs, int vpt, bool exact) {
  if (res)
    return exact ? pick_mode<true, true, DT>(mode, gs, vpt)
                 : pick_mode<true, false, DT>(mode, gs, vpt);
  return exact ? pick_mode<false, true, DT>(mode, gs, vpt)
               : pick_mode<false, false, DT>(mode, gs, vpt);
}

// The QK-norm + RoPE instantiation for (D, NEOX, heads per lane), one 16-bit type per table unit.
template <int DT, int D, bool NEOX>
const void* pick_rope_hpl(int hpl) {
  switch (hpl) {
    case 1: return reinterpret_cast<const void*>(&qk_norm_rope_kernel<D, NEOX, 1, DT>);
    case 2: return reinterpret_cast<const void*>(&qk_norm_rope_kernel<D, NEOX, 2, DT>);
    case 3: return reinterpret_cast<const void*>(&qk_norm_rope_kernel<D, NEOX, 3, DT>);
    case 4: return reinterpret_cast<const void*>(&qk_norm_rope_kernel<D, NEOX, 4, DT>);
    case 5: return reinterpret_cast<const void*>(&qk_norm_rope_kernel<D, NEOX, 5, DT>);
    case 6: return reinterpret_cast<const void*>(&qk_norm_rope_kernel<D, NEOX, 6, DT>);
    default: return nullptr;
  }
}

template <int DT>
const void* pick_rope(int D, bool neox, int hpl) {
  switch (D) {
    case 64: return neox ? pick_rope_hpl<DT, 64, true>(hpl) : pick_rope_hpl<DT, 64, false>(hpl);
    case 128:
      return neox ? pick_rope_hpl<DT, 128, true>(hpl) : pick_rope_hpl<DT, 128, false>(hpl);
    case 256:
      return neox ? pick_rope_hpl<DT, 256, true>(hpl) : pick_rope_hpl<DT, 256, false>(hpl);
    default: return nullptr;
  }
}

}  // namespace rmsq
