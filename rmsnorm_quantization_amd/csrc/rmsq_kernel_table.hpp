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
// (residual add ->) RMSNorm -> padded bf16 output (launches always masked)
const void* pad_kernel(bool res, int vpt);
// SiLU+Mul -> quantization, whole rows or row tiles
const void* act_kernel_bf16(bool tiled, bool exact, int mode, int gs, int vpt);
const void* act_kernel_f16(bool tiled, bool exact, int mode, int gs, int vpt);
// QK-norm + RoPE
const void* rope_kernel(int D, bool neox, int hpl);
// the diagnostic converters
const void* convert_kernel_ptr();

}  // namespace rmsq
