// table_misc.hip -- instantiations of the QK-norm + RoPE kernels for bf16, and the converter
// kernel.
#include "rmsq_kernel_table.hpp"

namespace rmsq {

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

const void* rope_kernel_bf16(int D, bool neox, int hpl) { return pick_rope<0>(D, neox, hpl); }

const void* convert_kernel_ptr() { return reinterpret_cast<const void*>(&convert_kernel); }

}  // namespace rmsq
