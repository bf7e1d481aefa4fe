// table_misc.hip -- instantiations of the QK-norm + RoPE kernels for bf16, the converter kernel
// and the FP4 global-scale reduction.
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
  } else if (fmt == RMSQ_CVT_E4M3_IN_RANGE) {
    reinterpret_cast<u32x2*>(out)[c] = (u32x2){fp8x4_in_range(v[0], v[1], v[2], v[3]),
                                               fp8x4_in_range(v[4], v[5], v[6], v[7])};
  } else if (fmt == RMSQ_CVT_E2M1) {
    reinterpret_cast<uint32_t*>(out)[c] = fp4x8(v);
  } else if (fmt == RMSQ_CVT_INV_SQRT) {
    float r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = inv_sqrt_f32((double)v[e]);
    reinterpret_cast<f32x4*>(out)[2 * c] = (f32x4){r[0], r[1], r[2], r[3]};
    reinterpret_cast<f32x4*>(out)[2 * c + 1] = (f32x4){r[4], r[5], r[6], r[7]};
  } else {
    reinterpret_cast<u32x4*>(out)[c] = (u32x4){pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                               pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
  }
}

const void* rope_kernel_bf16(int D, bool neox, int hpl) { return pick_rope<0>(D, neox, hpl); }

const void* convert_kernel_ptr() { return reinterpret_cast<const void*>(&convert_kernel); }

// One workgroup of 1024 threads: the largest of the row pass's T maxima, then the batch's FP4
// global scale.  Each thread takes every 1024th maximum, eight loads in flight per round (masked
// past T).  The launch costs ~3.5 us however the loads are arranged (mostly its own dispatch),
// which is why the block pass takes this reduction over wherever one round of loads suffices.
__global__ void __launch_bounds__(1024) fp4_global_scale_kernel(GArgs a) {
  __shared__ float s_mx[kMaxWavesPerBlock];
  constexpr int kLoads = 8;
  const int64_t stride = blockDim.x;
  float m = 0.0f;
  for (int64_t base = threadIdx.x; base < a.T; base += kLoads * stride) {
    float v[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int64_t i = base + u * stride;
      v[u] = (i < a.T) ? a.row_amax[i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kLoads; ++u) m = fmaxf(m, v[u]);
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) s_mx[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float amax = 0.0f;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) amax = fmaxf(amax, s_mx[i]);
    a.gs[0] = batch_fp4_scale(amax);
  }
}

const void* fp4_global_scale_kernel_ptr() {
  return reinterpret_cast<const void*>(&fp4_global_scale_kernel);
}

}  // namespace rmsq
