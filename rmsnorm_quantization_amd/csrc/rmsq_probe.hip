// rmsq_probe.hip -- the memory-only reference kernel declared in include/rmsq_probe.h.  It
// mirrors the fused kernel's row and chunk mapping (one workgroup per row, chunk c on thread
// c mod threads_per_row, 16-byte non-temporal loads and stores) so that the two differ only in
// the arithmetic.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "rmsq_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct ProbeArgs {
  const u32x4* in0;
  const u32x4* in1;
  u32x4* out0;
  uint8_t* out1;
  uint8_t* out2;
  int64_t nch;  // 16-byte chunks per row
  int32_t tpr;
  int32_t out2_shift;  // an out2 element per 2^shift chunks; -1: one per row
};

// Row base pointers are uniform over the workgroup (scalar registers) and each lane adds a 32-bit
// byte offset, the addressing form of the fused kernel.
template <class T>
__device__ __forceinline__ T* boff(T* p, uint32_t bytes) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(p) + bytes);
}
template <class T>
__device__ __forceinline__ const T* boff(const T* p, uint32_t bytes) {
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(p) + bytes);
}

// One row; IN1 / OUT0: whether the second input and the first output are present (uniform
// over the launch, so each combination is its own straight-line body).
template <int VPT, int OUT1, int OUT2, bool IN1, bool OUT0>
__device__ __forceinline__ void probe_row(const ProbeArgs& a) {
  const size_t base = (size_t)blockIdx.x * (size_t)a.nch;  // the row's first chunk
  const uint32_t lr = threadIdx.x;
  u32x4 v[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const uint32_t c = lr + (uint32_t)(k * a.tpr);
    v[k] = __builtin_nontemporal_load(boff(a.in0 + base, c << 4));
    if constexpr (IN1) v[k] ^= __builtin_nontemporal_load(boff(a.in1 + base, c << 4));
  }
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const uint32_t c = lr + (uint32_t)(k * a.tpr);
    if constexpr (OUT0) __builtin_nontemporal_store(v[k], boff(a.out0 + base, c << 4));
    if constexpr (OUT1 == 8) {
      __builtin_nontemporal_store((u32x2){v[k][0] ^ v[k][2], v[k][1] ^ v[k][3]},
                                  boff(reinterpret_cast<u32x2*>(a.out1) + base, c << 3));
    } else if constexpr (OUT1 == 4) {
      __builtin_nontemporal_store(v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3],
                                  boff(reinterpret_cast<uint32_t*>(a.out1) + base, c << 2));
    }
    if constexpr (OUT2 != 0) {  // scale-like stream: the lane that starts each element's chunks
      const bool per_row = a.out2_shift < 0;
      const uint32_t sh = per_row ? 0u : (uint32_t)a.out2_shift;
      if (per_row ? c == 0 : (c & ((1u << sh) - 1u)) == 0) {
        const size_t idx = per_row ? (size_t)blockIdx.x
                                   : (size_t)blockIdx.x * (size_t)(a.nch >> sh) + (c >> sh);
        const uint32_t val = v[k][0] ^ v[k][3];
        if constexpr (OUT2 == 4) reinterpret_cast<uint32_t*>(a.out2)[idx] = val;
        else a.out2[idx] = (uint8_t)val;
      }
    }
  }
}

template <int VPT, int OUT1, int OUT2>
__global__ void __launch_bounds__(1024) stream_probe_kernel(ProbeArgs a) {
  if (a.in1) {
    if (a.out0) probe_row<VPT, OUT1, OUT2, true, true>(a);
    else probe_row<VPT, OUT1, OUT2, true, false>(a);
  } else {
    if (a.out0) probe_row<VPT, OUT1, OUT2, false, true>(a);
    else probe_row<VPT, OUT1, OUT2, false, false>(a);
  }
}

template <int OUT1, int OUT2>
const void* pick(int vpt) {
  switch (vpt) {
    case 1: return reinterpret_cast<const void*>(&stream_probe_kernel<1, OUT1, OUT2>);
    case 2: return reinterpret_cast<const void*>(&stream_probe_kernel<2, OUT1, OUT2>);
    case 3: return reinterpret_cast<const void*>(&stream_probe_kernel<3, OUT1, OUT2>);
    case 4: return reinterpret_cast<const void*>(&stream_probe_kernel<4, OUT1, OUT2>);
    case 5: return reinterpret_cast<const void*>(&stream_probe_kernel<5, OUT1, OUT2>);
    case 6: return reinterpret_cast<const void*>(&stream_probe_kernel<6, OUT1, OUT2>);
    case 7: return reinterpret_cast<const void*>(&stream_probe_kernel<7, OUT1, OUT2>);
    case 8: return reinterpret_cast<const void*>(&stream_probe_kernel<8, OUT1, OUT2>);
    default: return nullptr;
  }
}

template <int OUT2>
const void* pick_out1(int ob, int vpt) {
  return ob == 8 ? pick<8, OUT2>(vpt) : ob == 4 ? pick<4, OUT2>(vpt) : pick<0, OUT2>(vpt);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" int rmsq_probe_stream(const void* in0, const void* in1, void* out0, void* out1,
                                 void* out2, int64_t rows, int64_t hidden,
                                 int out1_bytes_per_chunk, int out2_shift, int out2_bytes,
                                 int threads_per_row, int chunks_per_thread, void* start_event,
                                 void* stop_event, void* stream) {
  if (rows < 0 || rows > 0x7FFFFFFFLL || hidden < 8 || hidden % 8 != 0) return -1;
  if (threads_per_row < 64 || threads_per_row > 1024 || threads_per_row % 64 != 0) return -1;
  if (chunks_per_thread < 1 || chunks_per_thread > 8) return -1;
  if ((int64_t)threads_per_row * chunks_per_thread * 8 != hidden) return -1;
  if (out1_bytes_per_chunk != 0 && out1_bytes_per_chunk != 4 && out1_bytes_per_chunk != 8)
    return -1;
  if (out2) {
    if (out2_bytes != 1 && out2_bytes != 4) return -1;
    if (out2_shift < -1 || out2_shift > 6) return -1;
    if (out2_shift >= 0 && ((hidden / 8) & ((int64_t(1) << out2_shift) - 1)) != 0) return -1;
    if (out2_bytes == 4 && (reinterpret_cast<uintptr_t>(out2) & 3) != 0) return -2;
  }
  if (rows == 0) return 0;
  if (!in0) return -1;
  if (!aligned16(in0) || !aligned16(in1) || !aligned16(out0) || !aligned16(out1)) return -2;
  const int ob = out1 ? out1_bytes_per_chunk : 0;  // no out1 buffer: nothing written there
  const int o2 = out2 ? out2_bytes : 0;
  const void* fn = o2 == 4   ? pick_out1<4>(ob, chunks_per_thread)
                   : o2 == 1 ? pick_out1<1>(ob, chunks_per_thread)
                             : pick_out1<0>(ob, chunks_per_thread);
  ProbeArgs a;
  a.in0 = static_cast<const u32x4*>(in0);
  a.in1 = static_cast<const u32x4*>(in1);
  a.out0 = static_cast<u32x4*>(out0);
  a.out1 = ob ? static_cast<uint8_t*>(out1) : nullptr;
  a.out2 = static_cast<uint8_t*>(out2);
  a.nch = hidden / 8;
  a.tpr = threads_per_row;
  a.out2_shift = out2_shift;
  void* args[] = {&a};
  const hipError_t e = hipExtLaunchKernel(
      fn, dim3((uint32_t)rows), dim3((uint32_t)threads_per_row), args, 0,
      static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(start_event),
      static_cast<hipEvent_t>(stop_event), 0);
  return e == hipSuccess ? 0 : -5;
}
