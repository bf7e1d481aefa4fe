// table_act.hip -- instantiations of the SiLU+Mul -> quantization kernels.
#include "rmsq_kernel_table.hpp"

namespace rmsq {
namespace {

template <int MODE, int GS, bool EXACT, int DT>
const void* pick_act_vpt(int vpt) {
  switch (vpt) {
    case 1: return reinterpret_cast<const void*>(&silu_mul_kernel<MODE, 1, GS, EXACT, DT>);
    case 2: return reinterpret_cast<const void*>(&silu_mul_kernel<MODE, 2, GS, EXACT, DT>);
    case 3: return reinterpret_cast<const void*>(&silu_mul_kernel<MODE, 3, GS, EXACT, DT>);
    case 4: return reinterpret_cast<const void*>(&silu_mul_kernel<MODE, 4, GS, EXACT, DT>);
    case 5: return reinterpret_cast<const void*>(&silu_mul_kernel<MODE, 5, GS, EXACT, DT>);
    case 6: return reinterpret_cast<const void*>(&silu_mul_kernel<MODE, 6, GS, EXACT, DT>);
    case 7: return reinterpret_cast<const void*>(&silu_mul_kernel<MODE, 7, GS, EXACT, DT>);
    case 8: return reinterpret_cast<const void*>(&silu_mul_kernel<MODE, 8, GS, EXACT, DT>);
    default: return nullptr;
  }
}

template <int MODE, int GS, bool EXACT, int DT>
const void* pick_tile_vpt(int vpt) {
  switch (vpt) {
    case 1: return reinterpret_cast<const void*>(&silu_mul_tile_kernel<MODE, 1, GS, EXACT, DT>);
    case 2: return reinterpret_cast<const void*>(&silu_mul_tile_kernel<MODE, 2, GS, EXACT, DT>);
    case 4: return reinterpret_cast<const void*>(&silu_mul_tile_kernel<MODE, 4, GS, EXACT, DT>);
    default: return nullptr;
  }
}

template <bool EXACT, int DT>
const void* pick_tile_mode(int mode, int gs, int vpt) {
  switch (mode) {
    case RMSQ_FP8_STATIC: return pick_tile_vpt<RMSQ_FP8_STATIC, 0, EXACT, DT>(vpt);
    case RMSQ_FP8_GROUP:
      return gs == 64 ? pick_tile_vpt<RMSQ_FP8_GROUP, 64, EXACT, DT>(vpt)
                      : pick_tile_vpt<RMSQ_FP8_GROUP, 128, EXACT, DT>(vpt);
    case RMSQ_FP4_BLOCK16: return pick_tile_vpt<RMSQ_FP4_BLOCK16, 16, EXACT, DT>(vpt);
    default: return nullptr;
  }
}

template <bool EXACT, int DT>
const void* pick_act_mode(int mode, int gs, int vpt) {
  switch (mode) {
    case RMSQ_FP8_STATIC: return pick_act_vpt<RMSQ_FP8_STATIC, 0, EXACT, DT>(vpt);
    case RMSQ_FP8_TOKEN: return pick_act_vpt<RMSQ_FP8_TOKEN, 0, EXACT, DT>(vpt);
    case RMSQ_FP8_GROUP:
      return gs == 64 ? pick_act_vpt<RMSQ_FP8_GROUP, 64, EXACT, DT>(vpt)
                      : pick_act_vpt<RMSQ_FP8_GROUP, 128, EXACT, DT>(vpt);
    case RMSQ_FP4_BLOCK16: return pick_act_vpt<RMSQ_FP4_BLOCK16, 16, EXACT, DT>(vpt);
    default: return nullptr;
  }
}


}  // namespace

template <int DT>
const void* act_kernel_dt(bool tiled, bool exact, int mode, int gs, int vpt) {
  if (tiled)
    return exact ? pick_tile_mode<true, DT>(mode, gs, vpt)
                 : pick_tile_mode<false, DT>(mode, gs, vpt);
  return exact ? pick_act_mode<true, DT>(mode, gs, vpt) : pick_act_mode<false, DT>(mode, gs, vpt);
}

const void* act_kernel_bf16(bool tiled, bool exact, int mode, int gs, int vpt) {
  return act_kernel_dt<0>(tiled, exact, mode, gs, vpt);
}

const void* act_kernel_f16(bool tiled, bool exact, int mode, int gs, int vpt) {
  return act_kernel_dt<1>(tiled, exact, mode, gs, vpt);
}

}  // namespace rmsq
