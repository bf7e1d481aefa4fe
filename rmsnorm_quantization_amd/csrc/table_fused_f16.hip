// table_fused_f16.hip -- instantiations of fused_kernel for IEEE binary16 activations, and the
// padded-output mode for them.
#include "rmsq_kernel_table.hpp"

namespace rmsq {
namespace {

template <int MODE, bool RES, int GS, bool EXACT, int DT = 0>
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


}  // namespace

const void* fused_kernel_f16(int mode, bool res, int gs, int vpt, bool exact) {
  return pick_kernel_dt<1>(mode, res, gs, vpt, exact);
}

const void* pad_kernel_f16(bool res, int vpt) {
  return res ? pick_vpt<kModePad, true, 0, false, 1>(vpt)
             : pick_vpt<kModePad, false, 0, false, 1>(vpt);
}

const void* amax_kernel_f16(bool res, int vpt, bool exact) {
  if (res)
    return exact ? pick_vpt<kModeRowAmax, true, 0, true, 1>(vpt)
                 : pick_vpt<kModeRowAmax, true, 0, false, 1>(vpt);
  return exact ? pick_vpt<kModeRowAmax, false, 0, true, 1>(vpt)
               : pick_vpt<kModeRowAmax, false, 0, false, 1>(vpt);
}

}  // namespace rmsq
