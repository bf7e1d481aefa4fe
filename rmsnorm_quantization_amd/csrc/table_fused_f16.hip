// table_fused_f16.hip -- instantiations of fused_kernel for IEEE binary16 activations: the
// quantizing modes, the padded-output mode, the row-absmax mode and the batch-scale FP4 block
// pass.
#include "rmsq_kernel_table.hpp"

namespace rmsq {

const void* fused_kernel_f16(int mode, bool res, int gs, int vpt, bool exact) {
  return pick_kernel_dt<1>(mode, res, gs, vpt, exact);
}

const void* pad_kernel_f16(bool res, int vpt) {
  return res ? pick_vpt<kModePad, true, 0, false, 1>(vpt)
             : pick_vpt<kModePad, false, 0, false, 1>(vpt);
}

const void* batch_fp4_kernel_f16(int vpt, bool exact) {
  return exact ? pick_vpt<kModeFp4Batch, false, 16, true, 1>(vpt)
               : pick_vpt<kModeFp4Batch, false, 16, false, 1>(vpt);
}

const void* amax_kernel_f16(bool res, int vpt, bool exact) {
  if (res)
    return exact ? pick_vpt<kModeRowAmax, true, 0, true, 1>(vpt)
                 : pick_vpt<kModeRowAmax, true, 0, false, 1>(vpt);
  return exact ? pick_vpt<kModeRowAmax, false, 0, true, 1>(vpt)
               : pick_vpt<kModeRowAmax, false, 0, false, 1>(vpt);
}

}  // namespace rmsq
