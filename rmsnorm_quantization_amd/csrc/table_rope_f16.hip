// table_rope_f16.hip -- instantiations of the QK-norm + RoPE kernels for IEEE binary16.
#include "rmsq_kernel_table.hpp"

namespace rmsq {

const void* rope_kernel_f16(int D, bool neox, int hpl) { return pick_rope<1>(D, neox, hpl); }

}  // namespace rmsq
