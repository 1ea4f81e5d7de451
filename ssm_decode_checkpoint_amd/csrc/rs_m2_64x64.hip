// Mamba-2 kernels instantiated for dstate = 64, headdim = 64.
#include "rs_mamba2_kernels.h"

namespace rs {
template void m2_launch_shape<64, 64>(M2Op, const M2Args&, const M2Launch&, hipStream_t);
}  // namespace rs
