// Mamba-2 kernels instantiated for dstate = 16, headdim = 16.
#include "rs_mamba2_kernels.h"

namespace rs {
template void m2_launch_shape<16, 16>(M2Op, const M2Args&, const M2Launch&, hipStream_t);
}  // namespace rs
