// Mamba-2 kernels instantiated for dstate = 128, headdim = 128.
#include "rs_mamba2_kernels.h"

namespace rs {
template void m2_launch_shape<128, 128>(M2Op, const M2Args&, const M2Launch&, hipStream_t);
}  // namespace rs
