// Mamba-2 shape dispatch: each compiled (dstate, headdim) pair has its kernels
// instantiated in its own translation unit (rs_m2_<rows>x<cols>.hip).
#include "rs_internal.h"

namespace rs {

template <int NR, int NC>
void m2_launch_shape(M2Op op, const M2Args& a, const M2Launch& l, hipStream_t st);

extern template void m2_launch_shape<16, 16>(M2Op, const M2Args&, const M2Launch&, hipStream_t);
extern template void m2_launch_shape<64, 64>(M2Op, const M2Args&, const M2Launch&, hipStream_t);
extern template void m2_launch_shape<128, 64>(M2Op, const M2Args&, const M2Launch&, hipStream_t);
extern template void m2_launch_shape<128, 128>(M2Op, const M2Args&, const M2Launch&, hipStream_t);

// The compiled shapes are the ones m2_shape_supported (rs_host.cpp) accepts.
void m2_launch(M2Op op, const M2Args& a, const M2Launch& l, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (l.rows == 16 && l.cols == 16) m2_launch_shape<16, 16>(op, a, l, st);
  else if (l.rows == 64 && l.cols == 64) m2_launch_shape<64, 64>(op, a, l, st);
  else if (l.rows == 128 && l.cols == 64) m2_launch_shape<128, 64>(op, a, l, st);
  else if (l.rows == 128 && l.cols == 128) m2_launch_shape<128, 128>(op, a, l, st);
}

}  // namespace rs
