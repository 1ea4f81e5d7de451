// Gated DeltaNet decode kernels for gfx950 (placeholder shape table; kernels
// follow in this file).
#include "rs_device.h"
#include "rs_tile.h"
#include "rs_internal.h"

namespace rs {

bool gdn_shape_supported(int, int) { return false; }

void gdn_launch(GDNOp, const GDNArgs&, const GDNLaunch&, hipStream_t) {}

}  // namespace rs
