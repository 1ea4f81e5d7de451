// Buffer-counter advance after a step kernel. The step kernels only read the
// per-sequence counters (every workgroup of a sequence must see the values
// from before the step); this follow-up launch, one thread per sequence,
// applies the step's rule to them (sitech.ge ReplaySSM page, "How ReplaySSM
// works": append on a non-flush step; fold and clear on a flush; "Reducing
// state traffic and simplifying rollback": drafts held until verification).
// A sequence that broke the call's contract gets a sticky error bit and keeps
// its counters, exactly as the step kernel skipped it.
#include "rs_internal.h"

namespace rs {

__global__ __launch_bounds__(256) void meta_advance_kernel(rs_meta* meta, int batch, int op, int K) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  rs_meta* m = meta + b;
  const int len = m->len, nd = m->nd;
  switch (op) {
    case static_cast<int>(MetaOp::NonFlush):
      if (nd != 0) m->err |= RS_ERR_PENDING;
      else if (len > kRing - 2) m->err |= RS_ERR_FULL;
      else m->len = len + 1;
      break;
    case static_cast<int>(MetaOp::Flush):
      if (nd != 0) m->err |= RS_ERR_PENDING;
      else if (len > kRing - 1) m->err |= RS_ERR_FULL;
      else {
        m->n_ckpt = m->n_ckpt + len + 1;
        m->len = 0;
      }
      break;
    default:  // Append
      if (nd != 0 || len + K > kRing) m->err |= RS_ERR_OVERFLOW;
      else m->nd = K;
      break;
  }
}

void meta_advance(rs_meta* meta, int batch, MetaOp op, int K, hipStream_t st) {
  meta_advance_kernel<<<(batch + 255) / 256, 256, 0, st>>>(meta, batch, static_cast<int>(op), K);
}

}  // namespace rs
