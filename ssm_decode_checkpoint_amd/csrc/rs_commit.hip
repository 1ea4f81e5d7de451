// Speculative commit, counter part, for every layer kind (sitech.ge ReplaySSM
// page, "Reducing state traffic and simplifying rollback": the accepted prefix
// of the drafts is committed by moving the buffer pointer, no snapshot is
// saved or restored). Per sequence: len += accepted, nd = 0; a commit that
// leaves less room than the largest draft count folds the committed entries
// (n_ckpt += len, len = 0), and those sequences are listed, in ascending order,
// for the layer's fold kernel.
#include "rs_internal.h"

namespace rs {

// One workgroup of 1024 threads walks the batch in chunks; the list position
// of each folding sequence is an inclusive scan of the fold flags.
__global__ __launch_bounds__(1024) void commit_meta_kernel(CommitArgs a) {
  __shared__ int wsum[16];
  __shared__ int base;
  if (threadIdx.x == 0) base = 0;
  __syncthreads();
  for (int b0 = 0; b0 < a.batch; b0 += 1024) {
    const int b = b0 + threadIdx.x;
    int fold = 0, m = 0;
    long long nck = 0;
    if (b < a.batch) {
      rs_meta* mp = a.meta + b;
      const int k = a.accepted[b];
      const int nd = mp->nd;
      if (k < 0 || k > nd) {
        mp->err |= RS_ERR_COMMIT;
      } else {
        const int len = mp->len + k;
        mp->nd = 0;
        nck = mp->n_ckpt;
        if (len > kRing - a.kmax) {
          fold = 1;
          m = len;
          mp->n_ckpt = nck + len;
          mp->len = 0;
        } else {
          mp->len = len;
        }
      }
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = fold;
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int before = base;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    if (fold) {
      FoldItem it;
      it.b = b;
      it.m = m;
      it.nck = nck;
      a.work[before + incl - 1] = it;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int tot = 0;
      for (int w = 0; w < 16; ++w) tot += wsum[w];
      base += tot;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) *a.work_count = base;
}

void commit_meta(const CommitArgs& a, hipStream_t st) { commit_meta_kernel<<<1, 1024, 0, st>>>(a); }

// Slot reuse: a sequence slot that starts a new sequence gets empty counters
// (its buffer is empty; the caller writes the new checkpoint). The arrival
// counts are zero between calls and stay untouched.
__global__ __launch_bounds__(256) void reset_slots_kernel(rs_meta* meta, int batch, const int32_t* seqs, int count) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  const int b = seqs[i];
  if (b < 0 || b >= batch) return;
  rs_meta* m = meta + b;
  m->n_ckpt = 0;
  m->len = 0;
  m->nd = 0;
  m->err = 0;
}

void reset_slots(rs_meta* meta, int batch, const int32_t* seqs, int count, hipStream_t st) {
  reset_slots_kernel<<<(count + 255) / 256, 256, 0, st>>>(meta, batch, seqs, count);
}

}  // namespace rs
