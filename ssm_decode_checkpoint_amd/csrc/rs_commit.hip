// Per-sequence operations shared by every layer kind: the speculative commit's
// counter part, slot reuse and slot copies (prefix caching, forks).
//
// Speculative commit, counter part (sitech.ge ReplaySSM
// page, "Reducing state traffic and simplifying rollback": the accepted prefix
// of the drafts is committed by moving the buffer pointer, no snapshot is
// saved or restored). Per sequence: len += accepted, nd = 0; a commit that
// leaves less room than the largest draft count folds the committed entries
// (n_ckpt += len, len = 0), and those sequences are listed, in ascending order,
// for the layer's fold kernel.
#include <atomic>

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

void commit_meta(const CommitArgs& a, void* stream) {
  commit_meta_kernel<<<1, 1024, 0, static_cast<hipStream_t>(stream)>>>(a);
}

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

void reset_slots(rs_meta* meta, int batch, const int32_t* seqs, int count, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  reset_slots_kernel<<<(count + 255) / 256, 256, 0, st>>>(meta, batch, seqs, count);
}

// Prefix caching and forks: the state of a sequence at any token is its
// checkpoint, its buffer entries and its counters (sitech.ge ReplaySSM page,
// "Reducing state traffic and simplifying rollback": no per-token snapshot is
// kept), so saving or restoring it is a plain copy of those regions. One
// row of the grid per listed pair, blockIdx.x strides over the bytes.
__global__ __launch_bounds__(256) void copy_slots_kernel(CopyArgs a) {
  const int i = blockIdx.y;
  const int s = a.src_seqs[i], d = a.dst_seqs[i];
  if (s < 0 || s >= a.src_batch || d < 0 || d >= a.dst_batch) return;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  for (int r = 0; r < a.nreg; ++r) {
    const CopyRegion g = a.r[r];
    const char* src = g.src + static_cast<uint64_t>(s) * g.per;
    char* dst = g.dst + static_cast<uint64_t>(d) * g.per;
    if (g.per % 16 == 0) {
      const uint64_t n = g.per / 16;
      for (uint64_t k = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; k < n; k += stride)
        nt_store(nt_load(reinterpret_cast<const uint4*>(src) + k), reinterpret_cast<uint4*>(dst) + k);
    } else {
      const uint64_t n = g.per / 4;
      for (uint64_t k = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; k < n; k += stride)
        reinterpret_cast<uint32_t*>(dst)[k] = reinterpret_cast<const uint32_t*>(src)[k];
    }
  }
  if (a.dst_meta && blockIdx.x == 0 && threadIdx.x == 0) {
    const rs_meta* m = a.src_meta + s;
    rs_meta* o = a.dst_meta + d;
    o->n_ckpt = m->n_ckpt;
    o->len = m->len;
    o->nd = m->nd;
    o->err = m->err;
  }
}

void copy_slots(const CopyArgs& a, int blocks_per_pair, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  copy_slots_kernel<<<dim3(blocks_per_pair, a.count), 256, 0, st>>>(a);
}

rs_status launch_status() { return hipGetLastError() == hipSuccess ? RS_OK : RS_E_LAUNCH; }

// Fold list of rs_spec_commit_static: FoldItem[kStaticFoldSeqs] (128 KiB), then
// the count. Each device holds its own copy for the life of the process. In
// host code `scratch` names a host-side stand-in, so its device address is
// taken with hipGetSymbolAddress once per device (with that device current)
// and only that address is handed to kernels. commit_meta_kernel writes the
// count and the listed items on every call before the fold kernel reads them,
// so nothing needs clearing between calls; calls that overlap on one device
// share the array and race.
constexpr size_t kStaticListBytes = static_cast<size_t>(kStaticFoldSeqs) * sizeof(FoldItem);
static __device__ __align__(256) unsigned char scratch[kStaticListBytes + 256];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
}  // namespace

rs_status static_fold_list(FoldItem** list, int** count) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RS_E_LAUNCH;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return RS_E_LAUNCH;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *list = static_cast<FoldItem*>(p);
  *count = reinterpret_cast<int*>(static_cast<char*>(p) + kStaticListBytes);
  return RS_OK;
}

}  // namespace rs
