// Library-internal declarations shared by the host API and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rs.h"
#include "rs_device.h"

namespace rs {

constexpr int kMaxDraft = 8;
constexpr uint32_t kLayerMagic = 0x52534C31u;  // "RSL1"

// One sequence whose committed buffer entries a speculative commit folds.
struct FoldItem {
  int32_t b;      // sequence
  int32_t m;      // entries folded
  int64_t nck;    // n_ckpt before the fold (gives the ring slots)
};

// Kernel arguments for every Mamba-2 kernel (passed by value).
struct M2Args {
  int batch, nheads, ngroups, hpg, kmax, K, fuse_rc;
  StateBuf ck;          // checkpoint, or live state (conventional)
  StateBuf rc;          // NVFP4 read copy
  StateBuf rd;          // what non-flush / append read: rc or ck
  float* snap;          // snapshot baseline states
  void *rx, *rB, *rC, *rdt;
  rs_meta* meta;
  uint32_t* arrive;     // first-level arrival counters, arrive_groups(nheads) per sequence
  FoldItem* work;
  int* work_count;
  const void *x, *B, *C, *dt;
  const float *A, *D;
  float* y;
  const int32_t* accepted;
};

enum class M2Op { Conv, NonFlush, Flush, Auto, SpecAppend, CommitFold, ConvSpec, Restore, Requant };

struct M2Launch {
  int rows, cols;   // dstate, headdim
  bool in_bf16;
  int ckf, rdf;     // checkpoint format, format read by non-flush / append
  bool rc;          // read copy configured
  int grid;
};

// Per-sequence buffer counters, advanced inside the step kernels (sitech.ge
// ReplaySSM page, "How ReplaySSM works": append on a non-flush step; fold and
// clear on a flush; "Reducing state traffic and simplifying rollback": drafts
// held until verification). Every workgroup of a sequence first reads the
// sequence's counters; thread 0 then counts the workgroup in with a relaxed
// device-scope atomic whose operand depends on the values read, so it is
// issued only once the read has completed. Counting is two-level: workgroups
// arrive in groups of kArriveGroup on a counter of their own (one 128-byte
// line each, so that same-address atomics queue at most kArriveGroup deep;
// group sizes 4 to 32 time within 1%, the larger slightly ahead); the last
// of a group then arrives on the sequence's counter in rs_meta. The
// workgroup that arrives last there knows that all workgroups of its sequence
// have read the counters: it writes the advanced counters (or a sticky error
// bit, leaving them as they were, exactly as every workgroup skipped the
// sequence). Each last arriver clears the counter it closed for the next
// launch. The first-level atomic is issued after the state loads and its
// result is needed only at the end, so it costs the workgroup no wait.
enum class MetaOp { NonFlush = 0, Flush = 1, Append = 2 };

constexpr int kArriveGroup = 32;   // workgroups per first-level counter
constexpr int kArriveStride = 32;  // uint32 per first-level counter (128 bytes)

__host__ __device__ constexpr int arrive_groups(int nwg) { return (nwg + kArriveGroup - 1) / kArriveGroup; }

struct Arrival {
  uint32_t c;
  // wg: this workgroup's index among the nwg workgroups of its sequence;
  // ctr: the sequence's arrive_groups(nwg) first-level counters.
  __device__ __forceinline__ void arrive(uint32_t* ctr, int wg, long long nck, int len, int nd) {
    c = 0;
    if (threadIdx.x == 0) {
      uint32_t one = 1u;
      const int dep = static_cast<int>(nck) ^ len ^ nd;
      asm volatile("" : "+v"(one) : "v"(dep));   // the atomic waits for the counters read
      c = __hip_atomic_fetch_add(ctr + (wg / kArriveGroup) * kArriveStride, one, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // Called by every thread at the end; thread 0 of the last workgroup applies the rule.
  __device__ __forceinline__ void finish(rs_meta* m, uint32_t* ctr, int wg, int nwg, MetaOp op, int K,
                                         long long nck, int len, int nd) const {
    if (threadIdx.x != 0) return;
    const int g = wg / kArriveGroup;
    const int gsize = nwg - g * kArriveGroup < kArriveGroup ? nwg - g * kArriveGroup : kArriveGroup;
    if (c != static_cast<uint32_t>(gsize - 1)) return;
    __hip_atomic_store(ctr + g * kArriveStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int ng = arrive_groups(nwg);
    if (ng > 1) {
      const uint32_t c2 = __hip_atomic_fetch_add(&m->arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (c2 != static_cast<uint32_t>(ng - 1)) return;
      __hip_atomic_store(&m->arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    switch (op) {
      case MetaOp::NonFlush:
        if (nd != 0) m->err |= RS_ERR_PENDING;
        else if (len > kRing - 2) m->err |= RS_ERR_FULL;
        else m->len = len + 1;
        break;
      case MetaOp::Flush:
        if (nd != 0) m->err |= RS_ERR_PENDING;
        else if (len > kRing - 1) m->err |= RS_ERR_FULL;
        else {
          m->n_ckpt = nck + len + 1;
          m->len = 0;
        }
        break;
      case MetaOp::Append:
        if (nd != 0 || len + K > kRing) m->err |= RS_ERR_OVERFLOW;
        else m->nd = K;
        break;
    }
  }
};

bool m2_shape_supported(int dstate, int headdim);
void m2_launch(M2Op op, const M2Args& a, const M2Launch& l, hipStream_t st);

// Speculative commit, counter part (both layer kinds): len += accepted[b], nd = 0,
// and the ordered list of sequences whose committed entries must be folded now.
struct CommitArgs {
  int batch, kmax;
  rs_meta* meta;
  const int32_t* accepted;
  FoldItem* work;
  int* work_count;
};
void commit_meta(const CommitArgs& a, hipStream_t st);

// Clear the counters of the listed sequences (slot reuse); entries outside
// [0, batch) are skipped.
void reset_slots(rs_meta* meta, int batch, const int32_t* seqs, int count, hipStream_t st);

// Copy the whole state of listed sequences between two buffer sets of one
// layer configuration: every per-sequence region (checkpoint and its scales,
// read copy, ring arrays) is `per` bytes at src + seq * per, and the counters
// n_ckpt, len, nd, err of the meta record.
constexpr int kMaxCopyRegions = 16;
struct CopyRegion {
  const char* src;
  char* dst;
  uint64_t per;
};
struct CopyArgs {
  CopyRegion r[kMaxCopyRegions];
  int nreg, count, src_batch, dst_batch;
  const int32_t* src_seqs;
  const int32_t* dst_seqs;
  const rs_meta* src_meta;   // null in conventional mode
  rs_meta* dst_meta;
};
void copy_slots(const CopyArgs& a, int blocks_per_pair, hipStream_t st);

// Mamba-2 block: short causal convolution with its ring of recent inputs, and
// the gated RMS norm of the SSM output.
struct ConvArgs {
  int batch, channels, width, K;
  int d_inner, gn;         // x channels, then ngroups * dstate each for B and C
  const rs_meta* meta;     // positions n_ckpt + len
  void* ring;              // [batch][16][channels]
  const void* xbc;         // [K][batch][channels]
  const float* w;          // [channels][width]
  const float* bias;       // [channels] or null
  void* x;                 // [K][batch][d_inner]
  void* B;                 // [K][batch][gn]
  void* C;                 // [K][batch][gn]
};
void conv_step(const ConvArgs& a, bool bf, hipStream_t st);

struct NormArgs {
  int rows, d, gs;         // rows = K * batch, d = d_inner, gs = channels per group
  float eps;
  const float* y;          // [rows][d]
  const void* z;           // [rows][d], input type
  const float* w;          // [d]
  void* out;               // [rows][d], input type
};
void gated_norm(const NormArgs& a, bool bf, hipStream_t st);

// Gated DeltaNet
struct GDNArgs {
  int batch, nv, nqk, vpk;   // vpk = value heads per qk head
  int K, kmax;               // speculative: drafts in this call, configured maximum
  StateBuf ck;               // checkpoint, or live state (conventional)
  float* snap;               // snapshot baseline states [kmax][batch][nv][dk][dv]
  void *rq, *rk, *rv, *rg, *rbeta, *ru;
  rs_meta* meta;
  uint32_t* arrive;     // first-level arrival counters, arrive_groups(workgroups per sequence) each
  FoldItem* work;
  int* work_count;
  const int32_t* accepted;
  const void *q, *k, *v;     // one token, or K drafts stacked [K][batch][...]
  const float *g, *beta;
  float* o;                  // [batch][nv][dv], or [K][batch][nv][dv]
};

enum class GDNOp { Conv, NonFlush, Flush, Auto, SpecAppend, CommitFold, ConvSpec, Restore };

struct GDNLaunch {
  int dk, dv;
  bool in_bf16;
  bool vg;        // Kimi Delta Attention: per-key-channel gate
  int grid;
};

bool gdn_shape_supported(int dk, int dv);
void gdn_launch(GDNOp op, const GDNArgs& a, const GDNLaunch& l, hipStream_t st);

}  // namespace rs
