// Library-internal declarations shared by the host side of the C ABI
// (rs_host.cpp, plain C++ with no GPU headers) and the kernel files: layout
// constants, the argument blocks the kernels take by value, and the dispatch
// functions each kernel file exports. Streams cross this interface as void*
// (a hipStream_t, or null for the default stream).
#pragma once

#include <stdint.h>

#include "rs.h"

namespace rs {

constexpr int kRing = 16;
constexpr int kMaxDraft = 8;
constexpr uint32_t kLayerMagic = 0x52534C31u;  // "RSL1"

enum Fmt { FMT_F32 = 0, FMT_F16 = 1, FMT_FP8 = 2, FMT_NVFP4 = 3 };

// One layer's state buffer in a given format. `data` points at matrix 0;
// matrix t (t = b*heads + h) starts at t*rows*cols elements.
struct StateBuf {
  void* data;          // f32 / f16 values, E4M3 codes, or packed E2M1 codes
  uint8_t* nv_scale;   // NVFP4 block scales [t][rows][cols/16]
  float* tscale;       // FP8 per-matrix scale or NVFP4 tensor scale [t]
};

// One sequence whose committed buffer entries a speculative commit folds.
struct FoldItem {
  int32_t b;      // sequence
  int32_t m;      // entries folded
  int64_t nck;    // n_ckpt before the fold (gives the ring slots)
};

// First-level arrival counters of the step kernels (see rs_internal.h):
// workgroups of a sequence arrive in groups of kArriveGroup, one 128-byte
// counter per group.
constexpr int kArriveGroup = 32;   // workgroups per first-level counter
constexpr int kArriveStride = 32;  // uint32 per first-level counter (128 bytes)

constexpr int arrive_groups(int nwg) { return (nwg + kArriveGroup - 1) / kArriveGroup; }

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

bool m2_shape_supported(int dstate, int headdim);
void m2_launch(M2Op op, const M2Args& a, const M2Launch& l, void* stream);

// Speculative commit, counter part (both layer kinds): len += accepted[b], nd = 0,
// and the ordered list of sequences whose committed entries must be folded now.
struct CommitArgs {
  int batch, kmax;
  rs_meta* meta;
  const int32_t* accepted;
  FoldItem* work;
  int* work_count;
};
void commit_meta(const CommitArgs& a, void* stream);

// Clear the counters of the listed sequences (slot reuse); entries outside
// [0, batch) are skipped.
void reset_slots(rs_meta* meta, int batch, const int32_t* seqs, int count, void* stream);

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
void copy_slots(const CopyArgs& a, int blocks_per_pair, void* stream);

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
void conv_step(const ConvArgs& a, bool bf, void* stream);

struct NormArgs {
  int rows, d, gs;         // rows = K * batch, d = d_inner, gs = channels per group
  float eps;
  const float* y;          // [rows][d]
  const void* z;           // [rows][d], input type
  const float* w;          // [d]
  void* out;               // [rows][d], input type
};
void gated_norm(const NormArgs& a, bool bf, void* stream);

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
  StateBuf rc;               // NVFP4 read copy of the checkpoint (when configured)
};

// Requant: the read copy of every state from the checkpoint. RequantFolded:
// the states of sequences whose buffer is empty and holds no drafts, i.e.
// those a self-scheduling step has just flushed (an unchanged state
// requantizes to the same bytes, so the others it also takes cost only time).
// The flush and the commit fold write the copy of what they fold themselves.
enum class GDNOp { Conv, NonFlush, Flush, Auto, SpecAppend, CommitFold, ConvSpec, Restore, Requant, RequantFolded };

struct GDNLaunch {
  int dk, dv;
  bool in_bf16;
  bool vg;        // Kimi Delta Attention: per-key-channel gate
  bool rc;        // NVFP4 read copy: reads go to it, folds re-solve from the checkpoint
  int ckf;        // checkpoint format FMT_F32 / FMT_F16 / FMT_FP8 (without a read copy)
  int grid;
};

bool gdn_shape_supported(int dk, int dv);
void gdn_launch(GDNOp op, const GDNArgs& a, const GDNLaunch& l, void* stream);

// The speculative commit's fold list without caller memory: a static device
// array in rs_commit.hip holding FoldItem[kStaticFoldSeqs] and the list's
// count, one copy per device. Sets *list and *count to its address on the
// current device (resolved once per device); RS_E_LAUNCH if the runtime
// cannot give it.
constexpr int kStaticFoldSeqs = 8192;
rs_status static_fold_list(FoldItem** list, int** count);

// RS_OK if every launch so far succeeded, RS_E_LAUNCH otherwise (the runtime's
// last error, read and cleared; no synchronisation).
rs_status launch_status();

}  // namespace rs
