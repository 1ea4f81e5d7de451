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
  FoldItem* work;
  int* work_count;
  const void *x, *B, *C, *dt;
  const float *A, *D;
  float* y;
  const int32_t* accepted;
};

enum class M2Op { Conv, NonFlush, Flush, SpecAppend, CommitMeta, CommitFold, ConvSpec, Restore, Requant };

struct M2Launch {
  int rows, cols;   // dstate, headdim
  bool in_bf16;
  int ckf, rdf;     // checkpoint format, format read by non-flush / append
  bool rc;          // read copy configured
  int grid;
};

// Counter advance that follows a step kernel (the step kernels only read the counters).
enum class MetaOp { NonFlush = 0, Flush = 1, Append = 2 };
void meta_advance(rs_meta* meta, int batch, MetaOp op, int K, hipStream_t st);

bool m2_shape_supported(int dstate, int headdim);
void m2_launch(M2Op op, const M2Args& a, const M2Launch& l, hipStream_t st);

// Gated DeltaNet
struct GDNArgs {
  int batch, nv, nqk, vpk;   // vpk = value heads per qk head
  StateBuf ck;
  void *rq, *rk, *rv, *rg, *rbeta, *ru;
  rs_meta* meta;
  const void *q, *k, *v;
  const float *g, *beta;
  float* o;
};

enum class GDNOp { Conv, NonFlush, Flush };

struct GDNLaunch {
  int dk, dv;
  bool in_bf16;
  int grid;
};

bool gdn_shape_supported(int dk, int dv);
void gdn_launch(GDNOp op, const GDNArgs& a, const GDNLaunch& l, hipStream_t st);

}  // namespace rs
