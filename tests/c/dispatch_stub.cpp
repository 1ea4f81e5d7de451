// Host-only stand-in for the kernel files' dispatch functions (rs_host.h), for
// running the C ABI's host side without a GPU: each dispatch is recorded and
// checked for the invariants the kernels rely on, and nothing is launched.
// Linked with rs_host.cpp into the sanitizer build of the C ABI checks.
#include <cstdio>
#include <cstdlib>

#include "rs_host.h"

namespace {

int g_calls[16];

void require(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "dispatch stub: %s\n", what);
    std::abort();
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {
// Dispatches recorded so far by kind (see RS_STUB_* in abi_dispatch.c), and a reset.
int rs_stub_calls(int kind) { return kind >= 0 && kind < 16 ? g_calls[kind] : -1; }
void rs_stub_reset(void) {
  for (int& c : g_calls) c = 0;
}
}

namespace rs {

bool m2_shape_supported(int dstate, int headdim);

void m2_launch(M2Op op, const M2Args& a, const M2Launch& l, void*) {
  require(l.grid > 0, "m2 launch grid");
  if (op != M2Op::Requant)   // the quantizer reads only the two state buffers
    require(a.batch > 0 && a.nheads > 0 && a.hpg * a.ngroups == a.nheads, "m2 launch shape");
  require(m2_shape_supported(l.rows, l.cols), "m2 launch of an uncompiled shape");
  require(aligned16(a.ck.data), "m2 checkpoint alignment");
  if (op != M2Op::Conv && op != M2Op::ConvSpec && op != M2Op::Restore && op != M2Op::Requant)
    require(a.meta && a.arrive && a.rx && a.rB && a.rC && a.rdt, "m2 replay buffers");
  if (op == M2Op::Requant) require(a.rc.data && a.rc.nv_scale && a.rc.tscale, "m2 requant read copy");
  if (op == M2Op::SpecAppend || op == M2Op::ConvSpec) require(a.K >= 1 && a.K <= a.kmax, "m2 draft count");
  g_calls[0] += 1;
}

void gdn_launch(GDNOp op, const GDNArgs& a, const GDNLaunch& l, void*) {
  require(l.grid > 0 && a.batch > 0 && a.nv > 0, "gdn launch shape");
  if (op == GDNOp::Requant || op == GDNOp::RequantFolded) {   // the quantizer reads the states only
    require(l.rc && a.ck.data && a.rc.data && a.rc.nv_scale && a.rc.tscale, "gdn requant buffers");
    if (op == GDNOp::RequantFolded) require(a.meta != nullptr, "gdn requant counters");
    g_calls[1] += 1;
    return;
  }
  require(a.vpk * a.nqk == a.nv, "gdn head map");
  if (l.rc) require(a.rc.data && a.rc.nv_scale && a.rc.tscale, "gdn read copy");
  if (op == GDNOp::NonFlush || op == GDNOp::Flush || op == GDNOp::Auto || op == GDNOp::SpecAppend ||
      op == GDNOp::CommitFold)
    require(a.meta && a.arrive && a.rq && a.rk && a.rv && a.rg && a.rbeta && a.ru, "gdn replay buffers");
  g_calls[1] += 1;
}

void commit_meta(const CommitArgs& a, void*) {
  require(a.batch > 0 && a.meta && a.accepted && a.work && a.work_count, "commit arguments");
  g_calls[2] += 1;
}

void reset_slots(rs_meta* meta, int batch, const int32_t* seqs, int count, void*) {
  require(meta && batch > 0 && seqs && count > 0, "reset arguments");
  g_calls[3] += 1;
}

void copy_slots(const CopyArgs& a, int blocks_per_pair, void*) {
  require(a.nreg > 0 && a.nreg <= kMaxCopyRegions && a.count > 0 && blocks_per_pair >= 1, "copy arguments");
  for (int i = 0; i < a.nreg; ++i) require(a.r[i].src && a.r[i].dst && a.r[i].per % 4 == 0, "copy region");
  g_calls[4] += 1;
}

void conv_step(const ConvArgs& a, bool, void*) {
  require(a.batch > 0 && a.width >= 1 && a.width <= 4 && a.K >= 1 && a.d_inner % 8 == 0, "conv arguments");
  g_calls[5] += 1;
}

void gated_norm(const NormArgs& a, bool, void*) {
  require(a.rows > 0 && a.gs > 0 && a.d % a.gs == 0 && a.gs % 4 == 0, "norm arguments");
  g_calls[6] += 1;
}

rs_status launch_status() { return RS_OK; }

rs_status static_fold_list(FoldItem** list, int** count) {
  // a fake device address, never dereferenced on the host
  *list = reinterpret_cast<FoldItem*>(static_cast<uintptr_t>(0x7F0000000000ull));
  *count = reinterpret_cast<int*>(static_cast<uintptr_t>(0x7F0000000000ull + kStaticFoldSeqs * sizeof(FoldItem)));
  g_calls[7] += 1;
  return RS_OK;
}

}  // namespace rs
