// Host side of the C ABI: configuration checks, buffer layout, and the
// argument blocks of the kernels. Every entry point validates what the host
// can see, then hands its arguments to the dispatch functions of the kernel
// files (rs_host.h), which enqueue the kernels on the caller's stream and
// return without synchronising. Plain C++: no GPU header is included here.
#include <cstring>

#include "rs.h"
#include "rs_host.h"

using namespace rs;

namespace {

constexpr uint64_t kAlign = 256;

uint64_t align_up(uint64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Library work space inside the meta buffer, after rs_meta[batch]: the commit
// fold list (FoldItem[batch]) and its count, then the first-level arrival
// counters (arrive_groups of up to two workgroups per head, per sequence).
uint64_t arrive_off(const rs_layer& L) {
  return L.meta_work_off + align_up(static_cast<uint64_t>(L.cfg.batch) * sizeof(FoldItem)) + kAlign;
}
uint64_t arrive_bytes(const rs_layer& L) {
  return static_cast<uint64_t>(L.cfg.batch) * arrive_groups(2 * L.heads) * kArriveStride * sizeof(uint32_t);
}

int in_size(int32_t dt) { return dt == RS_F32 ? 4 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool need(const void* p) { return p != nullptr && aligned16(p); }

int fmt_of(int32_t dt) {
  switch (dt) {
    case RS_F16: return FMT_F16;
    case RS_FP8E4M3: return FMT_FP8;
    case RS_NVFP4: return FMT_NVFP4;
    default: return FMT_F32;
  }
}

// bytes of a [mats] x rows x cols state in a checkpoint format, and the
// offsets of its scale arrays
struct StateLayout {
  uint64_t bytes = 0, scale_off = 0, nv_scale_off = 0, tscale_off = 0;
};

StateLayout state_layout(int32_t dt, uint64_t mats, uint64_t rc) {
  StateLayout s;
  switch (dt) {
    case RS_F32: s.bytes = mats * rc * 4; break;
    case RS_F16: s.bytes = mats * rc * 2; break;
    case RS_FP8E4M3:
      s.scale_off = align_up(mats * rc);
      s.bytes = s.scale_off + mats * 4;
      break;
    case RS_NVFP4:
      s.nv_scale_off = align_up(mats * rc / 2);
      s.tscale_off = align_up(s.nv_scale_off + mats * rc / 16);
      s.bytes = s.tscale_off + mats * 4;
      break;
    default: break;
  }
  return s;
}

rs_status check_layer(const rs_layer* L) {
  if (!L || L->magic != kLayerMagic) return RS_E_ARG;
  return RS_OK;
}

rs_status launched() { return launch_status(); }


StateBuf ck_buf(const rs_layer* L, void* ckpt) {
  StateBuf s{ckpt, nullptr, nullptr};
  char* base = static_cast<char*>(ckpt);
  if (L->cfg.ckpt_dtype == RS_FP8E4M3) s.tscale = reinterpret_cast<float*>(base + L->ck_scale_off);
  if (L->cfg.ckpt_dtype == RS_NVFP4) {
    s.nv_scale = reinterpret_cast<uint8_t*>(base + L->ck_nv_scale_off);
    s.tscale = reinterpret_cast<float*>(base + L->ck_nv_tscale_off);
  }
  return s;
}

StateBuf rc_buf(const rs_layer* L, void* rcp) {
  StateBuf s{rcp, nullptr, nullptr};
  if (!rcp) return s;
  char* base = static_cast<char*>(rcp);
  s.nv_scale = reinterpret_cast<uint8_t*>(base + L->nv_scale_off);
  s.tscale = reinterpret_cast<float*>(base + L->nv_tscale_off);
  return s;
}

// Mamba-2 argument block common to every call
rs_status m2_args(const rs_layer* L, const rs_buffers* buf, M2Args* a, M2Launch* l) {
  const rs_config& c = L->cfg;
  if (!buf || !need(buf->ckpt)) return buf && buf->ckpt ? RS_E_ALIGN : RS_E_ARG;
  std::memset(a, 0, sizeof(*a));
  a->batch = c.batch;
  a->nheads = c.nheads;
  a->ngroups = c.ngroups;
  a->hpg = c.nheads / c.ngroups;
  a->kmax = c.max_draft;
  a->fuse_rc = c.fuse_requant;
  a->ck = ck_buf(L, buf->ckpt);
  a->rd = a->ck;
  if (c.mode == RS_REPLAY) {
    if (!buf->ring || !buf->meta) return RS_E_ARG;
    if (!aligned16(buf->ring) || !aligned16(buf->meta)) return RS_E_ALIGN;
    char* r = static_cast<char*>(buf->ring);
    a->rx = r + L->ring_x_off;
    a->rB = r + L->ring_B_off;
    a->rC = r + L->ring_C_off;
    a->rdt = r + L->ring_dt_off;
    a->meta = static_cast<rs_meta*>(buf->meta);
    a->arrive = reinterpret_cast<uint32_t*>(static_cast<char*>(buf->meta) + arrive_off(*L));
    char* w = static_cast<char*>(buf->meta) + L->meta_work_off;
    a->work = reinterpret_cast<FoldItem*>(w);
    a->work_count = reinterpret_cast<int*>(w + align_up(static_cast<uint64_t>(c.batch) * sizeof(FoldItem)));
    if (c.read_copy == RS_NVFP4) {
      if (!buf->read_copy) return RS_E_ARG;
      if (!aligned16(buf->read_copy)) return RS_E_ALIGN;
      a->rc = rc_buf(L, buf->read_copy);
      a->rd = a->rc;
    }
  } else if (c.max_draft > 0) {
    a->snap = static_cast<float*>(buf->snap);
  }
  l->rows = c.dstate;
  l->cols = c.headdim;
  l->in_bf16 = c.in_dtype == RS_BF16;
  l->ckf = fmt_of(c.ckpt_dtype);
  l->rc = c.read_copy == RS_NVFP4;
  l->rdf = l->rc ? FMT_NVFP4 : l->ckf;
  l->grid = c.batch * c.nheads;
  return RS_OK;
}

rs_status m2_inputs(const rs_inputs* in, const rs_params* prm, M2Args* a) {
  if (!in || !prm) return RS_E_ARG;
  if (!in->x || !in->B || !in->C || !in->dt || !prm->A || !prm->D) return RS_E_ARG;
  if (!aligned16(in->x) || !aligned16(in->B) || !aligned16(in->C) || !aligned16(in->dt) || !aligned16(prm->A) ||
      !aligned16(prm->D))
    return RS_E_ALIGN;
  a->x = in->x;
  a->B = in->B;
  a->C = in->C;
  a->dt = in->dt;
  a->A = prm->A;
  a->D = prm->D;
  return RS_OK;
}

GDNArgs gdn_args(const rs_layer* L, const rs_buffers* buf) {
  const rs_config& c = L->cfg;
  GDNArgs a;
  std::memset(&a, 0, sizeof(a));
  a.batch = c.batch;
  a.nv = c.n_v_heads;
  a.nqk = c.n_qk_heads;
  a.vpk = c.n_v_heads / c.n_qk_heads;
  a.kmax = c.max_draft;
  a.ck = ck_buf(L, buf->ckpt);
  if (c.read_copy == RS_NVFP4) a.rc = rc_buf(L, buf->read_copy);
  if (c.mode == RS_REPLAY) {
    char* r = static_cast<char*>(buf->ring);
    a.rq = r + L->ring_q_off;
    a.rk = r + L->ring_k_off;
    a.rv = r + L->ring_v_off;
    a.rg = r + L->ring_g_off;
    a.rbeta = r + L->ring_beta_off;
    a.ru = r + L->ring_u_off;
    a.meta = static_cast<rs_meta*>(buf->meta);
    a.arrive = reinterpret_cast<uint32_t*>(static_cast<char*>(buf->meta) + arrive_off(*L));
    char* w = static_cast<char*>(buf->meta) + L->meta_work_off;
    a.work = reinterpret_cast<FoldItem*>(w);
    a.work_count = reinterpret_cast<int*>(w + align_up(static_cast<uint64_t>(c.batch) * sizeof(FoldItem)));
  } else {
    a.snap = static_cast<float*>(buf->snap);
  }
  return a;
}

CommitArgs commit_args(const rs_layer* L, const rs_buffers* buf, const int32_t* accepted) {
  const rs_config& c = L->cfg;
  CommitArgs a;
  a.batch = c.batch;
  a.kmax = c.max_draft;
  a.meta = static_cast<rs_meta*>(buf->meta);
  a.accepted = accepted;
  char* w = static_cast<char*>(buf->meta) + L->meta_work_off;
  a.work = reinterpret_cast<FoldItem*>(w);
  a.work_count = reinterpret_cast<int*>(w + align_up(static_cast<uint64_t>(c.batch) * sizeof(FoldItem)));
  return a;
}

rs_status gdn_common(const rs_layer* L, const rs_buffers* buf, const rs_inputs* in, float* o, GDNArgs* a) {
  const rs_config& c = L->cfg;
  if (!buf || !in || !o) return RS_E_ARG;
  if (!buf->ckpt || !in->q || !in->k || !in->v || !in->g || !in->beta) return RS_E_ARG;
  if (c.mode == RS_REPLAY && (!buf->ring || !buf->meta)) return RS_E_ARG;
  const void* ps[] = {buf->ckpt, in->q, in->k, in->v, in->g, in->beta, o};
  for (const void* p : ps)
    if (!aligned16(p)) return RS_E_ALIGN;
  if (c.mode == RS_REPLAY && (!aligned16(buf->ring) || !aligned16(buf->meta))) return RS_E_ALIGN;
  if (c.read_copy == RS_NVFP4) {
    if (!buf->read_copy) return RS_E_ARG;
    if (!aligned16(buf->read_copy)) return RS_E_ALIGN;
  }
  *a = gdn_args(L, buf);
  a->q = in->q;
  a->k = in->k;
  a->v = in->v;
  a->g = static_cast<const float*>(in->g);
  a->beta = static_cast<const float*>(in->beta);
  a->o = o;
  return RS_OK;
}

GDNLaunch gdn_launch_cfg(const rs_layer* L);

// With a read copy, the self-scheduling step (whose flushes fold in column
// slices) is followed by the requant of the states it folded.
rs_status gdn_refresh_copy(const rs_layer* L, const GDNArgs& a, void* st) {
  if (L->cfg.read_copy != RS_NVFP4) return RS_OK;
  if (rs_status s = launch_status()) return s;
  gdn_launch(GDNOp::RequantFolded, a, gdn_launch_cfg(L), st);
  return RS_OK;
}

GDNLaunch gdn_launch_cfg(const rs_layer* L) {
  const rs_config& c = L->cfg;
  GDNLaunch l;
  l.dk = c.head_k_dim;
  l.dv = c.head_v_dim;
  l.in_bf16 = c.in_dtype == RS_BF16;
  l.vg = c.kind == RS_KDA;
  l.rc = c.read_copy == RS_NVFP4;
  l.ckf = fmt_of(c.ckpt_dtype);
  l.grid = c.batch * c.n_v_heads;
  return l;
}

}  // namespace

// The shapes the kernel files instantiate (rs_m2_<rows>x<cols>.hip; rs_gdn.hip).
bool rs::m2_shape_supported(int dstate, int headdim) {
  return (dstate == 16 && headdim == 16) || (dstate == 64 && headdim == 64) || (dstate == 128 && headdim == 64) ||
         (dstate == 128 && headdim == 128);
}

bool rs::gdn_shape_supported(int dk, int dv) {
  return (dk == 16 && dv == 16) || (dk == 64 && dv == 64) || (dk == 128 && dv == 128);
}

extern "C" {

rs_status rs_init(const rs_config* cfg, rs_layer* out) {
  if (!cfg || !out) return RS_E_ARG;
  const rs_config c = *cfg;
  if (c.kind != RS_MAMBA2 && c.kind != RS_GDN && c.kind != RS_KDA) return RS_E_ARG;
  if (c.mode != RS_REPLAY && c.mode != RS_CONVENTIONAL) return RS_E_MODE;
  if (c.batch < 1 || c.batch > (1 << 20)) return RS_E_ARG;
  if (c.ring != kRing) return RS_E_ARG;
  if (c.in_dtype != RS_F32 && c.in_dtype != RS_BF16) return RS_E_DTYPE;
  if (c.max_draft < 0 || c.max_draft > kMaxDraft) return RS_E_ARG;
  if (c.fuse_requant != 0 && c.fuse_requant != 1) return RS_E_ARG;
  if (c.read_copy != RS_NONE && c.read_copy != RS_NVFP4) return RS_E_DTYPE;
  rs_layer L;
  std::memset(&L, 0, sizeof(L));
  L.cfg = c;
  const uint64_t B = static_cast<uint64_t>(c.batch);
  const uint64_t sin = static_cast<uint64_t>(in_size(c.in_dtype));
  const bool replay = c.mode == RS_REPLAY;
  if (c.kind == RS_MAMBA2) {
    if (c.nheads < 1 || c.ngroups < 1 || c.headdim < 1 || c.dstate < 1) return RS_E_ARG;
    if (c.nheads % c.ngroups != 0) return RS_E_ARG;
    if (static_cast<uint64_t>(c.batch) * c.nheads > (1u << 30)) return RS_E_ARG;
    if (!m2_shape_supported(c.dstate, c.headdim)) return RS_E_UNSUPPORTED;
    if (c.ckpt_dtype != RS_F32 && c.ckpt_dtype != RS_F16 && c.ckpt_dtype != RS_FP8E4M3 && c.ckpt_dtype != RS_NVFP4)
      return RS_E_DTYPE;
    if (!replay && (c.ckpt_dtype != RS_F32 || c.read_copy != RS_NONE)) return RS_E_DTYPE;
    if (c.ckpt_dtype == RS_NVFP4 && c.read_copy != RS_NONE) return RS_E_DTYPE;
    L.heads = c.nheads;
    L.in_heads = c.ngroups;
    L.rows = c.dstate;
    L.cols = c.headdim;
  } else {
    if (c.n_qk_heads < 1 || c.n_v_heads < 1 || c.head_k_dim < 1 || c.head_v_dim < 1) return RS_E_ARG;
    if (c.n_v_heads % c.n_qk_heads != 0) return RS_E_ARG;
    if (static_cast<uint64_t>(c.batch) * c.n_v_heads > (1u << 30)) return RS_E_ARG;
    if (!gdn_shape_supported(c.head_k_dim, c.head_v_dim)) return RS_E_UNSUPPORTED;
    // FP16 / FP8 checkpoints: replay mode, without a read copy, on the 16 x 16 and
    // 128 x 128 states
    if (c.ckpt_dtype != RS_F32 && c.ckpt_dtype != RS_F16 && c.ckpt_dtype != RS_FP8E4M3) return RS_E_DTYPE;
    if (c.ckpt_dtype != RS_F32 && (!replay || c.read_copy != RS_NONE)) return RS_E_DTYPE;
    if (c.ckpt_dtype != RS_F32 && c.head_k_dim == 64) return RS_E_UNSUPPORTED;
    if (!replay && c.read_copy != RS_NONE) return RS_E_DTYPE;
    L.heads = c.n_v_heads;
    L.in_heads = c.n_qk_heads;
    L.rows = c.head_k_dim;
    L.cols = c.head_v_dim;
  }
  const uint64_t mats = B * L.heads;
  const uint64_t rc = static_cast<uint64_t>(L.rows) * L.cols;
  const StateLayout ck = state_layout(c.ckpt_dtype, mats, rc);
  L.ckpt_bytes = ck.bytes;
  L.ck_scale_off = ck.scale_off;
  L.ck_nv_scale_off = ck.nv_scale_off;
  L.ck_nv_tscale_off = ck.tscale_off;
  if (replay) {
    uint64_t off = 0;
    if (c.kind == RS_MAMBA2) {
      L.ring_x_off = off; off = align_up(off + B * c.nheads * kRing * c.headdim * sin);
      L.ring_B_off = off; off = align_up(off + B * c.ngroups * kRing * c.dstate * sin);
      L.ring_C_off = off; off = align_up(off + B * c.ngroups * kRing * c.dstate * sin);
      L.ring_dt_off = off; off = align_up(off + B * c.nheads * kRing * sin);
    } else {
      L.ring_q_off = off; off = align_up(off + B * c.n_qk_heads * kRing * c.head_k_dim * sin);
      L.ring_k_off = off; off = align_up(off + B * c.n_qk_heads * kRing * c.head_k_dim * sin);
      L.ring_v_off = off; off = align_up(off + B * c.n_v_heads * kRing * c.head_v_dim * sin);
      const uint64_t gw = c.kind == RS_KDA ? static_cast<uint64_t>(c.head_k_dim) : 1;   // gate width
      L.ring_g_off = off; off = align_up(off + B * c.n_v_heads * kRing * gw * 4);
      L.ring_beta_off = off; off = align_up(off + B * c.n_v_heads * kRing * 4);
      L.ring_u_off = off; off = align_up(off + B * c.n_v_heads * kRing * c.head_v_dim * 4);
    }
    L.ring_bytes = off;
    L.meta_work_off = align_up(B * sizeof(rs_meta));
    L.meta_bytes = arrive_off(L) + arrive_bytes(L);
    if (c.read_copy == RS_NVFP4) {
      const StateLayout r = state_layout(RS_NVFP4, mats, rc);
      L.read_copy_bytes = r.bytes;
      L.nv_scale_off = r.nv_scale_off;
      L.nv_tscale_off = r.tscale_off;
    }
  } else if (c.max_draft > 0) {
    L.snap_bytes = static_cast<uint64_t>(c.max_draft) * mats * rc * 4;
  }
  L.magic = kLayerMagic;
  *out = L;
  return RS_OK;
}

rs_status rs_step_conventional(const rs_layer* L, const rs_buffers* buf, const rs_inputs* in, const rs_params* prm,
                               float* y, void* stream) {
  if (rs_status s = check_layer(L)) return s;
  if (L->cfg.mode != RS_CONVENTIONAL) return RS_E_MODE;
  if (!y) return RS_E_ARG;
  if (!aligned16(y)) return RS_E_ALIGN;
  void* st = stream;
  if (L->cfg.kind != RS_MAMBA2) {
    GDNArgs a;
    if (rs_status s = gdn_common(L, buf, in, y, &a)) return s;
    gdn_launch(GDNOp::Conv, a, gdn_launch_cfg(L), st);
    return launched();
  }
  M2Args a;
  M2Launch l;
  if (rs_status s = m2_args(L, buf, &a, &l)) return s;
  if (rs_status s = m2_inputs(in, prm, &a)) return s;
  a.y = y;
  m2_launch(M2Op::Conv, a, l, st);
  return launched();
}

enum class StepKind { NonFlush, Flush, Auto };

static rs_status replay_step(const rs_layer* L, const rs_buffers* buf, const rs_inputs* in, const rs_params* prm,
                             float* y, void* stream, StepKind kind) {
  if (rs_status s = check_layer(L)) return s;
  if (L->cfg.mode != RS_REPLAY) return RS_E_MODE;
  if (!y) return RS_E_ARG;
  if (!aligned16(y)) return RS_E_ALIGN;
  void* st = stream;
  if (L->cfg.kind != RS_MAMBA2) {
    GDNArgs a;
    if (rs_status s = gdn_common(L, buf, in, y, &a)) return s;
    gdn_launch(kind == StepKind::Flush ? GDNOp::Flush : kind == StepKind::Auto ? GDNOp::Auto : GDNOp::NonFlush, a,
               gdn_launch_cfg(L), st);
    if (kind == StepKind::Auto)
      if (rs_status s = gdn_refresh_copy(L, a, st)) return s;
    return launched();
  }
  M2Args a;
  M2Launch l;
  if (rs_status s = m2_args(L, buf, &a, &l)) return s;
  if (rs_status s = m2_inputs(in, prm, &a)) return s;
  a.y = y;
  m2_launch(kind == StepKind::Flush ? M2Op::Flush : kind == StepKind::Auto ? M2Op::Auto : M2Op::NonFlush, a, l, st);
  return launched();
}

rs_status rs_step_nonflush(const rs_layer* L, const rs_buffers* buf, const rs_inputs* in, const rs_params* prm,
                           float* y, void* stream) {
  return replay_step(L, buf, in, prm, y, stream, StepKind::NonFlush);
}

rs_status rs_step_flush(const rs_layer* L, const rs_buffers* buf, const rs_inputs* in, const rs_params* prm, float* y,
                        void* stream) {
  return replay_step(L, buf, in, prm, y, stream, StepKind::Flush);
}

rs_status rs_step(const rs_layer* L, const rs_buffers* buf, const rs_inputs* in, const rs_params* prm, float* y,
                  void* stream) {
  return replay_step(L, buf, in, prm, y, stream, StepKind::Auto);
}

rs_status rs_reset_slots(const rs_layer* L, const rs_buffers* buf, const int32_t* seqs, int32_t count, void* stream) {
  if (rs_status s = check_layer(L)) return s;
  if (L->cfg.mode != RS_REPLAY) return RS_E_MODE;
  if (!buf || !buf->meta || count < 0 || (count > 0 && !seqs)) return RS_E_ARG;
  if (!aligned16(buf->meta)) return RS_E_ALIGN;
  if (count == 0) return RS_OK;
  reset_slots(static_cast<rs_meta*>(buf->meta), L->cfg.batch, seqs, count, stream);
  return launched();
}

namespace {

// Per-sequence regions of a layer's buffers, in the order rs_copy_slots copies them.
struct SeqRegion {
  int buf;           // 0 checkpoint, 1 ring, 2 read copy
  uint64_t off, per;
};

int seq_regions(const rs_layer* L, SeqRegion* out) {
  const rs_config& c = L->cfg;
  const uint64_t h = static_cast<uint64_t>(L->heads);
  const uint64_t rc = static_cast<uint64_t>(L->rows) * L->cols;
  const uint64_t sin = c.in_dtype == RS_BF16 ? 2 : 4;
  int n = 0;
  auto add = [&](int b, uint64_t off, uint64_t per) { out[n++] = SeqRegion{b, off, per}; };
  switch (c.ckpt_dtype) {
    case RS_F32: add(0, 0, h * rc * 4); break;
    case RS_F16: add(0, 0, h * rc * 2); break;
    case RS_FP8E4M3:
      add(0, 0, h * rc);
      add(0, L->ck_scale_off, h * 4);
      break;
    default:
      add(0, 0, h * rc / 2);
      add(0, L->ck_nv_scale_off, h * rc / 16);
      add(0, L->ck_nv_tscale_off, h * 4);
      break;
  }
  if (c.mode != RS_REPLAY) return n;
  if (c.kind == RS_MAMBA2) {
    add(1, L->ring_x_off, static_cast<uint64_t>(c.nheads) * kRing * c.headdim * sin);
    add(1, L->ring_B_off, static_cast<uint64_t>(c.ngroups) * kRing * c.dstate * sin);
    add(1, L->ring_C_off, static_cast<uint64_t>(c.ngroups) * kRing * c.dstate * sin);
    add(1, L->ring_dt_off, static_cast<uint64_t>(c.nheads) * kRing * sin);
  } else {
    const uint64_t gw = c.kind == RS_KDA ? static_cast<uint64_t>(c.head_k_dim) : 1;
    add(1, L->ring_q_off, static_cast<uint64_t>(c.n_qk_heads) * kRing * c.head_k_dim * sin);
    add(1, L->ring_k_off, static_cast<uint64_t>(c.n_qk_heads) * kRing * c.head_k_dim * sin);
    add(1, L->ring_v_off, static_cast<uint64_t>(c.n_v_heads) * kRing * c.head_v_dim * sin);
    add(1, L->ring_g_off, static_cast<uint64_t>(c.n_v_heads) * kRing * gw * 4);
    add(1, L->ring_beta_off, static_cast<uint64_t>(c.n_v_heads) * kRing * 4);
    add(1, L->ring_u_off, static_cast<uint64_t>(c.n_v_heads) * kRing * c.head_v_dim * 4);
  }
  if (c.read_copy == RS_NVFP4) {
    add(2, 0, h * rc / 2);
    add(2, L->nv_scale_off, h * rc / 16);
    add(2, L->nv_tscale_off, h * 4);
  }
  return n;
}

}  // namespace

rs_status rs_copy_slots(const rs_layer* Ls, const rs_buffers* src, const int32_t* src_seqs, const rs_layer* Ld,
                        const rs_buffers* dst, const int32_t* dst_seqs, int32_t count, void* stream) {
  if (rs_status s = check_layer(Ls)) return s;
  if (rs_status s = check_layer(Ld)) return s;
  rs_config cs = Ls->cfg;
  cs.batch = Ld->cfg.batch;
  if (std::memcmp(&cs, &Ld->cfg, sizeof(rs_config)) != 0) return RS_E_ARG;
  if (count < 0 || count > 65535 || (count > 0 && (!src_seqs || !dst_seqs))) return RS_E_ARG;
  if (!src || !dst || !src->ckpt || !dst->ckpt) return RS_E_ARG;
  const bool replay = Ls->cfg.mode == RS_REPLAY;
  if (replay && (!src->ring || !dst->ring || !src->meta || !dst->meta)) return RS_E_ARG;
  if (Ls->cfg.read_copy == RS_NVFP4 && (!src->read_copy || !dst->read_copy)) return RS_E_ARG;
  const void* ptrs[8] = {src->ckpt, dst->ckpt, src->ring, dst->ring, src->read_copy, dst->read_copy, src->meta,
                         dst->meta};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return RS_E_ALIGN;
  if (count == 0) return RS_OK;
  SeqRegion reg[kMaxCopyRegions], dreg[kMaxCopyRegions];
  const int nreg = seq_regions(Ls, reg);
  seq_regions(Ld, dreg);   // same regions and sizes; offsets of the other batch
  CopyArgs a{};
  uint64_t total = 0;
  for (int i = 0; i < nreg; ++i) {
    const char* sb = static_cast<const char*>(reg[i].buf == 0 ? src->ckpt : reg[i].buf == 1 ? src->ring
                                                                                              : src->read_copy);
    char* db = static_cast<char*>(reg[i].buf == 0 ? dst->ckpt : reg[i].buf == 1 ? dst->ring : dst->read_copy);
    if (reg[i].per % 4 != 0) return RS_E_UNSUPPORTED;
    a.r[i] = CopyRegion{sb + reg[i].off, db + dreg[i].off, reg[i].per};
    total += reg[i].per;
  }
  a.nreg = nreg;
  a.count = count;
  a.src_batch = Ls->cfg.batch;
  a.dst_batch = Ld->cfg.batch;
  a.src_seqs = src_seqs;
  a.dst_seqs = dst_seqs;
  a.src_meta = replay ? static_cast<const rs_meta*>(src->meta) : nullptr;
  a.dst_meta = replay ? static_cast<rs_meta*>(dst->meta) : nullptr;
  const uint64_t bpp = (total + 16383) / 16384;   // about four 16-byte chunks per thread
  copy_slots(a, static_cast<int>(bpp < 1 ? 1 : bpp > 1024 ? 1024 : bpp), stream);
  return launched();
}

rs_status rs_conv_step(const rs_layer* L, const rs_buffers* buf, void* conv_ring, const void* xbc, int32_t K,
                       const float* weight, const float* bias, int32_t width, void* x, void* Bo, void* Co,
                       void* stream) {
  if (rs_status s = check_layer(L)) return s;
  const rs_config& c = L->cfg;
  if (c.kind != RS_MAMBA2 || c.mode != RS_REPLAY) return RS_E_MODE;
  if (K < 1 || K > (c.max_draft > 1 ? c.max_draft : 1)) return RS_E_ARG;
  if (width < 1 || width > 4) return RS_E_ARG;
  if (!buf || !buf->meta || !conv_ring || !xbc || !weight || !x || !Bo || !Co) return RS_E_ARG;
  const int d_inner = c.nheads * c.headdim, gn = c.ngroups * c.dstate;
  if (d_inner % 8 != 0 || gn % 8 != 0) return RS_E_UNSUPPORTED;
  const void* ptrs[7] = {buf->meta, conv_ring, xbc, weight, x, Bo, Co};
  for (const void* p : ptrs)
    if (!aligned16(p)) return RS_E_ALIGN;
  if (bias && !aligned16(bias)) return RS_E_ALIGN;
  ConvArgs a{};
  a.batch = c.batch;
  a.channels = d_inner + 2 * gn;
  a.width = width;
  a.K = K;
  a.d_inner = d_inner;
  a.gn = gn;
  a.meta = static_cast<const rs_meta*>(buf->meta);
  a.ring = conv_ring;
  a.xbc = xbc;
  a.w = weight;
  a.bias = bias;
  a.x = x;
  a.B = Bo;
  a.C = Co;
  conv_step(a, c.in_dtype == RS_BF16, stream);
  return launched();
}

rs_status rs_gated_norm(const rs_layer* L, int32_t K, const float* y, const void* z, const float* weight,
                        int32_t norm_groups, float eps, void* out, void* stream) {
  if (rs_status s = check_layer(L)) return s;
  const rs_config& c = L->cfg;
  if (c.kind != RS_MAMBA2) return RS_E_MODE;
  const int d_inner = c.nheads * c.headdim;
  if (K < 1 || K > (c.max_draft > 1 ? c.max_draft : 1)) return RS_E_ARG;
  if (norm_groups < 1 || d_inner % norm_groups != 0 || !(eps >= 0.0f)) return RS_E_ARG;
  if (!y || !z || !weight || !out) return RS_E_ARG;
  if ((d_inner / norm_groups) % 4 != 0) return RS_E_UNSUPPORTED;
  if (!aligned16(y) || !aligned16(z) || !aligned16(weight) || !aligned16(out)) return RS_E_ALIGN;
  NormArgs a{};
  a.rows = K * c.batch;
  a.d = d_inner;
  a.gs = d_inner / norm_groups;
  a.eps = eps;
  a.y = y;
  a.z = z;
  a.w = weight;
  a.out = out;
  gated_norm(a, c.in_dtype == RS_BF16, stream);
  return launched();
}

rs_status rs_spec_append(const rs_layer* L, const rs_buffers* buf, const rs_inputs* drafts, int32_t K,
                         const rs_params* prm, float* y, void* stream) {
  if (rs_status s = check_layer(L)) return s;
  if (L->cfg.max_draft == 0) return RS_E_MODE;
  if (K < 1 || K > L->cfg.max_draft) return RS_E_ARG;
  if (!y) return RS_E_ARG;
  if (!aligned16(y)) return RS_E_ALIGN;
  if (L->cfg.kind != RS_MAMBA2) {
    GDNArgs a;
    if (rs_status s = gdn_common(L, buf, drafts, y, &a)) return s;
    a.K = K;
    void* st = stream;
    if (L->cfg.mode == RS_CONVENTIONAL) {
      if (!buf->snap) return RS_E_ARG;
      if (!aligned16(buf->snap)) return RS_E_ALIGN;
      gdn_launch(GDNOp::ConvSpec, a, gdn_launch_cfg(L), st);
    } else {
      gdn_launch(GDNOp::SpecAppend, a, gdn_launch_cfg(L), st);
    }
    return launched();
  }
  M2Args a;
  M2Launch l;
  if (rs_status s = m2_args(L, buf, &a, &l)) return s;
  if (rs_status s = m2_inputs(drafts, prm, &a)) return s;
  a.y = y;
  a.K = K;
  void* st = stream;
  if (L->cfg.mode == RS_CONVENTIONAL) {
    if (!buf->snap) return RS_E_ARG;
    if (!aligned16(buf->snap)) return RS_E_ALIGN;
    m2_launch(M2Op::ConvSpec, a, l, st);
  } else {
    m2_launch(M2Op::SpecAppend, a, l, st);
  }
  return launched();
}

// The speculative commit; the fold list lives in the meta buffer's work space,
// or, with use_static, in the library's static device array.
static rs_status spec_commit(const rs_layer* L, const rs_buffers* buf, const int32_t* accepted, const rs_params* prm,
                             void* stream, bool use_static) {
  if (rs_status s = check_layer(L)) return s;
  if (L->cfg.max_draft == 0) return RS_E_MODE;
  if (!accepted) return RS_E_ARG;
  if (!aligned16(accepted)) return RS_E_ALIGN;
  if (use_static && L->cfg.batch > kStaticFoldSeqs) return RS_E_ARG;
  void* st = stream;
  if (L->cfg.kind != RS_MAMBA2) {
    if (!buf || !buf->ckpt) return RS_E_ARG;
    if (L->cfg.mode == RS_REPLAY && (!buf->ring || !buf->meta)) return RS_E_ARG;
    if (!aligned16(buf->ckpt)) return RS_E_ALIGN;
    if (L->cfg.mode == RS_REPLAY && (!aligned16(buf->ring) || !aligned16(buf->meta))) return RS_E_ALIGN;
    if (L->cfg.read_copy == RS_NVFP4 && !buf->read_copy) return RS_E_ARG;
    if (L->cfg.read_copy == RS_NVFP4 && !aligned16(buf->read_copy)) return RS_E_ALIGN;
  } else if (!prm || !prm->A || !prm->D) {
    return RS_E_ARG;
  }
  FoldItem* list = nullptr;
  int* count = nullptr;
  if (use_static && L->cfg.mode == RS_REPLAY)
    if (rs_status s = static_fold_list(&list, &count)) return s;
  if (L->cfg.kind != RS_MAMBA2) {
    GDNArgs a = gdn_args(L, buf);
    a.accepted = accepted;
    GDNLaunch l = gdn_launch_cfg(L);
    if (L->cfg.mode == RS_CONVENTIONAL) {
      if (!buf->snap) return RS_E_ARG;
      if (!aligned16(buf->snap)) return RS_E_ALIGN;
      gdn_launch(GDNOp::Restore, a, l, st);
    } else {
      CommitArgs ca = commit_args(L, buf, accepted);
      if (list) {
        ca.work = a.work = list;
        ca.work_count = a.work_count = count;
      }
      commit_meta(ca, st);
      if (rs_status s = launch_status()) return s;
      gdn_launch(GDNOp::CommitFold, a, l, st);
    }
    return launched();
  }
  M2Args a;
  M2Launch l;
  if (rs_status s = m2_args(L, buf, &a, &l)) return s;
  a.accepted = accepted;
  a.A = prm->A;
  a.D = prm->D;
  if (L->cfg.mode == RS_CONVENTIONAL) {
    if (!buf->snap) return RS_E_ARG;
    if (!aligned16(buf->snap)) return RS_E_ALIGN;
    m2_launch(M2Op::Restore, a, l, st);
  } else {
    CommitArgs ca = commit_args(L, buf, accepted);
    if (list) {
      ca.work = a.work = list;
      ca.work_count = a.work_count = count;
    }
    commit_meta(ca, st);
    if (rs_status s = launch_status()) return s;
    const int tiles = L->cfg.batch * L->cfg.nheads;
    l.grid = tiles < 2048 ? tiles : 2048;
    m2_launch(M2Op::CommitFold, a, l, st);
  }
  return launched();
}

rs_status rs_spec_commit(const rs_layer* L, const rs_buffers* buf, const int32_t* accepted, const rs_params* prm,
                         void* stream) {
  return spec_commit(L, buf, accepted, prm, stream, false);
}

rs_status rs_spec_commit_static(const rs_layer* L, const rs_buffers* buf, const int32_t* accepted,
                                const rs_params* prm, void* stream) {
  return spec_commit(L, buf, accepted, prm, stream, true);
}

rs_status rs_requant_read_copy(const rs_layer* L, const rs_buffers* buf, void* stream) {
  if (rs_status s = check_layer(L)) return s;
  if (L->cfg.read_copy != RS_NVFP4) return RS_E_MODE;
  if (!buf || !buf->ckpt || !buf->read_copy) return RS_E_ARG;
  if (!aligned16(buf->ckpt) || !aligned16(buf->read_copy)) return RS_E_ALIGN;
  if (L->cfg.kind != RS_MAMBA2) {
    GDNArgs a;
    std::memset(&a, 0, sizeof(a));
    a.batch = L->cfg.batch;
    a.nv = L->cfg.n_v_heads;
    a.ck = StateBuf{buf->ckpt, nullptr, nullptr};
    a.rc = rc_buf(L, buf->read_copy);
    gdn_launch(GDNOp::Requant, a, gdn_launch_cfg(L), stream);
    return launched();
  }
  M2Args a;
  std::memset(&a, 0, sizeof(a));
  a.ck = ck_buf(L, buf->ckpt);
  a.rc = rc_buf(L, buf->read_copy);
  M2Launch l;
  l.rows = L->rows;
  l.cols = L->cols;
  l.in_bf16 = false;
  l.ckf = fmt_of(L->cfg.ckpt_dtype);
  l.rdf = FMT_NVFP4;
  l.rc = true;
  l.grid = L->cfg.batch * L->heads;
  m2_launch(M2Op::Requant, a, l, stream);
  return launched();
}

const char* rs_status_string(rs_status s) {
  switch (s) {
    case RS_OK: return "ok";
    case RS_E_ARG: return "invalid argument";
    case RS_E_DTYPE: return "unsupported dtype";
    case RS_E_ALIGN: return "pointer not 16-byte aligned";
    case RS_E_MODE: return "call not valid for this layer mode";
    case RS_E_LAUNCH: return "kernel launch failed";
    case RS_E_UNSUPPORTED: return "shape not compiled";
    default: return "unknown status";
  }
}

int32_t rs_version(void) { return 100; }

}  // extern "C"
