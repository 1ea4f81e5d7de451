/* The C ABI's host side against a recording stand-in for the kernel files
 * (dispatch_stub.cpp): every entry point is called with valid arguments and
 * must dispatch exactly once (two launches for a replay commit); then with
 * invalid ones, and must return the documented status without dispatching.
 * Device pointers are fake, 256-byte aligned addresses that the host side
 * never dereferences. Built and run under AddressSanitizer and
 * UndefinedBehaviorSanitizer; prints one line per check. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "rs.h"

int rs_stub_calls(int kind);
void rs_stub_reset(void);
enum { STUB_M2, STUB_GDN, STUB_COMMIT, STUB_RESET, STUB_COPY, STUB_CONV, STUB_NORM, STUB_STATIC, STUB_KINDS };

static int fails = 0;

static void expect(int cond, const char* what) {
  printf("%s %s\n", cond ? "ok" : "FAIL", what);
  if (!cond) fails++;
}

static void* dev(unsigned i) { return (void*)(uintptr_t)(0x100000000ull + (uint64_t)i * 0x40000000ull); }

/* status st, and the dispatch counts changed by exactly delta[] */
static void expect_call(rs_status st, rs_status want, const int* delta, const int* before, const char* what) {
  int ok = st == want;
  for (int k = 0; k < STUB_KINDS; ++k) ok = ok && rs_stub_calls(k) - before[k] == (delta ? delta[k] : 0);
  if (!ok) printf("  status %d (want %d)\n", (int)st, (int)want);
  expect(ok, what);
}

#define SNAP(b) int b[STUB_KINDS]; for (int k_ = 0; k_ < STUB_KINDS; ++k_) b[k_] = rs_stub_calls(k_)

static rs_config m2_cfg(int mode) {
  rs_config c;
  memset(&c, 0, sizeof c);
  c.kind = RS_MAMBA2;
  c.mode = mode;
  c.batch = 4;
  c.nheads = 128;
  c.headdim = 64;
  c.dstate = 128;
  c.ngroups = 8;
  c.ring = 16;
  c.max_draft = 4;
  c.in_dtype = RS_BF16;
  c.ckpt_dtype = RS_F32;
  c.read_copy = mode == RS_REPLAY ? RS_NVFP4 : RS_NONE;
  c.fuse_requant = 1;
  return c;
}

static rs_config delta_cfg(int kind, int mode) {
  rs_config c;
  memset(&c, 0, sizeof c);
  c.kind = kind;
  c.mode = mode;
  c.batch = 4;
  c.n_qk_heads = 2;
  c.n_v_heads = 4;
  c.head_k_dim = 128;
  c.head_v_dim = 128;
  c.ring = 16;
  c.max_draft = 4;
  c.in_dtype = RS_BF16;
  c.ckpt_dtype = RS_F32;
  return c;
}

int main(void) {
  const int M2[STUB_KINDS] = {1, 0, 0, 0, 0, 0, 0, 0};
  const int GD[STUB_KINDS] = {0, 1, 0, 0, 0, 0, 0, 0};
  const int M2C[STUB_KINDS] = {1, 0, 1, 0, 0, 0, 0, 0};
  const int GDC[STUB_KINDS] = {0, 1, 1, 0, 0, 0, 0, 0};
  const int M2S[STUB_KINDS] = {1, 0, 1, 0, 0, 0, 0, 1};
  const int RST[STUB_KINDS] = {0, 0, 0, 1, 0, 0, 0, 0};
  const int CPY[STUB_KINDS] = {0, 0, 0, 0, 1, 0, 0, 0};
  const int CNV[STUB_KINDS] = {0, 0, 0, 0, 0, 1, 0, 0};
  const int NRM[STUB_KINDS] = {0, 0, 0, 0, 0, 0, 1, 0};
  rs_stub_reset();

  /* ---- Mamba-2, replay mode, fp32 checkpoint with an NVFP4 read copy ---- */
  rs_config c = m2_cfg(RS_REPLAY);
  rs_layer L;
  expect(rs_init(&c, &L) == RS_OK, "mamba2 replay layer");
  rs_buffers buf = {dev(1), dev(2), dev(3), dev(4), NULL};
  rs_inputs in;
  memset(&in, 0, sizeof in);
  in.x = dev(5); in.B = dev(6); in.C = dev(7); in.dt = dev(8);
  rs_params prm = {(const float*)dev(9), (const float*)dev(10)};
  float* y = (float*)dev(11);
  int32_t* acc = (int32_t*)dev(12);
  {
    SNAP(b); expect_call(rs_step_nonflush(&L, &buf, &in, &prm, y, NULL), RS_OK, M2, b, "nonflush dispatches");
  }
  {
    SNAP(b); expect_call(rs_step_flush(&L, &buf, &in, &prm, y, NULL), RS_OK, M2, b, "flush dispatches");
  }
  {
    SNAP(b); expect_call(rs_step(&L, &buf, &in, &prm, y, NULL), RS_OK, M2, b, "self-scheduling step dispatches");
  }
  {
    SNAP(b); expect_call(rs_spec_append(&L, &buf, &in, 4, &prm, y, NULL), RS_OK, M2, b, "append of 4 drafts");
  }
  {
    SNAP(b); expect_call(rs_spec_commit(&L, &buf, acc, &prm, NULL), RS_OK, M2C, b, "commit: counters, then fold");
  }
  {
    SNAP(b); expect_call(rs_spec_commit_static(&L, &buf, acc, &prm, NULL), RS_OK, M2S, b,
                         "commit with the static fold list");
  }
  {
    rs_config big = c;
    big.batch = 8193;
    rs_layer LB;
    expect(rs_init(&big, &LB) == RS_OK, "a layer of 8193 sequences");
    SNAP(b); expect_call(rs_spec_commit_static(&LB, &buf, acc, &prm, NULL), RS_E_ARG, NULL, b,
                         "static fold list refused beyond 8192 sequences");
  }
  {
    SNAP(b); expect_call(rs_requant_read_copy(&L, &buf, NULL), RS_OK, M2, b, "requant dispatches");
  }
  {
    SNAP(b); expect_call(rs_step_conventional(&L, &buf, &in, &prm, y, NULL), RS_E_MODE, NULL, b,
                         "conventional step refused in replay mode");
  }
  {
    SNAP(b); expect_call(rs_spec_append(&L, &buf, &in, 5, &prm, y, NULL), RS_E_ARG, NULL, b, "5 drafts > max_draft");
  }
  {
    SNAP(b); expect_call(rs_spec_append(&L, &buf, &in, 0, &prm, y, NULL), RS_E_ARG, NULL, b, "0 drafts");
  }
  {
    SNAP(b); expect_call(rs_step_nonflush(&L, &buf, &in, &prm, (float*)((char*)y + 4), NULL), RS_E_ALIGN, NULL, b,
                         "misaligned output");
  }
  {
    rs_inputs bad = in;
    bad.B = (const char*)in.B + 8;
    SNAP(b); expect_call(rs_step_flush(&L, &buf, &bad, &prm, y, NULL), RS_E_ALIGN, NULL, b, "misaligned input");
  }
  {
    rs_inputs bad = in;
    bad.dt = NULL;
    SNAP(b); expect_call(rs_step_nonflush(&L, &buf, &bad, &prm, y, NULL), RS_E_ARG, NULL, b, "missing input");
  }
  {
    rs_buffers nb = buf;
    nb.read_copy = NULL;
    SNAP(b); expect_call(rs_step_nonflush(&L, &nb, &in, &prm, y, NULL), RS_E_ARG, NULL, b, "missing read copy");
  }
  {
    rs_buffers nb = buf;
    nb.meta = NULL;
    SNAP(b); expect_call(rs_spec_commit(&L, &nb, acc, &prm, NULL), RS_E_ARG, NULL, b, "commit without meta");
  }
  {
    rs_params np = {NULL, prm.D};
    SNAP(b); expect_call(rs_spec_commit(&L, &buf, acc, &np, NULL), RS_E_ARG, NULL, b, "commit without A");
  }
  {
    rs_layer junk = L;
    junk.magic = 0;
    SNAP(b); expect_call(rs_step_flush(&junk, &buf, &in, &prm, y, NULL), RS_E_ARG, NULL, b, "layer not from rs_init");
  }
  {
    int32_t* seqs = (int32_t*)dev(13);
    SNAP(b); expect_call(rs_reset_slots(&L, &buf, seqs, 2, NULL), RS_OK, RST, b, "reset of 2 slots");
  }
  {
    SNAP(b); expect_call(rs_reset_slots(&L, &buf, (int32_t*)dev(13), 0, NULL), RS_OK, NULL, b, "reset of none");
  }
  {
    SNAP(b); expect_call(rs_reset_slots(&L, &buf, (int32_t*)dev(13), -1, NULL), RS_E_ARG, NULL, b, "negative count");
  }
  {
    rs_config c8 = c;
    c8.batch = 8;
    rs_layer L8;
    expect(rs_init(&c8, &L8) == RS_OK, "a cache layer of 8 sequences");
    rs_buffers cache = {dev(20), dev(21), dev(22), dev(23), NULL};
    const int32_t* s = (const int32_t*)dev(24);
    const int32_t* d = (const int32_t*)dev(25);
    SNAP(b); expect_call(rs_copy_slots(&L, &buf, s, &L8, &cache, d, 3, NULL), RS_OK, CPY, b, "copy into the cache");
    rs_config cx = c8;
    cx.read_copy = RS_NONE;
    rs_layer LX;
    expect(rs_init(&cx, &LX) == RS_OK, "a layer without read copy");
    SNAP(b2); expect_call(rs_copy_slots(&L, &buf, s, &LX, &cache, d, 3, NULL), RS_E_ARG, NULL, b2,
                          "copy between different configurations");
    SNAP(b3); expect_call(rs_copy_slots(&L, &buf, s, &L8, &cache, d, 65536, NULL), RS_E_ARG, NULL, b3,
                          "copy count over 65535");
  }
  {
    void* ring = dev(30);
    SNAP(b); expect_call(rs_conv_step(&L, &buf, ring, dev(31), 1, (const float*)dev(32), NULL, 4, dev(33), dev(34),
                                      dev(35), NULL), RS_OK, CNV, b, "short convolution");
    SNAP(b2); expect_call(rs_conv_step(&L, &buf, ring, dev(31), 1, (const float*)dev(32), NULL, 5, dev(33), dev(34),
                                       dev(35), NULL), RS_E_ARG, NULL, b2, "convolution width 5");
    SNAP(b3); expect_call(rs_conv_step(&L, &buf, ring, dev(31), 5, (const float*)dev(32), NULL, 4, dev(33), dev(34),
                                       dev(35), NULL), RS_E_ARG, NULL, b3, "convolution of 5 drafts");
  }
  {
    SNAP(b); expect_call(rs_gated_norm(&L, 1, y, dev(40), (const float*)dev(41), 8, 1e-5f, dev(42), NULL), RS_OK,
                         NRM, b, "gated norm, 8 groups");
    SNAP(b2); expect_call(rs_gated_norm(&L, 1, y, dev(40), (const float*)dev(41), 3, 1e-5f, dev(42), NULL), RS_E_ARG,
                          NULL, b2, "gated norm, groups not dividing d_inner");
    SNAP(b3); expect_call(rs_gated_norm(&L, 1, y, dev(40), (const float*)dev(41), 8, -1.0f, dev(42), NULL), RS_E_ARG,
                          NULL, b3, "gated norm, negative eps");
  }

  /* ---- Mamba-2, conventional mode (the snapshot baseline) ---- */
  {
    rs_config cc = m2_cfg(RS_CONVENTIONAL);
    rs_layer LC;
    expect(rs_init(&cc, &LC) == RS_OK, "mamba2 conventional layer");
    expect(LC.snap_bytes == 4ull * 4 * 128 * 128 * 64 * 4, "snapshot bytes");
    rs_buffers cb = {dev(50), NULL, NULL, NULL, dev(51)};
    SNAP(b); expect_call(rs_step_conventional(&LC, &cb, &in, &prm, y, NULL), RS_OK, M2, b, "conventional step");
    SNAP(b2); expect_call(rs_step_nonflush(&LC, &cb, &in, &prm, y, NULL), RS_E_MODE, NULL, b2,
                          "non-flush refused in conventional mode");
    SNAP(b3); expect_call(rs_spec_append(&LC, &cb, &in, 4, &prm, y, NULL), RS_OK, M2, b3, "snapshot append");
    SNAP(b4); expect_call(rs_spec_commit(&LC, &cb, acc, &prm, NULL), RS_OK, M2, b4, "snapshot restore");
    rs_buffers nosnap = cb;
    nosnap.snap = NULL;
    SNAP(b5); expect_call(rs_spec_append(&LC, &nosnap, &in, 4, &prm, y, NULL), RS_E_ARG, NULL, b5,
                          "snapshot append without snapshots");
  }

  /* ---- Gated DeltaNet and KDA ---- */
  for (int kind = RS_GDN; kind <= RS_KDA; ++kind) {
    rs_config cg = delta_cfg(kind, RS_REPLAY);
    rs_layer G;
    expect(rs_init(&cg, &G) == RS_OK, kind == RS_GDN ? "gdn replay layer" : "kda replay layer");
    rs_buffers gb = {dev(60), dev(61), NULL, dev(62), NULL};
    rs_inputs gi;
    memset(&gi, 0, sizeof gi);
    gi.q = dev(63); gi.k = dev(64); gi.v = dev(65); gi.g = dev(66); gi.beta = dev(67);
    SNAP(b); expect_call(rs_step_nonflush(&G, &gb, &gi, NULL, y, NULL), RS_OK, GD, b, "delta-rule non-flush");
    SNAP(b2); expect_call(rs_step_flush(&G, &gb, &gi, NULL, y, NULL), RS_OK, GD, b2, "delta-rule flush");
    SNAP(b3); expect_call(rs_step(&G, &gb, &gi, NULL, y, NULL), RS_OK, GD, b3, "delta-rule self-scheduling step");
    SNAP(b4); expect_call(rs_spec_append(&G, &gb, &gi, 3, NULL, y, NULL), RS_OK, GD, b4, "delta-rule append");
    SNAP(b5); expect_call(rs_spec_commit(&G, &gb, acc, NULL, NULL), RS_OK, GDC, b5, "delta-rule commit");
    SNAP(b6); expect_call(rs_requant_read_copy(&G, &gb, NULL), RS_E_MODE, NULL, b6, "delta-rule requant refused");
    SNAP(b7); expect_call(rs_gated_norm(&G, 1, y, dev(40), (const float*)dev(41), 8, 1e-5f, dev(42), NULL),
                          RS_E_MODE, NULL, b7, "gated norm refused for a delta-rule layer");
    rs_inputs nb = gi;
    nb.beta = NULL;
    SNAP(b8); expect_call(rs_step_nonflush(&G, &gb, &nb, NULL, y, NULL), RS_E_ARG, NULL, b8, "missing beta");
  }

  /* ---- Gated DeltaNet and KDA with the NVFP4 read copy: the flush and the
   * commit fold write the copy themselves; the self-scheduling step is
   * followed by the copy's requant ---- */
  {
    const int GD2[STUB_KINDS] = {0, 2, 0, 0, 0, 0, 0, 0};
    for (int kind = RS_GDN; kind <= RS_KDA; ++kind) {
      rs_config cg = delta_cfg(kind, RS_REPLAY);
      cg.read_copy = RS_NVFP4;
      rs_layer G;
      expect(rs_init(&cg, &G) == RS_OK, "delta-rule layer with a read copy");
      expect(G.read_copy_bytes >= 4ull * 4 * (128 * 128 / 2 + 128 * 128 / 16 + 4), "delta-rule read copy bytes");
      rs_buffers gb = {dev(70), dev(71), dev(72), dev(73), NULL};
      rs_inputs gi;
      memset(&gi, 0, sizeof gi);
      gi.q = dev(74); gi.k = dev(75); gi.v = dev(76); gi.g = dev(77); gi.beta = dev(78);
      SNAP(b); expect_call(rs_step_nonflush(&G, &gb, &gi, NULL, y, NULL), RS_OK, GD, b, "non-flush reads the copy");
      SNAP(b2); expect_call(rs_step_flush(&G, &gb, &gi, NULL, y, NULL), RS_OK, GD, b2, "flush writes the copy");
      SNAP(b3); expect_call(rs_step(&G, &gb, &gi, NULL, y, NULL), RS_OK, GD2, b3, "self-scheduling step, then requant");
      SNAP(b4); expect_call(rs_spec_append(&G, &gb, &gi, 4, NULL, y, NULL), RS_OK, GD, b4, "append reads the copy");
      SNAP(b5); expect_call(rs_spec_commit(&G, &gb, acc, NULL, NULL), RS_OK, GDC, b5, "commit: counters, then the fold with the copy");
      SNAP(b6); expect_call(rs_requant_read_copy(&G, &gb, NULL), RS_OK, GD, b6, "delta-rule requant");
      rs_buffers nb = gb;
      nb.read_copy = NULL;
      SNAP(b7); expect_call(rs_step_nonflush(&G, &nb, &gi, NULL, y, NULL), RS_E_ARG, NULL, b7, "missing read copy");
      SNAP(b8); expect_call(rs_spec_commit(&G, &nb, acc, NULL, NULL), RS_E_ARG, NULL, b8, "commit without read copy");
      rs_config cc = delta_cfg(kind, RS_CONVENTIONAL);
      cc.read_copy = RS_NVFP4;
      rs_layer X;
      expect(rs_init(&cc, &X) == RS_E_DTYPE, "read copy refused in conventional mode");
    }
  }

  /* ---- rs_init refusals ---- */
  {
    rs_config bad = m2_cfg(RS_REPLAY);
    rs_layer X;
    bad.dstate = 96;
    expect(rs_init(&bad, &X) == RS_E_UNSUPPORTED, "uncompiled state shape");
    bad = m2_cfg(RS_REPLAY);
    bad.ckpt_dtype = RS_NVFP4;
    expect(rs_init(&bad, &X) == RS_E_DTYPE, "uniform NVFP4 checkpoint with a read copy");
    bad = m2_cfg(RS_REPLAY);
    bad.nheads = 100;
    expect(rs_init(&bad, &X) == RS_E_ARG, "heads not a multiple of groups");
    bad = m2_cfg(RS_REPLAY);
    bad.max_draft = 9;
    expect(rs_init(&bad, &X) == RS_E_ARG, "max_draft over 8");
    expect(rs_init(NULL, &X) == RS_E_ARG && rs_init(&bad, NULL) == RS_E_ARG, "null arguments");
  }
  printf("%d failed\n", fails);
  return fails != 0;
}
