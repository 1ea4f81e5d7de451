"""Unheld ring slots are never read.

Before every call, each ring slot of a sequence outside its held and pending
entries (slots (n_ckpt + i) mod 16 for i < len + nd) is filled with NaN in every
ring array: Mamba-2 x, B, C, dt; Gated DeltaNet and KDA q, k, v, g, beta and
the solved rows u (fp32 checkpoints with and without the NVFP4 read copy, FP16
and FP8 checkpoints). A twin layer runs
the same calls without poison. Outputs,
checkpoints, counters and the held slots must match bit for bit: a kernel that
touched an unheld slot, even to multiply it by zero, would carry a NaN into
them (sitech.ge ReplaySSM page, "How ReplaySSM works": a step reads the
checkpoint and the buffered entries only).
"""
import numpy as np
import pytest
import torch

import ssm_decode_checkpoint_amd as rs
import workloads as W
from gpu_harness import (gdn_drafts_dev, gdn_layer, gdn_tok_dev, load_state_f32, m2_drafts_dev, m2_layer, m2_tok_dev,
                         params_dev, read_meta, require_gpu, y_buf)
import lowprec_codes as LC

pytestmark = pytest.mark.gpu

M2_RING = ("x", "B", "C", "dt")
DELTA_RING = ("q", "k", "v", "g", "beta", "u")


def setup_module(_):
    require_gpu()


def _held(layer, bufs):
    nck, ln, nd, err, _ = read_meta(layer, bufs)
    held = np.zeros((layer.cfg.batch, 16), bool)
    for b in range(layer.cfg.batch):
        for i in range(int(ln[b]) + int(nd[b])):
            held[b, (int(nck[b]) + i) % 16] = True
    return held


def _names(layer):
    return M2_RING if layer.cfg.kind == rs.RS_MAMBA2 else DELTA_RING


def poison(layer, bufs):
    mask = torch.from_numpy(~_held(layer, bufs)).cuda()
    for n in _names(layer):
        v = rs.ring_view(layer, bufs, n)
        v.masked_fill_(mask.view(mask.shape[0], 1, 16, *([1] * (v.dim() - 3))), float("nan"))


def _bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


class Twin:
    """A poisoned and a clean layer driven by the same calls."""

    def __init__(self, make, load):
        self.p = make()
        self.c = make()
        for layer, bufs in (self.p, self.c):
            load(layer, bufs)
        self.calls = 0

    def call(self, fn, *out_shapes):
        """fn(layer, bufs, outs) on both layers; poison before the poisoned one's call."""
        poison(*self.p)
        outs_p = [y_buf(*s) for s in out_shapes]
        outs_c = [y_buf(*s) for s in out_shapes]
        fn(*self.p, outs_p)
        fn(*self.c, outs_c)
        self.calls += 1
        for a, b in zip(outs_p, outs_c):
            assert torch.isfinite(b).all()
            assert torch.equal(_bits(a), _bits(b)), f"call {self.calls}: outputs differ under poison"
        self.check()

    def check(self):
        (lp, bp), (lc, bc) = self.p, self.c
        assert torch.equal(bp.ckpt, bc.ckpt), f"call {self.calls}: checkpoint differs under poison"
        if bp.read_copy is not None:
            assert torch.equal(bp.read_copy, bc.read_copy)
        mp, mc = read_meta(lp, bp), read_meta(lc, bc)
        for a, b in zip(mp[:4], mc[:4]):
            assert np.array_equal(a, b)
        held = torch.from_numpy(_held(lc, bc)).cuda()
        for n in _names(lc):
            vp, vc = rs.ring_view(lp, bp, n), rs.ring_view(lc, bc, n)
            m = held.view(held.shape[0], 1, 16, *([1] * (vc.dim() - 3))).expand_as(vc)
            assert torch.equal(_bits(vp)[m], _bits(vc)[m]), f"call {self.calls}: held slots of ring {n} differ"


M2_CASES = [dict(), dict(batch=3, nheads=8, ngroups=2, dstate=128, headdim=64, in_dtype="bf16"),
            dict(batch=2, nheads=16, ngroups=1, dstate=128, headdim=64, in_dtype="bf16")]
M2_FORMATS = [(rs.RS_F32, rs.RS_NONE), (rs.RS_F32, rs.RS_NVFP4), (rs.RS_FP8E4M3, rs.RS_NONE)]


@pytest.mark.parametrize("ckpt,rc", M2_FORMATS)
@pytest.mark.parametrize("shape", M2_CASES)
def test_mamba2_decode_under_poison(shape, ckpt, rc):
    w = W.TINY_M2.with_(init_std=0.4, seed=180, **shape)
    p = W.m2_params(w)
    A, D = params_dev(p)
    H0 = W.m2_init_states(w, range(w.batch))

    def load(layer, bufs):
        if ckpt == rs.RS_F32:
            load_state_f32(layer, bufs, H0)
        if rc:
            rs.rs_requant_read_copy(layer, bufs)

    tw = Twin(lambda: m2_layer(w, ckpt_dtype=ckpt, read_copy=rc, fuse=1), load)
    yshape = (w.batch, w.nheads, w.headdim)
    for t in range(40):
        dtok = m2_tok_dev(W.m2_step(w, t, range(w.batch)), w.in_dtype)
        fn = rs.rs_step_flush if t % 16 == 15 else rs.rs_step_nonflush
        tw.call(lambda l, b, o: fn(l, b, dtok, A, D, o[0]), yshape)
    # the self-scheduling step, from a mid-window fill
    for t in range(40, 60):
        dtok = m2_tok_dev(W.m2_step(w, t, range(w.batch)), w.in_dtype)
        tw.call(lambda l, b, o: rs.rs_step(l, b, dtok, A, D, o[0]), yshape)


@pytest.mark.parametrize("shape", M2_CASES)
def test_mamba2_spec_under_poison(shape):
    w = W.TINY_M2.with_(init_std=0.4, seed=181, max_draft=4, **shape)
    p = W.m2_params(w)
    A, D = params_dev(p)
    H0 = W.m2_init_states(w, range(w.batch))
    tw = Twin(lambda: m2_layer(w), lambda l, b: load_state_f32(l, b, H0))
    K = 4
    for r in range(16):
        drafts = m2_drafts_dev([W.m2_step(w, 4000 + r * K + d, range(w.batch)) for d in range(K)], w.in_dtype)
        acc = torch.from_numpy(W.accepted_counts(w.seed, r, w.batch, K)).cuda()
        tw.call(lambda l, b, o: rs.rs_spec_append(l, b, drafts, K, A, D, o[0]), (w.batch, w.nheads, w.headdim, K))
        tw.call(lambda l, b, o: rs.rs_spec_commit(l, b, acc, A, D))


DELTA_CASES = [dict(), dict(batch=2, n_qk=2, n_v=4, dk=128, dv=128, in_dtype="bf16")]
# (checkpoint format, read copy): fp32 with and without the NVFP4 read copy, FP16 and FP8 checkpoints
DELTA_FORMATS = [(rs.RS_F32, rs.RS_NONE), (rs.RS_F32, rs.RS_NVFP4), (rs.RS_F16, rs.RS_NONE),
                 (rs.RS_FP8E4M3, rs.RS_NONE)]
_LC_FMT = {rs.RS_F16: "f16", rs.RS_FP8E4M3: "fp8"}


def _delta_load(S0, ckpt, rc):
    def load(layer, bufs):
        if ckpt == rs.RS_F32:
            load_state_f32(layer, bufs, S0)
        else:
            fmt = _LC_FMT[ckpt]
            enc = LC.encode(fmt, np.ascontiguousarray(np.swapaxes(np.asarray(S0, np.float32), -1, -2)))
            bufs.ckpt.copy_(torch.from_numpy(LC.to_device_bytes(layer, fmt, enc)).cuda())
        if rc:
            rs.rs_requant_read_copy(layer, bufs)
    return load


@pytest.mark.parametrize("ckpt,rc", DELTA_FORMATS)
@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("shape", DELTA_CASES)
def test_delta_decode_under_poison(shape, gate, ckpt, rc):
    base = W.TINY_GDN if gate == "scalar" else W.TINY_KDA
    w = base.with_(init_std=0.3, seed=182, **shape)
    gp = W.gdn_params(w)
    S0 = W.gdn_init_states(w, range(w.batch))
    tw = Twin(lambda: gdn_layer(w, read_copy=rc, ckpt_dtype=ckpt), _delta_load(S0, ckpt, rc))
    oshape = (w.batch, w.n_v, w.dv)
    for t in range(40):
        dtok = gdn_tok_dev(W.gdn_step(w, t, range(w.batch), gp), w.in_dtype)
        fn = rs.rs_step_flush if t % 16 == 15 else rs.rs_step_nonflush
        tw.call(lambda l, b, o: fn(l, b, dtok, None, None, o[0]), oshape)
    for t in range(40, 60):
        dtok = gdn_tok_dev(W.gdn_step(w, t, range(w.batch), gp), w.in_dtype)
        tw.call(lambda l, b, o: rs.rs_step(l, b, dtok, None, None, o[0]), oshape)


@pytest.mark.parametrize("ckpt,rc", DELTA_FORMATS)
@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("shape", DELTA_CASES)
def test_delta_spec_under_poison(shape, gate, ckpt, rc):
    base = W.TINY_GDN if gate == "scalar" else W.TINY_KDA
    w = base.with_(init_std=0.3, seed=183, max_draft=4, **shape)
    gp = W.gdn_params(w)
    S0 = W.gdn_init_states(w, range(w.batch))
    tw = Twin(lambda: gdn_layer(w, read_copy=rc, ckpt_dtype=ckpt), _delta_load(S0, ckpt, rc))
    K = 4
    for r in range(16):
        drafts = gdn_drafts_dev([W.gdn_step(w, 5000 + r * K + d, range(w.batch), gp) for d in range(K)], w.in_dtype)
        acc = torch.from_numpy(W.accepted_counts(w.seed, r, w.batch, K)).cuda()
        tw.call(lambda l, b, o: rs.rs_spec_append(l, b, drafts, K, None, None, o[0]), (w.batch, w.n_v, w.dv, K))
        tw.call(lambda l, b, o: rs.rs_spec_commit(l, b, acc, None, None))
