"""GPU parity of the Mamba-2 decode path against the fp64 oracle.

Floating point: rel-L2 of y per step (over all sequences, heads and headdim)
<= 1e-5 on fp32-input paths and <= 2e-3 on bf16-input paths (the oracle
consumes the same bf16-rounded inputs, so the GPU's error is its fp32
arithmetic only). Integer state: per-sequence counters and every held ring
slot are compared bit for bit with the oracle's buffer model and the inputs.
"""
import numpy as np
import pytest
import torch

import ssm_decode_checkpoint_amd as rs
import workloads as W
from oracle import decode
from oracle.ring import RingModel
from gpu_harness import (dev_in, load_state_f32, m2_layer, m2_tok_dev, params_dev, read_meta, read_state_f32,
                         rel_l2, require_gpu, y_buf, m2_drafts_dev)

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-3}


def setup_module(_):
    require_gpu()


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)).numpy()


def _in_bits(arr, in_dtype):
    arr = np.ascontiguousarray(arr, dtype=np.float32)
    return W.bf16_bits(arr).view(np.int16) if in_dtype == "bf16" else arr.view(np.int32)


class RingCheck:
    """Expected ring contents: which token each held slot must carry."""

    def __init__(self, w, batch):
        self.w = w
        self.model = RingModel(batch, max_draft=w.max_draft)
        self.slot_tok = [dict() for _ in range(batch)]

    def check(self, layer, bufs, tokens):
        nck, ln, nd, err, arrive = read_meta(layer, bufs)
        m = self.model
        assert list(nck) == m.n_ckpt and list(ln) == m.len and list(nd) == m.nd and list(err) == m.err
        assert not arrive.any()
        rx = _bits(rs.ring_view(layer, bufs, "x"))
        rB = _bits(rs.ring_view(layer, bufs, "B"))
        rC = _bits(rs.ring_view(layer, bufs, "C"))
        rdt = _bits(rs.ring_view(layer, bufs, "dt"))
        for b in range(len(m.len)):
            for s in m.live_slots(b):
                tk, bi = self.slot_tok[b][s]
                tok = tokens[tk]
                assert np.array_equal(rx[b, :, s], _in_bits(tok["x"][bi], self.w.in_dtype))
                assert np.array_equal(rB[b, :, s], _in_bits(tok["B"][bi], self.w.in_dtype))
                assert np.array_equal(rC[b, :, s], _in_bits(tok["C"][bi], self.w.in_dtype))
                assert np.array_equal(rdt[b, :, s], _in_bits(tok["dt"][bi], self.w.in_dtype))


def _init(w, std=None):
    w2 = w if std is None else w.with_(init_std=std)
    return W.m2_init_states(w2, range(w.batch))


@pytest.mark.parametrize("std", [0.0, 0.5])
def test_tiny_conventional(std):
    w = W.TINY_M2
    p = W.m2_params(w)
    A, D = params_dev(p)
    H0 = _init(w, std)
    layer, bufs = m2_layer(w, mode=rs.RS_CONVENTIONAL, max_draft=0)
    load_state_f32(layer, bufs, H0)
    ref = decode.M2Conventional(H0, p["A"], p["D"])
    worst = 0.0
    for t in range(w.steps):
        tok = W.m2_step(w, t, range(w.batch))
        y = y_buf(w.batch, w.nheads, w.headdim)
        rs.rs_step_conventional(layer, bufs, m2_tok_dev(tok, w.in_dtype), A, D, y)
        worst = max(worst, rel_l2(y.cpu().numpy(), ref.step(tok)))
    assert worst <= TOL["f32"], worst
    assert rel_l2(read_state_f32(layer, bufs), ref.H) <= TOL["f32"]


@pytest.mark.parametrize("std", [0.0, 0.5])
def test_tiny_replay(std):
    """64 steps from an empty buffer: 4 windows, flushes at t = 15, 31, 47, 63."""
    w = W.TINY_M2
    p = W.m2_params(w)
    A, D = params_dev(p)
    H0 = _init(w, std)
    layer, bufs = m2_layer(w)
    load_state_f32(layer, bufs, H0)
    ref = decode.M2Conventional(H0, p["A"], p["D"])
    rc = RingCheck(w, w.batch)
    tokens, worst, flushes = [], 0.0, []
    for t in range(w.steps):
        tok = W.m2_step(w, t, range(w.batch))
        tokens.append(tok)
        y = y_buf(w.batch, w.nheads, w.headdim)
        flush = rc.model.is_flush_step(0)
        if flush:
            rs.rs_step_flush(layer, bufs, m2_tok_dev(tok, w.in_dtype), A, D, y)
            for b in range(w.batch):
                rc.model.flush(b)
            flushes.append(t)
        else:
            rs.rs_step_nonflush(layer, bufs, m2_tok_dev(tok, w.in_dtype), A, D, y)
            for b in range(w.batch):
                rc.slot_tok[b][rc.model.nonflush(b)] = (t, b)
        yr = ref.step(tok)
        worst = max(worst, rel_l2(y.cpu().numpy(), yr))
        rc.check(layer, bufs, tokens)
        if flush:
            assert rel_l2(read_state_f32(layer, bufs), ref.H) <= TOL["f32"]
    assert flushes == [15, 31, 47, 63]
    assert worst <= TOL["f32"], worst


@pytest.mark.parametrize("fill", [0, 1, 6, 14])
def test_flush_at_any_fill(fill):
    w = W.TINY_M2
    p = W.m2_params(w)
    A, D = params_dev(p)
    H0 = _init(w, 0.5)
    layer, bufs = m2_layer(w)
    load_state_f32(layer, bufs, H0)
    ref = decode.M2Conventional(H0, p["A"], p["D"])
    model = RingModel(w.batch)
    worst = 0.0
    for t in range(40):
        tok = W.m2_step(w, t, range(w.batch))
        y = y_buf(w.batch, w.nheads, w.headdim)
        if t == fill or model.is_flush_step(0):
            rs.rs_step_flush(layer, bufs, m2_tok_dev(tok, w.in_dtype), A, D, y)
            for b in range(w.batch):
                model.flush(b)
        else:
            rs.rs_step_nonflush(layer, bufs, m2_tok_dev(tok, w.in_dtype), A, D, y)
            for b in range(w.batch):
                model.nonflush(b)
        worst = max(worst, rel_l2(y.cpu().numpy(), ref.step(tok)))
    nck, ln, *_ = read_meta(layer, bufs)
    assert list(nck) == model.n_ckpt and list(ln) == model.len
    assert worst <= TOL["f32"], worst


def _run_replay(w, layer, bufs, A, D, steps, t0=0, model=None):
    model = model or RingModel(layer.cfg.batch)
    ys = []
    for t in range(t0, t0 + steps):
        tok = W.m2_step(w, t, range(layer.cfg.batch))
        y = y_buf(layer.cfg.batch, w.nheads, w.headdim)
        if model.is_flush_step(0):
            rs.rs_step_flush(layer, bufs, m2_tok_dev(tok, w.in_dtype), A, D, y)
            for b in range(layer.cfg.batch):
                model.flush(b)
        else:
            rs.rs_step_nonflush(layer, bufs, m2_tok_dev(tok, w.in_dtype), A, D, y)
            for b in range(layer.cfg.batch):
                model.nonflush(b)
        ys.append(y.cpu().numpy())
    return ys, model


def test_determinism_and_resume():
    """Bit-identical outputs on a rerun, and after copying (checkpoint, ring, meta)
    into fresh buffers mid-window."""
    w = W.TINY_M2
    p = W.m2_params(w)
    A, D = params_dev(p)
    H0 = _init(w, 0.5)
    l1, b1 = m2_layer(w)
    load_state_f32(l1, b1, H0)
    ys1, _ = _run_replay(w, l1, b1, A, D, 40)
    l2, b2 = m2_layer(w)
    load_state_f32(l2, b2, H0)
    ys2a, model = _run_replay(w, l2, b2, A, D, 21)
    b3 = rs.alloc_buffers(l2)
    for name in ("ckpt", "ring", "meta"):
        getattr(b3, name).copy_(getattr(b2, name))
    ys2b, _ = _run_replay(w, l2, b3, A, D, 19, t0=21, model=model)
    for a, b in zip(ys1, ys2a + ys2b):
        assert np.array_equal(a.view(np.int32), b.view(np.int32))


def test_nemotron_batch256_sampled():
    """The 256 x 128-head, 64 x 128 bf16 layer: every sequence runs on the GPU;
    16 sequences spread over the batch are checked against the oracle for two
    full windows (30 non-flush steps and 2 flushes)."""
    w = W.M2_NEMOTRON
    steps = 32
    p = W.m2_params(w)
    A, D = params_dev(p)
    seqs = list(range(0, 256, 17))
    H0 = W.m2_init_states(w, range(w.batch))
    layer, bufs = m2_layer(w)
    load_state_f32(layer, bufs, H0)
    conv_l, conv_b = m2_layer(w, mode=rs.RS_CONVENTIONAL, max_draft=0)
    load_state_f32(conv_l, conv_b, H0)
    ref = decode.M2Conventional(H0[seqs], p["A"], p["D"])
    model = RingModel(w.batch)
    worst_r = worst_c = 0.0
    for t in range(steps):
        tok = W.m2_step(w, t, range(w.batch))
        dtok = m2_tok_dev(tok, w.in_dtype)
        y = y_buf(w.batch, w.nheads, w.headdim)
        yc = y_buf(w.batch, w.nheads, w.headdim)
        if model.is_flush_step(0):
            rs.rs_step_flush(layer, bufs, dtok, A, D, y)
            for b in range(w.batch):
                model.flush(b)
        else:
            rs.rs_step_nonflush(layer, bufs, dtok, A, D, y)
            for b in range(w.batch):
                model.nonflush(b)
        rs.rs_step_conventional(conv_l, conv_b, dtok, A, D, yc)
        yr = ref.step({k: v[seqs] for k, v in tok.items()})
        worst_r = max(worst_r, rel_l2(y.cpu().numpy()[seqs], yr))
        worst_c = max(worst_c, rel_l2(yc.cpu().numpy()[seqs], yr))
    print(f"nemotron b256: replay max rel-L2 {worst_r:.3e}, conventional {worst_c:.3e}")
    assert worst_r <= TOL["bf16"] and worst_c <= TOL["bf16"]
    assert worst_r <= 1e-5 and worst_c <= 1e-5     # fp32 arithmetic on exact bf16 inputs
    nck, ln, nd, err, arrive = read_meta(layer, bufs)
    assert (nck == 32).all() and (ln == 0).all() and not err.any() and not arrive.any()
    st = read_state_f32(layer, bufs, seqs)
    assert rel_l2(st, ref.H) <= 1e-5


def test_device_error_bits_leave_state_unchanged():
    w = W.TINY_M2.with_(max_draft=4)
    p = W.m2_params(w)
    A, D = params_dev(p)
    H0 = _init(w, 0.5)
    layer, bufs = m2_layer(w)
    load_state_f32(layer, bufs, H0)
    _run_replay(w, layer, bufs, A, D, 15)       # len = 15: the buffer is full
    ck = bufs.ckpt.clone()
    ring = bufs.ring.clone()
    y = y_buf(w.batch, w.nheads, w.headdim)
    rs.rs_step_nonflush(layer, bufs, m2_tok_dev(W.m2_step(w, 99, range(w.batch)), w.in_dtype), A, D, y)
    nck, ln, nd, err, arrive = read_meta(layer, bufs)
    assert (err == rs.RS_ERR_FULL).all() and (ln == 15).all() and not arrive.any()
    assert torch.isnan(y).all()
    assert torch.equal(ck, bufs.ckpt) and torch.equal(ring, bufs.ring)
    # appending drafts to a full buffer overflows; committing more than pending is refused
    yd = y_buf(w.batch, w.nheads, w.headdim, K=4)
    drafts = [W.m2_step(w, 200 + d, range(w.batch)) for d in range(4)]
    rs.rs_spec_append(layer, bufs, m2_drafts_dev(drafts, w.in_dtype), 4, A, D, yd)
    _, ln, nd, err, _ = read_meta(layer, bufs)
    assert (err == rs.RS_ERR_FULL | rs.RS_ERR_OVERFLOW).all() and (nd == 0).all()
    acc = torch.full((w.batch,), 2, dtype=torch.int32, device="cuda")
    rs.rs_spec_commit(layer, bufs, acc, A, D)
    _, ln, nd, err, _ = read_meta(layer, bufs)
    assert (err & rs.RS_ERR_COMMIT).all() and (ln == 15).all()
    assert torch.equal(ck, bufs.ckpt)


def test_spec_pending_blocks_plain_steps():
    w = W.TINY_M2.with_(max_draft=4)
    p = W.m2_params(w)
    A, D = params_dev(p)
    layer, bufs = m2_layer(w)
    load_state_f32(layer, bufs, _init(w, 0.5))
    drafts = [W.m2_step(w, d, range(w.batch)) for d in range(3)]
    rs.rs_spec_append(layer, bufs, m2_drafts_dev(drafts, w.in_dtype), 3, A, D,
                      y_buf(w.batch, w.nheads, w.headdim, K=3))
    y = y_buf(w.batch, w.nheads, w.headdim)
    rs.rs_step_nonflush(layer, bufs, m2_tok_dev(W.m2_step(w, 50, range(w.batch)), w.in_dtype), A, D, y)
    rs.rs_step_flush(layer, bufs, m2_tok_dev(W.m2_step(w, 51, range(w.batch)), w.in_dtype), A, D, y)
    nck, ln, nd, err, _ = read_meta(layer, bufs)
    assert (err == rs.RS_ERR_PENDING).all() and (nd == 3).all() and (ln == 0).all() and (nck == 0).all()
    assert torch.isnan(y).all()
