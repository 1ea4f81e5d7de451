"""GPU parity of the Gated DeltaNet decode path (conventional, and ReplaySSM in
UT form) against the fp64 oracle; buffer counters and ring slots bit-exact."""
import numpy as np
import pytest
import torch

import ssm_decode_checkpoint_amd as rs
import workloads as W
from oracle import decode
from oracle.ring import RingModel
from gpu_harness import (gdn_layer, gdn_tok_dev, load_state_f32, read_meta, read_state_f32, rel_l2, require_gpu,
                         y_buf)

pytestmark = pytest.mark.gpu


def setup_module(_):
    require_gpu()


def _bits(t):
    t = t.cpu()
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)).numpy()


def _in_bits(arr, in_dtype):
    arr = np.ascontiguousarray(arr, dtype=np.float32)
    return W.bf16_bits(arr).view(np.int16) if in_dtype == "bf16" else arr.view(np.int32)


def _init(w, std):
    return W.gdn_init_states(w.with_(init_std=std), range(w.batch))


@pytest.mark.parametrize("std", [0.0, 0.5])
def test_tiny_conventional(std):
    w = W.TINY_GDN
    gp = W.gdn_params(w)
    S0 = _init(w, std)
    layer, bufs = gdn_layer(w, mode=rs.RS_CONVENTIONAL)
    load_state_f32(layer, bufs, S0)
    ref = decode.GDNConventional(S0)
    worst = 0.0
    for t in range(w.steps):
        tok = W.gdn_step(w, t, range(w.batch), gp)
        o = y_buf(w.batch, w.n_v, w.dv)
        rs.rs_step_conventional(layer, bufs, gdn_tok_dev(tok, w.in_dtype), None, None, o)
        worst = max(worst, rel_l2(o.cpu().numpy(), ref.step(tok)))
    assert worst <= 1e-5, worst
    assert rel_l2(read_state_f32(layer, bufs), ref.S) <= 1e-5


@pytest.mark.parametrize("std", [0.0, 0.5])
def test_tiny_replay(std):
    w = W.TINY_GDN
    gp = W.gdn_params(w)
    S0 = _init(w, std)
    layer, bufs = gdn_layer(w)
    load_state_f32(layer, bufs, S0)
    ref = decode.GDNConventional(S0)
    model = RingModel(w.batch)
    slot_tok = [dict() for _ in range(w.batch)]
    toks = []
    worst = 0.0
    for t in range(w.steps):
        tok = W.gdn_step(w, t, range(w.batch), gp)
        toks.append(tok)
        o = y_buf(w.batch, w.n_v, w.dv)
        if model.is_flush_step(0):
            rs.rs_step_flush(layer, bufs, gdn_tok_dev(tok, w.in_dtype), None, None, o)
            for b in range(w.batch):
                model.flush(b)
        else:
            rs.rs_step_nonflush(layer, bufs, gdn_tok_dev(tok, w.in_dtype), None, None, o)
            for b in range(w.batch):
                slot_tok[b][model.nonflush(b)] = t
        worst = max(worst, rel_l2(o.cpu().numpy(), ref.step(tok)))
        nck, ln, nd, err, arrive = read_meta(layer, bufs)
        assert list(nck) == model.n_ckpt and list(ln) == model.len and not err.any() and not arrive.any()
        rings = {n: _bits(rs.ring_view(layer, bufs, n)) for n in ("q", "k", "v", "g", "beta")}
        for b in range(w.batch):
            for s in model.live_slots(b):
                tk = toks[slot_tok[b][s]]
                for n in ("q", "k", "v"):
                    assert np.array_equal(rings[n][b, :, s], _in_bits(tk[n][b], w.in_dtype)), (t, b, s, n)
                for n in ("g", "beta"):
                    assert np.array_equal(rings[n][b, :, s], tk[n][b].astype(np.float32).view(np.int32))
        if t % 16 == 15:
            assert rel_l2(read_state_f32(layer, bufs), ref.S) <= 1e-5
    assert worst <= 1e-5, worst


@pytest.mark.parametrize("fill", [0, 4, 13])
def test_flush_at_any_fill(fill):
    w = W.TINY_GDN
    gp = W.gdn_params(w)
    S0 = _init(w, 0.5)
    layer, bufs = gdn_layer(w)
    load_state_f32(layer, bufs, S0)
    ref = decode.GDNConventional(S0)
    model = RingModel(w.batch)
    worst = 0.0
    for t in range(36):
        tok = W.gdn_step(w, t, range(w.batch), gp)
        o = y_buf(w.batch, w.n_v, w.dv)
        if t == fill or model.is_flush_step(0):
            rs.rs_step_flush(layer, bufs, gdn_tok_dev(tok, w.in_dtype), None, None, o)
            for b in range(w.batch):
                model.flush(b)
        else:
            rs.rs_step_nonflush(layer, bufs, gdn_tok_dev(tok, w.in_dtype), None, None, o)
            for b in range(w.batch):
                model.nonflush(b)
        worst = max(worst, rel_l2(o.cpu().numpy(), ref.step(tok)))
    assert worst <= 1e-5, worst


def test_qwen_batch256_sampled():
    """256 sequences x 32 value heads of 128 x 128 fp32 state, bf16 q/k/v: all on
    the GPU; 8 sequences spread over the batch checked against the oracle over
    two windows, for both the ReplaySSM path and the conventional kernel."""
    w = W.GDN_QWEN
    steps = 32
    gp = W.gdn_params(w)
    seqs = list(range(0, 256, 37))
    S0 = W.gdn_init_states(w, range(w.batch))
    rl, rb = gdn_layer(w)
    load_state_f32(rl, rb, S0)
    cl, cb = gdn_layer(w, mode=rs.RS_CONVENTIONAL)
    load_state_f32(cl, cb, S0)
    ref = decode.GDNConventional(S0[seqs])
    model = RingModel(w.batch)
    worst_r = worst_c = 0.0
    for t in range(steps):
        tok = W.gdn_step(w, t, range(w.batch), gp)
        d = gdn_tok_dev(tok, w.in_dtype)
        o = y_buf(w.batch, w.n_v, w.dv)
        oc = y_buf(w.batch, w.n_v, w.dv)
        if model.is_flush_step(0):
            rs.rs_step_flush(rl, rb, d, None, None, o)
            for b in range(w.batch):
                model.flush(b)
        else:
            rs.rs_step_nonflush(rl, rb, d, None, None, o)
            for b in range(w.batch):
                model.nonflush(b)
        rs.rs_step_conventional(cl, cb, d, None, None, oc)
        orf = ref.step({k: v[seqs] for k, v in tok.items()})
        worst_r = max(worst_r, rel_l2(o.cpu().numpy()[seqs], orf))
        worst_c = max(worst_c, rel_l2(oc.cpu().numpy()[seqs], orf))
    print(f"gdn b256: replay max rel-L2 {worst_r:.3e}, conventional {worst_c:.3e}")
    assert worst_r <= 2e-3 and worst_c <= 2e-3
    assert worst_r <= 1e-5 and worst_c <= 1e-5
    nck, ln, nd, err, arrive = read_meta(rl, rb)
    assert (nck == 32).all() and (ln == 0).all() and not err.any() and not arrive.any()
    assert rel_l2(read_state_f32(rl, rb, seqs), ref.S) <= 1e-5


def test_error_bits_leave_state_unchanged_then_flush():
    """dk = dv = 128 (two column slices per state). A non-flush step on a full
    buffer is refused for every sequence: sticky RS_ERR_FULL, outputs not
    written, checkpoint and ring untouched, counters as they were. The flush
    that follows folds the 16 accepted tokens as if the refused one never came."""
    w = W.TINY_GDN.with_(batch=3, n_qk=2, n_v=4, dk=128, dv=128, init_std=0.3, seed=97)
    gp = W.gdn_params(w)
    S0 = W.gdn_init_states(w, range(w.batch))
    layer, bufs = gdn_layer(w)
    load_state_f32(layer, bufs, S0)
    ref = decode.GDNConventional(S0)
    for t in range(15):
        tok = W.gdn_step(w, t, range(w.batch), gp)
        o = y_buf(w.batch, w.n_v, w.dv)
        rs.rs_step_nonflush(layer, bufs, gdn_tok_dev(tok, w.in_dtype), None, None, o)
        assert rel_l2(o.cpu().numpy(), ref.step(tok)) <= 1e-5
    ck, ring = bufs.ckpt.clone(), bufs.ring.clone()
    o = y_buf(w.batch, w.n_v, w.dv)
    rs.rs_step_nonflush(layer, bufs, gdn_tok_dev(W.gdn_step(w, 99, range(w.batch), gp), w.in_dtype), None, None, o)
    nck, ln, nd, err, arrive = read_meta(layer, bufs)
    assert (err == rs.RS_ERR_FULL).all() and (ln == 15).all() and (nck == 0).all() and not arrive.any()
    assert torch.isnan(o).all()
    assert torch.equal(ck, bufs.ckpt) and torch.equal(ring, bufs.ring)
    tok = W.gdn_step(w, 15, range(w.batch), gp)
    o = y_buf(w.batch, w.n_v, w.dv)
    rs.rs_step_flush(layer, bufs, gdn_tok_dev(tok, w.in_dtype), None, None, o)
    assert rel_l2(o.cpu().numpy(), ref.step(tok)) <= 1e-5
    nck, ln, nd, err, arrive = read_meta(layer, bufs)
    assert (err == rs.RS_ERR_FULL).all() and (ln == 0).all() and (nck == 16).all() and not arrive.any()
    assert rel_l2(read_state_f32(layer, bufs), ref.S) <= 1e-5
