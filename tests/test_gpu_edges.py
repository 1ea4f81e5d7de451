"""GPU edge cases against the fp64 oracle:

* Largest sizes: 4096 sequences of the Nemotron-style Mamba-2 layer (a 16 GiB
  fp32 checkpoint: element offsets pass 2^31, byte offsets 2^34) and of the
  Qwen-style GDN and KDA layers (8 GiB), replay and conventional; sampled
  sequences include the last. Slot copies at the same size.
  Sequences other than the sampled ones reuse the sampled ones' inputs (their
  values do not matter here); the sampled sequences get exactly their own.
* Degenerate gates and steps: dt = 0 (no input, no decay) and decays that
  underflow fp32 (a state reset) for Mamba-2; alpha = 1 with beta in {0, 1} for
  Gated DeltaNet; per-channel gates of 0 beside gates that underflow for KDA.
"""
import numpy as np
import pytest
import torch

import ssm_decode_checkpoint_amd as rs
import workloads as W
from oracle import decode, gdn, kda
from gpu_harness import (DEV, dev_in, gdn_layer, gdn_tok_dev, load_state_f32, m2_layer, m2_tok_dev, params_dev,
                         read_meta, read_state_f32, rel_l2, require_gpu, y_buf)

pytestmark = pytest.mark.gpu

SEQS = [0, 1025, 2050, 4095]     # seqs[b % 4] == b for every sampled b
BIG = 4096


def setup_module(_):
    require_gpu()


def _spread(tok, in_dtype, keys, f32_keys=()):
    idx = torch.tensor([b % len(SEQS) for b in range(BIG)], device=DEV)
    out = {k: dev_in(tok[k], in_dtype).index_select(0, idx) for k in keys}
    for k in f32_keys:
        out[k] = torch.from_numpy(np.ascontiguousarray(tok[k], np.float32)).to(DEV).index_select(0, idx)
    return out


def test_mamba2_4096_sequences_past_32bit_offsets():
    w = W.M2_NEMOTRON.with_(batch=BIG, seed=180)
    p = W.m2_params(w)
    A, D = params_dev(p)
    H0 = W.m2_init_states(w, SEQS)
    layer, bufs = m2_layer(w)
    clayer, cbufs = m2_layer(w, mode=rs.RS_CONVENTIONAL)
    assert layer.ckpt_bytes == BIG * 128 * 64 * 128 * 4 > (1 << 34) - 1
    for lay, bf in ((layer, bufs), (clayer, cbufs)):
        ck = rs.ckpt_f32_view(lay, bf)
        for i, b in enumerate(SEQS):
            ck[b].copy_(torch.from_numpy(np.ascontiguousarray(H0[i].transpose(0, 2, 1))).to(DEV))
    ref = decode.M2Conventional(H0, p["A"], p["D"])
    cref = decode.M2Conventional(H0, p["A"], p["D"])
    worst = worst_c = 0.0
    for t in range(17):
        tok = W.m2_step(w, t, SEQS)
        dt = _spread(tok, w.in_dtype, ("x", "B", "C", "dt"))
        y = y_buf(BIG, w.nheads, w.headdim)
        (rs.rs_step_flush if t == 15 else rs.rs_step_nonflush)(layer, bufs, dt, A, D, y)
        worst = max(worst, rel_l2(y[SEQS].cpu().numpy(), ref.step(tok)))
        if t < 2:
            yc = y_buf(BIG, w.nheads, w.headdim)
            rs.rs_step_conventional(clayer, cbufs, dt, A, D, yc)
            worst_c = max(worst_c, rel_l2(yc[SEQS].cpu().numpy(), cref.step(tok)))
        if t == 15:
            assert rel_l2(read_state_f32(layer, bufs, SEQS), ref.H) <= 1e-5
    nck, ln, nd, err, arrive = read_meta(layer, bufs)
    assert (nck == 16).all() and (ln == 1).all() and not err.any() and not arrive.any()
    assert rel_l2(read_state_f32(clayer, cbufs, SEQS), cref.H) <= 1e-5
    assert worst <= 1e-5 and worst_c <= 1e-5, (worst, worst_c)


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_gdn_4096_sequences(gate):
    """Gated DeltaNet, and KDA (per-channel gate: a 1 GiB gate ring beside the 8 GiB state)."""
    w = W.GDN_QWEN.with_(batch=BIG, seed=181, gate=gate)
    gp = W.gdn_params(w)
    S0 = W.gdn_init_states(w, SEQS)
    layer, bufs = gdn_layer(w)
    ck = rs.ckpt_f32_view(layer, bufs)
    for i, b in enumerate(SEQS):
        ck[b].copy_(torch.from_numpy(np.ascontiguousarray(S0[i].transpose(0, 2, 1))).to(DEV))
    ref = decode.GDNConventional(S0, rule=kda if gate == "channel" else gdn)
    worst = 0.0
    for t in range(17):
        tok = W.gdn_step(w, t, SEQS, gp)
        dt = _spread(tok, w.in_dtype, ("q", "k", "v"), ("g", "beta"))
        o = y_buf(BIG, w.n_v, w.dv)
        (rs.rs_step_flush if t == 15 else rs.rs_step_nonflush)(layer, bufs, dt, None, None, o)
        worst = max(worst, rel_l2(o[SEQS].cpu().numpy(), ref.step(tok)))
        if t == 15:
            assert rel_l2(read_state_f32(layer, bufs, SEQS), ref.S) <= 1e-5
    nck, ln, nd, err, arrive = read_meta(layer, bufs)
    assert (nck == 16).all() and (ln == 1).all() and not err.any() and not arrive.any()
    assert worst <= 1e-5, worst


def test_copy_slots_past_32bit_offsets():
    """Slot copies at 4096 Nemotron-style sequences (checkpoint row offsets past 2^34
    bytes): the last sequence is forked into the first and the first into a middle
    slot; copies are bit-exact and untouched slots keep their bits."""
    w = W.M2_NEMOTRON.with_(batch=BIG, seed=186)
    layer, bufs = m2_layer(w)
    ck = rs.ckpt_f32_view(layer, bufs)
    g = torch.Generator(device=DEV).manual_seed(186)
    for b in (0, 1, 2047, 4095):
        ck[b].copy_(torch.randn(ck[b].shape, generator=g, device=DEV))
    ring = rs.ring_view(layer, bufs, "x")
    ring[4095].copy_(torch.randn(ring[4095].shape, generator=g, device=DEV).to(ring.dtype))
    meta_before = read_meta(layer, bufs)
    src_rows = {b: ck[b].clone() for b in (0, 1, 4095)}
    ring_src = ring[4095].clone()
    rs.rs_copy_slots(layer, bufs, torch.tensor([4095, 0], dtype=torch.int32, device=DEV), layer, bufs,
                     torch.tensor([1, 2047], dtype=torch.int32, device=DEV), 2)
    torch.cuda.synchronize()
    assert torch.equal(ck[1], src_rows[4095]) and torch.equal(ck[2047], src_rows[0])
    assert torch.equal(ck[0], src_rows[0]) and torch.equal(ck[4095], src_rows[4095])
    assert torch.equal(ring[1], ring_src)
    nck, ln, nd, err, arrive = read_meta(layer, bufs)
    assert (ln == meta_before[1]).all() and not arrive.any()


def test_mamba2_degenerate_steps():
    """dt = 0 on some steps (the state passes unchanged, y = H C + D x) and dt = 40 on
    others (exp(dt A) underflows fp32: the state restarts from the new input)."""
    w = W.TINY_M2.with_(init_std=0.5, seed=182)
    p = W.m2_params(w)
    A, D = params_dev(p)
    H0 = W.m2_init_states(w, range(w.batch))
    layer, bufs = m2_layer(w)
    load_state_f32(layer, bufs, H0)
    ref = decode.M2Conventional(H0, p["A"], p["D"])
    worst = 0.0
    for t in range(48):
        tok = W.m2_step(w, t, range(w.batch))
        if t % 3 == 0:
            tok["dt"] = np.zeros_like(tok["dt"])
        elif t % 7 == 1:
            tok["dt"] = np.full_like(tok["dt"], 40.0)
        y = y_buf(w.batch, w.nheads, w.headdim)
        (rs.rs_step_flush if t % 16 == 15 else rs.rs_step_nonflush)(layer, bufs, m2_tok_dev(tok, w.in_dtype), A, D, y)
        worst = max(worst, rel_l2(y.cpu().numpy(), ref.step(tok)))
    assert worst <= 1e-5, worst
    assert rel_l2(read_state_f32(layer, bufs), ref.H) <= 1e-5


def test_gdn_no_decay_and_extreme_beta():
    """alpha = 1 (g = 0) on every step; beta = 0 (no write) or 1 (exact write)."""
    w = W.TINY_GDN.with_(init_std=0.5, seed=183)
    gp = W.gdn_params(w)
    S0 = W.gdn_init_states(w, range(w.batch))
    layer, bufs = gdn_layer(w)
    load_state_f32(layer, bufs, S0)
    ref = decode.GDNConventional(S0)
    worst = 0.0
    for t in range(48):
        tok = W.gdn_step(w, t, range(w.batch), gp)
        tok["g"] = np.zeros_like(tok["g"])
        tok["beta"] = np.full_like(tok["beta"], 0.0 if t % 2 else 1.0)
        o = y_buf(w.batch, w.n_v, w.dv)
        (rs.rs_step_flush if t % 16 == 15 else rs.rs_step_nonflush)(layer, bufs, gdn_tok_dev(tok, w.in_dtype),
                                                                      None, None, o)
        worst = max(worst, rel_l2(o.cpu().numpy(), ref.step(tok)))
    assert worst <= 1e-5, worst
    assert rel_l2(read_state_f32(layer, bufs), ref.S) <= 1e-5


def test_kda_mixed_channel_gates():
    """Per-channel gates of 0 (no decay) beside -200 (exp underflows fp32: the channel
    forgets at once) in the same head."""
    w = W.TINY_KDA.with_(init_std=0.5, seed=184)
    gp = W.gdn_params(w)
    S0 = W.gdn_init_states(w, range(w.batch))
    layer, bufs = gdn_layer(w)
    load_state_f32(layer, bufs, S0)
    ref = decode.GDNConventional(S0, rule=kda)
    worst = 0.0
    chan = np.arange(w.dk)
    for t in range(48):
        tok = W.gdn_step(w, t, range(w.batch), gp)
        g = tok["g"].copy()
        g[..., chan % 4 == 0] = 0.0
        g[..., chan % 4 == 1] = -200.0
        tok["g"] = g.astype(np.float32)
        o = y_buf(w.batch, w.n_v, w.dv)
        (rs.rs_step_flush if t % 16 == 15 else rs.rs_step_nonflush)(layer, bufs, gdn_tok_dev(tok, w.in_dtype),
                                                                      None, None, o)
        worst = max(worst, rel_l2(o.cpu().numpy(), ref.step(tok)))
    assert worst <= 1e-5, worst
    assert rel_l2(read_state_f32(layer, bufs), ref.S) <= 1e-5
