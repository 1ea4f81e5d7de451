"""GPU parity of the Mamba-2 block calls around the SSM step against the fp64
oracle (oracle/block.py):

* rs_conv_step: the short causal convolution with its ring of recent inputs,
  over plain steps across flushes (positions come from the layer's counters),
  slot reuse, and speculative rounds (drafts, then a commit that only moves
  the position); its x / B / C outputs then drive the SSM step, checked
  against the oracle replay fed the same values. Sequences the SSM call would
  refuse are left untouched.
* rs_gated_norm: the gated RMS norm over channel groups, fp32 and bf16, plain
  and K-draft rows, on the tiny and the Nemotron-style shapes.

Tolerances: fp32 outputs within 1e-5 relative (+1e-6 absolute, for values
near zero after cancellation); bf16 outputs are the fp32 result rounded to
nearest even, so within half a bf16 step (2^-8 relative) of the exact value,
plus the same fp32 slack.
"""
import numpy as np
import pytest
import torch

import ssm_decode_checkpoint_amd as rs
import workloads as W
from oracle import block, decode
from gpu_harness import (DEV, dev_f32, dev_in, load_state_f32, m2_layer, params_dev, read_meta, rel_l2,
                         require_gpu, y_buf)

pytestmark = pytest.mark.gpu


def setup_module(_):
    require_gpu()


def _tdt(in_dtype):
    return torch.bfloat16 if in_dtype == "bf16" else torch.float32


def _close(got, ref, in_dtype):
    ref = np.asarray(ref, np.float64)
    rel = (2.0 ** -8 if in_dtype == "bf16" else 0.0) + 1e-5
    bad = np.abs(np.asarray(got, np.float64) - ref) > rel * np.abs(ref) + 1e-6
    assert not bad.any(), (int(bad.sum()), float(np.abs(got - ref)[bad].max()))


class _Conv:
    """Device side of one layer's convolution: ring, weights, output buffers."""

    def __init__(self, layer, w, bp, width):
        self.layer, self.w, self.width = layer, w, width
        self.ch = rs.conv_channels(layer)
        self.ring = torch.zeros(rs.conv_ring_bytes(layer), dtype=torch.uint8, device=DEV)
        self.cw, self.cb = dev_f32(np.ascontiguousarray(bp["conv_w"][:, :width])), dev_f32(bp["conv_b"])

    def run(self, bufs, xbc, K=None):
        """xbc: float32 [batch, ch] (a plain token), or [K, batch, ch] for K drafts,
        holding in_dtype values; outputs shaped the same way."""
        w, dt = self.w, _tdt(self.w.in_dtype)
        lead = (w.batch,) if K is None else (K, w.batch)
        x = torch.full(lead + (w.nheads, w.headdim), float("nan"), dtype=dt, device=DEV)
        B = torch.full(lead + (w.ngroups, w.dstate), float("nan"), dtype=dt, device=DEV)
        C = torch.full(lead + (w.ngroups, w.dstate), float("nan"), dtype=dt, device=DEV)
        rs.rs_conv_step(self.layer, bufs, self.ring, dev_in(xbc, w.in_dtype), 1 if K is None else K, self.cw,
                        self.cb, self.width, x, B, C)
        return x, B, C

    def flat(self, x, B, C):
        n = x.shape[:-2]
        return torch.cat([x.float().reshape(*n, -1), B.float().reshape(*n, -1), C.float().reshape(*n, -1)],
                         dim=-1).cpu().numpy()


def _split(w, v):
    """[..., ch] -> x [..., H, P], B, C [..., G, N] as float32."""
    d, gn = w.nheads * w.headdim, w.ngroups * w.dstate
    lead = v.shape[:-1]
    return (v[..., :d].reshape(*lead, w.nheads, w.headdim).astype(np.float32),
            v[..., d:d + gn].reshape(*lead, w.ngroups, w.dstate).astype(np.float32),
            v[..., d + gn:].reshape(*lead, w.ngroups, w.dstate).astype(np.float32))


@pytest.mark.parametrize("in_dtype,width", [("f32", 4), ("bf16", 4), ("bf16", 2), ("f32", 3), ("bf16", 1)])
def test_conv_then_ssm_steps(in_dtype, width):
    w = W.TINY_M2.with_(batch=4, init_std=0.4, seed=210, in_dtype=in_dtype)
    bp = W.block_params(w)
    p = W.m2_params(w)
    A, D = params_dev(p)
    layer, bufs = m2_layer(w)
    H0 = W.m2_init_states(w, range(w.batch))
    load_state_f32(layer, bufs, H0)
    cv = _Conv(layer, w, bp, width)
    conv_or = block.ConvState(w.batch, cv.ch, bp["conv_w"][:, :width], bp["conv_b"])
    ssm_or = decode.M2Replay(H0, p["A"], p["D"])
    worst = 0.0
    for t in range(40):                           # two flushes
        bt = W.block_step(w, t, range(w.batch))
        x, B, C = cv.run(bufs, bt["xbc"])
        got = cv.flat(x, B, C)
        _close(got, conv_or.step(bt["xbc"]), in_dtype)
        dt = W.m2_step(w, t, range(w.batch))["dt"]
        y = y_buf(w.batch, w.nheads, w.headdim)
        rs.rs_step(layer, bufs, {"x": x, "B": B, "C": C, "dt": dev_in(dt, in_dtype)}, A, D, y)
        gx, gB, gC = _split(w, got)
        worst = max(worst, rel_l2(y.cpu().numpy(), ssm_or.step({"x": gx, "B": gB, "C": gC, "dt": dt})))
    assert worst <= 1e-5, worst


def test_conv_slot_reuse():
    """A reused slot starts at position 0: its caller zeroes the history slots
    (positions -3..-1 = slots 13..15); the other sequences continue."""
    w = W.TINY_M2.with_(batch=4, init_std=0.0, seed=211, in_dtype="bf16")
    bp = W.block_params(w)
    layer, bufs = m2_layer(w)
    cv = _Conv(layer, w, bp, 4)
    conv_or = block.ConvState(w.batch, cv.ch, bp["conv_w"], bp["conv_b"])
    A, D = params_dev(W.m2_params(w))
    for t in range(30):
        if t == 19:
            rs.rs_reset_slots(layer, bufs, torch.tensor([2], dtype=torch.int32, device=DEV), 1)
            cv.ring.view(w.batch, -1)[2].zero_()
            conv_or.hist[2] = 0.0
        bt = W.block_step(w, t, range(w.batch))
        x, B, C = cv.run(bufs, bt["xbc"])
        _close(cv.flat(x, B, C), conv_or.step(bt["xbc"]), "bf16")
        dt = dev_in(W.m2_step(w, t, range(w.batch))["dt"], "bf16")
        rs.rs_step(layer, bufs, {"x": x, "B": B, "C": C, "dt": dt}, A, D, y_buf(w.batch, w.nheads, w.headdim))
    nck, ln, _, _, _ = read_meta(layer, bufs)
    assert nck[2] + ln[2] == 11 and nck[0] + ln[0] == 30


def test_conv_speculative_rounds():
    """K draft inputs convolve in order from the committed history; the commit
    only moves the position. A plain call with drafts pending changes nothing.
    Plain tokens before the first round and after the last (back-to-back rounds
    always have room for the next drafts)."""
    w = W.TINY_M2.with_(batch=4, init_std=0.4, seed=212, in_dtype="bf16", max_draft=4)
    bp = W.block_params(w)
    p = W.m2_params(w)
    A, D = params_dev(p)
    layer, bufs = m2_layer(w)
    H0 = W.m2_init_states(w, range(w.batch))
    load_state_f32(layer, bufs, H0)
    cv = _Conv(layer, w, bp, 4)
    conv_or = block.ConvState(w.batch, cv.ch, bp["conv_w"], bp["conv_b"])
    ssm_or = decode.M2Replay(H0, p["A"], p["D"], max_draft=4)
    state = {"t": 0, "worst": 0.0}

    def plain():
        t = state["t"]
        bt = W.block_step(w, t, range(w.batch))
        x, B, C = cv.run(bufs, bt["xbc"])
        got = cv.flat(x, B, C)
        _close(got, conv_or.step(bt["xbc"]), "bf16")
        dt = W.m2_step(w, t, range(w.batch))["dt"]
        y = y_buf(w.batch, w.nheads, w.headdim)
        rs.rs_step(layer, bufs, {"x": x, "B": B, "C": C, "dt": dev_in(dt, "bf16")}, A, D, y)
        gx, gB, gC = _split(w, got)
        state["worst"] = max(state["worst"],
                             rel_l2(y.cpu().numpy(), ssm_or.step({"x": gx, "B": gB, "C": gC, "dt": dt})))
        state["t"] = t + 1

    for _ in range(3):
        plain()
    for rnd in range(12):
        t, K = state["t"], 1 + rnd % 4
        xbcs = [W.block_step(w, 1000 + t + d, range(w.batch))["xbc"] for d in range(K)]
        x, B, C = cv.run(bufs, np.stack(xbcs), K=K)
        got = cv.flat(x, B, C)
        _close(got, conv_or.drafts(xbcs), "bf16")
        dts = [W.m2_step(w, 1000 + t + d, range(w.batch))["dt"] for d in range(K)]
        y = y_buf(w.batch, w.nheads, w.headdim, K=K)
        rs.rs_spec_append(layer, bufs, {"x": x, "B": B, "C": C, "dt": dev_in(np.stack(dts), "bf16")}, K, A, D, y)
        drafts = []
        for d in range(K):
            gx, gB, gC = _split(w, got[d])
            drafts.append({"x": gx, "B": gB, "C": gC, "dt": dts[d]})
        state["worst"] = max(state["worst"], rel_l2(y.cpu().numpy(), ssm_or.spec_append(drafts)))
        if rnd == 5:                               # drafts pending: a plain call is skipped
            ring0 = cv.ring.clone()
            xp, Bp, Cp = cv.run(bufs, W.block_step(w, 5000, range(w.batch))["xbc"])
            assert torch.isnan(xp.float()).all() and torch.isnan(Cp.float()).all()
            assert torch.equal(ring0, cv.ring)
        acc = W.accepted_counts(w.seed, rnd, w.batch, K)
        rs.rs_spec_commit(layer, bufs, torch.from_numpy(acc).to(DEV), A, D)
        ssm_or.spec_commit(acc)
        conv_or.commit(xbcs, acc)
        state["t"] = t + K
    for _ in range(6):
        plain()
    nck, ln, nd, err, _ = read_meta(layer, bufs)
    assert not err.any() and not nd.any()
    assert state["worst"] <= 1e-5, state["worst"]


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape,groups,K", [("tiny", 1, 1), ("tiny", 4, 3), ("nemotron", 8, 1), ("nemotron", 8, 2)])
def test_gated_norm(in_dtype, shape, groups, K):
    base = W.TINY_M2 if shape == "tiny" else W.M2_NEMOTRON
    w = base.with_(batch=3, in_dtype=in_dtype, seed=213, max_draft=4 if K > 1 else 0)
    layer, _ = m2_layer(w)
    bp = W.block_params(w)
    d = w.nheads * w.headdim
    g = np.random.default_rng(214)
    y = (g.standard_normal((K, w.batch, d)) * 0.5).astype(np.float32)
    z = np.stack([W.block_step(w, 7 + k, range(w.batch))["z"] for k in range(K)])
    out = torch.full((K, w.batch, d), float("nan"), dtype=_tdt(in_dtype), device=DEV)
    rs.rs_gated_norm(layer, K, dev_f32(y), dev_in(z, in_dtype), dev_f32(bp["norm_w"]), groups, 1e-5, out)
    ref = block.gated_rmsnorm(y.reshape(K * w.batch, d), z.reshape(K * w.batch, d), bp["norm_w"], groups, 1e-5)
    _close(out.float().cpu().numpy().reshape(K * w.batch, d), ref, in_dtype)
