"""GPU parity of the serving calls: the self-scheduling step (each sequence
flushes when its own buffer is full) over sequences at different fills, and
slot reuse (a slot's counters cleared and a new initial state written while the
other slots keep decoding). Every slot is checked against its own fp64 oracle:
the same-method replay (its own flush schedule) and the plain recurrence."""
import numpy as np
import pytest
import torch

import ssm_decode_checkpoint_amd as rs
import workloads as W
from oracle import decode, gdn, kda
from gpu_harness import (DEV, gdn_layer, gdn_tok_dev, m2_layer, m2_tok_dev, params_dev, read_meta, read_state_f32,
                         rel_l2, require_gpu, y_buf)

pytestmark = pytest.mark.gpu


def setup_module(_):
    require_gpu()


def _write_state(layer, bufs, b, logical):
    rs.ckpt_f32_view(layer, bufs)[b].copy_(
        torch.from_numpy(np.ascontiguousarray(np.swapaxes(np.asarray(logical, np.float32), -1, -2))).to(DEV))


def _reset_plan(batch, steps):
    """Slot b (b >= 1) starts a new sequence at step 3b + 1; slot 0 again at step 40."""
    plan = {}
    for b in range(1, batch):
        plan.setdefault(3 * b + 1, []).append(b)
    plan.setdefault(40, []).append(0)
    return {t: v for t, v in plan.items() if t < steps}


def _serve(kind, w, steps=64):
    if kind == "mamba2":
        p = W.m2_params(w)
        A, D = params_dev(p)
        init = lambda b, gen: W.m2_init_state(w.with_(seed=w.seed + 1000 * gen), b)
        layer, bufs = m2_layer(w)
        mk_rep = lambda st: decode.M2Replay(st[None], p["A"], p["D"])
        mk_conv = lambda st: decode.M2Conventional(st[None], p["A"], p["D"])
        step_in = lambda t: W.m2_step(w, t, range(w.batch))
        to_dev = lambda tok: m2_tok_dev(tok, w.in_dtype)
        out = lambda: y_buf(w.batch, w.nheads, w.headdim)
    else:
        rule = kda if w.gate == "channel" else gdn
        gp = W.gdn_params(w)
        A = D = None
        init = lambda b, gen: W.gdn_init_state(w.with_(seed=w.seed + 1000 * gen), b)
        layer, bufs = gdn_layer(w)
        mk_rep = lambda st: decode.GDNReplay(st[None], rule=rule)
        mk_conv = lambda st: decode.GDNConventional(st[None], rule=rule)
        step_in = lambda t: W.gdn_step(w, t, range(w.batch), gp)
        to_dev = lambda tok: gdn_tok_dev(tok, w.in_dtype)
        out = lambda: y_buf(w.batch, w.n_v, w.dv)
    reps, convs = [], []
    for b in range(w.batch):
        st = init(b, 0)
        _write_state(layer, bufs, b, st)
        reps.append(mk_rep(st))
        convs.append(mk_conv(st))
    plan = _reset_plan(w.batch, steps)
    worst_same = worst_exact = 0.0
    flushes_per_step = []
    for t in range(steps):
        if t in plan:
            seqs = plan[t]
            for b in seqs:
                st = init(b, t + 1)
                _write_state(layer, bufs, b, st)
                reps[b] = mk_rep(st)
                convs[b] = mk_conv(st)
            rs.rs_reset_slots(layer, bufs, torch.tensor(seqs, dtype=torch.int32, device=DEV), len(seqs))
        tok = step_in(t)
        y = out()
        flushes_per_step.append(sum(r.ring.len[0] == 15 for r in reps))
        rs.rs_step(layer, bufs, to_dev(tok), A, D, y)
        yg = y.cpu().numpy()
        for b in range(w.batch):
            tb = {k: v[b:b + 1] for k, v in tok.items()}
            worst_same = max(worst_same, rel_l2(yg[b:b + 1], reps[b].step(tb)))
            worst_exact = max(worst_exact, rel_l2(yg[b:b + 1], convs[b].step(tb)))
        nck, ln, nd, err, arrive = read_meta(layer, bufs)
        assert list(nck) == [r.ring.n_ckpt[0] for r in reps] and list(ln) == [r.ring.len[0] for r in reps]
        assert not err.any() and not arrive.any() and not nd.any()
    ck = read_state_f32(layer, bufs)
    worst_ck = max(rel_l2(ck[b:b + 1], reps[b].ckpt) for b in range(w.batch))
    return worst_same, worst_exact, worst_ck, flushes_per_step


def test_mamba2_staggered_slots():
    w = W.TINY_M2.with_(batch=8, init_std=0.4, seed=190)
    ws, we, wc, fl = _serve("mamba2", w)
    assert ws <= 1e-5 and we <= 1e-5 and wc <= 1e-5, (ws, we, wc)
    assert max(fl) < w.batch and sum(fl) > 8          # flushes happen, not all in one step


def test_mamba2_staggered_slots_nemotron_shapes():
    w = W.M2_NEMOTRON.with_(batch=6, init_std=0.1, seed=191)
    ws, we, wc, fl = _serve("mamba2", w, steps=48)
    assert ws <= 1e-5 and we <= 1e-5 and wc <= 1e-5, (ws, we, wc)


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_delta_rule_staggered_slots(gate):
    w = W.TINY_GDN.with_(batch=8, n_qk=2, n_v=4, dk=128, dv=128, in_dtype="bf16", init_std=0.3, seed=192,
                         gate=gate)
    ws, we, wc, fl = _serve("gdn", w)
    assert ws <= 1e-5 and we <= 1e-5 and wc <= 1e-5, (ws, we, wc)
    assert max(fl) < w.batch and sum(fl) > 8


def test_reset_slots_skips_out_of_range_and_keeps_others():
    w = W.TINY_M2.with_(batch=4, init_std=0.4, seed=193)
    p = W.m2_params(w)
    A, D = params_dev(p)
    layer, bufs = m2_layer(w)
    for t in range(5):
        rs.rs_step(layer, bufs, m2_tok_dev(W.m2_step(w, t, range(w.batch)), w.in_dtype), A, D,
                   y_buf(w.batch, w.nheads, w.headdim))
    before = read_meta(layer, bufs)
    rs.rs_reset_slots(layer, bufs, torch.tensor([2, -1, 7], dtype=torch.int32, device=DEV), 3)
    nck, ln, nd, err, _ = read_meta(layer, bufs)
    assert list(ln) == [5, 5, 0, 5] and list(nck) == [0, 0, 0, 0]
    assert np.array_equal(before[1][[0, 1, 3]], ln[[0, 1, 3]])
