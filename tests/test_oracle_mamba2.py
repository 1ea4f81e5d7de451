"""Pins for the Mamba-2 oracle: brute force, closed forms and method invariants.

None of these re-types the oracle's formulas: the brute force below is the
materialised (semiseparable) input-output map of the recurrence, written as
an O(T^2) sum with plain Python loops over scalars; the closed forms are
special cases worked out by hand.
"""
import math

import numpy as np
import pytest

import workloads as W
from oracle import decode, mamba2


def _rand_case(seed, b=2, h=4, g=2, P=3, N=4, T=20):
    r = np.random.default_rng(seed)
    H0 = r.standard_normal((b, h, P, N))
    toks = [{"x": r.standard_normal((b, h, P)), "B": r.standard_normal((b, g, N)),
             "C": r.standard_normal((b, g, N)), "dt": np.log1p(np.exp(r.standard_normal((b, h)) - 1))}
            for _ in range(T)]
    A = -np.exp(r.uniform(0, 2, size=h))
    D = r.standard_normal(h)
    return H0, toks, A, D


def _brute(H0, toks, A, D, groups):
    """y_t[p] = sum_{s<=t} (C_t.B_s) prod_{s<l<=t} a_l dt_s x_s[p]
              + prod_{l<=t} a_l (sum_n H0[p,n] C_t[n]) + D x_t[p], scalar loops."""
    b_, h_, P, N = H0.shape
    T = len(toks)
    out = np.zeros((T, b_, h_, P))
    for b in range(b_):
        for h in range(h_):
            g = groups[h]
            a = [math.exp(toks[t]["dt"][b, h] * A[h]) for t in range(T)]
            for t in range(T):
                Ct = toks[t]["C"][b, g]
                for p in range(P):
                    dec = 1.0
                    for l in range(t + 1):
                        dec *= a[l]
                    acc = dec * sum(H0[b, h, p, n] * Ct[n] for n in range(N))
                    for s in range(t + 1):
                        w = 1.0
                        for l in range(s + 1, t + 1):
                            w *= a[l]
                        cb = sum(Ct[n] * toks[s]["B"][b, g][n] for n in range(N))
                        acc += cb * w * toks[s]["dt"][b, h] * toks[s]["x"][b, h, p]
                    out[t, b, h, p] = acc + D[h] * toks[t]["x"][b, h, p]
    return out


def test_brute_force_semiseparable():
    H0, toks, A, D = _rand_case(0)
    ys, _ = mamba2.run(H0, toks, A, D)
    ref = _brute(H0, toks, A, D, groups=[0, 0, 1, 1])
    np.testing.assert_allclose(ys, ref, rtol=1e-11, atol=1e-11)


def test_group_map_is_contiguous():
    # 4 heads, 2 groups: heads 0,1 read group 0 and heads 2,3 read group 1.
    H0, toks, A, D = _rand_case(1, T=1)
    tk = dict(toks[0])
    B = tk["B"].copy()
    B[:, 1] = 0.0
    tk["B"] = B
    H1, _ = mamba2.step(H0, tk["x"], tk["B"], tk["C"], tk["dt"], A, D)
    a = np.exp(tk["dt"] * A)
    np.testing.assert_allclose(H1[:, 2:], a[:, 2:, None, None] * H0[:, 2:], rtol=1e-14)
    assert np.abs(H1[:, :2] - a[:, :2, None, None] * H0[:, :2]).max() > 1e-3


def test_closed_form_one_step_from_zero():
    H0, toks, A, D = _rand_case(2, T=1)
    tk = toks[0]
    _, y = mamba2.step(np.zeros_like(H0), tk["x"], tk["B"], tk["C"], tk["dt"], A, D)
    groups = [0, 0, 1, 1]
    for b in range(2):
        for h in range(4):
            bc = float(np.dot(tk["B"][b, groups[h]], tk["C"][b, groups[h]]))
            want = tk["dt"][b, h] * bc * tk["x"][b, h] + D[h] * tk["x"][b, h]
            np.testing.assert_allclose(y[b, h], want, rtol=1e-13)


def test_closed_form_dt_zero_keeps_state():
    H0, toks, A, D = _rand_case(3, T=1)
    tk = dict(toks[0])
    tk["dt"] = np.zeros_like(tk["dt"])
    H1, y = mamba2.step(H0, tk["x"], tk["B"], tk["C"], tk["dt"], A, D)
    np.testing.assert_array_equal(H1, H0)
    groups = [0, 0, 1, 1]
    for h in range(4):
        want = H0[:, h] @ tk["C"][:, groups[h]][:, :, None]
        np.testing.assert_allclose(y[:, h], want[..., 0] + D[h] * tk["x"][:, h], rtol=1e-13)


def test_closed_form_no_decay_is_running_sum():
    # A = 0: H_t = H0 + sum_s dt_s x_s B_s^T (unnormalised linear attention)
    H0, toks, A, D = _rand_case(4, T=12)
    A0 = np.zeros_like(A)
    _, H = mamba2.run(H0, toks, A0, D)
    want = H0.copy()
    groups = [0, 0, 1, 1]
    for tk in toks:
        for h in range(4):
            want[:, h] += tk["dt"][:, h, None, None] * tk["x"][:, h, :, None] * tk["B"][:, groups[h], None, :]
    np.testing.assert_allclose(H, want, rtol=1e-12, atol=1e-12)


def _tiny():
    w = W.TINY_M2
    p = W.m2_params(w)
    r = np.random.default_rng(7)
    H0 = r.standard_normal((w.batch, w.nheads, w.headdim, w.dstate)) * 0.3
    toks = [W.m2_step(w, t, range(w.batch)) for t in range(w.steps)]
    return w, p, H0, toks


def test_replay_equals_conventional():
    w, p, H0, toks = _tiny()
    conv = decode.M2Conventional(H0, p["A"], p["D"])
    rep = decode.M2Replay(H0, p["A"], p["D"])
    for t, tk in enumerate(toks):
        y1, y2 = conv.step(tk), rep.step(tk)
        assert np.linalg.norm(y2 - y1) <= 1e-12 * np.linalg.norm(y1), t
        np.testing.assert_allclose(rep.effective_state(), conv.H, rtol=1e-11, atol=1e-12)
    # four windows of 16 tokens: four checkpoint writes and an empty buffer at the end
    assert rep.ring.n_ckpt == [64] * w.batch and rep.ring.len == [0] * w.batch
    np.testing.assert_allclose(rep.ckpt, conv.H, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("fill", list(range(16)))
def test_flush_at_any_fill_leaves_outputs_unchanged(fill):
    w, p, H0, toks = _tiny()
    base = decode.M2Replay(H0, p["A"], p["D"])
    forced = decode.M2Replay(H0, p["A"], p["D"])
    for t, tk in enumerate(toks[:40]):
        y1 = base.step(tk)
        y2 = forced.step(tk, force_flush=(t == fill))
        assert np.linalg.norm(y2 - y1) <= 1e-12 * np.linalg.norm(y1)
    assert forced.ring.n_ckpt[0] != base.ring.n_ckpt[0] or fill == 15


def test_replay_forms_on_the_flush_window_directly():
    # y from (checkpoint, entries) equals y from the conventional state; the fold equals the state
    w, p, H0, toks = _tiny()
    H = H0.copy()
    for j in range(1, 17):
        H, y = mamba2.step(H, toks[j - 1]["x"], toks[j - 1]["B"], toks[j - 1]["C"], toks[j - 1]["dt"],
                           p["A"], p["D"])
        yr = mamba2.replay_output(H0, toks[:j], toks[j - 1]["C"], p["A"], p["D"])
        np.testing.assert_allclose(yr, y, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(mamba2.replay_fold(H0, toks[:j], p["A"]), H, rtol=1e-11, atol=1e-12)
