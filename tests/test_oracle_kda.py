"""Pins for the Kimi Delta Attention oracle (per-key-channel decay).

* A gate equal on every channel reduces the step to the Gated DeltaNet step
  (pinned on its own in test_oracle_gdn.py).
* Closed forms: beta = 0 is pure per-channel decay, S_T = S0 Diag(prod alpha);
  one step from zero state gives S = beta v k^T and o = beta (k . q) v.
* The delta-rule write property: with beta = 1 and |k| = 1 the new state maps k
  exactly to v whatever the decay (S_t k_t = v_t). It fixes the order of the
  decay and the projection: decaying after the projection breaks it.
* The triangular system equals numpy.linalg.solve of (I + L) U = B built as
  matrices; replay output / fold equal the plain recurrence.
"""
import numpy as np

import workloads as W
from oracle import decode, gdn, kda


def _rand(seed, b=2, nv=4, nqk=2, dv=8, dk=8):
    g = np.random.default_rng(seed)
    S = g.standard_normal((b, nv, dv, dk))
    k = g.standard_normal((b, nqk, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = g.standard_normal((b, nqk, dk))
    v = g.standard_normal((b, nv, dv))
    beta = 1.0 / (1.0 + np.exp(-g.standard_normal((b, nv))))
    gate = -np.abs(g.standard_normal((b, nv, dk))) * 0.5
    return S, q, k, v, gate, beta


def test_uniform_gate_is_gdn():
    S, q, k, v, gate, beta = _rand(1)
    gh = gate[:, :, 0]
    for _ in range(5):
        S1, o1 = kda.step(S, q, k, v, np.repeat(gh[:, :, None], S.shape[3], axis=2), beta)
        S2, o2 = gdn.step(S, q, k, v, gh, beta)
        np.testing.assert_allclose(S1, S2, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-13)
        S = S1


def test_pure_decay_and_first_step():
    S, q, k, v, gate, beta = _rand(2)
    S0 = S.copy()
    acc = np.ones_like(gate)
    for t in range(4):
        g_t = gate * (1 + 0.1 * t)
        S, _ = kda.step(S, q, k, v, g_t, np.zeros_like(beta))
        acc = acc * np.exp(g_t)
    np.testing.assert_allclose(S, S0 * acc[:, :, None, :], rtol=1e-13, atol=1e-14)
    Z = np.zeros_like(S0)
    S1, o1 = kda.step(Z, q, k, v, gate, beta)
    kk, qq = gdn.expand_qk(k, S.shape[1]), gdn.expand_qk(q, S.shape[1])
    np.testing.assert_allclose(S1, beta[:, :, None, None] * v[:, :, :, None] * kk[:, :, None, :], atol=1e-14)
    np.testing.assert_allclose(o1, (beta * np.sum(kk * qq, -1))[:, :, None] * v, atol=1e-13)


def test_delta_write_property_fixes_operator_order():
    S, q, k, v, gate, beta = _rand(3)
    Sn, _ = kda.step(S, q, k, v, gate, np.ones_like(beta))
    kk = gdn.expand_qk(k, S.shape[1])
    np.testing.assert_allclose(np.einsum("bhvk,bhk->bhv", Sn, kk), v, atol=1e-12)
    # the other order (project, then decay) does not have the property: the pin would catch it
    alpha = np.exp(gate)
    P = np.eye(S.shape[3]) - kk[:, :, :, None] * kk[:, :, None, :]
    wrong = np.matmul(np.matmul(S, P), alpha[..., None] * np.eye(S.shape[3])) + v[..., None] * kk[:, :, None, :]
    assert np.abs(np.einsum("bhvk,bhk->bhv", wrong, kk) - v).max() > 1e-3


def test_ut_solve_is_the_triangular_system():
    w = W.TINY_KDA.with_(batch=2, seed=21)
    gp = W.gdn_params(w)
    S0 = np.random.default_rng(22).standard_normal((w.batch, w.n_v, w.dv, w.dk))
    ents = [W.gdn_step(w, t, range(w.batch), gp) for t in range(7)]
    us = kda.ut_solve(S0, ents)
    m = len(ents)
    gamma, r = kda.window_decays(ents)
    ks = [gdn.expand_qk(e["k"], w.n_v) for e in ents]
    for b in range(w.batch):
        for h in range(w.n_v):
            L = np.zeros((m, m))
            rhs = np.zeros((m, w.dv))
            for t in range(m):
                bt = float(ents[t]["beta"][b, h])
                for i in range(t):
                    L[t, i] = bt * np.dot(ks[t][b, h], r[t][i][b, h] * ks[i][b, h])
                rhs[t] = bt * (ents[t]["v"][b, h] - S0[b, h] @ (gamma[t][b, h] * ks[t][b, h]))
            U = np.linalg.solve(np.eye(m) + L, rhs)
            for t in range(m):
                np.testing.assert_allclose(us[t][b, h], U[t], rtol=1e-10, atol=1e-12)


def test_replay_equals_recurrence():
    w = W.TINY_KDA.with_(seed=23)
    gp = W.gdn_params(w)
    S0 = np.random.default_rng(24).standard_normal((w.batch, w.n_v, w.dv, w.dk)) * 0.5
    conv = decode.GDNConventional(S0, rule=kda)
    rep = decode.GDNReplay(S0, rule=kda)
    for t in range(40):
        tk = W.gdn_step(w, t, range(w.batch), gp)
        o1, o2 = conv.step(tk), rep.step(tk)
        assert np.linalg.norm(o2 - o1) <= 1e-12 * np.linalg.norm(o1)
        if t % 16 == 15:
            np.testing.assert_allclose(rep.ckpt, conv.S, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(rep.effective_state(), conv.S, rtol=1e-11, atol=1e-12)


def test_channel_gates_differ_per_channel():
    """The workload's KDA gate really varies across key channels (else the GPU
    tests could not tell a per-channel decay from a per-head one)."""
    w = W.TINY_KDA
    tk = W.gdn_step(w, 0, range(w.batch), W.gdn_params(w))
    assert tk["g"].shape == (w.batch, w.n_v, w.dk)
    assert np.std(tk["g"], axis=-1).min() > 1e-3 and (tk["g"] <= 0).all()
