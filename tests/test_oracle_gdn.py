"""Pins for the Gated DeltaNet oracle.

* Brute force: the state after T steps as explicit dense transition products
  S_T = S0 M_1 ... M_T + sum_s beta_s v_s k_s^T M_{s+1} ... M_T with
  M_l = alpha_l (I - beta_l k_l k_l^T), built with plain matrix products.
* Closed forms: beta = 0 decays only; beta = 1 with a unit key stores v exactly
  under k ("replace"); orthonormal keys with no decay recall stored values.
* The UT system is also solved with numpy.linalg.solve.
* Replay equals conventional decode; a flush at any fill leaves outputs unchanged.
"""
import numpy as np
import pytest

import workloads as W
from oracle import decode, gdn


def _case(seed, b=2, nqk=2, nv=4, dk=5, dv=3, T=12, beta=None, g=None, unit=True):
    r = np.random.default_rng(seed)
    S0 = r.standard_normal((b, nv, dv, dk))
    toks = []
    for _ in range(T):
        k = r.standard_normal((b, nqk, dk))
        q = r.standard_normal((b, nqk, dk))
        if unit:
            k /= np.linalg.norm(k, axis=-1, keepdims=True)
        toks.append({"q": q, "k": k, "v": r.standard_normal((b, nv, dv)),
                     "g": (-r.uniform(0.0, 1.0, (b, nv)) if g is None else np.full((b, nv), g)),
                     "beta": (r.uniform(0.0, 1.0, (b, nv)) if beta is None else np.full((b, nv), beta))})
    return S0, toks


def test_brute_force_transition_products():
    S0, toks = _case(0)
    b_, nv, dv, dk = S0.shape
    _, S = gdn.run(S0, toks)
    qk_of = [0, 0, 1, 1]
    for b in range(b_):
        for h in range(nv):
            Ms = []
            for tk in toks:
                k = tk["k"][b, qk_of[h]]
                Ms.append(np.exp(tk["g"][b, h]) * (np.eye(dk) - tk["beta"][b, h] * np.outer(k, k)))
            want = S0[b, h].copy()
            for M in Ms:
                want = want @ M
            for s, tk in enumerate(toks):
                term = tk["beta"][b, h] * np.outer(tk["v"][b, h], tk["k"][b, qk_of[h]])
                for M in Ms[s + 1:]:
                    term = term @ M
                want = want + term
            np.testing.assert_allclose(S[b, h], want, rtol=1e-12, atol=1e-12)


def test_output_reads_updated_state():
    S0, toks = _case(1, T=1)
    S1, o = gdn.step(S0, **{k: toks[0][k] for k in ("q", "k", "v", "g", "beta")})
    qq = toks[0]["q"][:, [0, 0, 1, 1]]
    np.testing.assert_allclose(o, np.einsum("bhvk,bhk->bhv", S1, qq), rtol=1e-13)


def test_beta_zero_only_decays():
    S0, toks = _case(2, beta=0.0)
    outs, S = gdn.run(S0, toks)
    gam = np.exp(sum(tk["g"] for tk in toks))
    np.testing.assert_allclose(S, gam[:, :, None, None] * S0, rtol=1e-12)
    qq = toks[-1]["q"][:, [0, 0, 1, 1]]
    np.testing.assert_allclose(outs[-1], gam[:, :, None] * np.einsum("bhvk,bhk->bhv", S0, qq), rtol=1e-12)


def test_beta_one_unit_key_replaces_value():
    S0, toks = _case(3, beta=1.0)
    S = S0
    for tk in toks:
        S, _ = gdn.step(S, tk["q"], tk["k"], tk["v"], tk["g"], tk["beta"])
        kk = tk["k"][:, [0, 0, 1, 1]]
        np.testing.assert_allclose(np.einsum("bhvk,bhk->bhv", S, kk), tk["v"], rtol=1e-12, atol=1e-12)


def test_orthonormal_keys_recall():
    dk = 6
    r = np.random.default_rng(4)
    Q, _ = np.linalg.qr(r.standard_normal((dk, dk)))
    S = np.zeros((1, 1, 3, dk))
    vs = []
    for j in range(dk):
        v = r.standard_normal((1, 1, 3))
        vs.append(v)
        S, _ = gdn.step(S, Q[j][None, None], Q[j][None, None], v, np.zeros((1, 1)), np.ones((1, 1)))
    for j in range(dk):
        np.testing.assert_allclose(S[0, 0] @ Q[j], vs[j][0, 0], rtol=1e-12, atol=1e-12)


def test_ut_solve_matches_library_solve():
    S0, toks = _case(5, T=9)
    us = gdn.ut_solve(S0, toks)
    b_, nv, dv, dk = S0.shape
    m = len(toks)
    qk_of = [0, 0, 1, 1]
    for b in range(b_):
        for h in range(nv):
            al = [np.exp(tk["g"][b, h]) for tk in toks]
            K = np.stack([tk["k"][b, qk_of[h]] for tk in toks])
            V = np.stack([tk["v"][b, h] for tk in toks])
            be = np.array([tk["beta"][b, h] for tk in toks])
            gam = np.cumprod(al)
            Lm = np.zeros((m, m))
            for t in range(m):
                for i in range(t):
                    Lm[t, i] = be[t] * np.prod(al[i + 1:t + 1]) * (K[t] @ K[i])
            rhs = be[:, None] * (V - gam[:, None] * (K @ S0[b, h].T))
            U = np.linalg.solve(np.eye(m) + Lm, rhs)
            np.testing.assert_allclose(np.stack([u[b, h] for u in us]), U, rtol=1e-11, atol=1e-12)


def _tiny():
    w = W.TINY_GDN
    gp = W.gdn_params(w)
    r = np.random.default_rng(8)
    S0 = r.standard_normal((w.batch, w.n_v, w.dv, w.dk)) * 0.2
    toks = [W.gdn_step(w, t, range(w.batch), gp) for t in range(w.steps)]
    return w, S0, toks


def test_replay_equals_conventional():
    w, S0, toks = _tiny()
    conv, rep = decode.GDNConventional(S0), decode.GDNReplay(S0)
    for t, tk in enumerate(toks):
        o1, o2 = conv.step(tk), rep.step(tk)
        assert np.linalg.norm(o2 - o1) <= 1e-12 * np.linalg.norm(o1), t
        np.testing.assert_allclose(rep.effective_state(), conv.S, rtol=1e-11, atol=1e-12)
    assert rep.ring.n_ckpt == [64] * w.batch


@pytest.mark.parametrize("fill", [0, 3, 7, 14, 15])
def test_flush_at_any_fill(fill):
    w, S0, toks = _tiny()
    a, b = decode.GDNReplay(S0), decode.GDNReplay(S0)
    for t, tk in enumerate(toks[:34]):
        o1 = a.step(tk)
        o2 = b.step(tk, force_flush=(t == fill))
        assert np.linalg.norm(o2 - o1) <= 1e-12 * np.linalg.norm(o1)
