"""Pins for speculative rounds (Mamba-2, Gated DeltaNet and Kimi Delta
Attention) and the low-precision read copy in the oracle.

* commit(k) equals replaying the first k drafts: the replay driver's verify
  outputs and its effective state after each commit equal those of plain
  decode with per-draft snapshots (the definition stepped token by token).
* Rejected drafts never touch the checkpoint: a commit that does not fold
  leaves the checkpoint bits unchanged.
* Read-copy isolation: the checkpoint bits after every flush are identical
  with and without the NVFP4 read copy, while the outputs do differ (so the
  copy is really what the non-flush steps read).
"""
import numpy as np
import pytest

import workloads as W
from oracle import decode, gdn, kda


def _spec_case(batch=3, K=4, rounds=24):
    w = W.TINY_M2.with_(batch=batch, max_draft=K, seed=11)
    p = W.m2_params(w)
    H0 = np.random.default_rng(12).standard_normal((batch, w.nheads, w.headdim, w.dstate)) * 0.3
    return w, p, H0


def test_commit_equals_replaying_accepted_drafts():
    w, p, H0 = _spec_case()
    K = w.max_draft
    conv = decode.M2Conventional(H0, p["A"], p["D"])
    rep = decode.M2Replay(H0, p["A"], p["D"], max_draft=K)
    folds = 0
    for rnd in range(24):
        drafts = [W.m2_step(w, rnd * K + d, range(w.batch)) for d in range(K)]
        acc = W.accepted_counts(w.seed, rnd, w.batch, K)
        before = rep.ckpt.copy()
        y_rep = rep.spec_append(drafts)
        n0 = list(rep.ring.n_ckpt)
        rep.spec_commit(acc)
        y_conv = conv.spec_round(drafts, acc)
        assert np.linalg.norm(y_rep - y_conv) <= 1e-12 * np.linalg.norm(y_conv)
        np.testing.assert_allclose(rep.effective_state(), conv.H, rtol=1e-11, atol=1e-12)
        for b in range(w.batch):
            if rep.ring.n_ckpt[b] == n0[b]:
                assert np.array_equal(rep.ckpt[b], before[b])
            else:
                folds += 1
    assert folds > 0
    assert rep.ring.err == [0] * w.batch


def test_plain_steps_continue_after_spec():
    w, p, H0 = _spec_case(batch=2)
    K = w.max_draft
    conv = decode.M2Conventional(H0, p["A"], p["D"])
    rep = decode.M2Replay(H0, p["A"], p["D"], max_draft=K)
    for rnd in range(5):
        drafts = [W.m2_step(w, rnd * K + d, range(w.batch)) for d in range(K)]
        acc = W.accepted_counts(w.seed, rnd, w.batch, K)
        rep.spec_append(drafts)
        rep.spec_commit(acc)
        conv.spec_round(drafts, acc)
    for t in range(100, 140):
        tk = W.m2_step(w, t, range(w.batch))
        y1, y2 = conv.step(tk), rep.step(tk)
        assert np.linalg.norm(y2 - y1) <= 1e-12 * np.linalg.norm(y1)


def test_read_copy_isolation():
    w = W.TINY_M2.with_(seed=13)
    p = W.m2_params(w)
    H0 = np.random.default_rng(14).standard_normal((w.batch, w.nheads, w.headdim, w.dstate)).astype(np.float32)
    plain = decode.M2Replay(H0, p["A"], p["D"], ckpt_fmt="f32")
    rc = decode.M2Replay(H0, p["A"], p["D"], ckpt_fmt="f32", read_copy="nvfp4")
    differ = 0.0
    for t in range(48):
        tk = W.m2_step(w, t, range(w.batch))
        y1, y2 = plain.step(tk), rc.step(tk)
        differ = max(differ, np.abs(y1 - y2).max())
        assert np.array_equal(plain.ckpt, rc.ckpt)
    assert differ > 1e-4


def _gdn_spec_case(gate, batch=3, kmax=4):
    base = W.TINY_KDA if gate == "channel" else W.TINY_GDN
    w = base.with_(batch=batch, seed=15, init_std=0.3)
    gp = W.gdn_params(w)
    S0 = W.gdn_init_states(w, range(batch))
    return w, gp, S0, kmax, (kda if gate == "channel" else gdn)


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_gdn_commit_equals_replaying_accepted_drafts(gate):
    """Gated DeltaNet (per-head gate) and KDA (per-channel gate): verify outputs
    from checkpoint + buffer equal stepping the drafts with snapshots; after each
    commit the effective state equals the state after the accepted drafts;
    rejected drafts leave the checkpoint bits alone."""
    w, gp, S0, kmax, rule = _gdn_spec_case(gate)
    conv = decode.GDNConventional(S0, rule=rule)
    rep = decode.GDNReplay(S0, max_draft=kmax, rule=rule)
    folds = 0
    t = 0
    for rnd in range(30):
        K = (2, 3, 4)[rnd % 3]
        drafts = [W.gdn_step(w, t + d, range(w.batch), gp) for d in range(K)]
        t += K
        acc = W.accepted_counts(w.seed, rnd, w.batch, K)
        before = rep.ckpt.copy()
        o_rep = rep.spec_append(drafts)
        n0 = list(rep.ring.n_ckpt)
        rep.spec_commit(acc)
        o_conv = conv.spec_round(drafts, acc)
        assert np.linalg.norm(o_rep - o_conv) <= 1e-12 * np.linalg.norm(o_conv)
        np.testing.assert_allclose(rep.effective_state(), conv.S, rtol=1e-11, atol=1e-12)
        for b in range(w.batch):
            if rep.ring.n_ckpt[b] == n0[b]:
                assert np.array_equal(rep.ckpt[b], before[b])
            else:
                folds += 1
    assert folds > 0
    assert rep.ring.err == [0] * w.batch


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_gdn_plain_steps_continue_after_spec(gate):
    w, gp, S0, kmax, rule = _gdn_spec_case(gate, batch=2)
    conv = decode.GDNConventional(S0, rule=rule)
    rep = decode.GDNReplay(S0, max_draft=kmax, rule=rule)
    for rnd in range(6):
        drafts = [W.gdn_step(w, rnd * kmax + d, range(w.batch), gp) for d in range(kmax)]
        acc = W.accepted_counts(w.seed, rnd, w.batch, kmax)
        rep.spec_append(drafts)
        rep.spec_commit(acc)
        conv.spec_round(drafts, acc)
    for t in range(100, 140):
        tk = W.gdn_step(w, t, range(w.batch), gp)
        o1, o2 = conv.step(tk), rep.step(tk)
        assert np.linalg.norm(o2 - o1) <= 1e-12 * np.linalg.norm(o1)
