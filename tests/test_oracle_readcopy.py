"""Pins for the delta-rule oracle's low-precision read copy (Gated DeltaNet and
Kimi Delta Attention; sitech.ge ReplaySSM page, "Bounding quantization error":
a low-precision copy serves the reads while the recurrence keeps its own
precision).

* Isolation: the checkpoint after every flush and commit-fold is identical
  with and without the read copy, and equals conventional decoding.
* Closed form: with beta = 0 no entry writes, so every output is
  gamma_t S0 q_t (KDA: S0 (gamma_t * q_t)) with S0 read as the NVFP4 round
  trip of the stored matrix -- computed here from the quantizer directly.
* The copy is really read: outputs move away from exact decoding by the
  quantization error, and back to it without the copy.
"""
import numpy as np
import pytest

import workloads as W
from oracle import decode, gdn, kda, quant


def _nvfp4_view(S):
    """NVFP4 round trip of states [b, h, dv, dk], blocks along dv (stored [dk][dv])."""
    out = np.empty_like(S, dtype=np.float64)
    for b in range(S.shape[0]):
        for h in range(S.shape[1]):
            out[b, h] = quant.nvfp4_roundtrip(np.asarray(S[b, h], np.float32).T).T
    return out


WORKLOADS = {"gdn": (W.TINY_GDN, gdn), "kda": (W.TINY_KDA, kda)}


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_isolation_decode(kind):
    base, rule = WORKLOADS[kind]
    w = base.with_(init_std=0.5, seed=300)
    gp = W.gdn_params(w)
    S0 = W.gdn_init_states(w, range(w.batch))
    plain = decode.GDNReplay(S0, rule=rule)
    rc = decode.GDNReplay(S0, rule=rule, read_copy="nvfp4")
    conv = decode.GDNConventional(S0, rule=rule)
    gap = 0.0
    for t in range(48):
        tok = W.gdn_step(w, t, range(w.batch), gp)
        o_plain, o_rc, o_conv = plain.step(tok), rc.step(tok), conv.step(tok)
        np.testing.assert_allclose(o_plain, o_conv, rtol=1e-10, atol=1e-10)
        gap = max(gap, float(np.linalg.norm(o_rc - o_conv) / np.linalg.norm(o_conv)))
        if t % 16 == 15:
            assert np.array_equal(rc.ckpt, plain.ckpt)          # the copy never reaches the fold
            np.testing.assert_allclose(rc.ckpt, conv.S, rtol=1e-10, atol=1e-12)
            assert np.array_equal(rc.view, _nvfp4_view(rc.ckpt))  # and is refreshed from it
    assert gap > 1e-3            # outputs really read the 4-bit copy


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_isolation_speculative(kind):
    base, rule = WORKLOADS[kind]
    w = base.with_(init_std=0.5, seed=301, max_draft=4)
    gp = W.gdn_params(w)
    S0 = W.gdn_init_states(w, range(w.batch))
    plain = decode.GDNReplay(S0, rule=rule, max_draft=4)
    rc = decode.GDNReplay(S0, rule=rule, max_draft=4, read_copy="nvfp4")
    folds = 0
    for r in range(12):
        drafts = [W.gdn_step(w, 100 + 4 * r + d, range(w.batch), gp) for d in range(4)]
        acc = W.accepted_counts(w.seed, r, w.batch, 4)
        y_plain, y_rc = plain.spec_append(drafts), rc.spec_append(drafts)
        assert not np.allclose(y_plain, y_rc, rtol=1e-6, atol=1e-9)
        before = rc.ring.n_ckpt[:]
        plain.spec_commit(acc)
        rc.spec_commit(acc)
        folds += sum(a != b for a, b in zip(before, rc.ring.n_ckpt))
        assert np.array_equal(rc.ckpt, plain.ckpt)
        assert np.array_equal(rc.view, _nvfp4_view(rc.ckpt))
    assert folds > 0


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_no_writes_read_the_copy(kind):
    """beta = 0: o_t = gamma_t * S0_hat q_t (KDA: S0_hat (gamma_t * q_t)), S0_hat the NVFP4 round trip."""
    base, rule = WORKLOADS[kind]
    w = base.with_(init_std=0.5, seed=302)
    gp = W.gdn_params(w)
    S0 = W.gdn_init_states(w, range(w.batch))
    rc = decode.GDNReplay(S0, rule=rule, read_copy="nvfp4")
    Shat = _nvfp4_view(S0)
    logg = np.zeros((w.batch, w.n_v, w.dk)) if kind == "kda" else np.zeros((w.batch, w.n_v))
    for t in range(15):                  # one window, no flush
        tok = W.gdn_step(w, t, range(w.batch), gp)
        tok["beta"] = np.zeros_like(tok["beta"])
        logg = logg + np.asarray(tok["g"], np.float64)
        q = gdn.expand_qk(tok["q"], w.n_v)
        if kind == "kda":
            want = np.einsum("bhvk,bhk->bhv", Shat, np.exp(logg) * q)
        else:
            want = np.exp(logg)[:, :, None] * np.einsum("bhvk,bhk->bhv", Shat, q)
        np.testing.assert_allclose(rc.step(tok), want, rtol=1e-9, atol=1e-12)
