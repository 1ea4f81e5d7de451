"""GPU parity of the delta-rule layers' FP16 and FP8 checkpoints (Gated DeltaNet
and Kimi Delta Attention) from codes the oracle holds.

sitech.ge ReplaySSM page, "Bounding quantization error": the recurrence can be
kept in FP16 or FP8. Every window starts from a non-zero checkpoint whose codes
(and, for FP8, per-matrix scales) the oracle encoded, so the device reads
exactly the values the oracle reads and its outputs are gated at the fp32
tolerance. After each flush or speculative commit-fold the device's stored
codes are compared with the oracle's codes of its own float64 fold: only flips
next to a rounding boundary are allowed, and they are counted. The device is
then loaded with the oracle's codes, so the next window again reads identical
values. The FP8 folds store one scale per matrix, so the workgroup of a
state's first column slice folds both slices; the self-scheduling step and the
speculative commit take that path too.
"""
import numpy as np
import pytest
import torch

import ssm_decode_checkpoint_amd as rs
import workloads as W
from oracle import decode, gdn, kda
from gpu_harness import gdn_drafts_dev, gdn_layer, gdn_tok_dev, read_meta, rel_l2, require_gpu, y_buf
import lowprec_codes as LC

pytestmark = pytest.mark.gpu

TOL = 1e-5
CODE = {"f16": rs.RS_F16, "fp8": rs.RS_FP8E4M3}
SHAPES = [dict(), dict(batch=2, n_qk=2, n_v=4, dk=128, dv=128, in_dtype="bf16")]


def setup_module(_):
    require_gpu()


class FoldKeepingReplay(decode.GDNReplay):
    """The oracle's replay decode, keeping each sequence's last fold (float64,
    before storage rounding) so the test can encode it."""

    def __init__(self, *a, **k):
        super().__init__(*a, **k)
        self.folds = {}

    def _set_ckpt(self, b, Sn):
        self.folds[b] = np.asarray(Sn[0], np.float64).copy()
        super()._set_ckpt(b, Sn)


def _stored(logical):
    return np.ascontiguousarray(np.swapaxes(np.asarray(logical), -1, -2))


class Synced:
    def __init__(self, w, fmt, rule, S0):
        self.fmt = fmt
        self.layer, self.bufs = gdn_layer(w, ckpt_dtype=CODE[fmt])
        self.ref = FoldKeepingReplay(S0, max_draft=w.max_draft, rule=rule, ckpt_fmt=fmt)
        self.enc = LC.encode(fmt, _stored(np.asarray(S0, np.float32)))
        assert np.array_equal(LC.decode(fmt, self.enc).astype(np.float64), _stored(self.ref.ckpt))
        self.load()
        self.flips = LC.Flips()
        self.folds = 0

    def load(self):
        self.bufs.ckpt.copy_(torch.from_numpy(LC.to_device_bytes(self.layer, self.fmt, self.enc)).cuda())

    def after_fold(self, seqs):
        if not seqs:
            return
        self.folds += len(seqs)
        gpu = LC.from_device_bytes(self.layer, self.fmt, self.bufs.ckpt.cpu().numpy())
        fold = np.stack([_stored(self.ref.folds[b]) for b in seqs])
        ora = LC.encode(self.fmt, fold.astype(np.float32))
        fl = LC.compare(self.fmt, {k: v[seqs] for k, v in gpu.items()}, ora, fold, TOL)
        assert not fl.bad, fl.bad[:4]
        self.flips.add(fl)
        for k in self.enc:
            self.enc[k][seqs] = ora[k]
        self.load()

    def report(self):
        f = self.flips
        return f"{self.folds} folds: code flips {f.elements}/{f.total}, worst distance {f.worst:.2f} x tol"


def _case(gate, shape, seed, **kw):
    base, rule = (W.TINY_GDN, gdn) if gate == "scalar" else (W.TINY_KDA, kda)
    w = base.with_(init_std=0.4, seed=seed, **kw, **shape)
    return w, rule, W.gdn_params(w), W.gdn_init_states(w, range(w.batch))


@pytest.mark.parametrize("fmt", ["f16", "fp8"])
@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("auto", [False, True])
def test_delta_lowprec_decode_from_oracle_codes(fmt, gate, shape, auto):
    """48 decode steps (3 flushes) from a non-zero oracle-encoded checkpoint, by
    explicit non-flush / flush calls or by the self-scheduling step: every output
    within 1e-5 of the same-format oracle, post-fold codes flip only at rounding
    boundaries."""
    w, rule, gp, S0 = _case(gate, shape, 330)
    dev = Synced(w, fmt, rule, S0)
    worst = 0.0
    for t in range(48):
        tok = W.gdn_step(w, t, range(w.batch), gp)
        o = y_buf(w.batch, w.n_v, w.dv)
        flush = t % 16 == 15
        fn = rs.rs_step if auto else (rs.rs_step_flush if flush else rs.rs_step_nonflush)
        fn(dev.layer, dev.bufs, gdn_tok_dev(tok, w.in_dtype), None, None, o)
        e = rel_l2(o.cpu().numpy(), dev.ref.step(tok))
        assert e <= TOL, f"step {t}: rel-L2 {e:.3e} vs the same-format oracle"
        worst = max(worst, e)
        if flush:
            dev.after_fold(list(range(w.batch)))
    nck, ln, nd, err, _ = read_meta(dev.layer, dev.bufs)
    assert not err.any() and list(nck) == dev.ref.ring.n_ckpt and list(ln) == dev.ref.ring.len
    print(f"{fmt} {gate} {shape} auto={auto}: worst rel-L2 {worst:.2e}; {dev.report()}")


@pytest.mark.parametrize("fmt", ["f16", "fp8"])
@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("shape", SHAPES)
def test_delta_lowprec_spec_from_oracle_codes(fmt, gate, shape):
    """Speculative rounds (4 drafts, accepted counts ~U{0..4}) over the same
    checkpoints: verify outputs within 1e-5 of the same-format oracle;
    commit-folds checked like flushes."""
    w, rule, gp, S0 = _case(gate, shape, 331, max_draft=4)
    dev = Synced(w, fmt, rule, S0)
    K, worst = 4, 0.0
    for r in range(16):
        drafts = [W.gdn_step(w, 700 + K * r + d, range(w.batch), gp) for d in range(K)]
        acc = W.accepted_counts(w.seed, r, w.batch, K)
        o = y_buf(w.batch, w.n_v, w.dv, K=K)
        rs.rs_spec_append(dev.layer, dev.bufs, gdn_drafts_dev(drafts, w.in_dtype), K, None, None, o)
        e = rel_l2(o.cpu().numpy(), dev.ref.spec_append(drafts))
        assert e <= TOL, f"round {r}: verify rel-L2 {e:.3e}"
        worst = max(worst, e)
        nck0 = read_meta(dev.layer, dev.bufs)[0].copy()
        rs.rs_spec_commit(dev.layer, dev.bufs, torch.from_numpy(acc).cuda(), None, None)
        dev.ref.folds.clear()
        dev.ref.spec_commit(acc)
        nck, ln, nd, err, _ = read_meta(dev.layer, dev.bufs)
        assert not err.any() and not nd.any()
        folded = [b for b in range(w.batch) if nck[b] != nck0[b]]
        assert sorted(folded) == sorted(dev.ref.folds), (folded, sorted(dev.ref.folds))
        dev.after_fold(folded)
    assert dev.folds > 0
    print(f"spec {fmt} {gate} {shape}: worst rel-L2 {worst:.2e}; {dev.report()}")
