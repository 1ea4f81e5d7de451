"""GPU parity of the low-precision checkpoint read paths from codes the oracle holds.

Every window starts from a non-zero checkpoint whose codes and scales the
oracle encoded (fp16, fp8 with a matrix scale, the uniform NVFP4 checkpoint,
and fp32 with the NVFP4 read copy): the device reads exactly the values the
oracle reads, so its outputs are gated at the fp32 tolerance. After each flush
or speculative commit-fold, the device's stored codes are compared with the
oracle's codes of its own float64 fold: only flips next to a rounding boundary
are allowed, and they are counted (sitech.ge ReplaySSM page, "Bounding
quantization error"). The device is then loaded with the oracle's codes, so
the next window again reads identical values.
"""
import numpy as np
import pytest
import torch

import ssm_decode_checkpoint_amd as rs
import workloads as W
from oracle import decode
from gpu_harness import m2_drafts_dev, m2_layer, m2_tok_dev, params_dev, read_meta, rel_l2, require_gpu, y_buf
import lowprec_codes as LC

pytestmark = pytest.mark.gpu

TOL = 1e-5
CODE = {"f32": rs.RS_F32, "f16": rs.RS_F16, "fp8": rs.RS_FP8E4M3, "nvfp4": rs.RS_NVFP4}

# tiny layer; 128 x 64 heads four to a group (wavefront-per-head read kernel) with fp32 and
# bf16 inputs; 128 x 64 heads two to a group (workgroup-per-head kernel)
SHAPES = [dict(), dict(batch=3, nheads=8, ngroups=2, dstate=128, headdim=64),
          dict(batch=3, nheads=8, ngroups=2, dstate=128, headdim=64, in_dtype="bf16"),
          dict(batch=3, nheads=6, ngroups=3, dstate=128, headdim=64),
          # bf16 records with 8 or more heads per group: two heads per wavefront on FP8 / NVFP4 reads
          dict(batch=3, nheads=16, ngroups=1, dstate=128, headdim=64, in_dtype="bf16"),
          dict(batch=2, nheads=16, ngroups=2, dstate=128, headdim=64, in_dtype="bf16")]
FORMATS = [("f16", None), ("fp8", None), ("nvfp4", None), ("f16", "nvfp4"), ("fp8", "nvfp4"), ("f32", "nvfp4")]


def setup_module(_):
    require_gpu()


class FoldKeepingReplay(decode.M2Replay):
    """The oracle's replay decode, keeping each sequence's last fold (float64,
    before storage rounding) so the test can encode it."""

    def __init__(self, *a, **k):
        super().__init__(*a, **k)
        self.folds = {}

    def _set_ckpt(self, b, Hn):
        self.folds[b] = np.asarray(Hn[0], np.float64).copy()
        super()._set_ckpt(b, Hn)


def _stored(logical):
    return np.ascontiguousarray(np.swapaxes(np.asarray(logical), -1, -2))


class Synced:
    """A device layer whose checkpoint holds the oracle's codes at the start of each window."""

    def __init__(self, w, fmt, rc, p, H0):
        self.fmt, self.rc = fmt, rc
        self.layer, self.bufs = m2_layer(w, ckpt_dtype=CODE[fmt], read_copy=rs.RS_NVFP4 if rc else rs.RS_NONE,
                                         fuse=1)
        self.ref = FoldKeepingReplay(H0, p["A"], p["D"], max_draft=w.max_draft, ckpt_fmt=fmt, read_copy=rc)
        self.enc = LC.encode(fmt, _stored(np.asarray(H0, np.float32)))
        # the oracle reads exactly these codes' values
        assert np.array_equal(LC.decode(fmt, self.enc).astype(np.float64), _stored(self.ref.ckpt))
        self.load()
        self.flips = LC.Flips()
        self.rc_flips = LC.Flips()
        self.folds = 0

    def load(self):
        raw = LC.to_device_bytes(self.layer, self.fmt, self.enc)
        self.bufs.ckpt.copy_(torch.from_numpy(raw).cuda())
        if self.rc:
            rs.rs_requant_read_copy(self.layer, self.bufs)

    def after_fold(self, seqs):
        """Compare the device's codes of the sequences just folded with the oracle's,
        check the fused read copy, then give the device the oracle's codes."""
        if not seqs:
            return
        self.folds += len(seqs)
        gpu = LC.from_device_bytes(self.layer, self.fmt, self.bufs.ckpt.cpu().numpy())
        fold = np.stack([_stored(self.ref.folds[b]) for b in seqs])
        ora = LC.encode(self.fmt, fold.astype(np.float32))
        sub = {k: v[seqs] for k, v in gpu.items()}
        fl = LC.compare(self.fmt, sub, ora, fold, TOL)
        assert not fl.bad, fl.bad[:4]
        self.flips.add(fl)
        if self.rc:
            fused = self.bufs.read_copy.clone()
            rs.rs_requant_read_copy(self.layer, self.bufs)
            assert torch.equal(fused, self.bufs.read_copy), "fused read copy != standalone requant"
            if self.fmt == "f32":
                # over an fp32 checkpoint the copy is NVFP4 of the fold itself
                got = _read_copy(self.layer, self.bufs)
                rc_ora = LC.encode("nvfp4", fold.astype(np.float32))
                rfl = LC.compare("nvfp4", {k: v[seqs] for k, v in got.items()}, rc_ora, fold, TOL)
                assert not rfl.bad, rfl.bad[:4]
                self.rc_flips.add(rfl)
        for k in self.enc:
            self.enc[k][seqs] = ora[k]
        self.load()

    def report(self):
        f, r = self.flips, self.rc_flips
        s = (f"{self.folds} folds: checkpoint code flips {f.elements}/{f.total}, block scale flips {f.scales}, "
             f"worst distance {f.worst:.2f} x tol")
        if r.total:
            s += f"; read-copy code flips {r.elements}/{r.total}, block scale flips {r.scales}"
        return s


def _read_copy(layer, bufs):
    b, h, r, c = layer.cfg.batch, layer.heads, layer.rows, layer.cols
    raw = bufs.read_copy.cpu().numpy()
    n = b * h * r * c
    return {"codes": LC.quant.unpack_nibbles(raw[: n // 2].reshape(b, h, r, c // 2)),
            "scales": raw[layer.nv_scale_off: layer.nv_scale_off + n // 16].reshape(b, h, r, c // 16),
            "ts": raw[layer.nv_tscale_off: layer.nv_tscale_off + 4 * b * h].view(np.float32).reshape(b, h)}


@pytest.mark.parametrize("fmt,rc", FORMATS)
@pytest.mark.parametrize("shape", SHAPES)
def test_lowprec_decode_from_oracle_codes(fmt, rc, shape):
    """48 decode steps (3 flushes) from a non-zero oracle-encoded checkpoint: every
    output within 1e-5 of the same-format oracle, post-fold codes flip only at
    rounding boundaries."""
    w = W.TINY_M2.with_(init_std=0.5, seed=170, **shape)
    p = W.m2_params(w)
    A, D = params_dev(p)
    H0 = W.m2_init_states(w, range(w.batch))
    dev = Synced(w, fmt, rc, p, H0)
    worst = 0.0
    for t in range(48):
        tok = W.m2_step(w, t, range(w.batch))
        y = y_buf(w.batch, w.nheads, w.headdim)
        flush = t % 16 == 15
        (rs.rs_step_flush if flush else rs.rs_step_nonflush)(dev.layer, dev.bufs, m2_tok_dev(tok, w.in_dtype),
                                                             A, D, y)
        e = rel_l2(y.cpu().numpy(), dev.ref.step(tok))
        assert e <= TOL, f"step {t}: rel-L2 {e:.3e} vs the same-format oracle"
        worst = max(worst, e)
        if flush:
            dev.after_fold(list(range(w.batch)))
    print(f"{fmt}{' + nvfp4 reads' if rc else ''} {shape}: worst rel-L2 {worst:.2e}; {dev.report()}")


@pytest.mark.parametrize("fmt,rc", FORMATS)
@pytest.mark.parametrize("shape", SHAPES[:2])
def test_lowprec_spec_from_oracle_codes(fmt, rc, shape):
    """Speculative rounds (4 drafts, accepted ~U{0..4}) over the same checkpoints:
    verify outputs within 1e-5 of the same-format oracle; commit-folds checked
    like flushes."""
    w = W.TINY_M2.with_(init_std=0.5, seed=171, max_draft=4, **shape)
    p = W.m2_params(w)
    A, D = params_dev(p)
    H0 = W.m2_init_states(w, range(w.batch))
    dev = Synced(w, fmt, rc, p, H0)
    K, worst = 4, 0.0
    for r in range(20):
        drafts = [W.m2_step(w, 3000 + r * K + d, range(w.batch)) for d in range(K)]
        acc = W.accepted_counts(w.seed, r, w.batch, K)
        y = y_buf(w.batch, w.nheads, w.headdim, K=K)
        nck0 = read_meta(dev.layer, dev.bufs)[0].copy()
        rs.rs_spec_append(dev.layer, dev.bufs, m2_drafts_dev(drafts, w.in_dtype), K, A, D, y)
        e = rel_l2(y.cpu().numpy(), dev.ref.spec_append(drafts))
        assert e <= TOL, f"round {r}: verify rel-L2 {e:.3e}"
        worst = max(worst, e)
        rs.rs_spec_commit(dev.layer, dev.bufs, torch.from_numpy(acc).cuda(), A, D)
        dev.ref.folds.clear()
        dev.ref.spec_commit(acc)
        nck, ln, nd, err, _ = read_meta(dev.layer, dev.bufs)
        assert not err.any() and not nd.any()
        folded = [b for b in range(w.batch) if nck[b] != nck0[b]]
        assert sorted(folded) == sorted(dev.ref.folds), (folded, sorted(dev.ref.folds))
        dev.after_fold(folded)
    assert dev.folds > 0
    print(f"spec {fmt}{' + nvfp4 reads' if rc else ''} {shape}: worst rel-L2 {worst:.2e}; {dev.report()}")
