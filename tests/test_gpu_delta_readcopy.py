"""GPU parity of the NVFP4 read copy of the delta-rule layers (Gated DeltaNet
and Kimi Delta Attention; sitech.ge ReplaySSM page, "Bounding quantization
error": reads go to a 4-bit copy while the recurrence keeps fp32).

* The quantizer is bit-exact against the oracle's on GDN state shapes,
  including values on E2M1 rounding boundaries.
* Decode and speculative rounds against the oracle with the same read copy:
  each window starts from a copy the device and the oracle share (the device's
  is rewritten from the oracle's codes after each fold), so every output is
  gated at the fp32 tolerance; after each fold the device's fp32 checkpoint is
  compared with the oracle's (the folds re-solve their rows from the
  checkpoint, so they see no read error) and its fresh copy must be the
  quantizer's output for that checkpoint, bit for bit.
* Isolation: the checkpoints with and without a read copy agree to fp32
  rounding after every fold, and outputs really read the copy.
"""
import numpy as np
import pytest
import torch

import ssm_decode_checkpoint_amd as rs
import workloads as W
from oracle import decode, gdn, kda, quant
from gpu_harness import (gdn_drafts_dev, gdn_layer, gdn_tok_dev, load_state_f32, read_meta, read_state_f32, rel_l2, require_gpu,
                         y_buf)
import lowprec_codes as LC

pytestmark = pytest.mark.gpu
TOL = 1e-5


def setup_module(_):
    require_gpu()


def _layer(w, read_copy=True):
    return gdn_layer(w, read_copy=rs.RS_NVFP4 if read_copy else rs.RS_NONE)


def _read_copy(layer, bufs):
    b, h, r, c = layer.cfg.batch, layer.heads, layer.rows, layer.cols
    raw = bufs.read_copy.cpu().numpy()
    n = b * h * r * c
    return {"codes": quant.unpack_nibbles(raw[: n // 2].reshape(b, h, r, c // 2)),
            "scales": raw[layer.nv_scale_off: layer.nv_scale_off + n // 16].reshape(b, h, r, c // 16).copy(),
            "ts": raw[layer.nv_tscale_off: layer.nv_tscale_off + 4 * b * h].view(np.float32).reshape(b, h).copy()}


def _write_copy(layer, bufs, enc):
    raw = np.zeros(int(layer.read_copy_bytes), np.uint8)
    codes = quant.pack_nibbles(enc["codes"]).reshape(-1)
    raw[: codes.size] = codes
    sc = enc["scales"].reshape(-1)
    raw[layer.nv_scale_off: layer.nv_scale_off + sc.size] = sc
    ts = enc["ts"].reshape(-1).view(np.uint8)
    raw[layer.nv_tscale_off: layer.nv_tscale_off + ts.size] = ts
    bufs.read_copy.copy_(torch.from_numpy(raw).cuda())


def _stored(S):
    return np.ascontiguousarray(np.swapaxes(np.asarray(S), -1, -2))


SHAPES = [dict(), dict(batch=2, n_qk=2, n_v=4, dk=128, dv=128, in_dtype="bf16"),
          dict(batch=2, n_qk=1, n_v=2, dk=64, dv=64)]


@pytest.mark.parametrize("shape", SHAPES)
def test_requant_bit_exact_gdn_shapes(shape):
    w = W.TINY_GDN.with_(**shape)
    layer, bufs = _layer(w)
    tiles = W.state_tiles(60, 0, (w.batch, w.n_v, w.dk, w.dv), std=0.2, heavy_tail=True)
    tiles[0, 0] = 0.0
    rs.ckpt_f32_view(layer, bufs).copy_(torch.from_numpy(tiles).cuda())
    rs.rs_requant_read_copy(layer, bufs)
    got = _read_copy(layer, bufs)
    want = LC.encode("nvfp4", tiles)
    assert np.array_equal(got["ts"].view(np.uint32), want["ts"].view(np.uint32))
    assert np.array_equal(got["scales"], want["scales"])
    assert np.array_equal(got["codes"], want["codes"])


class Synced:
    """Device layer with a read copy, oracle with the same; after each fold the
    device takes the oracle's copy codes (its fp32 checkpoint stays its own)."""

    def __init__(self, w, S0, rule):
        self.layer, self.bufs = _layer(w)
        load_state_f32(self.layer, self.bufs, S0)
        rs.rs_requant_read_copy(self.layer, self.bufs)
        self.ref = decode.GDNReplay(S0, max_draft=w.max_draft, rule=rule, ckpt_fmt="f32", read_copy="nvfp4")
        self.sync()
        self.folds = 0
        self.worst_state = 0.0

    def sync(self):
        _write_copy(self.layer, self.bufs, LC.encode("nvfp4", _stored(self.ref.ckpt).astype(np.float32)))

    def after_fold(self, seqs):
        if not seqs:
            return
        self.folds += len(seqs)
        dev = read_state_f32(self.layer, self.bufs)
        self.worst_state = max(self.worst_state, rel_l2(dev[seqs], self.ref.ckpt[seqs]))
        assert self.worst_state <= TOL, self.worst_state
        # the copy the fold wrote is the quantizer's output for the device's checkpoint
        got = _read_copy(self.layer, self.bufs)
        want = LC.encode("nvfp4", _stored(dev).astype(np.float32))
        for k in want:
            assert np.array_equal(np.asarray(got[k])[seqs].view(np.uint8), np.asarray(want[k])[seqs].view(np.uint8)), k
        self.sync()


@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("shape", SHAPES)
def test_decode_reads_the_copy(shape, gate):
    base, rule = (W.TINY_GDN, gdn) if gate == "scalar" else (W.TINY_KDA, kda)
    w = base.with_(init_std=0.4, seed=310, **shape)
    gp = W.gdn_params(w)
    S0 = W.gdn_init_states(w, range(w.batch))
    dev = Synced(w, S0, rule)
    exact = decode.GDNConventional(S0, rule=rule)
    worst, gap = 0.0, 0.0
    for t in range(48):
        tok = W.gdn_step(w, t, range(w.batch), gp)
        o = y_buf(w.batch, w.n_v, w.dv)
        (rs.rs_step_flush if t % 16 == 15 else rs.rs_step_nonflush)(dev.layer, dev.bufs, gdn_tok_dev(tok, w.in_dtype),
                                                                     None, None, o)
        og = o.cpu().numpy()
        e = rel_l2(og, dev.ref.step(tok))
        assert e <= TOL, f"step {t}: {e:.3e}"
        worst = max(worst, e)
        gap = max(gap, rel_l2(og, exact.step(tok)))
        if t % 16 == 15:
            dev.after_fold(list(range(w.batch)))
    print(f"{gate} {shape}: worst rel-L2 vs same-copy oracle {worst:.2e}, state after folds {dev.worst_state:.2e}, "
          f"vs exact decoding {gap:.2e}")
    assert gap > 1e-3


@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("shape", SHAPES[:2])
def test_speculative_reads_the_copy(shape, gate):
    base, rule = (W.TINY_GDN, gdn) if gate == "scalar" else (W.TINY_KDA, kda)
    w = base.with_(init_std=0.4, seed=311, max_draft=4, **shape)
    gp = W.gdn_params(w)
    S0 = W.gdn_init_states(w, range(w.batch))
    dev = Synced(w, S0, rule)
    K, worst = 4, 0.0
    for r in range(16):
        drafts = [W.gdn_step(w, 500 + K * r + d, range(w.batch), gp) for d in range(K)]
        acc = W.accepted_counts(w.seed, r, w.batch, K)
        o = y_buf(w.batch, w.n_v, w.dv, K=K)
        rs.rs_spec_append(dev.layer, dev.bufs, gdn_drafts_dev(drafts, w.in_dtype), K, None, None, o)
        e = rel_l2(o.cpu().numpy(), dev.ref.spec_append(drafts))
        assert e <= TOL, f"round {r}: {e:.3e}"
        worst = max(worst, e)
        n0 = read_meta(dev.layer, dev.bufs)[0].copy()
        rs.rs_spec_commit(dev.layer, dev.bufs, torch.from_numpy(acc).cuda(), None, None)
        dev.ref.spec_commit(acc)
        nck, ln, nd, err, _ = read_meta(dev.layer, dev.bufs)
        assert not err.any() and not nd.any()
        assert list(nck) == dev.ref.ring.n_ckpt and list(ln) == dev.ref.ring.len
        dev.after_fold([b for b in range(w.batch) if nck[b] != n0[b]])
    assert dev.folds > 0
    print(f"spec {gate} {shape}: worst {worst:.2e}, state after folds {dev.worst_state:.2e}, folds {dev.folds}")


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_isolation_and_self_scheduling(gate):
    """The fp32 checkpoint with a read copy follows the one without it (to fp32
    rounding: the copy's folds re-solve their rows), through rs_step."""
    base = W.TINY_GDN if gate == "scalar" else W.TINY_KDA
    w = base.with_(batch=2, n_qk=2, n_v=4, dk=128, dv=128, in_dtype="bf16", init_std=0.4, seed=312)
    gp = W.gdn_params(w)
    S0 = W.gdn_init_states(w, range(w.batch))
    rc_l, rc_b = _layer(w)
    pl_l, pl_b = _layer(w, read_copy=False)
    for l, b in ((rc_l, rc_b), (pl_l, pl_b)):
        load_state_f32(l, b, S0)
    rs.rs_requant_read_copy(rc_l, rc_b)
    gap = 0.0
    for t in range(40):
        dtok = gdn_tok_dev(W.gdn_step(w, t, range(w.batch), gp), w.in_dtype)
        o1, o2 = y_buf(w.batch, w.n_v, w.dv), y_buf(w.batch, w.n_v, w.dv)
        rs.rs_step(rc_l, rc_b, dtok, None, None, o1)
        rs.rs_step(pl_l, pl_b, dtok, None, None, o2)
        gap = max(gap, rel_l2(o1.cpu().numpy(), o2.cpu().numpy()))
        if t % 16 == 15:
            assert rel_l2(read_state_f32(rc_l, rc_b), read_state_f32(pl_l, pl_b)) <= 1e-6
            fresh = rc_b.read_copy.clone()
            rs.rs_requant_read_copy(rc_l, rc_b)
            assert torch.equal(fresh, rc_b.read_copy)
    assert gap > 1e-3
