"""GPU parity over the rest of the compiled configurations: Mamba-2 state
shapes 64 x 64 and 128 x 128, GDN 64 x 64, bf16 inputs on small layers,
speculative rounds with 2 and 8 drafts, and speculative rounds over
low-precision checkpoints and the NVFP4 read copy (append reads the copy,
commit folds rewrite it)."""
import numpy as np
import pytest
import torch

import ssm_decode_checkpoint_amd as rs
import workloads as W
from oracle import decode
from oracle.ring import RingModel
from gpu_harness import (gdn_layer, gdn_tok_dev, load_state_f32, m2_drafts_dev, m2_layer, m2_tok_dev, params_dev,
                         read_meta, read_state_f32, rel_l2, require_gpu, y_buf)

pytestmark = pytest.mark.gpu


def setup_module(_):
    require_gpu()


def _replay_vs_conv(w, steps, tol):
    p = W.m2_params(w)
    A, D = params_dev(p)
    H0 = W.m2_init_states(w, range(w.batch))
    layer, bufs = m2_layer(w)
    load_state_f32(layer, bufs, H0)
    ref = decode.M2Conventional(H0, p["A"], p["D"])
    model = RingModel(w.batch)
    worst = 0.0
    for t in range(steps):
        tok = W.m2_step(w, t, range(w.batch))
        y = y_buf(w.batch, w.nheads, w.headdim)
        if model.is_flush_step(0):
            rs.rs_step_flush(layer, bufs, m2_tok_dev(tok, w.in_dtype), A, D, y)
            for b in range(w.batch):
                model.flush(b)
        else:
            rs.rs_step_nonflush(layer, bufs, m2_tok_dev(tok, w.in_dtype), A, D, y)
            for b in range(w.batch):
                model.nonflush(b)
        worst = max(worst, rel_l2(y.cpu().numpy(), ref.step(tok)))
    nck, ln, *_ = read_meta(layer, bufs)
    assert list(nck) == model.n_ckpt and list(ln) == model.len
    assert rel_l2(read_state_f32(layer, bufs), ref.H) <= tol
    return worst


@pytest.mark.parametrize("shape", [(64, 64, 8, 2), (128, 128, 8, 4), (128, 64, 16, 2), (16, 16, 6, 3)])
@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
def test_mamba2_shapes(shape, in_dtype):
    n, p, h, g = shape
    w = W.TINY_M2.with_(batch=3, nheads=h, headdim=p, dstate=n, ngroups=g, in_dtype=in_dtype, init_std=0.3,
                        seed=80 + n + p)
    worst = _replay_vs_conv(w, 48, 1e-5)      # ends on a flush: the checkpoint is the state
    assert worst <= 1e-5, worst


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
def test_gdn_64(in_dtype):
    w = W.TINY_GDN.with_(batch=3, n_qk=2, n_v=6, dk=64, dv=64, in_dtype=in_dtype, init_std=0.3, seed=90)
    gp = W.gdn_params(w)
    S0 = W.gdn_init_states(w, range(w.batch))
    layer, bufs = gdn_layer(w)
    load_state_f32(layer, bufs, S0)
    ref = decode.GDNConventional(S0)
    worst = 0.0
    for t in range(48):                      # ends on a flush: the checkpoint is the state
        tok = W.gdn_step(w, t, range(w.batch), gp)
        o = y_buf(w.batch, w.n_v, w.dv)
        fn = rs.rs_step_flush if t % 16 == 15 else rs.rs_step_nonflush
        fn(layer, bufs, gdn_tok_dev(tok, w.in_dtype), None, None, o)
        worst = max(worst, rel_l2(o.cpu().numpy(), ref.step(tok)))
    assert worst <= 1e-5, worst
    assert rel_l2(read_state_f32(layer, bufs), ref.S) <= 1e-5


def _spec(w, K, rounds, ckpt=rs.RS_F32, read_copy=rs.RS_NONE, oracle_fmt="f32_exact", oracle_rc=None):
    p = W.m2_params(w)
    A, D = params_dev(p)
    H0 = W.m2_init_states(w, range(w.batch))
    layer, bufs = m2_layer(w, ckpt_dtype=ckpt, read_copy=read_copy, fuse=1)
    if ckpt == rs.RS_F32:
        load_state_f32(layer, bufs, H0)
    if read_copy == rs.RS_NVFP4:
        rs.rs_requant_read_copy(layer, bufs)
    exact = decode.M2Conventional(H0, p["A"], p["D"])
    same = decode.M2Replay(H0, p["A"], p["D"], max_draft=w.max_draft, ckpt_fmt=oracle_fmt, read_copy=oracle_rc)
    model = RingModel(w.batch, max_draft=w.max_draft)
    worst_same = worst_exact = 0.0
    for r in range(rounds):
        drafts = [W.m2_step(w, 2000 + r * K + d, range(w.batch)) for d in range(K)]
        acc = W.accepted_counts(w.seed, r, w.batch, K)
        y = y_buf(w.batch, w.nheads, w.headdim, K=K)
        rs.rs_spec_append(layer, bufs, m2_drafts_dev(drafts, w.in_dtype), K, A, D, y)
        rs.rs_spec_commit(layer, bufs, torch.from_numpy(acc).cuda(), A, D)
        for b in range(w.batch):
            model.spec_append(b, K)
            model.spec_commit(b, int(acc[b]))
        yg = y.cpu().numpy()
        worst_same = max(worst_same, rel_l2(yg, same.spec_append(drafts)))
        same.spec_commit(acc)
        worst_exact = max(worst_exact, rel_l2(yg, exact.spec_round(drafts, acc)))
        nck, ln, nd, err, _ = read_meta(layer, bufs)
        assert list(nck) == model.n_ckpt and list(ln) == model.len and not err.any() and not nd.any()
    return worst_same, worst_exact, model


@pytest.mark.parametrize("K,kmax", [(2, 2), (8, 8), (3, 8)])
def test_spec_draft_counts(K, kmax):
    w = W.TINY_M2.with_(max_draft=kmax, init_std=0.4, seed=100 + K + kmax)
    ws, we, model = _spec(w, K, 24)
    assert ws <= 1e-5 and we <= 1e-5, (ws, we)
    assert max(model.n_ckpt) > 0


@pytest.mark.parametrize("ckpt,rc,fmt,gate", [(rs.RS_F32, rs.RS_NVFP4, "f32", 1e-4),
                                               (rs.RS_F16, rs.RS_NONE, "f16", 1e-4),
                                               (rs.RS_F16, rs.RS_NVFP4, "f16", 1e-2),
                                               (rs.RS_FP8E4M3, rs.RS_NONE, "fp8", 1e-2),
                                               (rs.RS_NVFP4, rs.RS_NONE, "nvfp4", 1e-2)])
def test_spec_low_precision(ckpt, rc, fmt, gate):
    """Zero initial state (as the low-precision workload); the GPU follows the
    oracle running the same storage formats."""
    w = W.TINY_M2.with_(max_draft=4, init_std=0.0, seed=110)
    ws, we, _ = _spec(w, 4, 20, ckpt=ckpt, read_copy=rc, oracle_fmt=fmt,
                      oracle_rc="nvfp4" if rc == rs.RS_NVFP4 else None)
    print(f"spec {fmt}{' + nvfp4 reads' if rc else ''}: vs same-format oracle {ws:.2e}, vs exact {we:.2e}")
    assert ws <= gate


def test_mamba2_batch1_full_heads():
    """One sequence of the 128-head Nemotron-style layer (the small end of the
    batch sweep): 128 workgroups share one sequence's counters."""
    w = W.M2_NEMOTRON.with_(batch=1, init_std=0.1, seed=120)
    worst = _replay_vs_conv(w, 32, 1e-5)
    assert worst <= 1e-5, worst
