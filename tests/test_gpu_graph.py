"""The decode calls inside a captured HIP graph (torch.cuda.CUDAGraph).

The library allocates nothing, never synchronises, issues no memset or copy,
and advances the per-sequence counters inside its own kernels, so a window of
steps can be captured once and replayed: each replay continues every
sequence's buffer from where the previous one left it. Checked the way such
graphs have to be checked: the graph is replayed several times with eager
work and synchronisations between the replays, and every replay's outputs,
and the state after it, must equal bit for bit an eager run of the same calls
on a second buffer set from the same initial state.

Cases: a Mamba-2 window of 15 non-flush steps and a flush; a Mamba-2
speculative round (append 4 drafts, commit); a Gated DeltaNet window through
the self-scheduling step.
"""
import numpy as np
import pytest
import torch

import ssm_decode_checkpoint_amd as rs
import workloads as W
from gpu_harness import (DEV, gdn_layer, gdn_tok_dev, load_state_f32, m2_drafts_dev, m2_layer, m2_tok_dev, params_dev,
                         read_meta, require_gpu, y_buf)

pytestmark = pytest.mark.gpu
RING = 16


def setup_module(_):
    require_gpu()


def _capture(calls):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    return g


def _busy():
    """Eager work of the program's own between replays."""
    a = torch.randn(512, 512, device=DEV)
    (a @ a).sum().item()


def test_mamba2_window_replays_match_eager():
    w = W.TINY_M2.with_(batch=6, init_std=0.3, seed=601, in_dtype="bf16")
    p = W.m2_params(w)
    A, D = params_dev(p)
    H0 = W.m2_init_states(w, range(w.batch))
    toks = [m2_tok_dev(W.m2_step(w, t, range(w.batch)), "bf16") for t in range(RING)]
    (lg, bg), (le, be) = m2_layer(w), m2_layer(w)
    load_state_f32(lg, bg, H0)
    load_state_f32(le, be, H0)
    yg = [y_buf(w.batch, w.nheads, w.headdim) for _ in range(RING)]
    ye = [y_buf(w.batch, w.nheads, w.headdim) for _ in range(RING)]

    def window(layer, bufs, ys):
        for t in range(RING):
            fn = rs.rs_step_flush if t == RING - 1 else rs.rs_step_nonflush
            fn(layer, bufs, toks[t], A, D, ys[t])

    g = _capture(lambda: window(lg, bg, yg))
    for rep in range(3):
        _busy()
        g.replay()
        torch.cuda.synchronize()
        window(le, be, ye)
        torch.cuda.synchronize()
        for t in range(RING):
            assert torch.equal(yg[t], ye[t]), (rep, t)
        assert torch.equal(rs.ckpt_f32_view(lg, bg), rs.ckpt_f32_view(le, be)), rep
        mg, me = read_meta(lg, bg), read_meta(le, be)
        for a, b in zip(mg, me):
            assert np.array_equal(a, b), rep
        assert mg[0][0] == RING * (rep + 1) and not mg[3].any()


def test_mamba2_spec_round_replays_match_eager():
    w = W.TINY_M2.with_(batch=5, init_std=0.3, seed=602, in_dtype="bf16", max_draft=4)
    p = W.m2_params(w)
    A, D = params_dev(p)
    H0 = W.m2_init_states(w, range(w.batch))
    K = 4
    drafts = m2_drafts_dev([W.m2_step(w, 100 + d, range(w.batch)) for d in range(K)], "bf16")
    acc = torch.from_numpy(W.accepted_counts(w.seed, 0, w.batch, K)).to(DEV)
    (lg, bg), (le, be) = m2_layer(w), m2_layer(w)
    load_state_f32(lg, bg, H0)
    load_state_f32(le, be, H0)
    yg, ye = y_buf(w.batch, w.nheads, w.headdim, K=K), y_buf(w.batch, w.nheads, w.headdim, K=K)

    def round_(layer, bufs, y):
        rs.rs_spec_append(layer, bufs, drafts, K, A, D, y)
        rs.rs_spec_commit(layer, bufs, acc, A, D)

    g = _capture(lambda: round_(lg, bg, yg))
    for rep in range(4):                 # enough rounds that commits fold
        _busy()
        g.replay()
        torch.cuda.synchronize()
        round_(le, be, ye)
        torch.cuda.synchronize()
        assert torch.equal(yg, ye), rep
        assert torch.equal(rs.ckpt_f32_view(lg, bg), rs.ckpt_f32_view(le, be)), rep
        for a, b in zip(read_meta(lg, bg), read_meta(le, be)):
            assert np.array_equal(a, b), rep
    assert not read_meta(lg, bg)[3].any()


def test_gdn_self_scheduling_window_replays_match_eager():
    w = W.TINY_GDN.with_(batch=4, init_std=0.3, seed=603, in_dtype="bf16")
    S0 = W.gdn_init_states(w, range(w.batch))
    toks = [gdn_tok_dev(W.gdn_step(w, t, range(w.batch)), "bf16") for t in range(RING)]
    (lg, bg), (le, be) = gdn_layer(w), gdn_layer(w)
    load_state_f32(lg, bg, S0)
    load_state_f32(le, be, S0)
    og = [y_buf(w.batch, w.n_v, w.dv) for _ in range(RING)]
    oe = [y_buf(w.batch, w.n_v, w.dv) for _ in range(RING)]

    def window(layer, bufs, os_):
        for t in range(RING):
            rs.rs_step(layer, bufs, toks[t], None, None, os_[t])

    g = _capture(lambda: window(lg, bg, og))
    for rep in range(3):
        _busy()
        g.replay()
        torch.cuda.synchronize()
        window(le, be, oe)
        torch.cuda.synchronize()
        for t in range(RING):
            assert torch.equal(og[t], oe[t]), (rep, t)
        assert torch.equal(rs.ckpt_f32_view(lg, bg), rs.ckpt_f32_view(le, be)), rep
