"""GPU checks of rs_copy_slots (prefix caching and forks).

A sequence's state at any token is its checkpoint, buffer entries and
counters, so a copied sequence must continue exactly as its source: same
outputs bit for bit (same kernels, same inputs, same flush schedule), and
against the fp64 oracle snapshotted at the time of the save (the same-method
replay and the plain recurrence). Covered: forks inside one buffer set, a
prefix cache of another batch (save, decode on, restore into other slots),
Mamba-2, Gated DeltaNet and KDA (their cached u rows travel with the entries),
an FP8 checkpoint with an NVFP4 read copy, conventional mode, and a copy taken
while drafts are pending.
"""
import copy

import numpy as np
import pytest
import torch

import ssm_decode_checkpoint_amd as rs
import workloads as W
from oracle import decode, gdn, kda
from gpu_harness import (DEV, gdn_drafts_dev, gdn_layer, gdn_tok_dev, load_state_f32, m2_layer, m2_tok_dev,
                         params_dev, read_meta, rel_l2, require_gpu, y_buf)

pytestmark = pytest.mark.gpu


def setup_module(_):
    require_gpu()


def _seqs(v):
    return torch.tensor(v, dtype=torch.int32, device=DEV)


def _dup_rows(tok, pairs):
    """Inputs where row d repeats row s for each (s, d)."""
    out = {k: v.copy() for k, v in tok.items()}
    for s, d in pairs:
        for k in out:
            out[k][d] = tok[k][s]
    return out


def _m2_case(w, **layer_kw):
    p = W.m2_params(w)
    A, D = params_dev(p)
    layer, bufs = m2_layer(w, **layer_kw)
    H0 = W.m2_init_states(w, range(w.batch))
    return p, A, D, layer, bufs, H0


def test_mamba2_fork_is_bit_exact_and_matches_oracle():
    w = W.TINY_M2.with_(batch=4, init_std=0.4, seed=200)
    p, A, D, layer, bufs, H0 = _m2_case(w)
    load_state_f32(layer, bufs, H0)
    rep = decode.M2Replay(H0, p["A"], p["D"])
    conv = decode.M2Conventional(H0, p["A"], p["D"])
    for t in range(21):                       # one flush, then 5 entries held
        tok = W.m2_step(w, t, range(w.batch))
        y = y_buf(w.batch, w.nheads, w.headdim)
        rs.rs_step(layer, bufs, m2_tok_dev(tok, w.in_dtype), A, D, y)
        rep.step(tok)
        conv.step(tok)
    pairs = [(0, 3), (1, 2)]
    rs.rs_copy_slots(layer, bufs, _seqs([s for s, _ in pairs]), layer, bufs, _seqs([d for _, d in pairs]), 2)
    nck, ln, nd, err, arrive = read_meta(layer, bufs)
    assert nck[3] == nck[0] and ln[3] == ln[0] == 5 and nck[2] == nck[1] and not arrive.any()
    worst = worst_c = 0.0
    for t in range(21, 60):
        tok = _dup_rows(W.m2_step(w, t, range(w.batch)), pairs)
        y = y_buf(w.batch, w.nheads, w.headdim)
        rs.rs_step(layer, bufs, m2_tok_dev(tok, w.in_dtype), A, D, y)
        yg = y.cpu().numpy()
        for s, d in pairs:
            assert np.array_equal(yg[d], yg[s]), (t, s, d)
        worst = max(worst, rel_l2(yg[:2], rep.step(tok)[:2]))
        worst_c = max(worst_c, rel_l2(yg[:2], conv.step(tok)[:2]))
    assert worst <= 1e-5 and worst_c <= 1e-5, (worst, worst_c)


def test_mamba2_prefix_cache_of_another_batch():
    """Save two sequences mid-window into a 3-slot cache, decode on past a flush,
    restore them into other slots, and continue from the saved prefixes."""
    w = W.TINY_M2.with_(batch=4, init_std=0.4, seed=201)
    p, A, D, layer, bufs, H0 = _m2_case(w)
    load_state_f32(layer, bufs, H0)
    cache_layer, cache = m2_layer(w, batch=3)
    rep = decode.M2Replay(H0, p["A"], p["D"])
    conv = decode.M2Conventional(H0, p["A"], p["D"])
    for t in range(7):
        tok = W.m2_step(w, t, range(w.batch))
        rs.rs_step(layer, bufs, m2_tok_dev(tok, w.in_dtype), A, D, y_buf(w.batch, w.nheads, w.headdim))
        rep.step(tok)
        conv.step(tok)
    rs.rs_copy_slots(layer, bufs, _seqs([1, 2]), cache_layer, cache, _seqs([2, 0]), 2)   # save
    saved_rep, saved_conv = copy.deepcopy(rep), copy.deepcopy(conv)
    saved_meta = read_meta(layer, bufs)
    for t in range(7, 19):                    # the live sequences flush in between
        tok = W.m2_step(w, t, range(w.batch))
        rs.rs_step(layer, bufs, m2_tok_dev(tok, w.in_dtype), A, D, y_buf(w.batch, w.nheads, w.headdim))
    rs.rs_copy_slots(cache_layer, cache, _seqs([0, 2]), layer, bufs, _seqs([3, 0]), 2)   # restore
    nck, ln, _, _, _ = read_meta(layer, bufs)
    assert (nck[3], ln[3]) == (saved_meta[0][2], saved_meta[1][2]) == (0, 7)
    assert (nck[0], ln[0]) == (saved_meta[0][1], saved_meta[1][1])
    back = {3: 2, 0: 1}                        # main slot -> the saved sequence it now continues
    worst = worst_c = 0.0
    for t in range(100, 130):
        tok = W.m2_step(w, t, range(w.batch))
        y = y_buf(w.batch, w.nheads, w.headdim)
        rs.rs_step(layer, bufs, m2_tok_dev(tok, w.in_dtype), A, D, y)
        yg = y.cpu().numpy()
        ts = _dup_rows(tok, [(d, s) for d, s in back.items()])   # saved row s gets main row d's input
        o_rep, o_conv = saved_rep.step(ts), saved_conv.step(ts)
        for d, s in back.items():
            worst = max(worst, rel_l2(yg[d], o_rep[s]))
            worst_c = max(worst_c, rel_l2(yg[d], o_conv[s]))
    assert worst <= 1e-5 and worst_c <= 1e-5, (worst, worst_c)


@pytest.mark.parametrize("gate", ["head", "channel"])
def test_delta_rule_fork_with_cached_rows(gate):
    w = W.TINY_GDN.with_(batch=4, n_qk=2, n_v=4, dk=128, dv=128, in_dtype="bf16", init_std=0.3, seed=202,
                         gate=gate)
    rule = kda if gate == "channel" else gdn
    gp = W.gdn_params(w)
    S0 = W.gdn_init_states(w, range(w.batch))
    layer, bufs = gdn_layer(w)
    load_state_f32(layer, bufs, S0)
    conv = decode.GDNConventional(S0, rule=rule)
    for t in range(9):
        tok = W.gdn_step(w, t, range(w.batch), gp)
        rs.rs_step(layer, bufs, gdn_tok_dev(tok, w.in_dtype), None, None, y_buf(w.batch, w.n_v, w.dv))
        conv.step(tok)
    pairs = [(2, 0), (1, 3)]
    rs.rs_copy_slots(layer, bufs, _seqs([s for s, _ in pairs]), layer, bufs, _seqs([d for _, d in pairs]), 2)
    fork = decode.GDNConventional(conv.S, rule=rule)   # copies the state
    for s, d in pairs:
        fork.S[d] = fork.S[s].copy()
    worst = 0.0
    for t in range(9, 40):
        tok = _dup_rows(W.gdn_step(w, t, range(w.batch), gp), pairs)
        o = y_buf(w.batch, w.n_v, w.dv)
        rs.rs_step(layer, bufs, gdn_tok_dev(tok, w.in_dtype), None, None, o)
        og = o.cpu().numpy()
        for s, d in pairs:
            assert np.array_equal(og[d], og[s]), (t, s, d)
        worst = max(worst, rel_l2(og, fork.step(tok)))
    assert worst <= 1e-5, worst


@pytest.mark.parametrize("ckpt,rc", [("fp8", True), ("nvfp4", False), ("f16", True)])
def test_low_precision_fork_copies_scales_and_read_copy(ckpt, rc):
    """Low-precision checkpoints (FP8 with its per-matrix scales, uniform NVFP4
    with block and tensor scales, FP16), with or without an NVFP4 read copy: the
    fork reads exactly what its source reads."""
    w = W.TINY_M2.with_(batch=4, init_std=0.0, seed=203)
    code = {"fp8": rs.RS_FP8E4M3, "nvfp4": rs.RS_NVFP4, "f16": rs.RS_F16}[ckpt]
    p, A, D, layer, bufs, _ = _m2_case(w, ckpt_dtype=code, read_copy=rs.RS_NVFP4 if rc else rs.RS_NONE)
    for t in range(20):
        tok = W.m2_step(w, t, range(w.batch))
        rs.rs_step(layer, bufs, m2_tok_dev(tok, w.in_dtype), A, D, y_buf(w.batch, w.nheads, w.headdim))
    pairs = [(0, 1), (3, 2)]
    rs.rs_copy_slots(layer, bufs, _seqs([s for s, _ in pairs]), layer, bufs, _seqs([d for _, d in pairs]), 2)
    for t in range(20, 50):
        tok = _dup_rows(W.m2_step(w, t, range(w.batch)), pairs)
        y = y_buf(w.batch, w.nheads, w.headdim)
        rs.rs_step(layer, bufs, m2_tok_dev(tok, w.in_dtype), A, D, y)
        yg = y.cpu().numpy()
        assert np.isfinite(yg).all()
        for s, d in pairs:
            assert np.array_equal(yg[d], yg[s]), (t, s, d)


def test_conventional_mode_and_skipped_pairs():
    """Conventional mode copies the live state; pairs out of range are skipped."""
    w = W.TINY_M2.with_(batch=3, init_std=0.4, seed=204)
    p, A, D, layer, bufs, H0 = _m2_case(w, mode=rs.RS_CONVENTIONAL)
    load_state_f32(layer, bufs, H0)
    conv = decode.M2Conventional(H0, p["A"], p["D"])
    for t in range(5):
        tok = W.m2_step(w, t, range(w.batch))
        rs.rs_step_conventional(layer, bufs, m2_tok_dev(tok, w.in_dtype), A, D, y_buf(w.batch, w.nheads, w.headdim))
        conv.step(tok)
    before = bufs.ckpt.clone()
    rs.rs_copy_slots(layer, bufs, _seqs([0, 5, -1]), layer, bufs, _seqs([2, 1, 1]), 3)
    row = bufs.ckpt.numel() // w.batch
    after = bufs.ckpt.view(w.batch, row)
    assert torch.equal(after[2], before.view(w.batch, row)[0]) and torch.equal(after[:2], before.view(w.batch, row)[:2])
    fork = copy.deepcopy(conv)
    fork.H[2] = fork.H[0].copy()
    worst = 0.0
    for t in range(5, 20):
        tok = _dup_rows(W.m2_step(w, t, range(w.batch)), [(0, 2)])
        y = y_buf(w.batch, w.nheads, w.headdim)
        rs.rs_step_conventional(layer, bufs, m2_tok_dev(tok, w.in_dtype), A, D, y)
        worst = max(worst, rel_l2(y.cpu().numpy(), fork.step(tok)))
    assert worst <= 1e-5, worst


def test_copy_with_pending_drafts():
    """A fork taken between append and commit carries the drafts: both copies
    commit the same accepted count and continue identically."""
    w = W.TINY_GDN.with_(batch=3, n_qk=2, n_v=4, dk=64, dv=64, init_std=0.3, max_draft=4, seed=205)
    gp = W.gdn_params(w)
    S0 = W.gdn_init_states(w, range(w.batch))
    layer, bufs = gdn_layer(w)
    load_state_f32(layer, bufs, S0)
    rep = decode.GDNReplay(S0, max_draft=4)
    for t in range(6):
        tok = W.gdn_step(w, t, range(w.batch), gp)
        rs.rs_step_nonflush(layer, bufs, gdn_tok_dev(tok, w.in_dtype), None, None, y_buf(w.batch, w.n_v, w.dv))
        rep.step(tok)
    drafts = [_dup_rows(W.gdn_step(w, 50 + d, range(w.batch), gp), [(0, 2)]) for d in range(3)]
    o = y_buf(w.batch, w.n_v, w.dv, K=3)
    rs.rs_spec_append(layer, bufs, gdn_drafts_dev(drafts, w.in_dtype), 3, None, None, o)
    rep.spec_append(drafts)
    rs.rs_copy_slots(layer, bufs, _seqs([0]), layer, bufs, _seqs([2]), 1)
    assert list(read_meta(layer, bufs)[2]) == [3, 3, 3]
    acc = np.array([2, 1, 2], np.int32)
    rs.rs_spec_commit(layer, bufs, torch.from_numpy(acc).to(DEV), None, None)
    rep.spec_commit(acc)
    worst = 0.0
    for t in range(60, 90):
        tok = _dup_rows(W.gdn_step(w, t, range(w.batch), gp), [(0, 2)])
        o = y_buf(w.batch, w.n_v, w.dv)
        rs.rs_step(layer, bufs, gdn_tok_dev(tok, w.in_dtype), None, None, o)
        og = o.cpu().numpy()
        assert np.array_equal(og[2], og[0]), t
        worst = max(worst, rel_l2(og[:2], rep.step(tok)[:2]))
    assert worst <= 1e-5, worst
