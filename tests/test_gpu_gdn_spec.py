"""GPU parity of Gated DeltaNet and Kimi Delta Attention speculative decoding
(append / verify, commit with folds, and the snapshot baseline) against the
fp64 oracle: verify outputs
against both the same-method oracle and stepping the drafts with snapshots,
counters bit-exact, draft records bit-exact in the ring, cached u rows against
the oracle's triangular solve, device error bits."""
import numpy as np
import pytest
import torch

import ssm_decode_checkpoint_amd as rs
import workloads as W
from oracle import decode, gdn, kda
from gpu_harness import (gdn_drafts_dev, gdn_layer, gdn_tok_dev, load_state_f32, read_meta, read_state_f32, rel_l2,
                         require_gpu, y_buf)

pytestmark = pytest.mark.gpu


def setup_module(_):
    require_gpu()


def _bits(t):
    t = t.cpu()
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)).numpy()


def _in_bits(arr, in_dtype):
    arr = np.ascontiguousarray(arr, dtype=np.float32)
    return W.bf16_bits(arr).view(np.int16) if in_dtype == "bf16" else arr.view(np.int32)


def _rule(w):
    return kda if w.gate == "channel" else gdn


def _check_ring(layer, bufs, same, w, seqs):
    """Every live slot's record bits, and its u row against the oracle's solve over
    the live entries from the oracle's checkpoint."""
    rings = {n: _bits(rs.ring_view(layer, bufs, n)) for n in ("q", "k", "v", "g", "beta")}
    ug = rs.ring_view(layer, bufs, "u").cpu().numpy()
    worst = 0.0
    for i, b in enumerate(seqs):
        slots = same.ring.live_slots(i)
        ents = [same.entries[i][s] for s in slots]
        for s, e in zip(slots, ents):
            for n in ("q", "k", "v"):
                assert np.array_equal(rings[n][b, :, s], _in_bits(e[n][0], w.in_dtype)), (b, s, n)
            for n in ("g", "beta"):
                assert np.array_equal(rings[n][b, :, s], e[n][0].astype(np.float32).view(np.int32)), (b, s, n)
        if ents:
            us = _rule(w).ut_solve(same.ckpt[i:i + 1], ents)
            for s, u in zip(slots, us):
                worst = max(worst, rel_l2(ug[b, :, s], u[0]))
    return worst


def _spec_run(w, rounds, Ks, seqs=None, t0=3000):
    seqs = list(range(w.batch)) if seqs is None else list(seqs)
    gp = W.gdn_params(w)
    S0 = W.gdn_init_states(w, range(w.batch))
    layer, bufs = gdn_layer(w)
    load_state_f32(layer, bufs, S0)
    exact = decode.GDNConventional(S0[seqs], rule=_rule(w))
    same = decode.GDNReplay(S0[seqs], max_draft=w.max_draft, rule=_rule(w))
    worst_same = worst_exact = worst_u = 0.0
    t = t0
    folds = 0
    for r in range(rounds):
        K = Ks[r % len(Ks)]
        drafts = [W.gdn_step(w, t + d, range(w.batch), gp) for d in range(K)]
        sub = [{k: v[seqs] for k, v in d.items()} for d in drafts]
        t += K
        acc = W.accepted_counts(w.seed, r, w.batch, K)
        o = y_buf(w.batch, w.n_v, w.dv, K=K)
        rs.rs_spec_append(layer, bufs, gdn_drafts_dev(drafts, w.in_dtype), K, None, None, o)
        og = o.cpu().numpy()[:, seqs]
        worst_same = max(worst_same, rel_l2(og, same.spec_append(sub)))
        nck, ln, nd, err, arrive = read_meta(layer, bufs)
        assert [int(nd[b]) for b in seqs] == same.ring.nd and not err.any() and not arrive.any()
        worst_u = max(worst_u, _check_ring(layer, bufs, same, w, seqs))
        n_before = list(same.ring.n_ckpt)
        rs.rs_spec_commit(layer, bufs, torch.from_numpy(acc).cuda(), None, None)
        same.spec_commit(acc[seqs])
        folds += sum(a != b for a, b in zip(same.ring.n_ckpt, n_before))
        worst_exact = max(worst_exact, rel_l2(og, exact.spec_round(sub, acc[seqs])))
        nck, ln, nd, err, arrive = read_meta(layer, bufs)
        assert [int(nck[b]) for b in seqs] == same.ring.n_ckpt and [int(ln[b]) for b in seqs] == same.ring.len
        assert not nd.any() and not err.any() and not arrive.any()
    worst_ck = rel_l2(read_state_f32(layer, bufs, seqs), same.ckpt)
    return worst_same, worst_exact, worst_u, worst_ck, folds


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K,kmax", [(4, 4), (2, 4), (8, 8)])
def test_tiny(K, kmax, in_dtype):
    """dk = dv = 16. With bf16 records the round's dots run on the matrix cores
    (one zero-padded 32-wide step; 8 drafts fill all 16 rows)."""
    w = W.TINY_GDN.with_(max_draft=kmax, init_std=0.4, seed=130 + K, in_dtype=in_dtype)
    ws, we, wu, wc, folds = _spec_run(w, 24, [K])
    assert ws <= 1e-5 and we <= 1e-5 and wu <= 1e-5 and wc <= 1e-5, (ws, we, wu, wc)
    assert folds > 0


def test_mixed_draft_counts_two_slices():
    """dk = dv = 128 (two column slices per state), bf16 q/k/v, K cycling 1..4."""
    w = W.TINY_GDN.with_(batch=3, n_qk=2, n_v=4, dk=128, dv=128, in_dtype="bf16", init_std=0.3, max_draft=4,
                         seed=140)
    ws, we, wu, wc, folds = _spec_run(w, 20, [1, 2, 3, 4])
    assert ws <= 1e-5 and we <= 1e-5 and wu <= 1e-5 and wc <= 1e-5, (ws, we, wu, wc)
    assert folds > 0


def test_eight_drafts_two_slices():
    """dk = dv = 128, bf16 records, up to 8 drafts per round: all 16 rows of the
    matrix-core dot block live (8 draft k, 8 draft q), the matvec on the VALU."""
    w = W.TINY_GDN.with_(batch=3, n_qk=2, n_v=4, dk=128, dv=128, in_dtype="bf16", init_std=0.3, max_draft=8,
                         seed=141)
    ws, we, wu, wc, folds = _spec_run(w, 12, [8, 5, 8, 3])
    assert ws <= 1e-5 and we <= 1e-5 and wu <= 1e-5 and wc <= 1e-5, (ws, we, wu, wc)
    assert folds > 0


def test_qwen_batch256_sampled():
    """The speculative Qwen-style workload at full size (256 sequences x 32 value
    heads of 128 x 128), 8 sequences spread over the batch checked each round."""
    w = W.GDN_SPEC
    seqs = [0, 37, 74, 111, 148, 185, 222, 255]
    ws, we, wu, wc, folds = _spec_run(w, 10, [4], seqs=seqs)
    print(f"gdn spec b256: vs same-method {ws:.2e}, vs snapshots {we:.2e}, u rows {wu:.2e}, checkpoint {wc:.2e}")
    assert ws <= 1e-5 and we <= 1e-5 and wu <= 1e-5 and wc <= 1e-5
    assert folds > 0


@pytest.mark.parametrize("K,kmax", [(4, 4), (2, 4), (8, 8)])
def test_kda_tiny(K, kmax):
    """Kimi Delta Attention (a decay per key channel), dk = dv = 16."""
    w = W.TINY_KDA.with_(max_draft=kmax, init_std=0.4, seed=170 + K)
    ws, we, wu, wc, folds = _spec_run(w, 24, [K])
    assert ws <= 1e-5 and we <= 1e-5 and wu <= 1e-5 and wc <= 1e-5, (ws, we, wu, wc)
    assert folds > 0


def test_kda_mixed_draft_counts_two_slices():
    w = W.TINY_KDA.with_(batch=3, n_qk=2, n_v=4, dk=128, dv=128, in_dtype="bf16", init_std=0.3, max_draft=4,
                         seed=175)
    ws, we, wu, wc, folds = _spec_run(w, 20, [1, 2, 3, 4])
    assert ws <= 1e-5 and we <= 1e-5 and wu <= 1e-5 and wc <= 1e-5, (ws, we, wu, wc)
    assert folds > 0


def test_kda_batch256_sampled():
    """KDA on the Qwen-style shapes at batch 256 with 4 drafts, 8 sequences checked."""
    w = W.KDA_B256.with_(max_draft=4)
    seqs = [0, 37, 74, 111, 148, 185, 222, 255]
    ws, we, wu, wc, folds = _spec_run(w, 10, [4], seqs=seqs)
    print(f"kda spec b256: vs same-method {ws:.2e}, vs snapshots {we:.2e}, u rows {wu:.2e}, checkpoint {wc:.2e}")
    assert ws <= 1e-5 and we <= 1e-5 and wu <= 1e-5 and wc <= 1e-5
    assert folds > 0


@pytest.mark.parametrize("gate", ["head", "channel"])
@pytest.mark.parametrize("K", [2, 4])
def test_snapshot_baseline(K, gate):
    w = W.TINY_GDN.with_(batch=3, n_qk=2, n_v=4, dk=128, dv=128, init_std=0.3, max_draft=4, seed=150, gate=gate)
    gp = W.gdn_params(w)
    S0 = W.gdn_init_states(w, range(w.batch))
    layer, bufs = gdn_layer(w, mode=rs.RS_CONVENTIONAL)
    load_state_f32(layer, bufs, S0)
    exact = decode.GDNConventional(S0, rule=_rule(w))
    worst = 0.0
    for r in range(10):
        drafts = [W.gdn_step(w, 500 + r * K + d, range(w.batch), gp) for d in range(K)]
        acc = W.accepted_counts(w.seed, r, w.batch, K)
        o = y_buf(w.batch, w.n_v, w.dv, K=K)
        rs.rs_spec_append(layer, bufs, gdn_drafts_dev(drafts, w.in_dtype), K, None, None, o)
        rs.rs_spec_commit(layer, bufs, torch.from_numpy(acc).cuda(), None, None)
        worst = max(worst, rel_l2(o.cpu().numpy(), exact.spec_round(drafts, acc)))
        assert rel_l2(read_state_f32(layer, bufs), exact.S) <= 1e-5
    assert worst <= 1e-5, worst


def test_error_bits():
    """Overflowing append, a plain step with drafts pending, and a commit of more
    than pending are refused per sequence with sticky bits, changing nothing;
    the valid calls around them follow the oracle."""
    w = W.TINY_GDN.with_(batch=3, n_qk=2, n_v=4, dk=128, dv=128, init_std=0.3, max_draft=4, seed=160)
    gp = W.gdn_params(w)
    S0 = W.gdn_init_states(w, range(w.batch))
    layer, bufs = gdn_layer(w)
    load_state_f32(layer, bufs, S0)
    same = decode.GDNReplay(S0, max_draft=4)
    for t in range(13):
        tok = W.gdn_step(w, t, range(w.batch), gp)
        o = y_buf(w.batch, w.n_v, w.dv)
        rs.rs_step_nonflush(layer, bufs, gdn_tok_dev(tok, w.in_dtype), None, None, o)
        assert rel_l2(o.cpu().numpy(), same.step(tok)) <= 1e-5
    ck, ring = bufs.ckpt.clone(), bufs.ring.clone()
    drafts = [W.gdn_step(w, 100 + d, range(w.batch), gp) for d in range(4)]
    o = y_buf(w.batch, w.n_v, w.dv, K=4)
    rs.rs_spec_append(layer, bufs, gdn_drafts_dev(drafts, w.in_dtype), 4, None, None, o)   # 13 + 4 > 16
    same.spec_append(drafts)
    nck, ln, nd, err, arrive = read_meta(layer, bufs)
    assert (err == rs.RS_ERR_OVERFLOW).all() and (nd == 0).all() and (ln == 13).all() and not arrive.any()
    assert torch.isnan(o).all() and torch.equal(ck, bufs.ckpt) and torch.equal(ring, bufs.ring)
    o = y_buf(w.batch, w.n_v, w.dv, K=3)
    rs.rs_spec_append(layer, bufs, gdn_drafts_dev(drafts[:3], w.in_dtype), 3, None, None, o)
    assert rel_l2(o.cpu().numpy(), same.spec_append(drafts[:3])) <= 1e-5
    tok = W.gdn_step(w, 200, range(w.batch), gp)
    o1 = y_buf(w.batch, w.n_v, w.dv)
    rs.rs_step_nonflush(layer, bufs, gdn_tok_dev(tok, w.in_dtype), None, None, o1)       # drafts pending
    same.step(tok)
    assert torch.isnan(o1).all()
    rs.rs_spec_commit(layer, bufs, torch.full((w.batch,), 5, dtype=torch.int32, device="cuda"), None, None)
    same.spec_commit(np.full(w.batch, 5))
    nck, ln, nd, err, _ = read_meta(layer, bufs)
    assert (err == rs.RS_ERR_OVERFLOW | rs.RS_ERR_PENDING | rs.RS_ERR_COMMIT).all() and (nd == 3).all()
    assert list(err) == same.ring.err
    rs.rs_spec_commit(layer, bufs, torch.full((w.batch,), 2, dtype=torch.int32, device="cuda"), None, None)
    same.spec_commit(np.full(w.batch, 2))                                                 # len 15 > 12: fold
    nck, ln, nd, err, arrive = read_meta(layer, bufs)
    assert list(nck) == same.ring.n_ckpt == [15] * w.batch and (ln == 0).all() and not arrive.any()
    assert rel_l2(read_state_f32(layer, bufs), same.ckpt) <= 1e-5
