"""GPU parity of speculative decoding (append K drafts, commit the accepted
prefix) for ReplaySSM and for the snapshot/restore baseline, against the fp64
oracle: verify outputs equal decoding the drafts from the committed state;
after commit(k) the state equals the state after the first k drafts; buffer
counters and ring slots are bit-exact with the oracle's buffer model."""
import numpy as np
import pytest
import torch

import ssm_decode_checkpoint_amd as rs
import workloads as W
from oracle import decode
from oracle.ring import RingModel
from gpu_harness import (load_state_f32, m2_drafts_dev, m2_layer, m2_tok_dev, params_dev, read_meta,
                         read_state_f32, rel_l2, require_gpu, y_buf)

pytestmark = pytest.mark.gpu


def setup_module(_):
    require_gpu()


def _bits_in(arr, in_dtype):
    arr = np.ascontiguousarray(arr, dtype=np.float32)
    return W.bf16_bits(arr).view(np.int16) if in_dtype == "bf16" else arr.view(np.int32)


def _ring_bits(layer, bufs, name):
    t = rs.ring_view(layer, bufs, name).cpu()
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)).numpy()


def _spec_run(w, rounds, K, seqs=None, check_ring=True, tol=1e-5):
    p = W.m2_params(w)
    A, D = params_dev(p)
    B = w.batch
    seqs = list(range(B)) if seqs is None else seqs
    H0 = W.m2_init_states(w, range(B))
    rl, rb = m2_layer(w)
    load_state_f32(rl, rb, H0)
    cl, cb = m2_layer(w, mode=rs.RS_CONVENTIONAL)
    load_state_f32(cl, cb, H0)
    ref = decode.M2Conventional(H0[seqs], p["A"], p["D"])          # definition (snapshot scheme)
    rep = decode.M2Replay(H0[seqs], p["A"], p["D"], max_draft=w.max_draft)
    model = RingModel(B, max_draft=w.max_draft)
    slot_tok = [dict() for _ in range(B)]
    worst_r = worst_c = 0.0
    history = {}
    for r in range(rounds):
        drafts = [W.m2_step(w, 1000 + r * K + d, range(B)) for d in range(K)]
        for d in range(K):
            history[(r, d)] = drafts[d]
        acc_np = W.accepted_counts(w.seed, r, B, K)
        dd = m2_drafts_dev(drafts, w.in_dtype)
        yr = y_buf(B, w.nheads, w.headdim, K=K)
        yc = y_buf(B, w.nheads, w.headdim, K=K)
        rs.rs_spec_append(rl, rb, dd, K, A, D, yr)
        rs.rs_spec_append(cl, cb, dd, K, A, D, yc)
        for b in range(B):
            for d, s in enumerate(model.spec_append(b, K)):
                slot_tok[b][s] = (r, d, b)
        if check_ring:
            _check_ring(rl, rb, model, slot_tok, history, w)
        acc = torch.from_numpy(acc_np).cuda()
        rs.rs_spec_commit(rl, rb, acc, A, D)
        rs.rs_spec_commit(cl, cb, acc, A, D)
        for b in range(B):
            model.spec_commit(b, int(acc_np[b]))
        sub = [{k: v[seqs] for k, v in dr.items()} for dr in drafts]
        y_ref = ref.spec_round(sub, acc_np[seqs])
        rep.spec_append(sub)
        rep.spec_commit(acc_np[seqs])
        worst_r = max(worst_r, rel_l2(yr.cpu().numpy()[:, seqs], y_ref))
        worst_c = max(worst_c, rel_l2(yc.cpu().numpy()[:, seqs], y_ref))
        nck, ln, nd, err, arrive = read_meta(rl, rb)
        assert list(nck) == model.n_ckpt and list(ln) == model.len and list(nd) == model.nd
        assert not err.any() and not arrive.any()
        assert rel_l2(read_state_f32(cl, cb, seqs), ref.H) <= tol
        assert rel_l2(read_state_f32(rl, rb, seqs), rep.ckpt) <= tol
        if check_ring:
            _check_ring(rl, rb, model, slot_tok, history, w)
    return worst_r, worst_c, model


def _check_ring(rl, rb, model, slot_tok, history, w):
    rx, rB, rdt = (_ring_bits(rl, rb, n) for n in ("x", "B", "dt"))
    for b in range(len(model.len)):
        for s in model.live_slots(b):
            r, d, bi = slot_tok[b][s]
            tok = history[(r, d)]
            assert np.array_equal(rx[b, :, s], _bits_in(tok["x"][bi], w.in_dtype))
            assert np.array_equal(rB[b, :, s], _bits_in(tok["B"][bi], w.in_dtype))
            assert np.array_equal(rdt[b, :, s], _bits_in(tok["dt"][bi], w.in_dtype))


@pytest.mark.parametrize("K", [4, 3, 1])
def test_spec_tiny(K):
    w = W.TINY_M2.with_(max_draft=4, init_std=0.5, seed=21 + K)
    worst_r, worst_c, model = _spec_run(w, rounds=20, K=K)
    assert worst_r <= 1e-5 and worst_c <= 1e-5, (worst_r, worst_c)
    assert max(model.n_ckpt) > 0       # folds happened


def test_spec_120b_shapes_sampled():
    """Batch 512, 128 heads, 64 x 128 states, 4 drafts per round: all sequences
    on the GPU, 16 spread over the batch checked against the oracle."""
    w = W.M2_SPEC
    seqs = list(range(0, 512, 33))
    worst_r, worst_c, model = _spec_run(w, rounds=6, K=4, seqs=seqs, check_ring=False, tol=1e-5)
    print(f"spec b512: replay max rel-L2 {worst_r:.3e}, snapshot baseline {worst_c:.3e}")
    assert worst_r <= 2e-3 and worst_c <= 2e-3
    assert worst_r <= 1e-5 and worst_c <= 1e-5
    assert max(model.n_ckpt) > 0


def test_spec_then_plain_steps():
    w = W.TINY_M2.with_(max_draft=4, init_std=0.5, seed=31)
    p = W.m2_params(w)
    A, D = params_dev(p)
    H0 = W.m2_init_states(w, range(w.batch))
    rl, rb = m2_layer(w)
    load_state_f32(rl, rb, H0)
    ref = decode.M2Conventional(H0, p["A"], p["D"])
    model = RingModel(w.batch, max_draft=4)
    for r in range(5):
        drafts = [W.m2_step(w, 500 + 4 * r + d, range(w.batch)) for d in range(4)]
        acc = W.accepted_counts(w.seed, r, w.batch, 4)
        rs.rs_spec_append(rl, rb, m2_drafts_dev(drafts, w.in_dtype), 4, A, D, y_buf(w.batch, w.nheads, w.headdim, K=4))
        rs.rs_spec_commit(rl, rb, torch.from_numpy(acc).cuda(), A, D)
        ref.spec_round(drafts, acc)
        for b in range(w.batch):
            model.spec_append(b, 4)
            model.spec_commit(b, int(acc[b]))
    # sequences now sit at different fills; a plain step must flush exactly those at len 15
    worst = 0.0
    for t in range(40):
        tok = W.m2_step(w, 900 + t, range(w.batch))
        y = y_buf(w.batch, w.nheads, w.headdim)
        full = [model.is_flush_step(b) for b in range(w.batch)]
        if all(full):
            rs.rs_step_flush(rl, rb, m2_tok_dev(tok, w.in_dtype), A, D, y)
            for b in range(w.batch):
                model.flush(b)
        elif not any(full):
            rs.rs_step_nonflush(rl, rb, m2_tok_dev(tok, w.in_dtype), A, D, y)
            for b in range(w.batch):
                model.nonflush(b)
        else:
            # mixed fills: flush everyone (a flush is valid at any fill)
            rs.rs_step_flush(rl, rb, m2_tok_dev(tok, w.in_dtype), A, D, y)
            for b in range(w.batch):
                model.flush(b)
        worst = max(worst, rel_l2(y.cpu().numpy(), ref.step(tok)))
        nck, ln, nd, err, _ = read_meta(rl, rb)
        assert list(nck) == model.n_ckpt and list(ln) == model.len and not err.any()
    assert worst <= 1e-5, worst
