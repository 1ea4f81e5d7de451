"""GPU parity of the Kimi Delta Attention decode path (per-key-channel decay):
conventional and ReplaySSM (UT form with per-channel decay products) against
the fp64 oracle; counters and ring slots bit-exact, including the gate rows."""
import numpy as np
import pytest
import torch

import ssm_decode_checkpoint_amd as rs
import workloads as W
from oracle import decode, kda
from oracle.ring import RingModel
from gpu_harness import (gdn_layer, gdn_tok_dev, load_state_f32, read_meta, read_state_f32, rel_l2, require_gpu,
                         y_buf)

pytestmark = pytest.mark.gpu


def setup_module(_):
    require_gpu()


def _bits(t):
    t = t.cpu()
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)).numpy()


def _in_bits(arr, in_dtype):
    arr = np.ascontiguousarray(arr, dtype=np.float32)
    return W.bf16_bits(arr).view(np.int16) if in_dtype == "bf16" else arr.view(np.int32)


def _conv(w, steps):
    gp = W.gdn_params(w)
    S0 = W.gdn_init_states(w, range(w.batch))
    layer, bufs = gdn_layer(w, mode=rs.RS_CONVENTIONAL)
    load_state_f32(layer, bufs, S0)
    ref = decode.GDNConventional(S0, rule=kda)
    worst = 0.0
    for t in range(steps):
        tok = W.gdn_step(w, t, range(w.batch), gp)
        o = y_buf(w.batch, w.n_v, w.dv)
        rs.rs_step_conventional(layer, bufs, gdn_tok_dev(tok, w.in_dtype), None, None, o)
        worst = max(worst, rel_l2(o.cpu().numpy(), ref.step(tok)))
    return worst, rel_l2(read_state_f32(layer, bufs), ref.S)


def _replay(w, steps, flush_at=(), check_ring=False, seqs=None):
    seqs = list(range(w.batch)) if seqs is None else list(seqs)
    gp = W.gdn_params(w)
    S0 = W.gdn_init_states(w, range(w.batch))
    layer, bufs = gdn_layer(w)
    load_state_f32(layer, bufs, S0)
    ref = decode.GDNConventional(S0[seqs], rule=kda)
    model = RingModel(w.batch)
    slot_tok = [dict() for _ in range(w.batch)]
    toks = []
    worst = 0.0
    for t in range(steps):
        tok = W.gdn_step(w, t, range(w.batch), gp)
        toks.append(tok)
        o = y_buf(w.batch, w.n_v, w.dv)
        if t in flush_at or model.is_flush_step(0):
            rs.rs_step_flush(layer, bufs, gdn_tok_dev(tok, w.in_dtype), None, None, o)
            for b in range(w.batch):
                model.flush(b)
        else:
            rs.rs_step_nonflush(layer, bufs, gdn_tok_dev(tok, w.in_dtype), None, None, o)
            for b in range(w.batch):
                slot_tok[b][model.nonflush(b)] = t
        sub = {k: v[seqs] for k, v in tok.items()}
        worst = max(worst, rel_l2(o.cpu().numpy()[seqs], ref.step(sub)))
        nck, ln, nd, err, arrive = read_meta(layer, bufs)
        assert list(nck) == model.n_ckpt and list(ln) == model.len and not err.any() and not arrive.any()
        if check_ring:
            rings = {n: _bits(rs.ring_view(layer, bufs, n)) for n in ("q", "k", "v", "g", "beta")}
            for b in seqs:
                for s in model.live_slots(b):
                    tk = toks[slot_tok[b][s]]
                    for n in ("q", "k", "v"):
                        assert np.array_equal(rings[n][b, :, s], _in_bits(tk[n][b], w.in_dtype)), (t, b, s, n)
                    assert np.array_equal(rings["g"][b, :, s], tk["g"][b].astype(np.float32).view(np.int32))
                    assert np.array_equal(rings["beta"][b, :, s], tk["beta"][b].astype(np.float32).view(np.int32))
    return worst, model, layer, bufs, ref, seqs


@pytest.mark.parametrize("std", [0.0, 0.5])
def test_tiny_conventional(std):
    worst, wst = _conv(W.TINY_KDA.with_(init_std=std), 40)
    assert worst <= 1e-5 and wst <= 1e-5, (worst, wst)


def test_conventional_128():
    worst, wst = _conv(W.TINY_KDA.with_(batch=3, n_qk=2, n_v=4, dk=128, dv=128, in_dtype="bf16", init_std=0.3,
                                        seed=170), 20)
    assert worst <= 1e-5 and wst <= 1e-5, (worst, wst)


@pytest.mark.parametrize("std", [0.0, 0.5])
def test_tiny_replay(std):
    w = W.TINY_KDA.with_(init_std=std)
    worst, model, layer, bufs, ref, _ = _replay(w, 48, check_ring=True)
    assert worst <= 1e-5, worst
    assert rel_l2(read_state_f32(layer, bufs), ref.S) <= 1e-5    # 48 steps end on a flush


@pytest.mark.parametrize("fill", [0, 5, 13])
def test_flush_at_any_fill(fill):
    w = W.TINY_KDA.with_(init_std=0.5, seed=171)
    worst, model, layer, bufs, ref, _ = _replay(w, 36, flush_at=(fill,))
    assert worst <= 1e-5, worst


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
def test_two_slices(in_dtype):
    """dk = dv = 128: two column slices per state, each with the full per-channel decay."""
    w = W.TINY_KDA.with_(batch=3, n_qk=2, n_v=4, dk=128, dv=128, in_dtype=in_dtype, init_std=0.3, seed=172)
    worst, model, layer, bufs, ref, _ = _replay(w, 48, check_ring=True)
    assert worst <= 1e-5, worst
    assert rel_l2(read_state_f32(layer, bufs), ref.S) <= 1e-5


def test_kda_batch256_sampled():
    """The KDA workload at full size (256 sequences x 32 value heads of 128 x 128):
    all on the GPU, 6 sequences checked against the oracle over two windows."""
    w = W.KDA_B256
    seqs = [0, 51, 102, 153, 204, 255]
    worst, model, layer, bufs, ref, seqs = _replay(w, 32, seqs=seqs)
    print(f"kda b256: max rel-L2 {worst:.3e}")
    assert worst <= 1e-5
    assert rel_l2(read_state_f32(layer, bufs, seqs), ref.S) <= 1e-5

