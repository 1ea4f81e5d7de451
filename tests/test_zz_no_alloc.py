"""rs_spec_commit_static (the speculative commit whose fold list lives in the
library's static device array) against rs_spec_commit (fold list in the meta
buffer's work space): twin layers take the same appends, one commits through
each entry point, and checkpoints, ring slots, read copies and counters must
match bit for bit after every commit. Calls alternate between a larger and a
smaller layer, so each call follows one that left a longer fold list in the
shared array; and a layer beyond the array's 8192 sequences is refused."""
import numpy as np
import pytest
import torch

import ssm_decode_checkpoint_amd as rs
import workloads as W
from gpu_harness import (gdn_drafts_dev, gdn_layer, load_state_f32, m2_drafts_dev, m2_layer, params_dev, read_meta,
                         require_gpu, y_buf)

pytestmark = pytest.mark.gpu


def setup_module(_):
    require_gpu()


def _same(t1, t2, what):
    (l1, b1), (l2, b2) = t1, t2
    for name in ("ckpt", "ring", "read_copy"):
        x, y = getattr(b1, name), getattr(b2, name)
        if x is not None:
            assert torch.equal(x, y), f"{what}: {name} differs"
    m1, m2 = read_meta(l1, b1), read_meta(l2, b2)
    for a, b in zip(m1[:4], m2[:4]):
        assert np.array_equal(a, b), f"{what}: counters differ"


def _accept(rnd, batch, K):
    # mostly long acceptances, so that many sequences fold on the same call
    g = np.random.default_rng([7, rnd, batch])
    return np.where(g.random(batch) < 0.8, K, g.integers(0, K + 1, batch)).astype(np.int32)


def test_static_commit_matches_meta_commit_mamba2():
    K = 4
    big = W.TINY_M2.with_(batch=24, nheads=8, ngroups=2, dstate=128, headdim=64, in_dtype="bf16", init_std=0.3,
                          seed=190, max_draft=K)
    small = big.with_(batch=7, seed=191)
    twins = {}
    for w in (big, small):
        p = W.m2_params(w)
        H0 = W.m2_init_states(w, range(w.batch))
        pair = []
        for _ in range(2):
            layer, bufs = m2_layer(w, ckpt_dtype=rs.RS_FP8E4M3, read_copy=rs.RS_NVFP4, fuse=1)
            load = torch.from_numpy(np.zeros(int(layer.ckpt_bytes), np.uint8)).cuda()
            bufs.ckpt.copy_(load)
            rs.rs_requant_read_copy(layer, bufs)
            pair.append((layer, bufs))
        twins[w.batch] = (w, params_dev(p), pair)
    folds = 0
    for r in range(8):
        for batch in (24, 7):                     # each call follows a longer list in the array
            w, (A, D), (ref, sta) = twins[batch]
            drafts = m2_drafts_dev([W.m2_step(w, 6000 + r * K + d, range(w.batch)) for d in range(K)], w.in_dtype)
            for layer, bufs in (ref, sta):
                y = y_buf(w.batch, w.nheads, w.headdim, K=K)
                rs.rs_spec_append(layer, bufs, drafts, K, A, D, y)
            acc = torch.from_numpy(_accept(r, w.batch, K)).cuda()
            n0 = read_meta(*ref)[0].copy()
            rs.rs_spec_commit(*ref, acc, A, D)
            rs.rs_spec_commit_static(*sta, acc, A, D)
            torch.cuda.synchronize()
            folds += int(np.count_nonzero(read_meta(*ref)[0] != n0))
            _same(ref, sta, f"round {r}, batch {batch}")
    assert folds >= 20, folds


def test_static_commit_matches_meta_commit_gdn():
    K = 4
    w = W.TINY_GDN.with_(batch=5, n_qk=2, n_v=4, dk=128, dv=128, in_dtype="bf16", init_std=0.3, seed=192,
                         max_draft=K)
    gp = W.gdn_params(w)
    S0 = W.gdn_init_states(w, range(w.batch))
    ref, sta = gdn_layer(w), gdn_layer(w)
    for layer, bufs in (ref, sta):
        load_state_f32(layer, bufs, S0)
    for r in range(6):
        drafts = gdn_drafts_dev([W.gdn_step(w, 7000 + r * K + d, range(w.batch), gp) for d in range(K)], w.in_dtype)
        for layer, bufs in (ref, sta):
            rs.rs_spec_append(layer, bufs, drafts, K, None, None, y_buf(w.batch, w.n_v, w.dv, K=K))
        acc = torch.from_numpy(_accept(r, w.batch, K)).cuda()
        rs.rs_spec_commit(*ref, acc, None, None)
        rs.rs_spec_commit_static(*sta, acc, None, None)
        torch.cuda.synchronize()
        _same(ref, sta, f"gdn round {r}")


def test_static_commit_refuses_beyond_its_array():
    w = W.TINY_M2.with_(batch=8193, max_draft=4)
    cfg = rs.make_config(rs.RS_MAMBA2, w.batch, nheads=w.nheads, headdim=w.headdim, dstate=w.dstate,
                         ngroups=w.ngroups, max_draft=4, in_dtype=rs.RS_F32)
    _, layer = rs.rs_init(cfg)
    bufs = rs.alloc_buffers(layer, "cuda")
    acc = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
    A = torch.zeros(w.nheads, device="cuda")
    st = rs.rs_spec_commit_static(layer, bufs, acc, A, A, raise_on_error=False)
    assert st == rs.RS_E_ARG
