"""GPU parity of the low-precision paths: the NVFP4 read-copy quantizer (bit
exact against the oracle's float32 emulation), non-flush steps that read the
copy, the fp16 / fp8 / uniform-NVFP4 checkpoints, the fused-vs-standalone
requant identity, and read-copy isolation (the fp32 checkpoint is bit-identical
with and without a read copy)."""
import numpy as np
import pytest
import torch

import ssm_decode_checkpoint_amd as rs
import workloads as W
from oracle import decode, quant
from gpu_harness import (load_state_f32, m2_layer, m2_tok_dev, params_dev, read_state_f32, rel_l2, require_gpu,
                         y_buf)

pytestmark = pytest.mark.gpu


def setup_module(_):
    require_gpu()


def _read_copy(layer, bufs):
    """(packed codes [b,h,rows,cols/2], block scales [b,h,rows,cols/16], tensor scales [b,h])."""
    b, h, r, c = layer.cfg.batch, layer.heads, layer.rows, layer.cols
    raw = bufs.read_copy.cpu().numpy()
    codes = raw[: b * h * r * c // 2].reshape(b, h, r, c // 2)
    sc = raw[layer.nv_scale_off: layer.nv_scale_off + b * h * r * c // 16].reshape(b, h, r, c // 16)
    ts = raw[layer.nv_tscale_off: layer.nv_tscale_off + 4 * b * h].view(np.float32).reshape(b, h)
    return codes, sc, ts


def _stored_tiles(layer, seed, std, heavy):
    shape = (layer.cfg.batch, layer.heads, layer.rows, layer.cols)
    x = W.state_tiles(seed, 0, shape, std=std, heavy_tail=heavy)
    x[0, 0] = 0.0                                 # an all-zero matrix
    x[0, 1, 3, :16] = 0.0                         # a zero block
    x[0, 1, 5, 16:32] *= 1e-9                     # a block far below the matrix max
    return x


def _oracle_copy(tiles):
    b, h = tiles.shape[:2]
    codes = np.empty(tiles.shape[:-1] + (tiles.shape[-1] // 2,), np.uint8)
    sc = np.empty(tiles.shape[:-1] + (tiles.shape[-1] // 16,), np.uint8)
    ts = np.empty((b, h), np.float32)
    for i in range(b):
        for j in range(h):
            c, s, t = quant.nvfp4_quantize(tiles[i, j])
            codes[i, j] = quant.pack_nibbles(c)
            sc[i, j] = s
            ts[i, j] = t
    return codes, sc, ts


@pytest.mark.parametrize("shape,heavy", [((4, 4, 16, 16, 1), True), ((2, 128, 128, 64, 8), True),
                                         ((2, 128, 128, 64, 8), False)])
def test_requant_bit_exact_from_f32(shape, heavy):
    b, h, n, p, g = shape
    w = W.TINY_M2.with_(batch=b, nheads=h, dstate=n, headdim=p, ngroups=g)
    layer, bufs = m2_layer(w, read_copy=rs.RS_NVFP4)
    tiles = _stored_tiles(layer, 40 + n, 0.1, heavy)
    rs.ckpt_f32_view(layer, bufs).copy_(torch.from_numpy(tiles).cuda())
    rs.rs_requant_read_copy(layer, bufs)
    got = _read_copy(layer, bufs)
    want = _oracle_copy(tiles)
    assert np.array_equal(got[2].view(np.uint32), want[2].view(np.uint32))
    assert np.array_equal(got[1], want[1])
    assert np.array_equal(got[0], want[0]), f"{np.count_nonzero(got[0] != want[0])} code bytes differ"


def _boundary_tiles(b, h, rows, cols, seed):
    """fp32 matrices whose elements sit on E2M1 rounding boundaries of their own
    block scale (ties, and one and two float32 steps either side), so that the
    codes depend on the quotient x / scale being rounded exactly as a float32
    division rounds it. The matrix max and each block's max are placed first,
    which fixes the tensor scale and every block scale (the oracle's formulas)."""
    g = np.random.default_rng(seed)
    F = np.float32
    x = np.zeros((b, h, rows, cols), F)
    bounds = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], F)
    for i in range(b):
        for j in range(h):
            amax = F(np.exp(g.uniform(np.log(0.3), np.log(300.0))))
            ts = F(amax / F(2688.0))
            d = F(F(6.0) * ts)
            for r in range(rows):
                for k in range(cols // 16):
                    bm = amax if (r == 0 and k == 0) else F(amax * F(g.uniform(0.02, 1.0)))
                    s = quant.e4m3_encode_mag(F(bm / d))
                    sd = F(quant.e4m3_decode(s) * ts)
                    blk = np.zeros(16, F)
                    blk[0] = bm
                    for e in range(1, 16):
                        q = F(bounds[g.integers(len(bounds))] * sd)
                        q = np.nextafter(q, F(np.inf) if g.integers(2) else F(0.0)) if g.integers(3) == 0 else q
                        if g.integers(4) == 0:
                            q = np.nextafter(np.nextafter(q, F(np.inf)), F(np.inf))
                        if abs(q) > bm:
                            q = F(0.0)
                        blk[e] = -q if g.integers(2) else q
                    g.shuffle(blk)
                    x[i, j, r, 16 * k: 16 * k + 16] = blk
    return x


def test_requant_codes_on_rounding_boundaries():
    """The GPU forms each quotient from one reciprocal per block plus a
    correction step; on values at and next to the code boundaries its codes must
    still equal those of the oracle's float32 division."""
    w = W.TINY_M2.with_(batch=2, nheads=8, dstate=128, headdim=64, ngroups=2)
    layer, bufs = m2_layer(w, read_copy=rs.RS_NVFP4)
    tiles = _boundary_tiles(w.batch, w.nheads, w.dstate, w.headdim, 47)
    rs.ckpt_f32_view(layer, bufs).copy_(torch.from_numpy(tiles).cuda())
    rs.rs_requant_read_copy(layer, bufs)
    got = _read_copy(layer, bufs)
    want = _oracle_copy(tiles)
    assert np.array_equal(got[2].view(np.uint32), want[2].view(np.uint32))
    assert np.array_equal(got[1], want[1])
    assert np.array_equal(got[0], want[0]), f"{np.count_nonzero(got[0] != want[0])} code bytes differ"


def test_requant_bit_exact_from_f16_and_fp8():
    w = W.TINY_M2.with_(batch=2, nheads=16, dstate=128, headdim=64, ngroups=2)
    # fp16 checkpoint (values rounded by torch's conversion)
    layer, bufs = m2_layer(w, ckpt_dtype=rs.RS_F16, read_copy=rs.RS_NVFP4)
    tiles = _stored_tiles(layer, 50, 0.3, True)
    t16 = torch.from_numpy(tiles).half()
    bufs.ckpt[: t16.numel() * 2].copy_(t16.view(torch.uint8).reshape(-1).cuda())
    rs.rs_requant_read_copy(layer, bufs)
    got = _read_copy(layer, bufs)
    want = _oracle_copy(t16.float().numpy())
    for a, b in zip(got, want):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
    # fp8 checkpoint: codes from torch's float8_e4m3fn conversion, one fp32 scale per matrix
    layer, bufs = m2_layer(w, ckpt_dtype=rs.RS_FP8E4M3, read_copy=rs.RS_NVFP4)
    x = torch.from_numpy(_stored_tiles(layer, 51, 0.3, False))
    sc = (x.abs().amax(dim=(2, 3)) / 448.0).float()
    sc = torch.where(sc == 0, torch.ones_like(sc), sc)
    codes = (x / sc[:, :, None, None]).to(torch.float8_e4m3fn)
    n = codes.numel()
    bufs.ckpt[:n].copy_(codes.view(torch.uint8).reshape(-1).cuda())
    bufs.ckpt[layer.ck_scale_off: layer.ck_scale_off + 4 * sc.numel()].copy_(sc.reshape(-1).view(torch.uint8).cuda())
    rs.rs_requant_read_copy(layer, bufs)
    got = _read_copy(layer, bufs)
    deq = (codes.float() * sc[:, :, None, None]).numpy()
    want = _oracle_copy(deq)
    for a, b in zip(got, want):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))


def _run(w, layer, bufs, A, D, steps, t0=0):
    ys = []
    for t in range(t0, t0 + steps):
        tok = W.m2_step(w, t, range(w.batch))
        y = y_buf(w.batch, w.nheads, w.headdim)
        if t % 16 == 15:
            rs.rs_step_flush(layer, bufs, m2_tok_dev(tok, w.in_dtype), A, D, y)
        else:
            rs.rs_step_nonflush(layer, bufs, m2_tok_dev(tok, w.in_dtype), A, D, y)
        ys.append(y.cpu().numpy())
    return ys


# tiny layer; 128 x 64 heads four to a group (the wavefront-per-head read kernel), fp32 and
# bf16 inputs; 128 x 64 heads two to a group (the workgroup-per-head kernel)
READ_SHAPES = [dict(), dict(batch=3, nheads=8, ngroups=2, dstate=128, headdim=64),
               dict(batch=3, nheads=8, ngroups=2, dstate=128, headdim=64, in_dtype="bf16"),
               dict(batch=3, nheads=6, ngroups=3, dstate=128, headdim=64),
               # bf16 records with 8 or more heads per group: two heads per wavefront on FP8 / NVFP4 reads
               dict(batch=3, nheads=16, ngroups=1, dstate=128, headdim=64, in_dtype="bf16"),
               dict(batch=2, nheads=16, ngroups=2, dstate=128, headdim=64, in_dtype="bf16")]


@pytest.mark.parametrize("shape", READ_SHAPES)
def test_nonflush_reads_copy_and_isolation(shape):
    w = W.TINY_M2.with_(init_std=0.5, seed=61, **shape)
    p = W.m2_params(w)
    A, D = params_dev(p)
    H0 = W.m2_init_states(w, range(w.batch))
    rl, rb = m2_layer(w, read_copy=rs.RS_NVFP4, fuse=1)
    pl, pb = m2_layer(w)
    load_state_f32(rl, rb, H0)
    load_state_f32(pl, pb, H0)
    rs.rs_requant_read_copy(rl, rb)
    ref = decode.M2Replay(H0, p["A"], p["D"], ckpt_fmt="f32", read_copy="nvfp4")
    exact = decode.M2Conventional(H0, p["A"], p["D"])
    before, after, lp_err = 0.0, 0.0, 0.0
    for t in range(40):
        tok = W.m2_step(w, t, range(w.batch))
        y = y_buf(w.batch, w.nheads, w.headdim)
        yp = y_buf(w.batch, w.nheads, w.headdim)
        fn = rs.rs_step_flush if t % 16 == 15 else rs.rs_step_nonflush
        fn(rl, rb, m2_tok_dev(tok, w.in_dtype), A, D, y)
        fn(pl, pb, m2_tok_dev(tok, w.in_dtype), A, D, yp)
        yr = ref.step(tok)
        ye = exact.step(tok)
        e = rel_l2(y.cpu().numpy(), yr)
        if t < 15:
            before = max(before, e)
        else:
            after = max(after, e)
        lp_err = max(lp_err, rel_l2(y.cpu().numpy(), ye))
        if t % 16 == 15:
            # read-copy isolation: the fp32 checkpoint does not see the read copy
            assert torch.equal(bufs_ck(rl, rb), bufs_ck(pl, pb))
            # fused requant == standalone requant, bit for bit
            fused = rb.read_copy.clone()
            rs.rs_requant_read_copy(rl, rb)
            assert torch.equal(fused, rb.read_copy)
    print(f"read-copy path: rel-L2 vs oracle before flush {before:.2e}, after {after:.2e}; "
          f"NVFP4-read error vs exact fp64 {lp_err:.2e}")
    assert before <= 1e-5 and after <= 1e-4
    assert lp_err > 1e-3          # the copy really is what non-flush steps read


def bufs_ck(layer, bufs):
    return bufs.ckpt[: layer.ckpt_bytes]


@pytest.mark.parametrize("fmt,rc,gate", [("f16", None, 1e-4), ("fp8", None, 2e-2), ("nvfp4", None, 2e-2),
                                         ("f16", "nvfp4", 2e-2), ("fp8", "nvfp4", 2e-2)])
@pytest.mark.parametrize("shape", READ_SHAPES[:2])
def test_low_precision_checkpoints(fmt, rc, gate, shape):
    """Zero initial state, 48 steps (3 flushes): GPU vs the oracle running the
    same storage formats; the error vs exact fp64 decoding is reported."""
    w = W.TINY_M2.with_(seed=70, **shape)
    p = W.m2_params(w)
    A, D = params_dev(p)
    code = {"f16": rs.RS_F16, "fp8": rs.RS_FP8E4M3, "nvfp4": rs.RS_NVFP4}[fmt]
    layer, bufs = m2_layer(w, ckpt_dtype=code, read_copy=rs.RS_NVFP4 if rc else rs.RS_NONE, fuse=1)
    H0 = W.m2_init_states(w, range(w.batch))
    ref = decode.M2Replay(H0, p["A"], p["D"], ckpt_fmt=fmt, read_copy=rc)
    exact = decode.M2Conventional(H0, p["A"], p["D"])
    worst, lp = 0.0, 0.0
    for t in range(48):
        tok = W.m2_step(w, t, range(w.batch))
        y = y_buf(w.batch, w.nheads, w.headdim)
        fn = rs.rs_step_flush if t % 16 == 15 else rs.rs_step_nonflush
        fn(layer, bufs, m2_tok_dev(tok, w.in_dtype), A, D, y)
        yg = y.cpu().numpy()
        worst = max(worst, rel_l2(yg, ref.step(tok)))
        lp = max(lp, rel_l2(yg, exact.step(tok)))
    print(f"{fmt} checkpoint{' + nvfp4 reads' if rc else ''}: vs same-format oracle {worst:.2e}, "
          f"vs exact fp64 {lp:.2e}")
    assert worst <= gate


LOWPREC_VARIANTS = [("f32", "nvfp4", 1e-4), ("f16", "nvfp4", 2e-2), ("fp8", "nvfp4", 2e-2), ("f16", None, 1e-4),
                    ("fp8", None, 2e-2), ("nvfp4", None, 2e-2)]


@pytest.mark.parametrize("fmt,rc,gate", LOWPREC_VARIANTS)
def test_lowprec_config_batch64_shortened(fmt, rc, gate):
    """The low-precision workload's own configuration (Nemotron-style shapes at
    batch 64, bf16 records, zero initial state), shortened to 48 steps (3
    flushes): the whole batch runs on the GPU, and two sequences are followed
    by the oracle running the same storage formats. The first window (before
    any fold quantizes) is held to 1e-5."""
    w = W.M2_LOWPREC
    seqs = [0, w.batch - 1]
    p = W.m2_params(w)
    A, D = params_dev(p)
    code = {"f32": rs.RS_F32, "f16": rs.RS_F16, "fp8": rs.RS_FP8E4M3, "nvfp4": rs.RS_NVFP4}[fmt]
    layer, bufs = m2_layer(w, ckpt_dtype=code, read_copy=rs.RS_NVFP4 if rc else rs.RS_NONE, fuse=1)
    if rc:
        rs.rs_requant_read_copy(layer, bufs)
    H0 = W.m2_init_states(w, seqs)
    ref = decode.M2Replay(H0, p["A"], p["D"], ckpt_fmt=fmt, read_copy=rc)
    first, worst = 0.0, 0.0
    for t in range(48):
        tok = W.m2_step(w, t, range(w.batch))
        y = y_buf(w.batch, w.nheads, w.headdim)
        fn = rs.rs_step_flush if t % 16 == 15 else rs.rs_step_nonflush
        fn(layer, bufs, m2_tok_dev(tok, w.in_dtype), A, D, y)
        e = rel_l2(y.cpu().numpy()[seqs], ref.step(W.m2_step(w, t, seqs)))
        if t < 15:
            first = max(first, e)
        worst = max(worst, e)
    print(f"batch-64 {fmt}{' + nvfp4 reads' if rc else ''}: first window {first:.2e}, worst {worst:.2e}")
    assert first <= 1e-5 and worst <= gate
