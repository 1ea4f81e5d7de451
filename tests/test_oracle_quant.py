"""Pins for the quantizer emulation.

* Format tables and round-to-nearest-even cases from the published format
  definitions (tests/golden/fp_formats.json).
* E4M3 encoding agrees with torch's float8_e4m3fn conversion (a library
  routine) wherever the value is in range; fp16 agrees with numpy.float16.
* NVFP4: representable inputs round-trip exactly, quantize(dequantize(q)) = q,
  every element error is within half an e2m1 step of its block scale, and
  the block scale is the E4M3 rounding of block-amax / (6 * tensor scale).
"""
import json
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import quant

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold():
    with open(os.path.join(GOLD, "fp_formats.json")) as f:
        return json.load(f)


def test_e2m1_table_and_ties():
    g = _gold()
    assert quant.e2m1_decode(np.arange(8)).tolist() == g["e2m1_magnitudes"]
    xs = np.array([a for a, _ in g["e2m1_round_nearest_even"]], np.float32)
    want = np.array([b for _, b in g["e2m1_round_nearest_even"]], np.float32)
    np.testing.assert_array_equal(quant.e2m1_decode(quant.e2m1_encode(xs)), want)


def test_e4m3_table_and_ties():
    g = _gold()
    for code, val in g["e4m3_code_values"]:
        assert float(quant.e4m3_decode(np.uint8(code))) == val
    for x, code in g["e4m3_round_nearest_even"]:
        assert int(quant.e4m3_encode_mag(np.float32(x))) == code


def test_e4m3_matches_torch_float8():
    r = np.random.default_rng(0)
    x = np.concatenate([np.exp2(r.uniform(-14, 8.8, 20000)), r.uniform(0, 448, 5000),
                        quant.E4M3_MAG.astype(np.float32)]).astype(np.float32)
    x = x[x <= 448]
    mine = quant.e4m3_encode_mag(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(mine, ref)


def test_e2m1_exhaustive_midpoints():
    mags = quant.E2M1_MAG.astype(np.float64)
    for i in range(7):
        lo, hi = mags[i], mags[i + 1]
        mid = (lo + hi) / 2
        assert quant.e2m1_decode(quant.e2m1_encode(np.float32(mid))) == (lo if i % 2 == 0 else hi)
        eps = (hi - lo) * 1e-3
        assert quant.e2m1_decode(quant.e2m1_encode(np.float32(mid - eps))) == lo
        assert quant.e2m1_decode(quant.e2m1_encode(np.float32(mid + eps))) == hi


def test_fp16_matches_numpy():
    x = W.state_tiles(1, 0, (64, 64), heavy_tail=True)
    np.testing.assert_array_equal(quant.fp16_roundtrip(x), x.astype(np.float16).astype(np.float32))


def test_nibble_packing():
    c = (np.arange(64, dtype=np.uint8) % 16).reshape(4, 16)
    p = quant.pack_nibbles(c)
    assert p[0, 0] == (0 | (1 << 4))
    np.testing.assert_array_equal(quant.unpack_nibbles(p), c)


@pytest.mark.parametrize("heavy", [False, True])
def test_nvfp4_properties(heavy):
    x = W.state_tiles(2, int(heavy), (32, 64), std=0.1, heavy_tail=heavy)
    codes, s, ts = quant.nvfp4_quantize(x)
    amax = np.float32(np.abs(x).max())
    assert ts == np.float32(amax / np.float32(2688.0))
    # block scale = E4M3(bamax / (6 ts)), checked with torch's conversion
    bamax = np.abs(x.reshape(32, 4, 16)).max(-1).astype(np.float32)
    q = (bamax / np.float32(np.float32(6.0) * ts)).astype(np.float32)
    ref_s = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(s, ref_s)
    xh = quant.nvfp4_dequantize(codes, s, ts)
    # idempotence, for blocks whose scale is a normal E4M3 number (in the subnormal
    # range the coarse scale grid can move the re-quantized block to another scale)
    c2, s2, ts2 = quant.nvfp4_quantize(xh)
    normal = np.repeat(s >= 8, 16, axis=1)
    assert normal.mean() > 0.5
    np.testing.assert_array_equal(quant.nvfp4_dequantize(c2, s2, ts2)[normal], xh[normal])
    # error within half a step of the e2m1 grid, per block scale
    sd = (quant.e4m3_decode(s) * ts).astype(np.float64)
    qv = np.abs(x.reshape(32, 4, 16).astype(np.float64)) / np.where(sd == 0, 1, sd)[..., None]
    gap = np.where(qv < 2, 0.5, np.where(qv < 4, 1.0, 2.0))
    err = np.abs(x.reshape(32, 4, 16) - xh.reshape(32, 4, 16))
    ax = np.abs(x.reshape(32, 4, 16))
    bound = np.where(qv <= 6, 0.5 * gap * sd[..., None], ax - 6 * sd[..., None])
    # a block whose scale underflows E4M3 (below half its smallest subnormal) reads as zero
    bound = np.where((sd == 0)[..., None], ax, bound)
    assert np.all(q[sd == 0] <= 2.0 ** -10)
    assert np.all(err <= bound + 1e-6 * sd[..., None] + 1e-30)


def test_nvfp4_representable_roundtrip():
    # values already on the NVFP4 grid of their own scales come back exactly
    r = np.random.default_rng(3)
    mags = quant.E2M1_MAG[r.integers(0, 8, (16, 64))]
    signs = np.where(r.random((16, 64)) < 0.5, -1, 1)
    x = (mags * signs).astype(np.float32)
    x[:, ::16] = 6.0                   # each block reaches 6 so its scale is exactly 1/448 * 448
    ts = np.float32(6.0 / 2688.0)
    codes, s, ts_ = quant.nvfp4_quantize(x)
    assert ts_ == np.float32(np.float32(6.0) / np.float32(2688.0))
    np.testing.assert_allclose(quant.nvfp4_dequantize(codes, s, ts_), x, rtol=2e-7)
    assert abs(float(ts_) - float(ts)) <= 1e-9


def test_nvfp4_zero_tile_and_zero_block():
    x = np.zeros((4, 32), np.float32)
    codes, s, ts = quant.nvfp4_quantize(x)
    assert ts == 1.0 and not codes.any() and not s.any()
    x[1, 20] = 3.0
    codes, s, ts = quant.nvfp4_quantize(x)
    assert quant.nvfp4_dequantize(codes, s, ts)[1, 20] == 3.0
    assert s[0].tolist() == [0, 0] and s[1, 0] == 0


def test_fp8_checkpoint_format():
    x = W.state_tiles(4, 0, (16, 64), std=0.5)
    codes, scale = quant.fp8_quantize(x)
    assert scale == np.float32(np.float32(np.abs(x).max()) / np.float32(448.0))
    ref = torch.from_numpy((np.abs(x) / scale).astype(np.float32)).to(torch.float8_e4m3fn)
    np.testing.assert_array_equal(codes & 0x7F, ref.view(torch.uint8).numpy())
    assert np.all((codes >> 7) == np.signbit(x))
    xh = quant.fp8_dequantize(codes, scale)
    assert np.all(np.abs(xh - x) <= np.abs(x) / 16 + 2.0 ** -9 * scale)


def test_saturation_over_the_whole_float32_range():
    """Both encoders saturate at their largest finite code for every magnitude
    above it, up to the largest float32 and infinity (the formats' saturating
    conversion); the sign is kept."""
    big = np.array([6.0, 6.5, 1e6, 1e16, 1e20, 1e30, 3.4e38, np.inf], np.float32)
    assert quant.e2m1_encode(big).tolist() == [7] * big.size
    assert quant.e2m1_encode(-big).tolist() == [15] * big.size
    big8 = np.array([448.0, 464.0, 1e6, 1e17, 1e20, 1e30, 3.4e38, np.inf], np.float32)
    assert quant.e4m3_encode_mag(big8).tolist() == [126] * big8.size
