"""The code-flip classifier used by the low-precision GPU tests, checked on the
CPU: identical codes pass, a flip next to a rounding boundary is allowed and
counted, and a flip away from a boundary, a jump over a code, a wrong scale or
a moved block are caught (mistakes planted on the oracle's own codes)."""
import numpy as np
import pytest

import ssm_decode_checkpoint_amd as rs
import lowprec_codes as LC
from oracle import quant

F32 = np.float32


def _tiles(seed, shape=(2, 3, 8, 32)):
    g = np.random.default_rng(seed)
    return (g.standard_normal(shape) * 0.3).astype(F32)


@pytest.mark.parametrize("fmt", ["f32", "f16", "fp8", "nvfp4"])
def test_identical_codes_pass_and_decode_matches_roundtrip(fmt):
    x = _tiles(1)
    enc = LC.encode(fmt, x)
    fl = LC.compare(fmt, enc, enc, x.astype(np.float64))
    assert not fl.bad and fl.elements == 0 and fl.scales == 0
    want = np.stack([np.stack([quant.roundtrip(fmt, x[i, j]) for j in range(x.shape[1])]) for i in range(x.shape[0])])
    assert np.array_equal(LC.decode(fmt, enc), want)


@pytest.mark.parametrize("fmt,code", [("f16", rs.RS_F16), ("fp8", rs.RS_FP8E4M3), ("nvfp4", rs.RS_NVFP4),
                                      ("f32", rs.RS_F32)])
def test_device_bytes_roundtrip(fmt, code):
    cfg = rs.make_config(rs.RS_MAMBA2, 2, nheads=3, headdim=16, dstate=16, ngroups=1, in_dtype=rs.RS_F32,
                         ckpt_dtype=code)
    _, layer = rs.rs_init(cfg)
    x = _tiles(2, (2, 3, 16, 16))
    enc = LC.encode(fmt, x)
    raw = LC.to_device_bytes(layer, fmt, enc)
    assert raw.size == layer.ckpt_bytes
    back = LC.from_device_bytes(layer, fmt, raw)
    for k in enc:
        assert np.array_equal(np.asarray(back[k]).view(np.uint8), np.asarray(enc[k]).view(np.uint8)), k


def _boundary_case_f16():
    """fp16 value m exactly between two fp16 numbers; the fold sits 1e-6 above it."""
    lo = np.float16(1.0)
    hi = np.nextafter(lo, np.float16(2.0))
    mid = (float(lo) + float(hi)) / 2
    x = np.full((1, 1, 1, 16), 0.5, np.float64)
    x[0, 0, 0, 3] = mid + 1e-6
    return x, lo, hi


def test_f16_flip_at_boundary_allowed_else_caught():
    x, lo, hi = _boundary_case_f16()
    ora = LC.encode("f16", x.astype(F32))
    assert ora["codes"][0, 0, 0, 3] == hi.view(np.uint16)      # the fold rounds up
    gpu = {"codes": ora["codes"].copy()}
    gpu["codes"][0, 0, 0, 3] = lo.view(np.uint16)                # device rounded down: allowed
    fl = LC.compare("f16", gpu, ora, x)
    assert not fl.bad and fl.elements == 1
    gpu["codes"][0, 0, 0, 5] = np.float16(0.5).view(np.uint16) + 1   # flip far from a boundary
    assert LC.compare("f16", gpu, ora, x).bad
    gpu = {"codes": ora["codes"].copy()}
    gpu["codes"][0, 0, 0, 3] = hi.view(np.uint16) + 1            # jumps a code
    assert LC.compare("f16", gpu, ora, x).bad


def test_fp8_scale_and_codes():
    x = _tiles(3).astype(np.float64)
    ora = LC.encode("fp8", x.astype(F32))
    gpu = {k: v.copy() for k, v in ora.items()}
    gpu["scale"][1, 2] *= F32(1.001)                             # wrong matrix scale
    assert LC.compare("fp8", gpu, ora, x).bad
    gpu = {k: v.copy() for k, v in ora.items()}
    c = gpu["codes"][0, 1, 2, 7]
    gpu["codes"][0, 1, 2, 7] = (c & 0x80) | ((c & 0x7F) + 1)     # one code up, not at a boundary
    assert LC.compare("fp8", gpu, ora, x).bad
    # at a boundary: put an element exactly between two e4m3 values of its matrix scale
    s = float(ora["scale"][0, 1])
    mid = (quant.E4M3_MAG[40] + quant.E4M3_MAG[41]) / 2 * s
    x2 = x.copy()
    x2[0, 1, 2, 7] = mid
    ora2 = LC.encode("fp8", x2.astype(F32))
    assert ora2["scale"][0, 1] == ora["scale"][0, 1]
    gpu = {k: v.copy() for k, v in ora2.items()}
    c = int(gpu["codes"][0, 1, 2, 7]) & 0x7F
    gpu["codes"][0, 1, 2, 7] = 41 if c == 40 else 40
    fl = LC.compare("fp8", gpu, ora2, x2)
    assert not fl.bad and fl.elements == 1


def test_nvfp4_codes_scales_and_moved_block():
    x = _tiles(4).astype(np.float64)
    ora = LC.encode("nvfp4", x.astype(F32))
    gpu = {k: v.copy() for k, v in ora.items()}
    gpu["scales"][0, 0, 1, 1] += 1                               # block scale off, away from its boundary
    assert LC.compare("nvfp4", gpu, ora, x).bad
    gpu = {k: v.copy() for k, v in ora.items()}
    gpu["codes"][1, 2, 3, 16:32] = ora["codes"][1, 2, 3, 0:16]   # a block written in the wrong place
    assert LC.compare("nvfp4", gpu, ora, x).bad
    gpu = {k: v.copy() for k, v in ora.items()}
    gpu["ts"][1, 1] = np.nextafter(gpu["ts"][1, 1], F32(1)) * F32(1.01)
    assert LC.compare("nvfp4", gpu, ora, x).bad
    # an element exactly on the 1.25 tie of its block: the neighbouring code is allowed
    sd = float(quant.e4m3_decode(ora["scales"][0, 0, 2, 0]) * ora["ts"][0, 0])
    x2 = x.copy()
    x2[0, 0, 2, 5] = 1.25 * sd
    ora2 = LC.encode("nvfp4", x2.astype(F32))
    assert ora2["scales"][0, 0, 2, 0] == ora["scales"][0, 0, 2, 0] and ora2["ts"][0, 0] == ora["ts"][0, 0]
    gpu = {k: v.copy() for k, v in ora2.items()}
    c = int(gpu["codes"][0, 0, 2, 5])
    assert c & 7 == 2                                             # ties to even: 1.0
    gpu["codes"][0, 0, 2, 5] = (c & 8) | 3
    fl = LC.compare("nvfp4", gpu, ora2, x2)
    assert not fl.bad and fl.elements == 1


def test_f32_fold_tolerance():
    x = _tiles(5).astype(np.float64)
    ora = LC.encode("f32", x.astype(F32))
    gpu = {"codes": ora["codes"].copy()}
    gpu["codes"][0, 0, 0, 0] += F32(1e-3)
    assert LC.compare("f32", gpu, ora, x).bad
