"""The bandwidth probes of librs_probe.so (include/rs_probe.h) do the work their
numbers are quoted for: every tile's loads are summed (rs_probe_read writes the
tile sum), and rs_probe_read_write stores its write_bytes per tile, each lane
16 bytes of its wavefront's sum. Checked against numpy on a small buffer of
seeded values; fp32 sums in the probe's order, so compared within 1e-4."""
import ctypes as C
import os

import numpy as np
import pytest
import torch

from gpu_harness import DEV, require_gpu

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def setup_module(_):
    require_gpu()


def _lib():
    lib = C.CDLL(os.path.join(ROOT, "ssm_decode_checkpoint_amd", "librs_probe.so"))
    lib.rs_probe_read.argtypes = [C.c_void_p, C.c_void_p, C.c_uint64, C.c_int32, C.c_int32, C.c_void_p]
    lib.rs_probe_read.restype = C.c_int32
    lib.rs_probe_read_write.argtypes = [C.c_void_p, C.c_void_p, C.c_uint64, C.c_int32, C.c_int32, C.c_int32,
                                        C.c_void_p]
    lib.rs_probe_read_write.restype = C.c_int32
    return lib


def _src(tiles, threads, per):
    n = tiles * threads * per * 4                       # floats
    host = np.random.default_rng(501).standard_normal(n).astype(np.float32)
    return host, torch.from_numpy(host).to(DEV)


def _stream():
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("threads,per", [(256, 8), (256, 4), (128, 16)])
def test_read_sums_every_tile(threads, per):
    tiles = 12
    host, src = _src(tiles, threads, per)
    out = torch.full((tiles,), float("nan"), dtype=torch.float32, device=DEV)
    assert _lib().rs_probe_read(src.data_ptr(), out.data_ptr(), src.numel() * 4, threads, per, _stream()) == 0
    torch.cuda.synchronize()
    ref = host.astype(np.float64).reshape(tiles, -1).sum(axis=1)
    np.testing.assert_allclose(out.cpu().numpy(), ref, rtol=1e-4, atol=1e-3)


@pytest.mark.parametrize("wbytes", [16, 416, 4096])
def test_read_write_stores_wave_sums(wbytes):
    threads, per, tiles = 256, 8, 12
    host, src = _src(tiles, threads, per)
    wvec = wbytes // 16
    dst = torch.full((tiles * wvec * 4,), float("nan"), dtype=torch.float32, device=DEV)
    st = _lib().rs_probe_read_write(src.data_ptr(), dst.data_ptr(), src.numel() * 4, threads, per, wbytes,
                                    _stream())
    assert st == 0
    torch.cuda.synchronize()
    got = dst.cpu().numpy().reshape(tiles, wvec, 4)
    # thread t of a tile reads the 16-byte vectors t + k * threads, k < per
    v = host.astype(np.float64).reshape(tiles, per, threads, 4)
    per_thread = v.sum(axis=(1, 3))                        # [tiles][threads]
    wave = per_thread.reshape(tiles, threads // 64, 64).sum(axis=2)
    for lane in range(wvec):
        exp = wave[:, lane // 64]
        for i in range(4):
            np.testing.assert_allclose(got[:, lane, i], exp, rtol=1e-4, atol=1e-3)


# variant -> (threads, 16-byte loads per thread) of its tile
VARIANTS = {0: (256, 8), 1: (256, 8), 2: (256, 16), 3: (256, 8), 4: (256, 16), 5: (256, 8)}


@pytest.mark.parametrize("variant", sorted(VARIANTS))
def test_read_variants_sum_every_tile(variant):
    """Each variant of rs_probe_read_variant reads every byte once per tile and
    writes the tile's sum. The persistent variant runs enough tile pairs (6000
    tiles) that every workgroup loops several times on this chip."""
    lib = _lib()
    lib.rs_probe_read_variant.argtypes = [C.c_void_p, C.c_void_p, C.c_uint64, C.c_int32, C.c_void_p]
    lib.rs_probe_read_variant.restype = C.c_int32
    threads, per = VARIANTS[variant]
    tiles = 6000 if variant == 5 else 12
    host, src = _src(tiles, threads, per)
    out = torch.full((tiles,), float("nan"), dtype=torch.float32, device=DEV)
    print(f"probe variant {variant}: {tiles} tiles of {threads * per * 16} bytes", flush=True)
    assert lib.rs_probe_read_variant(src.data_ptr(), out.data_ptr(), src.numel() * 4, variant, _stream()) == 0
    torch.cuda.synchronize()
    ref = host.astype(np.float64).reshape(tiles, -1).sum(axis=1)
    np.testing.assert_allclose(out.cpu().numpy(), ref, rtol=1e-4, atol=1e-3)
