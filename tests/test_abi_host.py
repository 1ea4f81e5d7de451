"""Host-only checks of the C ABI: the library loads, exports every entry point
include/rs.h declares, sizes buffers as the header documents, and rejects
invalid configurations and arguments before launching anything. No device
call is made here."""
import ctypes as C
import re
import os

import pytest

import ssm_decode_checkpoint_amd as rs

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "rs.h")


def _declared():
    src = open(HDR).read()
    return sorted(set(re.findall(r"^\s*(?:rs_status|const char\*|int32_t)\s+(rs_\w+)\s*\(", src, re.M)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) >= {"rs_init", "rs_step_conventional", "rs_step_nonflush", "rs_step_flush",
                          "rs_spec_append", "rs_spec_commit", "rs_requant_read_copy"}
    lib = rs.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert rs.rs_version() >= 100
    assert rs.status_string(rs.RS_E_ALIGN).startswith("pointer")


def test_probe_library_exports_and_checks_arguments():
    """librs_probe.so (the read-stream measurement helper) exports what
    include/rs_probe.h declares and rejects bad arguments before launching."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    hdr = open(os.path.join(root, "include", "rs_probe.h")).read()
    names = re.findall(r"^\s*int32_t\s+(rs_\w+)\s*\(", hdr, re.M)
    assert names == ["rs_probe_read", "rs_probe_read_write", "rs_probe_read_variant"]
    lib = C.CDLL(os.path.join(root, "ssm_decode_checkpoint_amd", "librs_probe.so"))
    f = lib.rs_probe_read
    f.argtypes = [C.c_void_p, C.c_void_p, C.c_uint64, C.c_int32, C.c_int32, C.c_void_p]
    f.restype = C.c_int32
    p = C.c_void_p(0x10000)
    assert f(None, p, 1 << 20, 256, 8, None) == -1
    assert f(C.c_void_p(0x10004), p, 1 << 20, 256, 8, None) == -1
    assert f(p, p, (1 << 20) + 16, 256, 8, None) == -2 and f(p, p, 0, 256, 4, None) == -2
    assert f(p, p, 1 << 20, 64, 8, None) == -4
    g = lib.rs_probe_read_write
    g.argtypes = [C.c_void_p, C.c_void_p, C.c_uint64, C.c_int32, C.c_int32, C.c_int32, C.c_void_p]
    g.restype = C.c_int32
    assert g(p, None, 1 << 20, 256, 8, 256, None) == -1
    assert g(p, C.c_void_p(0x10008), 1 << 20, 256, 8, 256, None) == -1
    assert g(p, p, (1 << 20) + 16, 256, 8, 256, None) == -2
    for wb in (0, -16, 8, 24, 256 * 16 + 16):
        assert g(p, p, 1 << 20, 256, 8, wb, None) == -5, wb
    assert g(p, p, 1 << 20, 128, 16, 128 * 16 + 16, None) == -5
    assert g(p, p, 1 << 20, 64, 8, 256, None) == -4
    v = lib.rs_probe_read_variant
    v.argtypes = [C.c_void_p, C.c_void_p, C.c_uint64, C.c_int32, C.c_void_p]
    v.restype = C.c_int32
    assert v(None, p, 1 << 20, 0, None) == -1 and v(C.c_void_p(0x10004), p, 1 << 20, 0, None) == -1
    assert v(p, p, 1 << 20, -1, None) == -4 and v(p, p, 1 << 20, 6, None) == -4
    assert v(p, p, 32 << 10, 2, None) == -2 and v(p, p, 32 << 10, 4, None) == -2   # 64 KiB tiles
    assert v(p, p, 32 << 10, 5, None) == -2 and v(p, p, 96 << 10, 5, None) == -2   # whole tile pairs
    assert v(p, p, 0, 0, None) == -2


def test_struct_sizes_match_header():
    assert C.sizeof(rs.RsConfig) == 17 * 4
    assert C.sizeof(rs.RsBuffers) == 5 * 8
    assert C.sizeof(rs.RsInputs) == 9 * 8


def _m2(**kw):
    base = dict(batch=256, nheads=128, headdim=64, dstate=128, ngroups=8)
    base.update(kw)
    b = base.pop("batch")
    return rs.make_config(rs.RS_MAMBA2, b, **base)


def test_mamba2_layout_sizes():
    st, L = rs.rs_init(_m2())
    assert st == rs.RS_OK
    assert L.ckpt_bytes == 256 * 128 * 64 * 128 * 4          # 4 MiB per sequence, fp32
    assert (L.heads, L.in_heads, L.rows, L.cols) == (128, 8, 128, 64)
    ring = 256 * 16 * (128 * 64 + 2 * 8 * 128 + 128) * 2    # x, B, C, dt bf16, 16 slots
    assert ring <= L.ring_bytes < ring + 4 * 256
    assert L.ring_x_off == 0 and L.ring_B_off >= 256 * 128 * 16 * 64 * 2
    assert L.meta_bytes >= 256 * 32 and L.read_copy_bytes == 0 and L.snap_bytes == 0
    st, L = rs.rs_init(_m2(read_copy=rs.RS_NVFP4))
    mats = 256 * 128
    assert L.read_copy_bytes >= mats * (8192 // 2 + 8192 // 16 + 4)
    assert L.nv_scale_off >= mats * 4096 and L.nv_tscale_off >= L.nv_scale_off + mats * 512
    st, L = rs.rs_init(_m2(mode=rs.RS_CONVENTIONAL, max_draft=4, batch=512))
    assert L.snap_bytes == 4 * 512 * 128 * 64 * 128 * 4 and L.ring_bytes == 0
    st, L = rs.rs_init(_m2(ckpt_dtype=rs.RS_FP8E4M3))
    assert L.ckpt_bytes >= mats * 8192 + mats * 4 and L.ck_scale_off >= mats * 8192


def test_gdn_layout_sizes():
    cfg = rs.make_config(rs.RS_GDN, 256, n_qk_heads=16, n_v_heads=32, head_k_dim=128, head_v_dim=128)
    st, L = rs.rs_init(cfg, raise_on_error=False)
    assert st == rs.RS_OK or st == rs.RS_E_UNSUPPORTED
    if st == rs.RS_OK:
        assert L.ckpt_bytes == 256 * 32 * 128 * 128 * 4


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_delta_rule_low_precision_checkpoints(kind):
    """FP16 / FP8 checkpoints of the delta-rule layers: replay mode without a read
    copy, on the 16 x 16 and 128 x 128 states; the stored matrix in 2 or 1 bytes
    per element, FP8 with one fp32 scale per matrix after the codes."""
    k = rs.RS_KDA if kind == "kda" else rs.RS_GDN
    kw = dict(n_qk_heads=2, n_v_heads=4, head_k_dim=128, head_v_dim=128)
    mats = 8 * 4
    _, L32 = rs.rs_init(rs.make_config(k, 8, **kw))
    _, L16 = rs.rs_init(rs.make_config(k, 8, ckpt_dtype=rs.RS_F16, **kw))
    _, L8 = rs.rs_init(rs.make_config(k, 8, ckpt_dtype=rs.RS_FP8E4M3, **kw))
    assert L32.ckpt_bytes == mats * 128 * 128 * 4
    assert L16.ckpt_bytes >= mats * 128 * 128 * 2
    assert L8.ck_scale_off >= mats * 128 * 128 and L8.ckpt_bytes >= L8.ck_scale_off + mats * 4
    assert L16.ring_bytes == L32.ring_bytes and L8.meta_bytes == L32.meta_bytes
    tiny = dict(n_qk_heads=1, n_v_heads=2, head_k_dim=16, head_v_dim=16)
    for dt in (rs.RS_F16, rs.RS_FP8E4M3):
        assert rs.rs_init(rs.make_config(k, 2, ckpt_dtype=dt, **tiny), raise_on_error=False)[0] == rs.RS_OK
        assert rs.rs_init(rs.make_config(k, 2, ckpt_dtype=dt, mode=rs.RS_CONVENTIONAL, **tiny),
                          raise_on_error=False)[0] == rs.RS_E_DTYPE
        assert rs.rs_init(rs.make_config(k, 2, ckpt_dtype=dt, read_copy=rs.RS_NVFP4, **tiny),
                          raise_on_error=False)[0] == rs.RS_E_DTYPE
        assert rs.rs_init(rs.make_config(k, 2, ckpt_dtype=dt, n_qk_heads=1, n_v_heads=2, head_k_dim=64,
                                         head_v_dim=64), raise_on_error=False)[0] == rs.RS_E_UNSUPPORTED
    assert rs.rs_init(rs.make_config(k, 2, ckpt_dtype=rs.RS_NVFP4, **tiny), raise_on_error=False)[0] == rs.RS_E_DTYPE


def test_reset_slots_host_checks():
    """rs_reset_slots: argument and mode checks happen on the host; count == 0 launches nothing."""
    lib = rs.lib()
    _, L = rs.rs_init(_m2(batch=2, nheads=8, headdim=16, dstate=16, ngroups=1))
    bufs = rs.RsBuffers(0x1000, 0x2000, None, 0x3000, None)
    assert lib.rs_reset_slots(C.byref(L), C.byref(bufs), C.c_void_p(0x1000), 0, None) == rs.RS_OK
    assert lib.rs_reset_slots(C.byref(L), C.byref(bufs), None, 2, None) == rs.RS_E_ARG
    assert lib.rs_reset_slots(C.byref(L), C.byref(bufs), C.c_void_p(0x1000), -1, None) == rs.RS_E_ARG
    nometa = rs.RsBuffers(0x1000, 0x2000, None, None, None)
    assert lib.rs_reset_slots(C.byref(L), C.byref(nometa), C.c_void_p(0x1000), 1, None) == rs.RS_E_ARG
    _, Lc = rs.rs_init(_m2(batch=2, nheads=8, headdim=16, dstate=16, ngroups=1, mode=rs.RS_CONVENTIONAL))
    assert lib.rs_reset_slots(C.byref(Lc), C.byref(bufs), C.c_void_p(0x1000), 1, None) == rs.RS_E_MODE
    assert lib.rs_step(C.byref(Lc), C.byref(bufs), C.byref(rs.RsInputs()), C.byref(rs.RsParams()), C.c_void_p(0x1000),
                       None) == rs.RS_E_MODE


def test_copy_slots_host_checks():
    """rs_copy_slots: configurations must match except batch; pointer, count and
    alignment checks happen on the host; count == 0 launches nothing."""
    lib = rs.lib()
    kw = dict(nheads=8, headdim=16, dstate=16, ngroups=1)
    _, L = rs.rs_init(_m2(batch=4, **kw))
    _, Lc = rs.rs_init(_m2(batch=2, **kw))                      # a cache of another batch: fine
    _, Lx = rs.rs_init(_m2(batch=2, nheads=4, headdim=16, dstate=16, ngroups=1))
    _, Lf = rs.rs_init(_m2(batch=2, ckpt_dtype=rs.RS_F16, **kw))
    bufs = rs.RsBuffers(0x1000, 0x2000, None, 0x3000, None)
    seqs = C.c_void_p(0x4000)

    def call(Ls, Ld, b1=bufs, b2=bufs, s1=seqs, s2=seqs, n=1):
        return lib.rs_copy_slots(C.byref(Ls), C.byref(b1), s1, C.byref(Ld), C.byref(b2), s2, n, None)

    assert call(L, Lc, n=0) == rs.RS_OK
    assert call(L, Lx, n=0) == rs.RS_E_ARG and call(L, Lf, n=0) == rs.RS_E_ARG
    assert call(L, Lc, s1=None) == rs.RS_E_ARG and call(L, Lc, n=-1) == rs.RS_E_ARG
    assert call(L, Lc, n=65536) == rs.RS_E_ARG
    assert call(L, Lc, b2=rs.RsBuffers(0x1000, None, None, 0x3000, None)) == rs.RS_E_ARG   # no ring
    assert call(L, Lc, b2=rs.RsBuffers(0x1004, 0x2000, None, 0x3000, None)) == rs.RS_E_ALIGN
    _, Lr = rs.rs_init(_m2(batch=4, read_copy=rs.RS_NVFP4, **kw))
    assert call(Lr, Lr) == rs.RS_E_ARG                                                   # no read copy
    L.magic = 0
    assert call(L, Lc, n=0) == rs.RS_E_ARG


def test_block_calls_host_checks():
    """rs_conv_step / rs_gated_norm: kind, mode, K, width, group and pointer checks on the host."""
    lib = rs.lib()
    kw = dict(nheads=8, headdim=16, dstate=16, ngroups=1)
    _, L = rs.rs_init(_m2(batch=2, **kw))
    _, Ls = rs.rs_init(_m2(batch=2, max_draft=4, **kw))
    _, Lc = rs.rs_init(_m2(batch=2, mode=rs.RS_CONVENTIONAL, **kw))
    _, G = rs.rs_init(rs.make_config(rs.RS_GDN, 2, n_qk_heads=1, n_v_heads=2, head_k_dim=16, head_v_dim=16))
    bufs = rs.RsBuffers(0x1000, 0x2000, None, 0x3000, None)
    p = C.c_void_p(0x4000)

    def conv(Lx, K=1, width=4, ring=p, x=p, bb=bufs):
        return lib.rs_conv_step(C.byref(Lx), C.byref(bb), ring, p, K, p, None, width, x, p, p, None)

    assert conv(Lc) == rs.RS_E_MODE and conv(G) == rs.RS_E_MODE
    assert conv(L, K=2) == rs.RS_E_ARG and conv(Ls, K=5) == rs.RS_E_ARG and conv(L, K=0) == rs.RS_E_ARG
    assert conv(L, width=5) == rs.RS_E_ARG and conv(L, width=0) == rs.RS_E_ARG
    assert conv(L, ring=None) == rs.RS_E_ARG and conv(L, x=C.c_void_p(0x4004)) == rs.RS_E_ALIGN
    assert conv(L, bb=rs.RsBuffers(0x1000, 0x2000, None, None, None)) == rs.RS_E_ARG

    def norm(Lx, K=1, groups=1, eps=1e-5, out=p):
        return lib.rs_gated_norm(C.byref(Lx), K, p, p, p, groups, C.c_float(eps), out, None)

    assert norm(G) == rs.RS_E_MODE and norm(L, K=2) == rs.RS_E_ARG
    assert norm(L, groups=3) == rs.RS_E_ARG and norm(L, groups=0) == rs.RS_E_ARG
    assert norm(L, eps=-1.0) == rs.RS_E_ARG and norm(L, eps=float("nan")) == rs.RS_E_ARG
    assert norm(L, out=None) == rs.RS_E_ARG
    assert rs.conv_channels(L) == 8 * 16 + 2 * 16 and rs.conv_ring_bytes(L) == 2 * 16 * 160 * 2   # bf16


def test_kda_layout_sizes():
    """Kimi Delta Attention: the GDN layout with a dk-wide gate per ring entry;
    speculative configs get the GDN snapshot area (conventional mode)."""
    kw = dict(n_qk_heads=16, n_v_heads=32, head_k_dim=128, head_v_dim=128)
    _, G = rs.rs_init(rs.make_config(rs.RS_GDN, 4, **kw))
    _, K = rs.rs_init(rs.make_config(rs.RS_KDA, 4, **kw))
    assert K.ckpt_bytes == G.ckpt_bytes == 4 * 32 * 128 * 128 * 4
    gdn_g = G.ring_beta_off - G.ring_g_off
    kda_g = K.ring_beta_off - K.ring_g_off
    assert gdn_g >= 4 * 32 * 16 * 4 and kda_g >= 4 * 32 * 16 * 128 * 4 and kda_g < 4 * 32 * 16 * 128 * 4 + 256
    _, Ks = rs.rs_init(rs.make_config(rs.RS_KDA, 4, max_draft=4, mode=rs.RS_CONVENTIONAL, **kw))
    _, Gs = rs.rs_init(rs.make_config(rs.RS_GDN, 4, max_draft=4, mode=rs.RS_CONVENTIONAL, **kw))
    assert Ks.snap_bytes == Gs.snap_bytes == 4 * K.ckpt_bytes
    st, _ = rs.rs_init(rs.make_config(4, 4, **kw), raise_on_error=False)
    assert st == rs.RS_E_ARG


@pytest.mark.parametrize("kw,code", [
    (dict(ring=8), rs.RS_E_ARG),
    (dict(batch=0), rs.RS_E_ARG),
    (dict(ngroups=3), rs.RS_E_ARG),
    (dict(dstate=96), rs.RS_E_UNSUPPORTED),
    (dict(in_dtype=rs.RS_F16), rs.RS_E_DTYPE),
    (dict(ckpt_dtype=rs.RS_BF16), rs.RS_E_DTYPE),
    (dict(read_copy=rs.RS_F16), rs.RS_E_DTYPE),
    (dict(ckpt_dtype=rs.RS_NVFP4, read_copy=rs.RS_NVFP4), rs.RS_E_DTYPE),
    (dict(mode=rs.RS_CONVENTIONAL, ckpt_dtype=rs.RS_F16), rs.RS_E_DTYPE),
    (dict(mode=7), rs.RS_E_MODE),
    (dict(max_draft=9), rs.RS_E_ARG),
    (dict(fuse_requant=2), rs.RS_E_ARG),
])
def test_init_rejects(kw, code):
    st, _ = rs.rs_init(_m2(**kw), raise_on_error=False)
    assert st == code


def test_calls_reject_before_launch():
    _, L = rs.rs_init(_m2(batch=2, nheads=8, headdim=16, dstate=16, ngroups=1))
    lib = rs.lib()
    y = C.c_void_p(0x1000)
    bufs = rs.RsBuffers(0x1000, 0x2000, None, 0x3000, None)
    inp = rs.RsInputs(0x1000, 0x1000, 0x1000, 0x1000, None, None, None, None, None)
    prm = rs.RsParams(0x1000, 0x1000)
    # uninitialised layer
    assert lib.rs_step_nonflush(C.byref(rs.RsLayer()), C.byref(bufs), C.byref(inp), C.byref(prm), y, None) == rs.RS_E_ARG
    # null output / null input pointers
    assert lib.rs_step_nonflush(C.byref(L), C.byref(bufs), C.byref(inp), C.byref(prm), None, None) == rs.RS_E_ARG
    bad = rs.RsInputs(0x1000, None, 0x1000, 0x1000, None, None, None, None, None)
    assert lib.rs_step_flush(C.byref(L), C.byref(bufs), C.byref(bad), C.byref(prm), y, None) == rs.RS_E_ARG
    # misaligned pointers
    mis = rs.RsInputs(0x1004, 0x1000, 0x1000, 0x1000, None, None, None, None, None)
    assert lib.rs_step_nonflush(C.byref(L), C.byref(bufs), C.byref(mis), C.byref(prm), y, None) == rs.RS_E_ALIGN
    assert lib.rs_step_nonflush(C.byref(L), C.byref(bufs), C.byref(inp), C.byref(prm), C.c_void_p(0x1008), None) == rs.RS_E_ALIGN
    misb = rs.RsBuffers(0x1010, 0x2004, None, 0x3000, None)
    assert lib.rs_step_nonflush(C.byref(L), C.byref(misb), C.byref(inp), C.byref(prm), y, None) == rs.RS_E_ALIGN
    # mode mismatches
    assert lib.rs_step_conventional(C.byref(L), C.byref(bufs), C.byref(inp), C.byref(prm), y, None) == rs.RS_E_MODE
    assert lib.rs_spec_append(C.byref(L), C.byref(bufs), C.byref(inp), 2, C.byref(prm), y, None) == rs.RS_E_MODE
    assert lib.rs_spec_commit(C.byref(L), C.byref(bufs), C.c_void_p(0x1000), C.byref(prm), None) == rs.RS_E_MODE
    assert lib.rs_requant_read_copy(C.byref(L), C.byref(bufs), None) == rs.RS_E_MODE
    # draft count out of range on a speculative layer
    _, Ls = rs.rs_init(_m2(batch=2, nheads=8, headdim=16, dstate=16, ngroups=1, max_draft=4))
    assert lib.rs_spec_append(C.byref(Ls), C.byref(bufs), C.byref(inp), 5, C.byref(prm), y, None) == rs.RS_E_ARG
    assert lib.rs_spec_append(C.byref(Ls), C.byref(bufs), C.byref(inp), 0, C.byref(prm), y, None) == rs.RS_E_ARG
    # conventional spec layer without snapshot buffer
    _, Lc = rs.rs_init(_m2(batch=2, nheads=8, headdim=16, dstate=16, ngroups=1, max_draft=4,
                           mode=rs.RS_CONVENTIONAL))
    nosnap = rs.RsBuffers(0x1000, None, None, None, None)
    assert lib.rs_spec_append(C.byref(Lc), C.byref(nosnap), C.byref(inp), 4, C.byref(prm), y, None) == rs.RS_E_ARG
    assert lib.rs_step_nonflush(C.byref(Lc), C.byref(nosnap), C.byref(inp), C.byref(prm), y, None) == rs.RS_E_MODE
    # replay layer without ring/meta
    noring = rs.RsBuffers(0x1000, None, None, None, None)
    assert lib.rs_step_nonflush(C.byref(L), C.byref(noring), C.byref(inp), C.byref(prm), y, None) == rs.RS_E_ARG
    # read copy configured but missing
    _, Lr = rs.rs_init(_m2(batch=2, nheads=8, headdim=16, dstate=16, ngroups=1, read_copy=rs.RS_NVFP4))
    assert lib.rs_step_nonflush(C.byref(Lr), C.byref(bufs), C.byref(inp), C.byref(prm), y, None) == rs.RS_E_ARG
    assert lib.rs_requant_read_copy(C.byref(Lr), C.byref(bufs), None) == rs.RS_E_ARG
