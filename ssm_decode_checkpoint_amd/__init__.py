"""ReplaySSM SSM-layer decode step on AMD MI355X (gfx950): Python binding.

A thin ctypes layer over the C ABI in include/rs.h (librs.so, built in-tree by
``ssm_decode_checkpoint_amd.build``). Every function here only marshals
arguments: it takes torch tensors for device memory, passes their data
pointers and the current HIP stream, and returns the library's status. All
arithmetic runs in the HIP kernels. There is no fallback: if librs.so is
missing or the GPU is absent, calls raise.

Names mirror the C entry points: rs_init, rs_step_conventional,
rs_step_nonflush, rs_step_flush, rs_spec_append, rs_spec_commit,
rs_requant_read_copy.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Dict, Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librs.so")

# status codes, kinds, modes, dtypes, device error bits (include/rs.h)
RS_OK, RS_E_ARG, RS_E_DTYPE, RS_E_ALIGN, RS_E_MODE, RS_E_LAUNCH, RS_E_UNSUPPORTED = 0, -1, -2, -3, -4, -5, -6
RS_MAMBA2, RS_GDN, RS_KDA = 1, 2, 3
RS_REPLAY, RS_CONVENTIONAL = 0, 1
RS_NONE, RS_F32, RS_BF16, RS_F16, RS_FP8E4M3, RS_NVFP4 = 0, 1, 2, 3, 4, 5
RS_ERR_FULL, RS_ERR_OVERFLOW, RS_ERR_COMMIT, RS_ERR_PENDING = 1, 2, 4, 8

EXPORTS = ("rs_init", "rs_step_conventional", "rs_step_nonflush", "rs_step_flush", "rs_step", "rs_spec_append",
           "rs_spec_commit", "rs_spec_commit_static", "rs_requant_read_copy", "rs_reset_slots", "rs_copy_slots", "rs_conv_step",
           "rs_gated_norm", "rs_status_string", "rs_version")


class RsConfig(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "kind", "mode", "batch", "nheads", "headdim", "dstate", "ngroups", "n_qk_heads", "n_v_heads",
        "head_k_dim", "head_v_dim", "ring", "max_draft", "in_dtype", "ckpt_dtype", "read_copy", "fuse_requant")]


class RsLayer(C.Structure):
    _fields_ = [("cfg", RsConfig), ("heads", C.c_int32), ("in_heads", C.c_int32), ("rows", C.c_int32),
                ("cols", C.c_int32)] + [(n, C.c_uint64) for n in (
                    "ckpt_bytes", "ring_bytes", "read_copy_bytes", "meta_bytes", "snap_bytes",
                    "ring_x_off", "ring_B_off", "ring_C_off", "ring_dt_off",
                    "ring_q_off", "ring_k_off", "ring_v_off", "ring_g_off", "ring_beta_off", "ring_u_off",
                    "ck_scale_off", "ck_nv_scale_off", "ck_nv_tscale_off", "nv_scale_off", "nv_tscale_off",
                    "meta_work_off")] + [("magic", C.c_uint32), ("reserved", C.c_uint32)]


class RsBuffers(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("ckpt", "ring", "read_copy", "meta", "snap")]


class RsInputs(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("x", "B", "C", "dt", "q", "k", "v", "g", "beta")]


class RsParams(C.Structure):
    _fields_ = [("A", C.c_void_p), ("D", C.c_void_p)]


META_DTYPE_FIELDS = ("n_ckpt", "len", "nd", "err", "arrive")  # rs_meta: int64, 4 x int32, 2 x int32 reserved
META_BYTES = 32

_lib: Optional[C.CDLL] = None


class RsError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")
        self.status = status


def lib() -> C.CDLL:
    """Load librs.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m ssm_decode_checkpoint_amd.build`")
        L = C.CDLL(LIB_PATH)
        P = C.POINTER
        L.rs_init.argtypes = [P(RsConfig), P(RsLayer)]
        for name in ("rs_step_conventional", "rs_step_nonflush", "rs_step_flush", "rs_step"):
            getattr(L, name).argtypes = [P(RsLayer), P(RsBuffers), P(RsInputs), P(RsParams), C.c_void_p, C.c_void_p]
        L.rs_spec_append.argtypes = [P(RsLayer), P(RsBuffers), P(RsInputs), C.c_int32, P(RsParams), C.c_void_p,
                                     C.c_void_p]
        L.rs_spec_commit.argtypes = [P(RsLayer), P(RsBuffers), C.c_void_p, P(RsParams), C.c_void_p]
        L.rs_spec_commit_static.argtypes = [P(RsLayer), P(RsBuffers), C.c_void_p, P(RsParams), C.c_void_p]
        L.rs_requant_read_copy.argtypes = [P(RsLayer), P(RsBuffers), C.c_void_p]
        L.rs_reset_slots.argtypes = [P(RsLayer), P(RsBuffers), C.c_void_p, C.c_int32, C.c_void_p]
        L.rs_copy_slots.argtypes = [P(RsLayer), P(RsBuffers), C.c_void_p, P(RsLayer), P(RsBuffers), C.c_void_p,
                                    C.c_int32, C.c_void_p]
        L.rs_conv_step.argtypes = [P(RsLayer), P(RsBuffers), C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p,
                                   C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
        L.rs_gated_norm.argtypes = [P(RsLayer), C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_float,
                                    C.c_void_p, C.c_void_p]
        for name in EXPORTS:
            if name not in ("rs_status_string", "rs_version"):
                getattr(L, name).restype = C.c_int32
        L.rs_status_string.argtypes = [C.c_int32]
        L.rs_status_string.restype = C.c_char_p
        L.rs_version.restype = C.c_int32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().rs_status_string(status).decode()


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def _check(fn: str, status: int, raise_on_error: bool) -> int:
    if status != RS_OK and raise_on_error:
        raise RsError(fn, status)
    return status


# ---------------------------------------------------------------------------
# configuration
# ---------------------------------------------------------------------------

def make_config(kind: int, batch: int, *, mode: int = RS_REPLAY, nheads=0, headdim=0, dstate=0, ngroups=0,
                n_qk_heads=0, n_v_heads=0, head_k_dim=0, head_v_dim=0, ring=16, max_draft=0,
                in_dtype=RS_BF16, ckpt_dtype=RS_F32, read_copy=RS_NONE, fuse_requant=0) -> RsConfig:
    return RsConfig(kind, mode, batch, nheads, headdim, dstate, ngroups, n_qk_heads, n_v_heads, head_k_dim,
                    head_v_dim, ring, max_draft, in_dtype, ckpt_dtype, read_copy, fuse_requant)


def rs_init(cfg: RsConfig, raise_on_error: bool = True):
    """Validate a config and return (status, RsLayer)."""
    out = RsLayer()
    st = lib().rs_init(C.byref(cfg), C.byref(out))
    _check("rs_init", st, raise_on_error)
    return st, out


# ---------------------------------------------------------------------------
# device buffers (torch allocates; the library only sees pointers)
# ---------------------------------------------------------------------------

@dataclass
class Buffers:
    ckpt: object
    ring: object = None
    read_copy: object = None
    meta: object = None
    snap: object = None

    def c(self) -> RsBuffers:
        return RsBuffers(_ptr(self.ckpt), _ptr(self.ring), _ptr(self.read_copy), _ptr(self.meta), _ptr(self.snap))


def alloc_buffers(layer: RsLayer, device="cuda") -> Buffers:
    """Zero-filled uint8 device tensors of the sizes rs_init computed."""
    import torch

    def z(n):
        return torch.zeros(int(n), dtype=torch.uint8, device=device) if n else None

    return Buffers(ckpt=z(layer.ckpt_bytes), ring=z(layer.ring_bytes), read_copy=z(layer.read_copy_bytes),
                   meta=z(layer.meta_bytes), snap=z(layer.snap_bytes))


def _inputs(d: Dict[str, object]) -> RsInputs:
    return RsInputs(*[_ptr(d.get(n)) for n in ("x", "B", "C", "dt", "q", "k", "v", "g", "beta")])


def _params(A=None, D=None) -> RsParams:
    return RsParams(_ptr(A), _ptr(D))


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def rs_step_conventional(layer: RsLayer, bufs: Buffers, inputs: Dict[str, object], A, D, y, stream=None,
                         raise_on_error: bool = True) -> int:
    st = lib().rs_step_conventional(C.byref(layer), C.byref(bufs.c()), C.byref(_inputs(inputs)),
                                    C.byref(_params(A, D)), _ptr(y), _stream(stream))
    return _check("rs_step_conventional", st, raise_on_error)


def rs_step_nonflush(layer: RsLayer, bufs: Buffers, inputs: Dict[str, object], A, D, y, stream=None,
                     raise_on_error: bool = True) -> int:
    st = lib().rs_step_nonflush(C.byref(layer), C.byref(bufs.c()), C.byref(_inputs(inputs)),
                                C.byref(_params(A, D)), _ptr(y), _stream(stream))
    return _check("rs_step_nonflush", st, raise_on_error)


def rs_step_flush(layer: RsLayer, bufs: Buffers, inputs: Dict[str, object], A, D, y, stream=None,
                  raise_on_error: bool = True) -> int:
    st = lib().rs_step_flush(C.byref(layer), C.byref(bufs.c()), C.byref(_inputs(inputs)),
                             C.byref(_params(A, D)), _ptr(y), _stream(stream))
    return _check("rs_step_flush", st, raise_on_error)


def rs_step(layer: RsLayer, bufs: Buffers, inputs: Dict[str, object], A, D, y, stream=None,
            raise_on_error: bool = True) -> int:
    st = lib().rs_step(C.byref(layer), C.byref(bufs.c()), C.byref(_inputs(inputs)), C.byref(_params(A, D)),
                       _ptr(y), _stream(stream))
    return _check("rs_step", st, raise_on_error)


def rs_reset_slots(layer: RsLayer, bufs: Buffers, seqs, count: int, stream=None, raise_on_error: bool = True) -> int:
    st = lib().rs_reset_slots(C.byref(layer), C.byref(bufs.c()), _ptr(seqs), int(count), _stream(stream))
    return _check("rs_reset_slots", st, raise_on_error)


def rs_copy_slots(src_layer: RsLayer, src: Buffers, src_seqs, dst_layer: RsLayer, dst: Buffers, dst_seqs, count: int,
                  stream=None, raise_on_error: bool = True) -> int:
    st = lib().rs_copy_slots(C.byref(src_layer), C.byref(src.c()), _ptr(src_seqs), C.byref(dst_layer),
                             C.byref(dst.c()), _ptr(dst_seqs), int(count), _stream(stream))
    return _check("rs_copy_slots", st, raise_on_error)


def rs_spec_append(layer: RsLayer, bufs: Buffers, drafts: Dict[str, object], K: int, A, D, y, stream=None,
                   raise_on_error: bool = True) -> int:
    st = lib().rs_spec_append(C.byref(layer), C.byref(bufs.c()), C.byref(_inputs(drafts)), int(K),
                              C.byref(_params(A, D)), _ptr(y), _stream(stream))
    return _check("rs_spec_append", st, raise_on_error)


def rs_spec_commit(layer: RsLayer, bufs: Buffers, accepted, A, D, stream=None, raise_on_error: bool = True) -> int:
    st = lib().rs_spec_commit(C.byref(layer), C.byref(bufs.c()), _ptr(accepted), C.byref(_params(A, D)),
                              _stream(stream))
    return _check("rs_spec_commit", st, raise_on_error)


def rs_spec_commit_static(layer: RsLayer, bufs: Buffers, accepted, A, D, stream=None,
                          raise_on_error: bool = True) -> int:
    st = lib().rs_spec_commit_static(C.byref(layer), C.byref(bufs.c()), _ptr(accepted), C.byref(_params(A, D)),
                                     _stream(stream))
    return _check("rs_spec_commit_static", st, raise_on_error)


def rs_conv_step(layer: RsLayer, bufs: Buffers, conv_ring, xbc, K: int, weight, bias, width: int, x, B, Cm,
                 stream=None, raise_on_error: bool = True) -> int:
    st = lib().rs_conv_step(C.byref(layer), C.byref(bufs.c()), _ptr(conv_ring), _ptr(xbc), int(K), _ptr(weight),
                            _ptr(bias), int(width), _ptr(x), _ptr(B), _ptr(Cm), _stream(stream))
    return _check("rs_conv_step", st, raise_on_error)


def rs_gated_norm(layer: RsLayer, K: int, y, z, weight, norm_groups: int, eps: float, out, stream=None,
                  raise_on_error: bool = True) -> int:
    st = lib().rs_gated_norm(C.byref(layer), int(K), _ptr(y), _ptr(z), _ptr(weight), int(norm_groups), float(eps),
                             _ptr(out), _stream(stream))
    return _check("rs_gated_norm", st, raise_on_error)


def conv_channels(layer: RsLayer) -> int:
    c = layer.cfg
    return c.nheads * c.headdim + 2 * c.ngroups * c.dstate


def conv_ring_bytes(layer: RsLayer) -> int:
    """Bytes of the convolution ring: batch x 16 x channels inputs."""
    return layer.cfg.batch * 16 * conv_channels(layer) * (2 if layer.cfg.in_dtype == RS_BF16 else 4)


def rs_requant_read_copy(layer: RsLayer, bufs: Buffers, stream=None, raise_on_error: bool = True) -> int:
    st = lib().rs_requant_read_copy(C.byref(layer), C.byref(bufs.c()), _stream(stream))
    return _check("rs_requant_read_copy", st, raise_on_error)


def rs_version() -> int:
    return int(lib().rs_version())


# ---------------------------------------------------------------------------
# views of the device layouts (include/rs.h), for loading state and reading results
# ---------------------------------------------------------------------------

def meta_view(layer: RsLayer, bufs: Buffers):
    """(n_ckpt int64 [batch], int32 [batch, 6]: len, nd, err, arrive, reserved x2)."""
    import torch
    b = layer.cfg.batch
    raw = bufs.meta[: b * META_BYTES].view(b, META_BYTES)
    return raw[:, :8].contiguous().view(torch.int64).view(b), raw[:, 8:].contiguous().view(torch.int32)


def ckpt_f32_view(layer: RsLayer, bufs: Buffers):
    """fp32 checkpoint as [batch, heads, rows, cols] (stored layout)."""
    import torch
    c = layer.cfg
    n = c.batch * layer.heads * layer.rows * layer.cols
    return bufs.ckpt[: n * 4].view(torch.float32).view(c.batch, layer.heads, layer.rows, layer.cols)


def ring_view(layer: RsLayer, bufs: Buffers, name: str):
    """One ring array as a typed tensor: Mamba-2 x [b,H,16,P], B/C [b,G,16,N], dt [b,H,16];
    GDN q/k [b,Hk,16,dk], v [b,Hv,16,dv], g/beta [b,Hv,16], u [b,Hv,16,dv] (fp32);
    KDA as GDN with g [b,Hv,16,dk]."""
    import torch
    c = layer.cfg
    b = c.batch
    esz = 4 if c.in_dtype == RS_F32 else 2
    edt = torch.float32 if c.in_dtype == RS_F32 else torch.bfloat16
    if c.kind == RS_MAMBA2:
        shapes = {"x": (b, c.nheads, 16, c.headdim), "B": (b, c.ngroups, 16, c.dstate),
                  "C": (b, c.ngroups, 16, c.dstate), "dt": (b, c.nheads, 16)}
    else:
        shapes = {"q": (b, c.n_qk_heads, 16, c.head_k_dim), "k": (b, c.n_qk_heads, 16, c.head_k_dim),
                  "v": (b, c.n_v_heads, 16, c.head_v_dim), "g": (b, c.n_v_heads, 16),
                  "beta": (b, c.n_v_heads, 16), "u": (b, c.n_v_heads, 16, c.head_v_dim)}
        if c.kind == RS_KDA:
            shapes["g"] = (b, c.n_v_heads, 16, c.head_k_dim)
    shp = shapes[name]
    dt, sz = (torch.float32, 4) if name in ("g", "beta", "u") else (edt, esz)
    off = getattr(layer, f"ring_{name}_off")
    n = 1
    for s in shp:
        n *= s
    return bufs.ring[off: off + n * sz].view(dt).view(*shp)
