"""Helpers for the GPU parity tests: move seeded workload inputs to the device in
the layouts of include/rs.h, drive the library through its Python binding, and
read results back. No decode arithmetic happens here."""
from __future__ import annotations

import numpy as np
import torch

import ssm_decode_checkpoint_amd as rs
import workloads as W

DEV = "cuda"


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need an MI355X; torch.cuda.is_available() is False")
    rs.lib()


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def dev_in(arr: np.ndarray, in_dtype: str) -> torch.Tensor:
    """float32 array holding in_dtype values -> device tensor of that dtype (bit exact)."""
    arr = np.ascontiguousarray(arr, dtype=np.float32)
    if in_dtype == "bf16":
        bits = W.bf16_bits(arr).view(np.int16)
        return torch.from_numpy(bits.copy()).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(arr.copy()).to(DEV)


def dev_f32(arr: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32).copy()).to(DEV)


def m2_tok_dev(tok: dict, in_dtype: str) -> dict:
    return {k: dev_in(tok[k], in_dtype) for k in ("x", "B", "C", "dt")}


def m2_drafts_dev(drafts: list, in_dtype: str) -> dict:
    return {k: dev_in(np.stack([d[k] for d in drafts]), in_dtype) for k in ("x", "B", "C", "dt")}


def gdn_drafts_dev(drafts: list, in_dtype: str) -> dict:
    d = {k: dev_in(np.stack([t[k] for t in drafts]), in_dtype) for k in ("q", "k", "v")}
    d["g"] = dev_f32(np.stack([t["g"] for t in drafts]))
    d["beta"] = dev_f32(np.stack([t["beta"] for t in drafts]))
    return d


def gdn_tok_dev(tok: dict, in_dtype: str) -> dict:
    d = {k: dev_in(tok[k], in_dtype) for k in ("q", "k", "v")}
    d["g"] = dev_f32(tok["g"])
    d["beta"] = dev_f32(tok["beta"])
    return d


def m2_layer(w: W.Mamba2Workload, mode=rs.RS_REPLAY, ckpt_dtype=rs.RS_F32, read_copy=rs.RS_NONE, fuse=1,
             max_draft=None, batch=None):
    cfg = rs.make_config(rs.RS_MAMBA2, w.batch if batch is None else batch, mode=mode, nheads=w.nheads,
                         headdim=w.headdim, dstate=w.dstate, ngroups=w.ngroups,
                         max_draft=w.max_draft if max_draft is None else max_draft,
                         in_dtype=rs.RS_BF16 if w.in_dtype == "bf16" else rs.RS_F32,
                         ckpt_dtype=ckpt_dtype, read_copy=read_copy, fuse_requant=fuse)
    _, layer = rs.rs_init(cfg)
    return layer, rs.alloc_buffers(layer, DEV)


def gdn_layer(w: W.GDNWorkload, mode=rs.RS_REPLAY, batch=None, max_draft=None, read_copy=rs.RS_NONE,
              ckpt_dtype=rs.RS_F32):
    """A Gated DeltaNet layer, or a Kimi Delta Attention layer for a per-channel gate."""
    kind = rs.RS_KDA if w.gate == "channel" else rs.RS_GDN
    cfg = rs.make_config(kind, w.batch if batch is None else batch, mode=mode, n_qk_heads=w.n_qk,
                         n_v_heads=w.n_v, head_k_dim=w.dk, head_v_dim=w.dv,
                         max_draft=w.max_draft if max_draft is None else max_draft,
                         in_dtype=rs.RS_BF16 if w.in_dtype == "bf16" else rs.RS_F32, read_copy=read_copy,
                         ckpt_dtype=ckpt_dtype)
    _, layer = rs.rs_init(cfg)
    return layer, rs.alloc_buffers(layer, DEV)


def load_state_f32(layer, bufs, logical: np.ndarray):
    """Write a logical state [b, heads, P|dv, N|dk] into the fp32 checkpoint (stored transposed)."""
    st = np.ascontiguousarray(np.swapaxes(np.asarray(logical, np.float32), -1, -2))
    rs.ckpt_f32_view(layer, bufs).copy_(torch.from_numpy(st).to(DEV))


def read_state_f32(layer, bufs, seqs=None) -> np.ndarray:
    """fp32 checkpoint (optionally only some sequences) in logical layout [b, heads, P|dv, N|dk]."""
    v = rs.ckpt_f32_view(layer, bufs)
    if seqs is not None:
        v = v[torch.as_tensor(seqs, device=v.device)]
    return np.swapaxes(v.cpu().numpy(), -1, -2)


def read_meta(layer, bufs):
    nck, rest = rs.meta_view(layer, bufs)
    r = rest.cpu().numpy()
    return nck.cpu().numpy(), r[:, 0], r[:, 1], r[:, 2], r[:, 3]


def params_dev(p: dict):
    return dev_f32(p["A"]), dev_f32(p["D"])


def y_buf(batch, heads, width, K=None):
    shape = (batch, heads, width) if K is None else (K, batch, heads, width)
    return torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)
