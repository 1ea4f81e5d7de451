"""Low-precision checkpoint codes for the GPU parity tests.

Encodes a stored state (fp32, stored orientation [b, heads, rows, cols]) with the
oracle's quantizers into the device byte layout of include/rs.h, reads the
device's codes back, and classifies the places where the device's codes differ
from the oracle's.

A flush folds in float32 on the device and in float64 in the oracle, so the two
folds differ by float32 rounding, and a value that sits next to a rounding
boundary of the storage format may take the neighbouring code on one side. Such
flips are allowed, counted and reported; any other difference is a failure
(sitech.ge ReplaySSM page, "Bounding quantization error", for the formats; the
reading that only boundary flips are allowed is the survey's rounding-parity
reading). A flip is allowed when the two codes are adjacent in the format's
value order and the float64 fold lies within `tol * amax` of the midpoint
between them (amax: the matrix's largest magnitude), widened by how far the
two sides' matrix scales differ.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from oracle import quant

F32 = np.float32


# ---------------------------------------------------------------------------
# encode / device bytes
# ---------------------------------------------------------------------------

def encode(fmt: str, stored: np.ndarray) -> dict:
    """Oracle codes of fp32 matrices stored [b, h, rows, cols] in checkpoint format fmt."""
    x = np.asarray(stored, F32)
    b, h, r, c = x.shape
    if fmt == "f32":
        return {"codes": x.copy()}
    if fmt == "f16":
        return {"codes": x.astype(np.float16).view(np.uint16)}
    if fmt == "fp8":
        codes = np.empty(x.shape, np.uint8)
        scale = np.empty((b, h), F32)
        for i in range(b):
            for j in range(h):
                codes[i, j], scale[i, j] = quant.fp8_quantize(x[i, j])
        return {"codes": codes, "scale": scale}
    if fmt == "nvfp4":
        codes = np.empty(x.shape, np.uint8)
        sc = np.empty((b, h, r, c // 16), np.uint8)
        ts = np.empty((b, h), F32)
        for i in range(b):
            for j in range(h):
                codes[i, j], sc[i, j], ts[i, j] = quant.nvfp4_quantize(x[i, j])
        return {"codes": codes, "scales": sc, "ts": ts}
    raise ValueError(fmt)


def decode(fmt: str, enc: dict) -> np.ndarray:
    """Values (float32, stored orientation) of encoded matrices."""
    if fmt == "f32":
        return enc["codes"].copy()
    if fmt == "f16":
        return enc["codes"].view(np.float16).astype(F32)
    if fmt == "fp8":
        return (quant.e4m3_decode(enc["codes"]) * enc["scale"][:, :, None, None]).astype(F32)
    if fmt == "nvfp4":
        b, h = enc["ts"].shape
        out = np.empty(enc["codes"].shape, F32)
        for i in range(b):
            for j in range(h):
                out[i, j] = quant.nvfp4_dequantize(enc["codes"][i, j], enc["scales"][i, j], enc["ts"][i, j])
        return out
    raise ValueError(fmt)


def to_device_bytes(layer, fmt: str, enc: dict) -> np.ndarray:
    """The checkpoint buffer (ckpt_bytes) holding enc in the layout of include/rs.h."""
    out = np.zeros(int(layer.ckpt_bytes), np.uint8)
    if fmt in ("f32", "f16"):
        raw = enc["codes"].reshape(-1).view(np.uint8)
        out[: raw.size] = raw
    elif fmt == "fp8":
        raw = enc["codes"].reshape(-1)
        out[: raw.size] = raw
        s = enc["scale"].reshape(-1).view(np.uint8)
        out[layer.ck_scale_off: layer.ck_scale_off + s.size] = s
    elif fmt == "nvfp4":
        raw = quant.pack_nibbles(enc["codes"]).reshape(-1)
        out[: raw.size] = raw
        s = enc["scales"].reshape(-1)
        out[layer.ck_nv_scale_off: layer.ck_nv_scale_off + s.size] = s
        t = enc["ts"].reshape(-1).view(np.uint8)
        out[layer.ck_nv_tscale_off: layer.ck_nv_tscale_off + t.size] = t
    else:
        raise ValueError(fmt)
    return out


def from_device_bytes(layer, fmt: str, raw: np.ndarray) -> dict:
    """Inverse of to_device_bytes."""
    b, h, r, c = layer.cfg.batch, layer.heads, layer.rows, layer.cols
    n = b * h * r * c
    if fmt == "f32":
        return {"codes": raw[: 4 * n].view(F32).reshape(b, h, r, c).copy()}
    if fmt == "f16":
        return {"codes": raw[: 2 * n].view(np.uint16).reshape(b, h, r, c).copy()}
    if fmt == "fp8":
        return {"codes": raw[:n].reshape(b, h, r, c).copy(),
                "scale": raw[layer.ck_scale_off: layer.ck_scale_off + 4 * b * h].view(F32).reshape(b, h).copy()}
    if fmt == "nvfp4":
        codes = quant.unpack_nibbles(raw[: n // 2].reshape(b, h, r, c // 2))
        sc = raw[layer.ck_nv_scale_off: layer.ck_nv_scale_off + n // 16].reshape(b, h, r, c // 16).copy()
        ts = raw[layer.ck_nv_tscale_off: layer.ck_nv_tscale_off + 4 * b * h].view(F32).reshape(b, h).copy()
        return {"codes": codes, "scales": sc, "ts": ts}
    raise ValueError(fmt)


# ---------------------------------------------------------------------------
# code comparison
# ---------------------------------------------------------------------------

def _ord_f16(bits):
    bits = bits.astype(np.int64)
    mag = bits & 0x7FFF
    return np.where(bits & 0x8000, -mag, mag)


def _ord_signmag(codes, sign_bit, mag_mask):
    codes = codes.astype(np.int64)
    mag = codes & mag_mask
    return np.where(codes & sign_bit, -mag, mag)


@dataclass
class Flips:
    elements: int = 0          # element codes that differ (all allowed)
    scales: int = 0            # block scale codes that differ (all allowed)
    total: int = 0             # codes compared
    worst: float = 0.0         # largest distance of a flipped value from its midpoint, in units of tol*amax
    bad: list = field(default_factory=list)

    def add(self, other: "Flips"):
        self.elements += other.elements
        self.scales += other.scales
        self.total += other.total
        self.worst = max(self.worst, other.worst)
        self.bad += other.bad


def _check_flips(name, where, ord_g, ord_o, mid, x, slack, flips: Flips):
    """Every differing code must be adjacent and x must lie within slack of the midpoint."""
    diff = ord_g != ord_o
    n = int(np.count_nonzero(diff))
    if not n:
        return 0
    adj = np.abs(ord_g - ord_o) == 1
    dist = np.abs(x - mid)
    ok = adj & (dist <= slack)
    bad = diff & ~ok
    if np.any(bad):
        idx = np.argwhere(bad)[:4]
        flips.bad.append(f"{name} {where}: {int(np.count_nonzero(bad))} codes differ away from a rounding "
                         f"boundary, first at {idx.tolist()}")
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(diff & adj, dist / np.maximum(slack, 1e-300), 0.0)
    flips.worst = max(flips.worst, float(np.max(r)))
    return n


def compare(fmt: str, gpu: dict, ora: dict, fold64: np.ndarray, tol: float = 1e-5) -> Flips:
    """Classify the differences between the device's codes and the oracle's codes of
    its own float64 fold (fold64: float64, stored orientation [b, h, rows, cols])."""
    fl = Flips()
    x = np.asarray(fold64, np.float64)
    b, h = x.shape[:2]
    for i in range(b):
        for j in range(h):
            where = f"matrix ({i}, {j})"
            xm = x[i, j]
            amax = float(np.max(np.abs(xm)))
            if fmt == "f32":
                err = float(np.max(np.abs(gpu["codes"][i, j].astype(np.float64) - xm)))
                fl.total += xm.size
                if err > tol * amax:
                    fl.bad.append(f"f32 {where}: fold differs by {err:.3e} (amax {amax:.3e})")
            elif fmt == "f16":
                cg, co = gpu["codes"][i, j], ora["codes"][i, j]
                fl.total += cg.size
                vg = cg.view(np.float16).astype(np.float64)
                vo = co.view(np.float16).astype(np.float64)
                fl.elements += _check_flips("f16", where, _ord_f16(cg), _ord_f16(co), (vg + vo) / 2, xm,
                                            tol * amax, fl)
            elif fmt == "fp8":
                sg, so = float(gpu["scale"][i, j]), float(ora["scale"][i, j])
                srel = abs(sg / so - 1.0)
                if srel > tol:
                    fl.bad.append(f"fp8 {where}: matrix scale {sg!r} vs {so!r}")
                cg, co = gpu["codes"][i, j], ora["codes"][i, j]
                fl.total += cg.size
                vg = quant.e4m3_decode(cg).astype(np.float64)
                vo = quant.e4m3_decode(co).astype(np.float64)
                fl.elements += _check_flips("fp8", where, _ord_signmag(cg, 0x80, 0x7F), _ord_signmag(co, 0x80, 0x7F),
                                            (vg + vo) / 2, xm / so, 448.0 * (tol + srel), fl)
            elif fmt == "nvfp4":
                tg, to = float(gpu["ts"][i, j]), float(ora["ts"][i, j])
                trel = abs(tg / to - 1.0)
                if trel > tol:
                    fl.bad.append(f"nvfp4 {where}: tensor scale {tg!r} vs {to!r}")
                sg, so = gpu["scales"][i, j], ora["scales"][i, j]
                fl.total += sg.size
                blocks = xm.reshape(xm.shape[0], -1, 16)
                bamax = np.max(np.abs(blocks), axis=-1)
                eg = quant.e4m3_decode(sg).astype(np.float64)
                eo = quant.e4m3_decode(so).astype(np.float64)
                fl.scales += _check_flips("nvfp4 block scale", where, sg.astype(np.int64), so.astype(np.int64),
                                          (eg + eo) / 2, bamax / (6.0 * to), 448.0 * (tol + trel), fl)
                same = sg == so
                cg = gpu["codes"][i, j].reshape(blocks.shape)
                co = ora["codes"][i, j].reshape(blocks.shape)
                fl.total += int(np.count_nonzero(same)) * 16
                sd = (eo * to)[..., None]
                vg = quant.e2m1_decode(cg).astype(np.float64)
                vo = quant.e2m1_decode(co).astype(np.float64)
                with np.errstate(divide="ignore", invalid="ignore"):
                    q = np.where(sd > 0, blocks / sd, 0.0)
                    slack = np.where(sd > 0, tol * amax / sd, np.inf) + 6.0 * trel
                m = np.broadcast_to(same[..., None], cg.shape)
                fl.elements += _check_flips("nvfp4", where, np.where(m, _ord_signmag(cg, 8, 7), 0),
                                            np.where(m, _ord_signmag(co, 8, 7), 0), (vg + vo) / 2, q, slack, fl)
                # blocks whose scale flipped: each element within the quantizer's error bound
                if not np.all(same):
                    sdg = (eg * tg)[..., None]
                    err = np.abs(vg * sdg - blocks)
                    bound = sdg + np.maximum(0.0, np.abs(blocks) - 6.0 * sdg) + tol * amax
                    badb = (~m) & (err > bound)
                    if np.any(badb):
                        fl.bad.append(f"nvfp4 {where}: {int(np.count_nonzero(badb))} elements of rescaled "
                                      f"blocks outside the quantizer's error bound")
            else:
                raise ValueError(fmt)
    return fl
