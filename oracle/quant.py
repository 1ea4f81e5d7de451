"""Low-precision checkpoint and read-copy formats (oracle; test infrastructure only).

sitech.ge ReplaySSM page, "Bounding quantization error": a quantized SSM state
fed back through the recurrence accumulates rounding error, so the method keeps
a high-precision checkpoint for the recurrence and a low-precision copy for
reads (NVFP4 reads over an FP32 recurrence; FP16 or FP8 recurrences; a generic,
uniformly NVFP4 checkpoint as the comparator).

Formats, and the readings taken where the pages are silent:

* NVFP4 read copy. A "tensor" is one (sequence, head) state matrix as stored
  (rows = dstate / key index, columns = headdim / value index, columns
  innermost). Blocks are 16 consecutive elements of a row. In float32, with
  each operation rounded to float32 in this order:
      amax = max |x|;  ts = amax / 2688 (= 6 * 448), or 1 if that is 0
      per block: d = 6 * ts;  s = e4m3(max|block| / d);  sd = value(s) * ts
      code = e2m1(x / sd)  (all codes 0 if sd = 0)
      dequant: value(code) * sd
  e2m1 holds magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6} (code = sign << 3 |
  index); e4m3 is OCP E4M3FN (bias 7, max 448, subnormal step 2^-9). Both
  round to nearest with ties to the even code and saturate at their maximum.
  Codes pack two per byte, the even column in the low nibble.
* FP16 checkpoint: IEEE binary16, round to nearest even.
* FP8 checkpoint: e4m3 codes with one fp32 scale per matrix, scale = amax/448
  (1 if amax = 0), code = sign | e4m3(|x| / scale), dequant value * scale.
* Uniform NVFP4 checkpoint: the checkpoint itself stored in NVFP4.

The encoders below are written as "nearest entry of the value table, ties to
the even code", which is the plain definition of round-to-nearest-even for a
format this small.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32

E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)


def _e4m3_table() -> np.ndarray:
    """Values of the 127 non-negative finite OCP E4M3FN codes (0x00 .. 0x7E)."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        if e == 0:
            vals.append(m * 2.0 ** -9)
        else:
            vals.append((1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


E4M3_MAG = _e4m3_table()          # E4M3_MAG[126] = 448


def _nearest_even(mag: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the nearest table entry to each |value|; ties go to the even index;
    values beyond the last entry take the last entry (saturation)."""
    # Clamping first is the saturation itself; it also keeps the distances below
    # from losing every table entry to float64 rounding for huge magnitudes.
    mag = np.minimum(np.asarray(mag, dtype=np.float64), table[-1])
    d = np.abs(mag[..., None] - table.astype(np.float64))
    best = d.min(axis=-1, keepdims=True)
    hit = d == best
    idx = np.arange(table.size)
    # among the (at most two adjacent) nearest entries prefer the even index
    score = np.where(hit, np.where(idx % 2 == 0, 0, 1), 2)
    return np.argmin(score, axis=-1)


def e2m1_encode(x) -> np.ndarray:
    """float32 -> 4-bit e2m1 code (sign bit 3), round to nearest even, saturating at 6."""
    x = np.asarray(x, dtype=F32)
    idx = _nearest_even(np.abs(x), E2M1_MAG)
    return (idx | (np.signbit(x).astype(np.int64) << 3)).astype(np.uint8)


def e2m1_decode(code) -> np.ndarray:
    code = np.asarray(code, dtype=np.uint8)
    mag = E2M1_MAG[code & 7]
    return np.where(code & 8, -mag, mag).astype(F32)


def e4m3_encode_mag(x) -> np.ndarray:
    """Non-negative float32 -> E4M3FN code 0..126, round to nearest even, saturating at 448."""
    x = np.asarray(x, dtype=F32)
    return _nearest_even(x, E4M3_MAG).astype(np.uint8)


def e4m3_decode(code) -> np.ndarray:
    code = np.asarray(code, dtype=np.uint8)
    mag = E4M3_MAG[code & 0x7F].astype(F32)
    return np.where(code & 0x80, -mag, mag).astype(F32)


# ---------------------------------------------------------------------------
# NVFP4 read copy
# ---------------------------------------------------------------------------

def nvfp4_quantize(tile):
    """Quantize one stored state matrix [rows, cols] (cols % 16 == 0).

    Returns (codes uint8 [rows, cols], block scale codes uint8 [rows, cols/16],
    tensor scale float32).
    """
    x = np.asarray(tile, dtype=F32)
    rows, cols = x.shape
    amax = F32(np.max(np.abs(x))) if x.size else F32(0)
    ts = F32(amax / F32(2688.0))
    if ts == 0:
        ts = F32(1.0)
    blocks = x.reshape(rows, cols // 16, 16)
    bamax = np.max(np.abs(blocks), axis=-1).astype(F32)
    d = F32(F32(6.0) * ts)
    s = e4m3_encode_mag((bamax / d).astype(F32))
    sd = (e4m3_decode(s) * ts).astype(F32)                    # [rows, nblk]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (blocks / sd[..., None]).astype(F32)
    codes = e2m1_encode(q)
    codes = np.where((sd == 0)[..., None], np.uint8(0), codes)
    return codes.reshape(rows, cols).astype(np.uint8), s, ts


def nvfp4_dequantize(codes, scales, ts):
    codes = np.asarray(codes, dtype=np.uint8)
    rows, cols = codes.shape
    sd = (e4m3_decode(scales) * F32(ts)).astype(F32)
    v = e2m1_decode(codes).reshape(rows, cols // 16, 16)
    return (v * sd[..., None]).astype(F32).reshape(rows, cols)


def nvfp4_roundtrip(tile) -> np.ndarray:
    return nvfp4_dequantize(*nvfp4_quantize(tile))


def pack_nibbles(codes) -> np.ndarray:
    """Two 4-bit codes per byte, the even column in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# ---------------------------------------------------------------------------
# FP16 and FP8 checkpoints
# ---------------------------------------------------------------------------

def fp16_roundtrip(x) -> np.ndarray:
    """Round to IEEE binary16 (nearest even) and back to float32."""
    return np.asarray(x, dtype=F32).astype(np.float16).astype(F32)


def fp8_quantize(tile):
    """One stored matrix -> (E4M3FN codes with sign, fp32 scale = amax / 448)."""
    x = np.asarray(tile, dtype=F32)
    amax = F32(np.max(np.abs(x))) if x.size else F32(0)
    scale = F32(amax / F32(448.0))
    if scale == 0:
        scale = F32(1.0)
    mag = e4m3_encode_mag((np.abs(x) / scale).astype(F32))
    codes = (mag | (np.signbit(x).astype(np.uint8) << 7)).astype(np.uint8)
    return codes, scale


def fp8_dequantize(codes, scale) -> np.ndarray:
    return (e4m3_decode(codes) * F32(scale)).astype(F32)


def fp8_roundtrip(tile) -> np.ndarray:
    return fp8_dequantize(*fp8_quantize(tile))


def roundtrip(fmt: str, tile) -> np.ndarray:
    """Stored-then-read value of a [rows, cols] matrix in checkpoint format fmt."""
    if fmt == "f32":
        return np.asarray(tile, dtype=F32).copy()
    if fmt == "f16":
        return fp16_roundtrip(tile)
    if fmt == "fp8":
        return fp8_roundtrip(tile)
    if fmt == "nvfp4":
        return nvfp4_roundtrip(tile)
    raise ValueError(fmt)
