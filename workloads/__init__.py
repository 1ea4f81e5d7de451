"""Seeded synthetic workloads for the ReplaySSM SSM-layer decode step.

This module only draws inputs. It holds none of the decode arithmetic: no
recurrence, no decay product, no quantizer. Both the fp64 oracle (through the
tests) and the HIP path consume what it returns, so the two sides see the very
same numbers.

Shapes and value distributions follow the workloads described for the method
(ReplaySSM news coverage, sitech.ge page, "How ReplaySSM works" and "Reducing
state traffic" sections: batch 256 serving, a 16-entry buffer, Mamba-2 and Gated
DeltaNet layers). The exact distributions are the build's stated recipe:

* Mamba-2: x ~ N(0,1); B, C ~ N(0,1)/sqrt(N); dt = softplus(N(0,1) - 2);
  A = -exp(U(log 1, log 16)) per head; D ~ N(0,1) per head; initial state
  N(0, std^2) with std 0.1 (or zero).
* Gated DeltaNet: q, k ~ N(0,1), L2-normalised in fp32; v ~ N(0,1);
  beta = sigmoid(N(0,1)); g = -exp(a) * softplus(N(0,1)) with a ~ U(-3, 0) per
  v-head (alpha = exp(g)); initial state N(0, std^2).

Every draw comes from ``numpy.random.Generator(PCG64(SeedSequence(key)))`` with
a key that names what is drawn, so any subset of sequences or steps can be
regenerated on its own:

* step inputs of sequence b at step t: ``[seed, t, b]``
* per-head parameters: ``[seed, 2**31]``
* initial state of sequence b: ``[seed, 2**31 + 1, b]``
* accepted draft counts of speculative round r: ``[seed, 2**31 + 2, r]``
* a test tile of arbitrary values: ``[seed, 2**31 + 3, i]``

bf16 inputs are produced by round-to-nearest-even from the fp32 draw; the
arrays returned hold those rounded values as float32, and ``bf16_bits`` gives
the 16-bit patterns that are uploaded to the device.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Iterable, Sequence, Tuple

import numpy as np

KEY_PARAMS = 2**31
KEY_INIT = 2**31 + 1
KEY_ACCEPT = 2**31 + 2
KEY_TILE = 2**31 + 3
KEY_BLOCK = 2**31 + 4


def rng_for(*key: int) -> np.random.Generator:
    """A PCG64 generator seeded by the integer key tuple."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


# --------------------------------------------------------------------------
# bf16 round-to-nearest-even (input preparation, not decode arithmetic)
# --------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Expand bf16 bit patterns to the float32 values they denote."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array of the bf16-rounded values of x."""
    return bf16_to_f32(bf16_bits(x))


def _softplus(z: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, z)


def _sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


# --------------------------------------------------------------------------
# workload shapes
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Mamba2Workload:
    name: str
    batch: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    in_dtype: str  # "f32" or "bf16"
    init_std: float
    steps: int
    seed: int
    max_draft: int = 0
    a_range: Tuple[float, float] = (1.0, 16.0)   # |A| is log-uniform on this range

    def with_(self, **kw) -> "Mamba2Workload":
        return replace(self, **kw)


@dataclass(frozen=True)
class GDNWorkload:
    name: str
    batch: int
    n_qk: int
    n_v: int
    dk: int
    dv: int
    in_dtype: str
    init_std: float
    steps: int
    seed: int
    max_draft: int = 0
    gate: str = "head"   # "head": one decay per value head (Gated DeltaNet); "channel": per key channel (KDA)

    def with_(self, **kw) -> "GDNWorkload":
        return replace(self, **kw)


# Tiny Mamba-2 layer: every input fp32, zero initial state, 64 steps (4 flushes).
TINY_M2 = Mamba2Workload("tiny_mamba2", batch=4, nheads=4, headdim=16, dstate=16, ngroups=1,
                         in_dtype="f32", init_std=0.0, steps=64, seed=1)
# Nemotron-style Mamba-2 layer at serving batch 256: 4 MiB fp32 state per sequence.
M2_NEMOTRON = Mamba2Workload("mamba2_nemotron_b256", batch=256, nheads=128, headdim=64,
                             dstate=128, ngroups=8, in_dtype="bf16", init_std=0.1,
                             steps=256, seed=2)
# Qwen3.5-style Gated DeltaNet layer at batch 256: 16 q/k heads, 32 v heads, 128x128 states.
GDN_QWEN = GDNWorkload("gdn_qwen_b256", batch=256, n_qk=16, n_v=32, dk=128, dv=128,
                       in_dtype="bf16", init_std=0.1, steps=256, seed=3)
# Speculative decode on 120B-class Mamba-2 shapes: batch 512, 4 drafts per round, 64 rounds.
M2_SPEC = Mamba2Workload("mamba2_spec_b512", batch=512, nheads=128, headdim=64, dstate=128,
                         ngroups=8, in_dtype="bf16", init_std=0.1, steps=64, seed=4,
                         max_draft=4)
# Speculative decode on the Qwen-style GDN shapes: batch 256, 4 drafts per round, 64 rounds.
GDN_SPEC = GDNWorkload("gdn_qwen_spec_b256", batch=256, n_qk=16, n_v=32, dk=128, dv=128,
                       in_dtype="bf16", init_std=0.1, steps=64, seed=7, max_draft=4)
# Kimi Delta Attention (per-key-channel decay) on the Qwen-style GDN shapes at batch 256.
KDA_B256 = GDNWorkload("kda_b256", batch=256, n_qk=16, n_v=32, dk=128, dv=128, in_dtype="bf16",
                       init_std=0.1, steps=256, seed=8, gate="channel")
# Low-precision reads on the Nemotron-style shapes at batch 64 (zero initial state).
M2_LOWPREC = Mamba2Workload("mamba2_lowprec_b64", batch=64, nheads=128, headdim=64,
                            dstate=128, ngroups=8, in_dtype="bf16", init_std=0.0,
                            steps=16384, seed=5)
# Tiny Gated DeltaNet layer for brute-force checks: fp32, zero initial state.
TINY_GDN = GDNWorkload("tiny_gdn", batch=4, n_qk=2, n_v=4, dk=16, dv=16, in_dtype="f32",
                       init_std=0.0, steps=64, seed=6)
# Tiny KDA layer for brute-force checks: fp32, zero initial state, per-channel gate.
TINY_KDA = GDNWorkload("tiny_kda", batch=4, n_qk=2, n_v=4, dk=16, dv=16, in_dtype="f32",
                       init_std=0.0, steps=64, seed=9, gate="channel")


def _as_in(x: np.ndarray, in_dtype: str) -> np.ndarray:
    x = x.astype(np.float32)
    return round_bf16(x) if in_dtype == "bf16" else x


# --------------------------------------------------------------------------
# Mamba-2 draws
# --------------------------------------------------------------------------

def m2_params(w: Mamba2Workload) -> Dict[str, np.ndarray]:
    """Per-head fp32 A (< 0) and D."""
    g = rng_for(w.seed, KEY_PARAMS)
    A = -np.exp(g.uniform(np.log(w.a_range[0]), np.log(w.a_range[1]), size=w.nheads))
    D = g.standard_normal(w.nheads)
    return {"A": A.astype(np.float32), "D": D.astype(np.float32)}


def m2_init_state(w: Mamba2Workload, b: int) -> np.ndarray:
    """Initial fp32 state of sequence b, logical layout [nheads, headdim, dstate]."""
    shape = (w.nheads, w.headdim, w.dstate)
    if w.init_std == 0.0:
        return np.zeros(shape, np.float32)
    g = rng_for(w.seed, KEY_INIT, b)
    return (g.standard_normal(shape) * w.init_std).astype(np.float32)


def m2_init_states(w: Mamba2Workload, seqs: Iterable[int]) -> np.ndarray:
    return np.stack([m2_init_state(w, b) for b in seqs])


def m2_token(w: Mamba2Workload, t: int, b: int) -> Dict[str, np.ndarray]:
    """Inputs (x, B, C, dt) of sequence b at step t, as float32 holding in_dtype values."""
    g = rng_for(w.seed, t, b)
    x = g.standard_normal((w.nheads, w.headdim))
    B = g.standard_normal((w.ngroups, w.dstate)) / np.sqrt(w.dstate)
    C = g.standard_normal((w.ngroups, w.dstate)) / np.sqrt(w.dstate)
    dt = _softplus(g.standard_normal(w.nheads) - 2.0)
    return {k: _as_in(v, w.in_dtype) for k, v in (("x", x), ("B", B), ("C", C), ("dt", dt))}


def m2_step(w: Mamba2Workload, t: int, seqs: Sequence[int]) -> Dict[str, np.ndarray]:
    """Batched inputs of step t for the listed sequences: x [nb,H,P], B/C [nb,G,N], dt [nb,H]."""
    toks = [m2_token(w, t, b) for b in seqs]
    return {k: np.stack([tk[k] for tk in toks]) for k in ("x", "B", "C", "dt")}


def accepted_counts(seed: int, rnd: int, batch: int, max_draft: int) -> np.ndarray:
    """Accepted draft count per sequence for speculative round rnd, uniform on {0..max_draft}."""
    g = rng_for(seed, KEY_ACCEPT, rnd)
    return g.integers(0, max_draft + 1, size=batch).astype(np.int32)


# --------------------------------------------------------------------------
# Mamba-2 block draws (short convolution and gated norm around the SSM)
# --------------------------------------------------------------------------

def block_params(w: Mamba2Workload, width: int = 4) -> Dict[str, np.ndarray]:
    """Convolution weights [channels, width] (~ 1/sqrt(width)), bias [channels] and
    norm weights [d_inner], fp32; channels = d_inner + 2 ngroups dstate."""
    g = rng_for(w.seed, KEY_BLOCK)
    ch = w.nheads * w.headdim + 2 * w.ngroups * w.dstate
    return {"conv_w": (g.standard_normal((ch, width)) / np.sqrt(width)).astype(np.float32),
            "conv_b": (0.1 * g.standard_normal(ch)).astype(np.float32),
            "norm_w": (1.0 + 0.1 * g.standard_normal(w.nheads * w.headdim)).astype(np.float32)}


def block_token(w: Mamba2Workload, t: int, b: int) -> Dict[str, np.ndarray]:
    """Pre-convolution channels xbc [channels] and gate z [d_inner] of sequence b at
    step t, as float32 holding in_dtype values."""
    g = rng_for(w.seed, KEY_BLOCK, t, b)
    ch = w.nheads * w.headdim + 2 * w.ngroups * w.dstate
    return {"xbc": _as_in(g.standard_normal(ch), w.in_dtype),
            "z": _as_in(g.standard_normal(w.nheads * w.headdim), w.in_dtype)}


def block_step(w: Mamba2Workload, t: int, seqs: Sequence[int]) -> Dict[str, np.ndarray]:
    toks = [block_token(w, t, b) for b in seqs]
    return {k: np.stack([tk[k] for tk in toks]) for k in ("xbc", "z")}


# --------------------------------------------------------------------------
# Gated DeltaNet draws
# --------------------------------------------------------------------------

def gdn_params(w: GDNWorkload) -> Dict[str, np.ndarray]:
    """Per-v-head decay log-rate a ~ U(-3, 0)."""
    g = rng_for(w.seed, KEY_PARAMS)
    return {"a": g.uniform(-3.0, 0.0, size=w.n_v).astype(np.float32)}


def gdn_init_state(w: GDNWorkload, b: int) -> np.ndarray:
    """Initial fp32 state of sequence b, logical layout [n_v, dv, dk]."""
    shape = (w.n_v, w.dv, w.dk)
    if w.init_std == 0.0:
        return np.zeros(shape, np.float32)
    g = rng_for(w.seed, KEY_INIT, b)
    return (g.standard_normal(shape) * w.init_std).astype(np.float32)


def gdn_init_states(w: GDNWorkload, seqs: Iterable[int]) -> np.ndarray:
    return np.stack([gdn_init_state(w, b) for b in seqs])


def _l2n(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.float32)
    n = np.sqrt(np.sum(z * z, axis=-1, keepdims=True, dtype=np.float32))
    return (z / n).astype(np.float32)


def gdn_token(w: GDNWorkload, t: int, b: int, params: Dict[str, np.ndarray] | None = None
              ) -> Dict[str, np.ndarray]:
    """Inputs (q, k, v, g, beta) of sequence b at step t.

    q, k: [n_qk, dk] (in_dtype values); v: [n_v, dv] (in_dtype values);
    g: [n_v] fp32, or [n_v, dk] for a per-channel gate; beta: [n_v] fp32.
    """
    if params is None:
        params = gdn_params(w)
    gen = rng_for(w.seed, t, b)
    q = _l2n(gen.standard_normal((w.n_qk, w.dk)))
    k = _l2n(gen.standard_normal((w.n_qk, w.dk)))
    v = gen.standard_normal((w.n_v, w.dv))
    beta = _sigmoid(gen.standard_normal(w.n_v))
    if w.gate == "channel":
        gate = -np.exp(params["a"].astype(np.float64))[:, None] * _softplus(gen.standard_normal((w.n_v, w.dk)))
    else:
        gate = -np.exp(params["a"].astype(np.float64)) * _softplus(gen.standard_normal(w.n_v))
    return {"q": _as_in(q, w.in_dtype), "k": _as_in(k, w.in_dtype), "v": _as_in(v, w.in_dtype),
            "g": gate.astype(np.float32), "beta": beta.astype(np.float32)}


def gdn_step(w: GDNWorkload, t: int, seqs: Sequence[int],
             params: Dict[str, np.ndarray] | None = None) -> Dict[str, np.ndarray]:
    if params is None:
        params = gdn_params(w)
    toks = [gdn_token(w, t, b, params) for b in seqs]
    return {k: np.stack([tk[k] for tk in toks]) for k in ("q", "k", "v", "g", "beta")}


# --------------------------------------------------------------------------
# generic tiles (quantizer tests)
# --------------------------------------------------------------------------

def state_tiles(seed: int, i: int, shape: Sequence[int], std: float = 1.0,
                heavy_tail: bool = False) -> np.ndarray:
    """fp32 tiles of N(0, std^2) values; heavy_tail multiplies each 16-block by a
    log-uniform factor in [2^-20, 2^4] so block scales span the e4m3 range."""
    g = rng_for(seed, KEY_TILE, i)
    x = g.standard_normal(tuple(shape)) * std
    if heavy_tail:
        nblk = x.shape[-1] // 16
        f = np.exp2(g.uniform(-20.0, 4.0, size=x.shape[:-1] + (nblk, 1)))
        x = (x.reshape(x.shape[:-1] + (nblk, 16)) * f).reshape(x.shape)
    return x.astype(np.float32)
