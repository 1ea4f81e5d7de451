"""The Mamba-2 block's other per-token state and its output gate, in fp64
(oracle; test infrastructure only).

Definitions (the Mamba-2 block of Dao and Gu, "Transformers are SSMs", 2024;
not given on the ReplaySSM pages, which name the layer type only):

* Short causal convolution. Before the SSM, the concatenated channels
  xBC = [x | B | C] (d_inner + 2 ngroups dstate channels) go through a
  depthwise causal convolution of width W (4 in the published models) with a
  bias, then SiLU:
      out_t[c] = silu(bias[c] + sum_{k<W} w[c][k] * xBC_{t-W+1+k}[c])
  so w[c][W-1] weighs the current token and w[c][0] the oldest. Inputs before
  the first token are zero. Its decode state is the last W-1 inputs, a short
  buffer of recent inputs like the ReplaySSM buffer (sitech.ge ReplaySSM page,
  "How ReplaySSM works"), and the same rollback question arises for drafts
  (same page, "Reducing state traffic and simplifying rollback").
* Gated RMS norm after the SSM (the gate applied before the norm):
      v = y * silu(z);  out = v / sqrt(mean_group(v^2) + eps) * weight
  over groups of d_inner / ngroups consecutive channels of the flattened
  y [nheads * headdim].

silu(u) = u / (1 + exp(-u)).
"""
from __future__ import annotations

import numpy as np


def silu(u):
    u = np.asarray(u, dtype=np.float64)
    return u / (1.0 + np.exp(-u))


def causal_conv(seq, weight, bias=None):
    """Whole-sequence causal depthwise convolution + SiLU: seq [T, ..., C] over the
    time axis 0, weight [C, W], bias [C] or None. Returns [T, ..., C] fp64."""
    seq = np.asarray(seq, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    T, W = seq.shape[0], w.shape[1]
    out = np.zeros_like(seq)
    for t in range(T):
        acc = np.zeros(seq.shape[1:]) if bias is None else np.broadcast_to(np.asarray(bias, np.float64),
                                                                            seq.shape[1:]).copy()
        for k in range(W):
            src = t - (W - 1) + k
            if src >= 0:
                acc = acc + w[:, k] * seq[src]
        out[t] = silu(acc)
    return out


class ConvState:
    """Decode form: the last W-1 inputs per sequence (zeros before the first token).
    step(xbc [batch, C]) -> conv output [batch, C]."""

    def __init__(self, batch: int, channels: int, weight, bias=None, history=None):
        self.w = np.asarray(weight, dtype=np.float64)
        self.b = None if bias is None else np.asarray(bias, dtype=np.float64)
        W = self.w.shape[1]
        self.hist = np.zeros((batch, W - 1, channels)) if history is None else \
            np.asarray(history, dtype=np.float64).copy()      # oldest first

    def step(self, xbc):
        x = np.asarray(xbc, dtype=np.float64)
        window = np.concatenate([self.hist, x[:, None, :]], axis=1)      # [b, W, C], oldest first
        acc = np.einsum("bkc,ck->bc", window, self.w)
        if self.b is not None:
            acc = acc + self.b
        self.hist = window[:, 1:, :]
        return silu(acc)

    def drafts(self, xbcs):
        """Outputs for K draft inputs in order, without keeping them (the state is
        unchanged); commit(xbcs[:k]) keeps the first k."""
        saved = self.hist.copy()
        outs = [self.step(x) for x in xbcs]
        self.hist = saved
        return np.stack(outs)

    def commit(self, xbcs, accepted):
        """Keep the first accepted[b] of the draft inputs of sequence b."""
        for b, k in enumerate(np.asarray(accepted)):
            for d in range(int(k)):
                self.hist[b] = np.concatenate([self.hist[b, 1:], np.asarray(xbcs[d], np.float64)[b][None]], axis=0)


def gated_rmsnorm(y, z, weight, ngroups: int, eps: float = 1e-5):
    """y, z [batch, d_inner] (flattened heads x headdim), weight [d_inner]."""
    y = np.asarray(y, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    b, d = y.shape
    v = (y * silu(z)).reshape(b, ngroups, d // ngroups)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    out = v / np.sqrt(ms + eps)
    return out.reshape(b, d) * np.asarray(weight, dtype=np.float64)
