"""Mamba-2 decode in fp64 (oracle; test infrastructure only).

Definition (the recurrent decode form of the Mamba-2 / SSD layer, Dao and Gu,
"Transformers are SSMs", 2024), per sequence b and head h, with group
g(h) = h // (nheads // ngroups):

    a_t = exp(dt_t * A_h)
    H_t = a_t * H_{t-1} + dt_t * x_t B_t^T          (H is headdim x dstate)
    y_t = H_t C_t + D_h * x_t

The state is updated first and then read. The ReplaySSM pages name Mamba-2 as
one of the SSM layer types the method serves (news.hamidun.com ReplaySSM page,
"Why hybrid models became the norm").

Checkpoint-plus-buffer forms (sitech.ge ReplaySSM page, "How ReplaySSM works":
the state is a checkpoint plus a buffer of recent inputs; non-flush steps
compute the output from both without storing state; a flush folds the buffer
into the checkpoint once). With checkpoint H0 and buffer entries i = 1..j
(entry j is the current token), unrolling the recurrence gives

    l_j     = prod_{1<=l<=j} a_l
    w_{j,i} = prod_{i<l<=j} a_l                      (w_{j,j} = 1)
    y_j     = l_j (H0 C_j) + sum_{i<=j} w_{j,i} dt_i (B_i . C_j) x_i + D x_j
    H_m     = l_m H0 + sum_{i<=m} w_{m,i} dt_i x_i B_i^T   (the fold)

Arrays use the logical layout: states [batch, nheads, headdim, dstate]; x
[batch, nheads, headdim]; B, C [batch, ngroups, dstate]; dt [batch, nheads];
A, D [nheads]. Everything is converted to float64 on entry.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def group_of_head(nheads: int, ngroups: int) -> np.ndarray:
    """Head h reads group h // (nheads // ngroups): groups are contiguous head ranges."""
    if nheads % ngroups:
        raise ValueError("nheads must be a multiple of ngroups")
    return np.arange(nheads) // (nheads // ngroups)


def expand_groups(Bg: np.ndarray, nheads: int) -> np.ndarray:
    """[batch, ngroups, N] -> [batch, nheads, N] by the contiguous head-to-group map."""
    return _f64(Bg)[:, group_of_head(nheads, Bg.shape[1]), :]


def step(H, x, B, C, dt, A, D):
    """One conventional decode step: returns (H_t, y_t), both fp64.

    Reads and writes the full state, which is what conventional decoding does
    at every step (sitech.ge ReplaySSM page, "How ReplaySSM works").
    """
    H, x, dt, A, D = _f64(H), _f64(x), _f64(dt), _f64(A), _f64(D)
    nh = H.shape[1]
    Bh, Ch = expand_groups(B, nh), expand_groups(C, nh)
    a = np.exp(dt * A[None, :])                                   # [b, h]
    Hn = a[:, :, None, None] * H + (dt[:, :, None] * x)[:, :, :, None] * Bh[:, :, None, :]
    y = np.einsum("bhpn,bhn->bhp", Hn, Ch) + D[None, :, None] * x
    return Hn, y


def run(H0, tokens: Sequence[dict], A, D):
    """Conventional decode over a token list; returns (ys [T, b, h, P], final state)."""
    H = _f64(H0)
    ys = []
    for tk in tokens:
        H, y = step(H, tk["x"], tk["B"], tk["C"], tk["dt"], A, D)
        ys.append(y)
    return np.stack(ys), H


def decays(dts: Sequence[np.ndarray], A) -> list:
    """a_i = exp(dt_i * A) for each buffer entry, fp64 [b, h]."""
    A = _f64(A)
    return [np.exp(_f64(dt) * A[None, :]) for dt in dts]


def window_weights(a: Sequence[np.ndarray], j: int):
    """(l_j, [w_{j,1} .. w_{j,j}]) as direct products of the per-entry factors."""
    w = [None] * j
    acc = np.ones_like(a[0])
    for i in range(j, 0, -1):          # w_{j,i} = prod over l = i+1 .. j
        w[i - 1] = acc.copy()
        acc = acc * a[i - 1]
    return acc, w                      # acc now holds prod over l = 1 .. j


def replay_output(H0, entries: Sequence[dict], C_j, A, D):
    """y_j from the checkpoint and buffer entries 1..j (entry j is the current token).

    No state is formed: the checkpoint is read as is and the buffer term is a
    sum of j rank-one contributions (the non-flush step).
    """
    H0 = _f64(H0)
    j = len(entries)
    nh = H0.shape[1]
    Cj = expand_groups(C_j, nh)
    a = decays([e["dt"] for e in entries], A)
    l_j, w = window_weights(a, j)
    y = l_j[:, :, None] * np.einsum("bhpn,bhn->bhp", H0, Cj)
    for i, e in enumerate(entries):
        Bi = expand_groups(e["B"], nh)
        s = w[i] * _f64(e["dt"]) * np.einsum("bhn,bhn->bh", Bi, Cj)
        y = y + s[:, :, None] * _f64(e["x"])
    y = y + _f64(D)[None, :, None] * _f64(entries[-1]["x"])
    return y


def replay_fold(H0, entries: Sequence[dict], A):
    """H_m = l_m H0 + sum_i w_{m,i} dt_i x_i B_i^T over buffer entries 1..m (the flush fold)."""
    H0 = _f64(H0)
    m = len(entries)
    nh = H0.shape[1]
    a = decays([e["dt"] for e in entries], A)
    l_m, w = window_weights(a, m)
    H = l_m[:, :, None, None] * H0
    for i, e in enumerate(entries):
        Bi = expand_groups(e["B"], nh)
        xt = (w[i] * _f64(e["dt"]))[:, :, None] * _f64(e["x"])
        H = H + xt[:, :, :, None] * Bi[:, :, None, :]
    return H
