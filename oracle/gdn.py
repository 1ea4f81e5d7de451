"""Gated DeltaNet decode in fp64 (oracle; test infrastructure only).

Definition (the gated delta rule of Gated DeltaNet, Yang, Kautz and
Hatamizadeh, 2024), per sequence b and value head h, with key/query head
kappa(h) = h // (n_v // n_qk):

    alpha_t = exp(g_t)
    S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T   (S is dv x dk)
    o_t = S_t q_t

No query scaling and no normalisation happen inside the layer step; the
inputs arrive normalised. The ReplaySSM pages name Gated DeltaNet as one of the
SSM layer types the method serves (news.hamidun.com ReplaySSM page, "Why hybrid
models became the norm").

UT / WY form over a buffer (the non-flush output and the flush fold of
sitech.ge ReplaySSM page, "How ReplaySSM works", written for the delta rule).
Define u_t = beta_t (v_t - alpha_t S_{t-1} k_t); then S_t = alpha_t S_{t-1} +
u_t k_t^T, and from the checkpoint S0, with entries i = 1..m of the buffer,

    gamma_t = prod_{l<=t} alpha_l,   r_{t,i} = prod_{i<l<=t} alpha_l
    S_t     = gamma_t S0 + sum_{i<=t} r_{t,i} u_i k_i^T
    u_t + sum_{i<t} beta_t r_{t,i} (k_t . k_i) u_i = beta_t (v_t - gamma_t S0 k_t)
    o_t     = gamma_t S0 q_t + sum_{i<=t} r_{t,i} (k_i . q_t) u_i

The u_t are found by forward substitution of the unit lower-triangular system
(I + L) U = diag(beta) (V - diag(gamma) K S0^T), L_{t,i} = beta_t r_{t,i} (k_t . k_i).

Arrays: states [batch, n_v, dv, dk]; q, k [batch, n_qk, dk]; v [batch, n_v, dv];
g, beta [batch, n_v]. Everything is converted to float64 on entry.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def qk_head_of_v_head(n_v: int, n_qk: int) -> np.ndarray:
    """Value head h reads key/query head h // (n_v // n_qk): contiguous sharing."""
    if n_v % n_qk:
        raise ValueError("n_v must be a multiple of n_qk")
    return np.arange(n_v) // (n_v // n_qk)


def expand_qk(z: np.ndarray, n_v: int) -> np.ndarray:
    """[batch, n_qk, dk] -> [batch, n_v, dk]."""
    return _f64(z)[:, qk_head_of_v_head(n_v, z.shape[1]), :]


def step(S, q, k, v, g, beta):
    """One conventional decode step: returns (S_t, o_t), fp64. Reads and writes the full state."""
    S, v, g, beta = _f64(S), _f64(v), _f64(g), _f64(beta)
    nv, dk = S.shape[1], S.shape[3]
    kk, qq = expand_qk(k, nv), expand_qk(q, nv)
    alpha = np.exp(g)
    eye = np.eye(dk)
    P = eye[None, None] - beta[:, :, None, None] * kk[:, :, :, None] * kk[:, :, None, :]
    Sn = alpha[:, :, None, None] * np.matmul(S, P) \
        + beta[:, :, None, None] * v[:, :, :, None] * kk[:, :, None, :]
    o = np.einsum("bhvk,bhk->bhv", Sn, qq)
    return Sn, o


def run(S0, tokens: Sequence[dict]):
    """Conventional decode over a token list; returns (os [T, b, h, dv], final state)."""
    S = _f64(S0)
    outs = []
    for tk in tokens:
        S, o = step(S, tk["q"], tk["k"], tk["v"], tk["g"], tk["beta"])
        outs.append(o)
    return np.stack(outs), S


def window_gates(entries: Sequence[dict]):
    """gamma_t and r_{t,i} (t, i = 1..m) as direct products of alpha_l = exp(g_l).

    Returns (gamma [m][b,h], r[t][i] [b,h] for i <= t), 0-based lists.
    """
    alphas = [np.exp(_f64(e["g"])) for e in entries]
    m = len(alphas)
    gamma = []
    acc = np.ones_like(alphas[0])
    for t in range(m):
        acc = acc * alphas[t]
        gamma.append(acc.copy())
    r = []
    for t in range(m):
        row = [None] * (t + 1)
        prod = np.ones_like(alphas[0])
        for i in range(t, -1, -1):     # r_{t,i} = prod over l = i+1 .. t
            row[i] = prod.copy()
            prod = prod * alphas[i]
        r.append(row)
    return gamma, r


def ut_solve(S0, entries: Sequence[dict]) -> list:
    """u_1..u_m by forward substitution of (I + L) U = diag(beta)(V - diag(gamma) K S0^T)."""
    S0 = _f64(S0)
    nv = S0.shape[1]
    gamma, r = window_gates(entries)
    ks = [expand_qk(e["k"], nv) for e in entries]
    us = []
    for t, e in enumerate(entries):
        beta = _f64(e["beta"])
        rhs = _f64(e["v"]) - gamma[t][:, :, None] * np.einsum("bhvk,bhk->bhv", S0, ks[t])
        u = beta[:, :, None] * rhs
        for i in range(t):
            kk = np.einsum("bhk,bhk->bh", ks[t], ks[i])
            u = u - (beta * r[t][i] * kk)[:, :, None] * us[i]
        us.append(u)
    return us


def replay_output(S0, entries: Sequence[dict], q_j):
    """o_j from the checkpoint and buffer entries 1..j (entry j is the current token)."""
    S0 = _f64(S0)
    nv = S0.shape[1]
    j = len(entries)
    gamma, r = window_gates(entries)
    us = ut_solve(S0, entries)
    qq = expand_qk(q_j, nv)
    o = gamma[j - 1][:, :, None] * np.einsum("bhvk,bhk->bhv", S0, qq)
    for i, e in enumerate(entries):
        kq = np.einsum("bhk,bhk->bh", expand_qk(e["k"], nv), qq)
        o = o + (r[j - 1][i] * kq)[:, :, None] * us[i]
    return o


def replay_fold(S0, entries: Sequence[dict]):
    """S_m = gamma_m S0 + sum_i r_{m,i} u_i k_i^T over buffer entries 1..m (the flush fold)."""
    S0 = _f64(S0)
    nv = S0.shape[1]
    m = len(entries)
    gamma, r = window_gates(entries)
    us = ut_solve(S0, entries)
    S = gamma[m - 1][:, :, None, None] * S0
    for i, e in enumerate(entries):
        ki = expand_qk(e["k"], nv)
        S = S + r[m - 1][i][:, :, None, None] * us[i][:, :, :, None] * ki[:, :, None, :]
    return S
