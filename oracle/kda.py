"""Kimi Delta Attention decode in fp64 (oracle; test infrastructure only).

Definition (Kimi Delta Attention of the Kimi Linear architecture, Moonshot AI,
2025: the gated delta rule with a decay per key channel instead of one per
head), per sequence b and value head h, with key/query head
kappa(h) = h // (n_v // n_qk), written for the stored orientation of this
library (S is dv x dk, so the paper's dk x dv state transposed):

    alpha_t = exp(g_t)                      (a vector over the dk key channels)
    S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
    o_t = S_t q_t

With every channel of alpha_t equal this is the Gated DeltaNet step. The
ReplaySSM pages name KDA as the third SSM layer type beside Mamba-2 and Gated
DeltaNet (news.hamidun.com ReplaySSM page, "Why hybrid models became the
norm"), and a model family that verifies draft inputs in KDA layers (sitech.ge
ReplaySSM page, "Availability"); they give no formula.

Checkpoint + buffer form (the non-flush output and flush fold of sitech.ge
ReplaySSM page, "How ReplaySSM works", written for this rule). Define
u_t = beta_t (v_t - S_{t-1} Diag(alpha_t) k_t); then
S_t = S_{t-1} Diag(alpha_t) + u_t k_t^T, and from the checkpoint S0 over
buffer entries i = 1..m, with the per-channel products

    gamma_t = prod_{l<=t} alpha_l,   r_{t,i} = prod_{i<l<=t} alpha_l   (vectors)
    S_t     = S0 Diag(gamma_t) + sum_{i<=t} u_i (r_{t,i} * k_i)^T
    u_t + sum_{i<t} beta_t <k_t, r_{t,i} * k_i> u_i = beta_t (v_t - S0 (gamma_t * k_t))
    o_t     = S0 (gamma_t * q_t) + sum_{i<=t} <q_t, r_{t,i} * k_i> u_i

(* is the elementwise product, <,> the dot product). As for Gated DeltaNet,
u_t depends only on S0 and entries <= t.

Arrays: states [batch, n_v, dv, dk]; q, k [batch, n_qk, dk]; v [batch, n_v, dv];
g [batch, n_v, dk]; beta [batch, n_v]. Everything is converted to float64.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

from .gdn import expand_qk


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def step(S, q, k, v, g, beta):
    """One conventional decode step: returns (S_t, o_t), fp64. Reads and writes the full state."""
    S, v, g, beta = _f64(S), _f64(v), _f64(g), _f64(beta)
    nv, dk = S.shape[1], S.shape[3]
    kk, qq = expand_qk(k, nv), expand_qk(q, nv)
    alpha = np.exp(g)                                                   # [b, h, dk]
    eye = np.eye(dk)
    P = eye[None, None] - beta[:, :, None, None] * kk[:, :, :, None] * kk[:, :, None, :]
    Sn = np.matmul(S * alpha[:, :, None, :], P) + beta[:, :, None, None] * v[:, :, :, None] * kk[:, :, None, :]
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


def window_decays(entries: Sequence[dict]):
    """gamma_t and r_{t,i} (t, i = 1..m) per key channel, as direct products of
    alpha_l = exp(g_l). Returns (gamma [m][b,h,dk], r[t][i] [b,h,dk] for i <= t)."""
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
    """u_1..u_m by forward substitution (entries in buffer order)."""
    S0 = _f64(S0)
    nv = S0.shape[1]
    gamma, r = window_decays(entries)
    ks = [expand_qk(e["k"], nv) for e in entries]
    us = []
    for t, e in enumerate(entries):
        beta = _f64(e["beta"])
        rhs = _f64(e["v"]) - np.einsum("bhvk,bhk->bhv", S0, gamma[t] * ks[t])
        u = beta[:, :, None] * rhs
        for i in range(t):
            w = np.einsum("bhk,bhk->bh", ks[t], r[t][i] * ks[i])
            u = u - (beta * w)[:, :, None] * us[i]
        us.append(u)
    return us


def replay_output(S0, entries: Sequence[dict], q_j):
    """o_j from the checkpoint and buffer entries 1..j (entry j is the current token)."""
    S0 = _f64(S0)
    nv = S0.shape[1]
    j = len(entries)
    gamma, r = window_decays(entries)
    us = ut_solve(S0, entries)
    qq = expand_qk(q_j, nv)
    o = np.einsum("bhvk,bhk->bhv", S0, gamma[j - 1] * qq)
    for i, e in enumerate(entries):
        w = np.einsum("bhk,bhk->bh", qq, r[j - 1][i] * expand_qk(e["k"], nv))
        o = o + w[:, :, None] * us[i]
    return o


def replay_fold(S0, entries: Sequence[dict]):
    """S_m = S0 Diag(gamma_m) + sum_i u_i (r_{m,i} * k_i)^T over entries 1..m (the flush fold)."""
    S0 = _f64(S0)
    nv = S0.shape[1]
    m = len(entries)
    gamma, r = window_decays(entries)
    us = ut_solve(S0, entries)
    S = S0 * gamma[m - 1][:, :, None, :]
    for i, e in enumerate(entries):
        kr = r[m - 1][i] * expand_qk(e["k"], nv)
        S = S + us[i][:, :, :, None] * kr[:, :, None, :]
    return S
