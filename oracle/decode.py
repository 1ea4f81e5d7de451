"""Token-by-token decode drivers in fp64 (oracle; test infrastructure only).

* ``M2Conventional`` / ``GDNConventional``: the layer's plain recurrence, which
  reads and writes the full state every step (sitech.ge ReplaySSM page, "How
  ReplaySSM works", conventional decoding). Speculative rounds here follow the
  snapshot/restore scheme that the pages contrast with ReplaySSM: each draft's
  state is kept, and the state after the last accepted draft becomes live
  (news.hamidun.com ReplaySSM page, "Where the state problem appears": rollback
  needs per-step copies of the state).
* ``M2Replay`` / ``GDNReplay``: ReplaySSM decode. The state is a checkpoint
  plus a ring of recent input records driven by ``ring.RingModel``; non-flush
  steps compute the output from checkpoint + buffer and store no state; a flush
  folds the buffer into the checkpoint (sitech.ge ReplaySSM page, "How
  ReplaySSM works"). Speculative rounds append drafts and commit the accepted
  prefix by moving the buffer pointer, with no snapshot (same page, "Reducing
  state traffic and simplifying rollback"). Optional low-precision formats
  (same page, "Bounding quantization error"): the checkpoint may be stored as
  fp16, fp8 or NVFP4 (the last being the uniform comparator), and reads may go
  through an NVFP4 copy of the stored checkpoint while the fold keeps reading
  the checkpoint itself.

Inputs are batched token dicts as drawn by the workload generators (arrays
with a leading batch axis). The replay drivers loop over sequences so that
each one follows its own buffer position.
"""
from __future__ import annotations

from typing import Dict, List, Sequence

import numpy as np

from . import gdn, kda, mamba2, quant
from .ring import RingModel, R


def _slice(tok: Dict[str, np.ndarray], b: int) -> Dict[str, np.ndarray]:
    return {k: np.asarray(v)[b:b + 1] for k, v in tok.items()}


def _stored(fmt: str, state: np.ndarray) -> np.ndarray:
    """Stored-then-read value of a state in checkpoint format fmt, per stored matrix.

    The stored matrix is the state transposed to [dstate or dk, headdim or dv]
    (the stored layout), so quantizer blocks run along headdim / dv.
    """
    if fmt == "f32_exact":
        return np.array(state, dtype=np.float64, copy=True)
    st = np.asarray(state, dtype=np.float64).astype(np.float32)
    out = np.empty(st.shape, dtype=np.float64)
    for b in range(st.shape[0]):
        for h in range(st.shape[1]):
            out[b, h] = quant.roundtrip(fmt, st[b, h].T).T
    return out


class M2Conventional:
    def __init__(self, H0, A, D):
        self.H = np.asarray(H0, dtype=np.float64).copy()
        self.A, self.D = A, D

    def step(self, tok) -> np.ndarray:
        self.H, y = mamba2.step(self.H, tok["x"], tok["B"], tok["C"], tok["dt"], self.A, self.D)
        return y

    def spec_round(self, drafts: Sequence[dict], accepted: np.ndarray) -> np.ndarray:
        """Verify K drafts from the live state (keeping a snapshot per draft), then make
        the snapshot after draft k[b] live. Returns the K outputs [K, b, h, P]."""
        H = self.H
        snaps, ys = [], []
        for d in drafts:
            H, y = mamba2.step(H, d["x"], d["B"], d["C"], d["dt"], self.A, self.D)
            snaps.append(H)
            ys.append(y)
        for b, k in enumerate(np.asarray(accepted)):
            if k >= 1:
                self.H[b] = snaps[k - 1][b]
        return np.stack(ys)


class M2Replay:
    """ReplaySSM decode of a Mamba-2 layer in fp64.

    ckpt_fmt: "f32_exact" (fp64 checkpoint, the method without storage rounding),
    "f32", "f16", "fp8" or "nvfp4" (uniform comparator). read_copy: None or "nvfp4".
    """

    def __init__(self, H0, A, D, max_draft: int = 0, ckpt_fmt: str = "f32_exact",
                 read_copy=None, ring: int = R):
        self.A, self.D = A, D
        self.ckpt_fmt, self.read_copy = ckpt_fmt, read_copy
        self.batch = H0.shape[0]
        self.ring = RingModel(self.batch, ring, max_draft)
        self.entries: List[Dict[int, dict]] = [dict() for _ in range(self.batch)]
        self.ckpt = _stored(ckpt_fmt, H0)
        self.view = self._read_view(self.ckpt)

    def _read_view(self, ckpt):
        if self.read_copy == "nvfp4" and self.ckpt_fmt != "nvfp4":
            return _stored("nvfp4", ckpt)
        return ckpt

    def _buffer(self, b: int, slots) -> List[dict]:
        return [self.entries[b][s] for s in slots]

    def step(self, tok, force_flush: bool = False) -> np.ndarray:
        """One decode step for every sequence: flush when the buffer fills (or when
        forced), otherwise a non-flush step. Returns y [b, h, P]."""
        ys = []
        for b in range(self.batch):
            tb = _slice(tok, b)
            if force_flush or self.ring.is_flush_step(b):
                ys.append(self._flush(b, tb))
            else:
                ys.append(self._nonflush(b, tb))
        return np.concatenate(ys)

    def _nonflush(self, b, tb):
        held = self._buffer(b, self.ring.committed_slots(b))
        s = self.ring.nonflush(b)
        if s is None:
            return np.full((1,) + tb["x"].shape[1:], np.nan)
        self.entries[b][s] = tb
        return mamba2.replay_output(self.view[b:b + 1], held + [tb], tb["C"], self.A, self.D)

    def _flush(self, b, tb):
        held = self._buffer(b, self.ring.committed_slots(b))
        if self.ring.flush(b) is None:
            return np.full((1,) + tb["x"].shape[1:], np.nan)
        Hn = mamba2.replay_fold(self.ckpt[b:b + 1], held + [tb], self.A)
        y = np.einsum("bhpn,bhn->bhp", Hn, mamba2.expand_groups(tb["C"], Hn.shape[1])) \
            + np.asarray(self.D, np.float64)[None, :, None] * np.asarray(tb["x"], np.float64)
        self._set_ckpt(b, Hn)
        return y

    def _set_ckpt(self, b, Hn):
        self.ckpt[b:b + 1] = _stored(self.ckpt_fmt, Hn)
        self.view[b:b + 1] = self._read_view(self.ckpt[b:b + 1])

    def spec_append(self, drafts: Sequence[dict]) -> np.ndarray:
        """Append K drafts and return their verify outputs [K, b, h, P]; no state is formed."""
        K = len(drafts)
        out = []
        for b in range(self.batch):
            held = self._buffer(b, self.ring.committed_slots(b))
            slots = self.ring.spec_append(b, K)
            dr = [_slice(d, b) for d in drafts]
            if slots is None:
                out.append(np.full((K, 1) + dr[0]["x"].shape[1:], np.nan))
                continue
            for s, d in zip(slots, dr):
                self.entries[b][s] = d
            ys = [mamba2.replay_output(self.view[b:b + 1], held + dr[:i + 1], dr[i]["C"],
                                       self.A, self.D) for i in range(K)]
            out.append(np.stack(ys))
        return np.concatenate(out, axis=1)

    def spec_commit(self, accepted) -> None:
        """Commit the first accepted[b] drafts of each sequence; fold when room runs short."""
        for b, k in enumerate(np.asarray(accepted)):
            folded = self.ring.spec_commit(b, int(k))
            if folded:
                ents = self._buffer(b, folded)
                self._set_ckpt(b, mamba2.replay_fold(self.ckpt[b:b + 1], ents, self.A))

    def effective_state(self) -> np.ndarray:
        """fold(checkpoint, committed buffer): the state conventional decode would hold."""
        out = np.empty_like(self.ckpt)
        for b in range(self.batch):
            held = self._buffer(b, self.ring.committed_slots(b))
            out[b] = self.ckpt[b] if not held else mamba2.replay_fold(self.ckpt[b:b + 1], held, self.A)[0]
        return out


class GDNConventional:
    """Plain decode of a delta-rule layer: rule = gdn (Gated DeltaNet) or kda
    (Kimi Delta Attention, per-key-channel decay)."""

    def __init__(self, S0, rule=gdn):
        self.S = np.asarray(S0, dtype=np.float64).copy()
        self.rule = rule

    def step(self, tok) -> np.ndarray:
        self.S, o = self.rule.step(self.S, tok["q"], tok["k"], tok["v"], tok["g"], tok["beta"])
        return o

    def spec_round(self, drafts: Sequence[dict], accepted: np.ndarray) -> np.ndarray:
        """Verify K drafts from the live state (keeping a snapshot per draft), then make
        the snapshot after draft k[b] live. Returns the K outputs [K, b, n_v, dv]."""
        S = self.S
        snaps, os_ = [], []
        for d in drafts:
            S, o = self.rule.step(S, d["q"], d["k"], d["v"], d["g"], d["beta"])
            snaps.append(S)
            os_.append(o)
        for b, k in enumerate(np.asarray(accepted)):
            if k >= 1:
                self.S[b] = snaps[k - 1][b]
        return np.stack(os_)


class GDNReplay:
    """ReplaySSM decode of a delta-rule layer in fp64; rule = gdn or kda as for
    GDNConventional.

    ckpt_fmt: "f32_exact" (fp64 checkpoint, the method without storage
    rounding) or "f32" (the checkpoint rounded to float32 at every write).
    read_copy: None or "nvfp4". With a read copy, every output (non-flush
    steps and speculative verify) is computed from the NVFP4 copy of the stored
    checkpoint, the solved rows u included, while every fold (flush, commit)
    solves its rows from the checkpoint itself, so read error never enters the
    recurrence (sitech.ge ReplaySSM page, "Bounding quantization error"). The
    copy quantizes the stored matrix [dk][dv] (value index innermost, the
    layout the checkpoint is stored in), so its 16-element blocks run along dv.
    """

    def __init__(self, S0, ring: int = R, max_draft: int = 0, rule=gdn, ckpt_fmt: str = "f32_exact",
                 read_copy=None):
        self.rule = rule
        self.ckpt_fmt, self.read_copy = ckpt_fmt, read_copy
        self.batch = S0.shape[0]
        self.ckpt = _stored(ckpt_fmt, S0)
        self.view = self._read_view(self.ckpt)
        self.ring = RingModel(self.batch, ring, max_draft)
        self.entries: List[Dict[int, dict]] = [dict() for _ in range(self.batch)]

    def _read_view(self, ckpt):
        if self.read_copy == "nvfp4":
            return _stored("nvfp4", ckpt)
        return ckpt

    def _set_ckpt(self, b, Sn):
        self.ckpt[b:b + 1] = _stored(self.ckpt_fmt, Sn)
        self.view[b:b + 1] = self._read_view(self.ckpt[b:b + 1])

    def spec_append(self, drafts: Sequence[dict]) -> np.ndarray:
        """Append K drafts after the committed entries and return their verify outputs
        [K, b, n_v, dv], each from the checkpoint and the buffer up to that draft; no
        state is formed."""
        K = len(drafts)
        out = []
        for b in range(self.batch):
            held = [self.entries[b][s] for s in self.ring.committed_slots(b)]
            slots = self.ring.spec_append(b, K)
            dr = [_slice(d, b) for d in drafts]
            if slots is None:
                out.append(np.full((K, 1) + dr[0]["v"].shape[1:], np.nan))
                continue
            for s, d in zip(slots, dr):
                self.entries[b][s] = d
            os_ = [self.rule.replay_output(self.view[b:b + 1], held + dr[:i + 1], dr[i]["q"]) for i in range(K)]
            out.append(np.stack(os_))
        return np.concatenate(out, axis=1)

    def spec_commit(self, accepted) -> None:
        """Commit the first accepted[b] drafts of each sequence (a pointer move); fold
        the committed entries into the checkpoint when room for the next round runs short."""
        for b, k in enumerate(np.asarray(accepted)):
            folded = self.ring.spec_commit(b, int(k))
            if folded:
                ents = [self.entries[b][s] for s in folded]
                self._set_ckpt(b, self.rule.replay_fold(self.ckpt[b:b + 1], ents))

    def step(self, tok, force_flush: bool = False) -> np.ndarray:
        outs = []
        for b in range(self.batch):
            tb = _slice(tok, b)
            held = [self.entries[b][s] for s in self.ring.committed_slots(b)]
            if force_flush or self.ring.is_flush_step(b):
                if self.ring.flush(b) is None:
                    outs.append(np.full((1,) + tb["v"].shape[1:], np.nan))
                    continue
                Sn = self.rule.replay_fold(self.ckpt[b:b + 1], held + [tb])
                o = np.einsum("bhvk,bhk->bhv", Sn, gdn.expand_qk(tb["q"], Sn.shape[1]))
                self._set_ckpt(b, Sn)
            else:
                s = self.ring.nonflush(b)
                if s is None:
                    outs.append(np.full((1,) + tb["v"].shape[1:], np.nan))
                    continue
                self.entries[b][s] = tb
                o = self.rule.replay_output(self.view[b:b + 1], held + [tb], tb["q"])
            outs.append(o)
        return np.concatenate(outs)

    def effective_state(self) -> np.ndarray:
        out = self.ckpt.copy()
        for b in range(self.batch):
            held = [self.entries[b][s] for s in self.ring.committed_slots(b)]
            if held:
                out[b] = self.rule.replay_fold(self.ckpt[b:b + 1], held)[0]
        return out
