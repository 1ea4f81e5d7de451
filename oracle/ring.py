"""Integer state machine of the ReplaySSM input buffer (oracle; test infrastructure only).

sitech.ge ReplaySSM page, "How ReplaySSM works": the state is a checkpoint plus
a buffer of recent input records; most steps (non-flush) append the current
input; when the 16-entry buffer fills, a flush step folds the buffered inputs
into the checkpoint, writes it once and clears the buffer. Same page, "Reducing
state traffic and simplifying rollback": for speculative decoding, draft-token
inputs are appended until verification and the accepted prefix is committed by
moving a pointer, with no state snapshot saved or restored.

Readings taken where the pages are silent:

* Per sequence the machine holds n_ckpt (tokens folded into the checkpoint),
  len (committed buffer entries) and nd (pending draft entries).
* Buffer entry i (0-based, i < len + nd) lives in slot (n_ckpt + i) mod R,
  i.e. the global token index modulo the ring size R = 16.
* Plain decode: a step with len = R - 1 is the flush; it folds the R - 1
  stored entries plus the current token (R entries). Any other step with
  len <= R - 2 is a non-flush step that writes the current token to slot
  (n_ckpt + len) mod R. A flush may also be forced at any fill f <= R - 1; it
  folds f + 1 entries.
* Every step emits an output, flush steps included.
* Speculative append of K drafts needs nd = 0 and len + K <= R; it sets nd = K.
  Commit of k needs 0 <= k <= nd; it sets len += k and nd = 0, and then, if
  len > R - K_max, folds the len committed entries (n_ckpt += len, len = 0), so
  that the next round's K_max drafts fit.
* A call that breaks these rules sets a sticky error bit for that sequence
  and leaves it unchanged: 1 = non-flush on a full buffer, 2 = append
  overflow, 4 = commit count outside [0, nd], 8 = a plain step while drafts
  are pending.

Plain Python integers only, so the model can be read line by line.
"""
from __future__ import annotations

from typing import List

R = 16

ERR_FULL = 1
ERR_OVERFLOW = 2
ERR_COMMIT = 4
ERR_PENDING = 8


class RingModel:
    def __init__(self, batch: int, ring: int = R, max_draft: int = 0):
        self.ring = ring
        self.max_draft = max_draft
        self.n_ckpt = [0] * batch
        self.len = [0] * batch
        self.nd = [0] * batch
        self.err = [0] * batch

    def slot(self, b: int, i: int) -> int:
        """Ring slot of buffer entry i of sequence b."""
        return (self.n_ckpt[b] + i) % self.ring

    def committed_slots(self, b: int) -> List[int]:
        return [self.slot(b, i) for i in range(self.len[b])]

    def live_slots(self, b: int) -> List[int]:
        return [self.slot(b, i) for i in range(self.len[b] + self.nd[b])]

    # -- plain decode ------------------------------------------------------
    def nonflush(self, b: int):
        """Append the current token. Returns its slot, or None on a contract violation."""
        if self.nd[b]:
            self.err[b] |= ERR_PENDING
            return None
        if self.len[b] > self.ring - 2:
            self.err[b] |= ERR_FULL
            return None
        s = self.slot(b, self.len[b])
        self.len[b] += 1
        return s

    def flush(self, b: int):
        """Fold the stored entries plus the current token. Returns the folded slots
        (the current token is not stored), or None on a contract violation."""
        if self.nd[b]:
            self.err[b] |= ERR_PENDING
            return None
        folded = self.committed_slots(b)
        self.n_ckpt[b] += self.len[b] + 1
        self.len[b] = 0
        return folded

    def is_flush_step(self, b: int) -> bool:
        """The plain decode schedule: flush exactly when the buffer would fill."""
        return self.len[b] == self.ring - 1

    # -- speculative decode -------------------------------------------------
    def spec_append(self, b: int, K: int):
        """Append K drafts. Returns their slots, or None on a contract violation."""
        if self.nd[b] or self.len[b] + K > self.ring or K < 1 or K > self.max_draft:
            self.err[b] |= ERR_OVERFLOW
            return None
        slots = [self.slot(b, self.len[b] + d) for d in range(K)]
        self.nd[b] = K
        return slots

    def spec_commit(self, b: int, k: int):
        """Commit the first k drafts. Returns the folded slots if the commit folds,
        [] if it does not, or None on a contract violation."""
        if k < 0 or k > self.nd[b]:
            self.err[b] |= ERR_COMMIT
            return None
        self.len[b] += k
        self.nd[b] = 0
        if self.len[b] > self.ring - self.max_draft:
            folded = self.committed_slots(b)
            self.n_ckpt[b] += self.len[b]
            self.len[b] = 0
            return folded
        return []
