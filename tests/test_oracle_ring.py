"""Pins for the buffer state machine.

* Plain decode from an empty buffer has a closed form: step t is a flush iff
  t mod 16 = 15, a non-flush step writes slot t mod 16, and after step t the
  buffer holds (t+1) mod 16 entries over a checkpoint of 16 floor((t+1)/16)
  tokens (tests/golden/flush_schedule.json holds the tiny Mamba-2 case).
* Speculative rounds are checked against a second model written differently:
  each sequence keeps the list of global token indices held in its buffer,
  and a token's slot is its global index mod 16.
"""
import json
import os
import random

from oracle.ring import RingModel, ERR_COMMIT, ERR_FULL, ERR_OVERFLOW, ERR_PENDING

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_plain_schedule_closed_form():
    m = RingModel(1)
    for t in range(200):
        flush = m.is_flush_step(0)
        assert flush == (t % 16 == 15)
        if flush:
            m.flush(0)
        else:
            assert m.nonflush(0) == t % 16
        assert m.len[0] == (t + 1) % 16
        assert m.n_ckpt[0] == 16 * ((t + 1) // 16)


def test_golden_tiny_schedule():
    with open(os.path.join(GOLD, "flush_schedule.json")) as f:
        g = json.load(f)
    m = RingModel(1)
    flushes, slots = [], []
    for t in range(g["steps"]):
        if m.is_flush_step(0):
            m.flush(0)
            flushes.append(t)
        else:
            slots.append(m.nonflush(0))
    assert flushes == g["flush_steps"]
    assert slots[:20] == g["first_nonflush_slots"]
    assert m.n_ckpt[0] == g["final_n_ckpt"] and m.len[0] == g["final_len"]


class ListModel:
    """Second model: the buffer is a list of global token indices."""

    def __init__(self, kmax):
        self.kmax = kmax
        self.next_global = 0      # global index of the next token to enter
        self.committed = []
        self.pending = []

    def append(self, K):
        if self.pending or len(self.committed) + K > 16:
            return None
        self.pending = [self.next_global + len(self.committed) + d for d in range(K)]
        return [g % 16 for g in self.pending]

    def commit(self, k):
        if k < 0 or k > len(self.pending):
            return None
        self.committed += self.pending[:k]
        self.pending = []
        if len(self.committed) > 16 - self.kmax:
            out = [g % 16 for g in self.committed]
            self.next_global += len(self.committed)
            self.committed = []
            return out
        return []


def test_spec_matches_list_model():
    rnd = random.Random(0)
    for kmax in (1, 2, 4, 6):
        m, ref = RingModel(1, max_draft=kmax), ListModel(kmax)
        for _ in range(400):
            K = rnd.randint(1, kmax)
            assert m.spec_append(0, K) == ref.append(K)
            k = rnd.randint(0, K)
            assert m.spec_commit(0, k) == ref.commit(k)
            assert m.len[0] == len(ref.committed) and m.nd[0] == 0
            assert m.n_ckpt[0] == ref.next_global
            assert m.committed_slots(0) == [g % 16 for g in ref.committed]
        assert m.err == [0]


def test_plain_steps_after_spec_rounds():
    m = RingModel(1, max_draft=4)
    m.spec_append(0, 4)
    m.spec_commit(0, 3)
    assert m.len[0] == 3 and m.nonflush(0) == 3
    assert m.committed_slots(0) == [0, 1, 2, 3]


def test_error_bits_leave_state_unchanged():
    m = RingModel(1, max_draft=4)
    for _ in range(15):
        m.nonflush(0)
    snap = (m.n_ckpt[0], m.len[0], m.nd[0])
    assert m.nonflush(0) is None and m.err[0] & ERR_FULL
    assert (m.n_ckpt[0], m.len[0], m.nd[0]) == snap
    assert m.spec_append(0, 4) is None and m.err[0] & ERR_OVERFLOW
    m2 = RingModel(1, max_draft=4)
    m2.spec_append(0, 2)
    assert m2.spec_commit(0, 3) is None and m2.err[0] & ERR_COMMIT
    assert m2.nonflush(0) is None and m2.err[0] & ERR_PENDING
    assert m2.flush(0) is None
    assert (m2.len[0], m2.nd[0]) == (0, 2)
