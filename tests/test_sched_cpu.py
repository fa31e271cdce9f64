"""CPU tests of the slot manager (mllm_sched_* through the binding).

The policy under test is the one microLLM-rocm ARCHITECTURE.md ("Tensor
ownership boundary") gives its continuous-batch scheduler: admission only at
step boundaries, first in first out into the lowest free slot, a row reset on
length / stop / cancel, the shared allocation persisting while rows return to
position zero, and max_sequence_length bounding every request (zero keeps the
cache's maximum).  Hand scenarios pin each rule; a long randomized trace is
compared boundary by boundary with `PolicyModel`, a plain Python statement of
the same rules.  The caller's kernels are simulated by setting row lengths
(a prefill sets the prompt length, a decode step adds one).
"""
import ctypes
import random

import pytest

import positions_aware_cached_amd as pac
from test_abi_cpu import FakeCache

LENGTH, STOP, CANCEL = 1, 2, 3


def run_plan(cache, admitted, decode):
    """What the caller's kernels do to the row lengths in one step."""
    for _, row, prompt in admitted:
        cache.set_row_length(row, prompt)
    for _, row, pos in decode:
        cache.set_row_length(row, pos + 1)


def test_lowest_free_slot_fifo_and_grouping():
    fc = FakeCache(S=3, C=64)
    s = pac.Scheduler(fc.cache)
    assert s.max_sequence_length == 64
    for rid, p in [(10, 7), (11, 5), (12, 7), (13, 4)]:
        s.submit(rid, p, 3)
    adm, dec, ret = s.boundary()
    # FIFO into rows 0, 1, 2; listed by prompt length, then row
    assert adm == [(11, 1, 5), (10, 0, 7), (12, 2, 7)]
    assert dec == [] and ret == []
    assert s.counts() == (1, 3)
    run_plan(fc.cache, adm, dec)
    s.cancel(11)                       # active: leaves at the next boundary
    adm, dec, ret = s.boundary()
    assert ret == [(11, 1, CANCEL)]
    assert fc.cache.row_length(1) == 0  # reset on the way out
    assert dec == [(10, 0, 7), (12, 2, 7)]
    assert adm == [(13, 1, 4)]          # the lowest free row
    run_plan(fc.cache, adm, dec)
    adm, dec, ret = s.boundary()
    assert dec == [(10, 0, 8), (13, 1, 4), (12, 2, 8)] and adm == [] and ret == []


def test_retire_on_length_stop_and_zero_new_tokens():
    fc = FakeCache(S=2, C=32)
    s = pac.Scheduler(fc.cache, 20)
    s.submit(1, 5, 2)
    s.submit(2, 3, 0)                  # nothing to generate: done once prefilled
    adm, dec, ret = s.boundary()
    run_plan(fc.cache, adm, dec)
    adm, dec, ret = s.boundary()
    assert ret == [(2, 1, LENGTH)] and dec == [(1, 0, 5)]
    run_plan(fc.cache, adm, dec)
    adm, dec, ret = s.boundary()
    assert ret == [] and dec == [(1, 0, 6)]
    run_plan(fc.cache, adm, dec)       # row 0 now holds 5 + 2 positions
    adm, dec, ret = s.boundary()
    assert ret == [(1, 0, LENGTH)] and dec == []
    assert fc.cache.row_length(0) == 0 and s.counts() == (0, 0)
    s.submit(3, 4, 9)
    adm, _, _ = s.boundary()
    run_plan(fc.cache, adm, [])
    s.stop(3)
    adm, dec, ret = s.boundary()
    assert ret == [(3, 0, STOP)] and dec == []


def test_admission_only_at_boundaries():
    fc = FakeCache(S=2, C=32)
    s = pac.Scheduler(fc.cache)
    s.submit(1, 4, 1)
    assert s.counts() == (1, 0)
    adm, _, _ = s.boundary()
    assert [a[0] for a in adm] == [1]
    s.submit(2, 4, 1)                  # free row exists, but waits for the next boundary
    assert s.counts() == (1, 1)
    adm, _, _ = s.boundary()
    assert adm == [(2, 1, 4)]


def test_cancel_queued_and_errors():
    fc = FakeCache(S=1, C=16)
    s = pac.Scheduler(fc.cache, 12)
    s.submit(1, 4, 4)
    s.submit(2, 4, 4)
    s.cancel(2)                        # queued: removed at once
    assert s.counts() == (1, 0)
    adm, _, _ = s.boundary()
    assert adm == [(1, 0, 4)] and s.counts() == (0, 1)
    for args, name in [((3, 0, 1), "INVALID_ARG"), ((3, 1, -1), "INVALID_ARG"),
                       ((3, 9, 4), "OUT_OF_RANGE"), ((1, 2, 2), "INVALID_ARG")]:
        with pytest.raises(pac.MllmError) as e:
            s.submit(*args)
        assert e.value.name == name, args
    s.submit(3, 8, 4)                  # exactly max_sequence_length
    for f in (s.stop, s.cancel):
        with pytest.raises(pac.MllmError) as e:
            f(99)
        assert e.value.name == "INVALID_ARG"
    # plan arrays smaller than the slot count: rejected, nothing changed
    L = pac.load()
    a = (pac.SchedEntry * 1)()
    n = ctypes.c_int32()
    st = L.mllm_sched_boundary(s.handle, a, 0, ctypes.byref(n), a, 1, ctypes.byref(n), a, 1,
                               ctypes.byref(n))
    assert pac.STATUS[st] == "INVALID_ARG"
    assert s.counts() == (1, 1)


def test_boundary_refused_after_cache_free():
    fc = FakeCache(S=2, C=16)
    s = pac.Scheduler(fc.cache)
    s.submit(1, 4, 2)
    fc.cache.free()
    with pytest.raises(RuntimeError):
        s.boundary()


def test_create_rules():
    fc = FakeCache(S=2, C=16)
    with pytest.raises(pac.MllmError) as e:
        pac.Scheduler(fc.cache, 17)
    assert e.value.name == "OUT_OF_RANGE"
    fc.cache.set_row_length(1, 3)
    with pytest.raises(pac.MllmError) as e:
        pac.Scheduler(fc.cache)
    assert e.value.name == "ROW_BUSY"
    fc.cache.reset_row(1)
    assert pac.Scheduler(fc.cache, 0).max_sequence_length == 16
    with pytest.raises(pac.MllmError) as e:
        fc.cache.set_row_length(0, 17)
    assert e.value.name == "OUT_OF_RANGE"


class PolicyModel:
    """The pages' scheduler rules, stated plainly (test-side model)."""

    def __init__(self, slots, max_seq):
        self.slots, self.max_seq = slots, max_seq
        self.queue, self.reqs, self.rows = [], {}, [None] * slots

    def submit(self, rid, prompt, new):
        if prompt < 1 or new < 0:
            return "INVALID_ARG"
        if prompt + new > self.max_seq:
            return "OUT_OF_RANGE"
        if rid in self.reqs:
            return "INVALID_ARG"
        self.reqs[rid] = dict(prompt=prompt, new=new, row=None, planned=False, stop=False,
                              cancel=False)
        self.queue.append(rid)
        return "OK"

    def end(self, rid, cancel):
        if rid not in self.reqs:
            return "INVALID_ARG"
        if cancel and self.reqs[rid]["row"] is None:
            self.queue.remove(rid)
            del self.reqs[rid]
        else:
            self.reqs[rid]["cancel" if cancel else "stop"] = True
        return "OK"

    def boundary(self, lengths):
        retired = []
        for r, rid in enumerate(self.rows):
            if rid is None:
                continue
            q = self.reqs[rid]
            why = (CANCEL if q["cancel"] else STOP if q["stop"] else
                   LENGTH if q["planned"] and lengths[r] >= q["prompt"] + q["new"] else 0)
            if why:
                retired.append((rid, r, why))
                self.rows[r] = None
                del self.reqs[rid]
        decode = [(rid, r, lengths[r]) for r, rid in enumerate(self.rows)
                  if rid is not None and self.reqs[rid]["planned"]]
        admitted = []
        while self.queue and None in self.rows:
            rid = self.queue.pop(0)
            r = self.rows.index(None)
            self.rows[r] = rid
            self.reqs[rid]["row"] = r
            admitted.append((rid, r, self.reqs[rid]["prompt"]))
        admitted.sort(key=lambda e: (e[2], e[1]))
        for rid, _, _ in admitted:
            self.reqs[rid]["planned"] = True
        return admitted, decode, retired


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_trace_matches_policy(seed):
    rng = random.Random(seed)
    S, C, max_seq = 5, 64, 40
    fc = FakeCache(S=S, C=C)
    s = pac.Scheduler(fc.cache, max_seq)
    m = PolicyModel(S, max_seq)
    next_id, live = 0, []
    for step in range(600):
        for _ in range(rng.choice([0, 0, 1, 2, 3])):
            prompt = rng.choice([0, 1, 2, 5, 8, 13, 20, 33, 40])
            new = rng.choice([-1, 0, 1, 2, 4, 7, 12])
            rid = rng.choice(live) if live and rng.random() < 0.05 else next_id
            want = m.submit(rid, prompt, new)
            try:
                s.submit(rid, prompt, new)
                got = "OK"
            except pac.MllmError as e:
                got = e.name
            assert got == want, (step, rid, prompt, new)
            if got == "OK":
                live.append(rid)
                next_id += 1
        if live and rng.random() < 0.3:
            rid = rng.choice(live + [10 ** 9])
            cancel = rng.random() < 0.5
            want = m.end(rid, cancel)
            try:
                (s.cancel if cancel else s.stop)(rid)
                got = "OK"
            except pac.MllmError as e:
                got = e.name
            assert got == want
        lengths = [fc.cache.row_length(r) for r in range(S)]
        got = s.boundary()
        want = m.boundary(lengths)
        assert got == want, (step, got, want)
        for rid, _, _ in got[2]:
            live.remove(rid)
        for r in range(S):
            if m.rows[r] is None:
                assert fc.cache.row_length(r) == 0
        run_plan(fc.cache, got[0], got[1])
        q, a = s.counts()
        assert (q, a) == (len(m.queue), len(m.reqs) - len(m.queue))
