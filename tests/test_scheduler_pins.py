"""Pins of the hybrid-scheduling reference model on its own (CPU only).

The model (oracle/scheduler_ref.py) follows the policy the pages state in
words ([zh] §2.2, [de] §2 Scheduling-Strategien, [fr] §2.B; asynchronous
compression [zh] §2.1, [fr] §2.D). It is pinned here without the library:

  * hand-derived step plans for five tiny pools (tests/golden/
    scheduler_traces.json): basic decoding and compression, preemption of
    slot-free requests, restricted steps, the slot-free stop at N_max*b - w
    and compression into a target block after a shared prefix;
  * invariants checked on the model over seeded workloads: only the first M
    running requests hold slots; only slot-free requests are preempted,
    newest first; a step is restricted only when no slot-free request is
    left; every block is free or held, with counts equal to its holders; no
    compression without w captured queries (counted from the plans); FIFO
    admission with preempted requests at the front; decode and compression
    lengths within the trigger rules;
  * planted mistakes in the model, each caught by one of the above.
"""

import json
import os
from collections import deque
from unittest import mock

import numpy as np
import pytest

import oracle.scheduler_ref as SR
import oracle.zipage_ref as ZR
from oracle.scheduler_ref import Scheduler

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "scheduler_traces.json")


def _load():
    with open(GOLDEN) as f:
        return json.load(f)["scenarios"]


def _plan_rows(p):
    return {
        "restricted": bool(p.restricted),
        "admitted": [[a["id"], a["len"], a["slot"], a["table"], a["shared"]]
                     for a in p.admitted],
        "new_slots": list(p.new_slots),
        "decode": [[d["id"], d["slot"], d["len"], d["pos"], d["table"]] for d in p.decode],
        "compress": [[c["id"], c["slot"], c["len"], c["pos"], c["src"], c["dst"], c["pinned"]]
                     for c in p.compress],
        "preempted": list(p.preempted),
    }


def _expected_rows(step):
    return {
        "restricted": step.get("restricted", False),
        "admitted": step.get("admitted", []),
        "new_slots": step.get("new_slots", []),
        "decode": step.get("decode", []),
        "compress": step.get("compress", []),
        "preempted": step.get("preempted", []),
    }


def _run_golden(sc):
    c = sc["config"]
    m = Scheduler(c["num_blocks"], c["b"], c["n_max"], c["w"], c["slots"], c["max_running"])
    for blocks in sc["prefixes"]:
        m.add_prefix(blocks)
    for rid, prompt, gen, group in sc["requests"]:
        m.submit(rid, prompt, gen, group)
    for i, step in enumerate(sc["steps"]):
        got = _plan_rows(m.step())
        want = _expected_rows(step)
        assert got == want, f"{sc['name']}: step {i}\n got  {got}\n want {want}"
        m.complete()
    for key, val in sc["stats"].items():
        assert m.stats[key] == val, f"{sc['name']}: stats[{key}] {m.stats[key]} != {val}"
    assert m.pool.stack == sc["free_stack"], sc["name"]
    return m


@pytest.mark.parametrize("idx", range(5))
def test_golden_trace(idx):
    _run_golden(_load()[idx])


def test_golden_traces_cover_every_branch():
    sc = _load()
    steps = [s for x in sc for s in x["steps"]]
    assert any(s.get("preempted") for s in steps)
    assert any(s.get("restricted") for s in steps)
    assert any(c[6] > 0 for s in steps for c in s.get("compress", []))
    assert any(s.get("new_slots") and not s.get("admitted") for s in steps)


# ------------------------------------------------------------ invariants ---

WORKLOADS = [
    # seed, blocks, b, n_max, w, M, max_running, requests, prompt range,
    # gen range, prefix groups (blocks), long prompts
    (21, 400, 16, 8, 8, 4, 16, 24, (5, 60), (20, 200), [], False),
    (22, 70, 16, 6, 8, 3, 20, 30, (5, 40), (40, 160), [], False),
    (1, 16, 16, 6, 8, 3, 20, 14, (5, 40), (20, 70), [], False),    # restricted steps
    (24, 160, 16, 8, 8, 4, 12, 20, (40, 90), (30, 150), [2, 3], False),
    (25, 220, 16, 8, 4, 5, 10, 16, (20, 150), (10, 90), [], True),
    (26, 12, 16, 4, 16, 1, 8, 12, (3, 30), (20, 80), [1], False),
    (27, 40, 4, 5, 6, 2, 8, 20, (2, 15), (10, 60), [], False),   # w > b
    (28, 30, 4, 4, 3, 2, 6, 14, (2, 12), (8, 40), [2], False),
]


class Invariants:
    """Runs the model and checks every step; the checks use the plans and the
    model's public state only."""

    def __init__(self, wl):
        (seed, nb, b, n_max, w, M, maxrun, nreq, prange, grange, prefixes, longp) = wl
        self.nb, self.b, self.n_max, self.w, self.M = nb, b, n_max, w, M
        rng = np.random.default_rng(seed)
        self.m = Scheduler(nb, b, n_max, w, M, maxrun)
        self.prefix_blocks = []
        groups = []
        for pb in prefixes:
            g, ids = self.m.add_prefix(pb)
            self.prefix_blocks += ids
            groups.append((g, pb))
        self.queue = deque()
        for rid in range(nreq):
            prompt = int(rng.integers(*prange))
            if longp and rid % 4 == 1:
                prompt = n_max * b + int(rng.integers(1, 40))
            gen = int(rng.integers(*grange))
            group = -1
            if groups and rid % 3 == 0:
                group, pb = groups[rid % len(groups)]
                prompt = max(prompt, pb * b + 1)
            self.m.submit(rid, prompt, gen, group)
            self.queue.append(rid)
        self.nreq = nreq
        self.captured = {}
        self.slot_of = {}
        self.seen = dict(preempt=0, restricted=0, compress=0, late_slot=0)

    def step(self):
        m = self.m
        trig = self.n_max * self.b
        before = list(m.running)
        plan = m.step()
        # S1: slot holders are exactly the first M running requests
        holders = {r for r in m.running if m.reqs[r].slot >= 0}
        assert holders == set(m.running[:self.M]), "slots not on the first M"
        slots = [m.reqs[r].slot for r in holders]
        assert len(set(slots)) == len(slots), "a slot held twice"
        # S5: preempted requests were slot-free, newest first
        pos = {r: i for i, r in enumerate(before)}
        for r in plan.preempted:
            assert r in pos and m.reqs[r].slot < 0, "a slot holder was preempted"
        order = [pos[r] for r in plan.preempted]
        assert order == sorted(order, reverse=True), "preemption not newest first"
        if plan.preempted:
            # a request preempted for its own block can be re-admitted in the
            # same step (its blocks came back): it is not a survivor
            oldest_cut = min(order)
            readmitted = {a["id"] for a in plan.admitted}
            for r in m.running:
                if r in pos and r not in readmitted and m.reqs[r].slot < 0:
                    assert pos[r] < oldest_cut, "a newer slot-free request survived"
        # restricted only when no slot-free request is left to preempt
        if plan.restricted:
            assert all(m.reqs[r].slot >= 0 for r in m.running), "restricted with a slot-free request"
            assert not plan.admitted
        # FIFO admission, preempted requests back at the front
        for r in plan.preempted:
            self.queue.appendleft(r)
        for a in plan.admitted:
            assert self.queue.popleft() == a["id"], "admission out of FIFO order"
        # the captured-query count, derived from the plans alone
        for a in plan.admitted:
            self.slot_of[a["id"]] = a["slot"]
            self.captured[a["id"]] = min(self.w, a["len"]) if a["slot"] >= 0 else 0
        for row in plan.decode + plan.compress:
            rid = row["id"]
            if row["slot"] >= 0 and self.slot_of.get(rid, -1) < 0:
                self.captured[rid] = 0           # slot handed out this step
                self.seen["late_slot"] += 1
            self.slot_of[rid] = row["slot"]
        for c in plan.compress:
            assert c["slot"] >= 0 and c["len"] >= trig
            assert self.captured[c["id"]] >= self.w, "compressed without a full window"
            table = c["src"]
            S = 0
            while S < self.n_max - 1 and m.pool.refcount[table[S]] > 1:
                S += 1
            assert c["pinned"] == S
        for d in plan.decode:
            limit = trig if d["slot"] >= 0 else trig - self.w
            assert d["len"] < limit, "decoded past the slot rule"
            assert len(d["table"]) * self.b >= d["len"] + 1
        ids = [d["id"] for d in plan.decode] + [c["id"] for c in plan.compress]
        assert len(ids) == len(set(ids)), "a request both decodes and compresses"
        m.complete()
        for d in plan.decode:
            if d["slot"] >= 0:
                self.captured[d["id"]] = self.captured.get(d["id"], 0) + 1
        for r in plan.preempted:
            self.slot_of[r] = -1
        self.seen["preempt"] += len(plan.preempted)
        self.seen["restricted"] += int(plan.restricted)
        self.seen["compress"] += len(plan.compress)
        self._check_blocks()

    def _check_blocks(self):
        m = self.m
        held = [0] * self.nb
        for r in m.running:
            for bid in m.reqs[r].table:
                held[bid] += 1
        for bid in self.prefix_blocks:
            held[bid] += 1
        assert m.pool.refcount == held, "refcounts differ from the holders"
        assert sorted(m.pool.stack) == [i for i in range(self.nb) if held[i] == 0]

    def run(self, max_steps=4000):
        for _ in range(max_steps):
            self.step()
            if self.m.stats["finished"] == self.nreq:
                return True
        return False


@pytest.mark.parametrize("wl", WORKLOADS, ids=[f"seed{w[0]}" for w in WORKLOADS])
def test_invariants_on_seeded_workloads(wl):
    inv = Invariants(wl)
    assert inv.run(), "not every request finished"
    assert not inv.m.running and not inv.m.waiting


def test_invariant_workloads_take_every_branch():
    seen = dict(preempt=0, restricted=0, late_slot=0, compress=0)
    for wl in WORKLOADS:
        inv = Invariants(wl)
        inv.run()
        for k in seen:
            seen[k] += inv.seen[k]
    assert all(v > 0 for v in seen.values()), seen


# -------------------------------------------------------- planted mistakes ---

def _slots_to_last_m(self):
    return self.running[-self.M:]


def _stop_one_late(self):
    return self.n_max * self.b - self.w + 1


def _stop_at_trigger(self):
    # the pages' wording without the window rule: decode until N_max blocks
    # are full -- a request that gets its slot then has no captured window
    return self.n_max * self.b


def _preempt_any(self, plan, skip):
    for rid in reversed(self.running):
        if rid in skip:
            continue
        r = self.reqs[rid]
        self._release(r.table)
        r.table, r.n = [], 0
        if r.slot >= 0:
            self.free_slots.add(r.slot)
            r.slot = -1
        self.running.remove(rid)
        self.waiting.appendleft(rid)
        plan.preempted.append(rid)
        self.stats["preemptions"] += 1
        return rid
    return None


def _preempt_oldest(self, plan, skip):
    for rid in list(self.running):
        r = self.reqs[rid]
        if r.slot >= 0 or rid in skip:
            continue
        self._release(r.table)
        r.table, r.n = [], 0
        self.running.remove(rid)
        self.waiting.appendleft(rid)
        plan.preempted.append(rid)
        self.stats["preemptions"] += 1
        return rid
    return None


def _fifo_alloc(self, n):
    if n > len(self.stack):
        raise MemoryError("free list exhausted")
    out = [self.stack.pop(0) for _ in range(n)]
    for bid in out:
        self.refcount[bid] = 1
    return out


def _caught(patches):
    """True when a golden trace or an invariant fails under the patches."""
    with contextlib_exit(patches):
        for sc in _load():
            try:
                _run_golden(sc)
            except (AssertionError, MemoryError, KeyError, ValueError):
                return True
        for wl in WORKLOADS:
            try:
                Invariants(wl).run(max_steps=600)
            except (AssertionError, MemoryError, KeyError, ValueError):
                return True
    return False


class contextlib_exit:
    def __init__(self, patches):
        self.patches = patches

    def __enter__(self):
        for p in self.patches:
            p.start()

    def __exit__(self, *exc):
        for p in reversed(self.patches):
            p.stop()
        return False


MUTANTS = [
    ("slots to the last M running", lambda: [mock.patch.object(Scheduler, "_slot_holders", _slots_to_last_m)]),
    ("slot-free stop one token late", lambda: [mock.patch.object(Scheduler, "_slot_free_stop", _stop_one_late)]),
    ("slot-free decode up to the trigger", lambda: [mock.patch.object(Scheduler, "_slot_free_stop", _stop_at_trigger)]),
    ("a slot holder preempted", lambda: [mock.patch.object(Scheduler, "_preempt_latest", _preempt_any)]),
    ("oldest slot-free request preempted", lambda: [mock.patch.object(Scheduler, "_preempt_latest", _preempt_oldest)]),
    ("FIFO free list", lambda: [mock.patch.object(ZR.BlockPool, "alloc", _fifo_alloc)]),
]


def test_the_real_model_passes_every_pin():
    assert not _caught([])


@pytest.mark.parametrize("name,make", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_scheduler_mistake_is_caught(name, make):
    assert _caught(make()), f"'{name}' slipped past the golden traces and invariants"
