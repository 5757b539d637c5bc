"""The library's hybrid scheduler against the reference model, step by step.

Seeded workloads sized so that every branch of the policy is taken: query
slots handed out and freed, slot-free decoding and waiting for a slot,
compressions in place, after a prefill overshoot and with a shared prefix
(target blocks), preemption of slot-free requests (including the requester
itself) and restricted steps. Every field of every plan must agree exactly,
and so must the final counters. CPU only (no GPU calls).
"""

import numpy as np
import pytest

import kv_cache_compression_paged_amd as Z
from oracle.scheduler_ref import Scheduler as RefScheduler


def _rows(tab):
    return [[int(x) for x in row if x >= 0] for row in tab]


def _compare(step, got, want):
    where = f"step {step}"
    assert got.restricted == want.restricted, where
    assert got.preempt_id.tolist() == want.preempted, where
    assert got.new_slot.tolist() == want.new_slots, where
    assert got.admit_id.tolist() == [a["id"] for a in want.admitted], where
    assert got.admit_len.tolist() == [a["len"] for a in want.admitted], where
    assert got.admit_slot.tolist() == [a["slot"] for a in want.admitted], where
    assert got.admit_shared.tolist() == [a["shared"] for a in want.admitted], where
    assert _rows(got.admit_table) == [a["table"] for a in want.admitted], where
    assert got.decode_id.tolist() == [d["id"] for d in want.decode], where
    assert got.decode_slot.tolist() == [d["slot"] for d in want.decode], where
    assert got.decode_len.tolist() == [d["len"] for d in want.decode], where
    assert got.decode_pos.tolist() == [d["pos"] for d in want.decode], where
    assert _rows(got.decode_table) == [d["table"] for d in want.decode], where
    assert got.compress_id.tolist() == [c["id"] for c in want.compress], where
    assert got.compress_slot.tolist() == [c["slot"] for c in want.compress], where
    assert got.compress_len.tolist() == [c["len"] for c in want.compress], where
    assert got.compress_pos.tolist() == [c["pos"] for c in want.compress], where
    assert _rows(got.compress_src) == [c["src"] for c in want.compress], where
    assert got.compress_dst.tolist() == [c["dst"] for c in want.compress], where
    assert got.compress_pinned.tolist() == [c["pinned"] for c in want.compress], where


WORKLOADS = [
    # name, seed, blocks, b, n_max, w, M, max_running, requests, prompt range,
    # gen range, prefix groups (blocks), long prompts
    ("roomy", 11, 400, 16, 8, 8, 4, 16, 24, (5, 60), (20, 200), [], False),
    ("tight: preemption", 12, 70, 16, 6, 8, 3, 20, 30, (5, 40), (40, 160), [], False),
    # fewer blocks than M * N_max: slot holders outgrow the pool for a while
    # and the step runs restricted until one of them finishes
    ("starved: restricted steps", 1, 16, 16, 6, 8, 3, 20, 14, (5, 40), (20, 70), [],
     False),
    ("shared prefixes", 13, 160, 16, 8, 8, 4, 12, 20, (40, 90), (30, 150), [2, 3], False),
    ("long prompts overshoot", 14, 220, 16, 8, 4, 5, 10, 16, (20, 150), (10, 90), [], True),
    ("one slot, small pool", 15, 12, 16, 4, 16, 1, 8, 12, (3, 30), (20, 80), [1], False),
]


@pytest.mark.parametrize("wl", WORKLOADS, ids=[w[0] for w in WORKLOADS])
def test_scheduler_matches_reference(wl):
    (name, seed, nb, b, n_max, w, M, maxrun, nreq, prange, grange, prefixes, longp) = wl
    rng = np.random.default_rng(seed)
    max_blocks = 24
    lib_s = Z.Scheduler(nb, b, n_max, w, M, maxrun, max_blocks)
    ref = RefScheduler(nb, b, n_max, w, M, maxrun)
    groups = []
    for pb in prefixes:
        g1, ids1 = lib_s.add_prefix(pb)
        g2, ids2 = ref.add_prefix(pb)
        assert g1 == g2 and ids1.tolist() == ids2
        groups.append((g1, pb))
    for rid in range(nreq):
        prompt = int(rng.integers(*prange))
        if longp and rid % 4 == 1:
            prompt = n_max * b + int(rng.integers(1, 40))       # prefill overshoot
        gen = int(rng.integers(*grange))
        gen = min(gen, max_blocks * b - prompt)
        group = -1
        if groups and rid % 3 == 0:
            group, pb = groups[rid % len(groups)]
            prompt = max(prompt, pb * b + 1)
        lib_s.submit(rid, prompt, gen, group)
        ref.submit(rid, prompt, gen, group)
    seen = dict(compress=0, preempt=0, restricted=0, pinned=0, overshoot=0, wait=0)
    for step in range(3000):
        got, want = lib_s.step(), ref.step()
        _compare(step, got, want)
        seen["compress"] += len(want.compress)
        seen["preempt"] += len(want.preempted)
        seen["restricted"] += int(want.restricted)
        seen["pinned"] += sum(1 for c in want.compress if c["pinned"] > 0)
        seen["overshoot"] += sum(1 for c in want.compress if c["len"] > n_max * b)
        lib_s.complete()
        ref.complete()
        st = lib_s.stats()
        if st["finished"] == nreq:
            break
    st = lib_s.stats()
    assert st["finished"] == nreq, f"not all requests finished: {st}"
    for key in ("steps", "tokens", "compressions", "preemptions", "restricted_steps",
                "admitted", "finished"):
        assert st[key] == ref.stats[key], key
    assert seen["compress"] > 0
    if "preemption" in name or "small" in name:
        assert seen["preempt"] > 0, seen
    if "restricted" in name:
        assert seen["restricted"] > 0, seen
    if prefixes:
        assert seen["pinned"] > 0, seen
    if longp:
        assert seen["overshoot"] > 0, seen
    # every block is back: prefixes stay cached, nothing else is held
    assert st["running"] == 0 and st["waiting"] == 0
    assert st["free_blocks"] == nb - sum(prefixes)


def test_scheduler_rejects_bad_use():
    s = Z.Scheduler(64, 16, 4, 8, 2, 4, 8)
    with pytest.raises(Z.ZipageError):
        s.submit(0, 100, 100)                  # beyond max_blocks * b
    with pytest.raises(Z.ZipageError):
        s.submit(0, 10, 10, group=3)           # no such prefix group
    s.submit(0, 10, 10)
    with pytest.raises(Z.ZipageError):
        s.submit(0, 10, 10)                    # id already used
    with pytest.raises(Z.ZipageError):
        s.complete()                           # nothing pending
    s.step()
    with pytest.raises(Z.ZipageError):
        s.step()                               # previous step not completed
    s.complete()
    with pytest.raises(Z.ZipageError):
        Z.Scheduler(64, 16, 4, 100, 2, 4, 8)   # window beyond n_max * b
    with pytest.raises(Z.ZipageError):
        Z.Scheduler(64, 1 << 16, 4, 8, 2, 4, 1 << 16)   # lengths past int32 range
