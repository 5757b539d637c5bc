"""Reference model of hybrid scheduling (host policy, no GPU).

TEST INFRASTRUCTURE ONLY: used by the tests to check the library's native
scheduler decision by decision. It shares no code with the library.

The pages describe the policy in words ([zh] §2.2 hybrid scheduling, [de] §2
scheduling strategies, [fr] §2.B; asynchronous compression [zh] §2.1,
[fr] §2.D):
  * only the first M running requests receive query slots for compression;
  * requests that hold fewer than N_max blocks, or whose last block still has
    room, decode without a slot;
  * when no block can be allocated, requests without a slot are preempted
    first; once none is left the system falls back to a restricted mode;
  * compression runs beside decoding: requests that need no compression do
    not wait, compressed requests rejoin the decode steps afterwards.

Readings taken where the words leave the mechanics open (each is one rule
below):
  S1 slot holders are the first M running requests in admission order; a
     slot, once held, stays until the request finishes;
  S2 a request needs its last w queries captured before it compresses, so a
     slot-free request stops decoding once its cache reaches N_max*b - w
     tokens and waits for a slot; slot holders capture every decoded token,
     and an admitted slot holder has its prompt's last min(w, len) queries.
     This is stricter than the pages, which let a slot-free request decode
     until it holds N_max blocks and its last block is full ([de] §2,
     [zh] §2.2): it stops w tokens earlier (for w > b, whole blocks
     earlier), because a request that got its slot only at the trigger
     would hold no captured window to score with;
  S3 a slot holder compresses in the step after its cache reaches N_max*b
     tokens (or at admission, for a longer prompt), provided it has w
     captured queries; it does not decode in that step;
  S4 a shared-prefix compression needs N_max-1-S target blocks; slot-free
     requests are preempted for them; if still short, no request compresses
     this step and the step is restricted;
  S5 decode order is admission order; a token at a block boundary takes one
     block; when none is free the most recently admitted slot-free running
     request (possibly the requester) is preempted: its blocks are released,
     it goes to the front of the waiting queue and will be prefilled again
     with prompt + generated tokens; with no such request left the requester
     waits and the step is restricted;
  S6 admission is FIFO and stops at the first request that does not fit: it
     needs ceil(len/b) blocks minus its group's cached prefix, and a prompt of
     at least N_max*b - w tokens needs a slot (admitted only while fewer than M
     requests run); nothing is admitted in a restricted step;
  S7 free slots are handed out lowest first; the free list is the oracle's
     LIFO block pool.
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field
from typing import Dict, List, Optional

from .zipage_ref import BlockPool


@dataclass
class _Req:
    rid: int
    prompt: int
    gen: int
    group: int
    generated: int = 0
    n: int = 0
    seq: int = 0
    slot: int = -1
    captured: int = 0
    table: List[int] = field(default_factory=list)


@dataclass
class StepPlan:
    restricted: bool
    admitted: List[dict]        # id, len, slot, table, shared (tokens)
    new_slots: List[int]
    decode: List[dict]          # id, slot, len, pos, table
    compress: List[dict]        # id, slot, len, pos, src, dst, pinned
    preempted: List[int]


class Scheduler:
    def __init__(self, num_blocks: int, b: int, n_max: int, w: int, slots: int,
                 max_running: int):
        self.pool = BlockPool(num_blocks)
        self.b, self.n_max, self.w, self.M = b, n_max, w, slots
        self.max_running = max_running
        self.reqs: Dict[int, _Req] = {}
        self.running: List[int] = []
        self.waiting: deque = deque()
        self.free_slots = set(range(slots))
        self.prefixes: List[List[int]] = []
        self._pending = None
        self.stats = dict(steps=0, tokens=0, compressions=0, preemptions=0,
                          restricted_steps=0, admitted=0, finished=0)

    # --------------------------------------------------------------- setup
    def add_prefix(self, blocks: int) -> (int, List[int]):
        ids = self.pool.alloc(blocks)
        self.prefixes.append(ids)
        return len(self.prefixes) - 1, ids

    def submit(self, rid: int, prompt: int, gen: int, group: int = -1) -> None:
        self.reqs[rid] = _Req(rid, prompt, gen, group)
        self.waiting.append(rid)

    # ------------------------------------------------------------ helpers
    def _slot_holders(self) -> List[int]:
        """S1: the first M running requests, in admission order."""
        return self.running[:self.M]

    def _slot_free_stop(self) -> int:
        """S2: a request without a slot decodes only below this many tokens."""
        return self.n_max * self.b - self.w

    def _release(self, table: List[int]) -> None:
        for bid in table:
            self.pool.refcount[bid] -= 1
            if self.pool.refcount[bid] == 0:
                self.pool.stack.append(bid)

    def _take_slot(self) -> int:
        s = min(self.free_slots)
        self.free_slots.remove(s)
        return s

    def _preempt_latest(self, plan: StepPlan, skip: set) -> Optional[int]:
        for rid in reversed(self.running):
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

    # --------------------------------------------------------------- step
    def step(self) -> StepPlan:
        assert self._pending is None, "previous step not completed"
        b, w, nmax = self.b, self.w, self.n_max
        trig = nmax * b
        plan = StepPlan(False, [], [], [], [], [])
        # S1: slots for the first M running requests
        for rid in self._slot_holders():
            r = self.reqs[rid]
            if r.slot < 0:
                r.slot, r.captured = self._take_slot(), 0
                plan.new_slots.append(r.slot)
        # S3/S4: compressions
        comp = [rid for rid in self.running
                if self.reqs[rid].slot >= 0 and self.reqs[rid].n >= trig
                and self.reqs[rid].captured >= w]
        skip = set(comp)
        bm_plan = None
        if comp:
            need = 0
            for rid in comp:
                sb = self.pool.shared_prefix(self.reqs[rid].table, nmax)
                need += (nmax - 1 - sb) if sb > 0 else 0
            while len(self.pool.stack) < need:
                if self._preempt_latest(plan, skip) is None:
                    break
            if len(self.pool.stack) < need:
                plan.restricted = True
                skip.clear()
                comp = []
        skip.update(plan.preempted)
        if comp:
            bm_plan = self.pool.plan_compress([self.reqs[rid].table for rid in comp],
                                              [self.reqs[rid].n for rid in comp], nmax, b)
            for i, rid in enumerate(comp):
                r = self.reqs[rid]
                plan.compress.append(dict(id=rid, slot=r.slot, len=r.n, pos=r.seq,
                                          src=list(r.table),
                                          dst=[int(x) for x in bm_plan.dst_tables[i]],
                                          pinned=int(bm_plan.n_pinned[i])))
        # S2/S5: decoding
        dec: List[int] = []
        for rid in list(self.running):
            if rid in skip:
                continue
            r = self.reqs[rid]
            if r.slot < 0 and r.n >= self._slot_free_stop():
                continue
            if r.slot >= 0 and r.n >= trig:
                continue
            if r.n == len(r.table) * b:          # the token opens a block
                while not self.pool.stack:
                    v = self._preempt_latest(plan, skip)
                    if v is None:
                        break
                    skip.add(v)
                    if v in dec:
                        dec.remove(v)
                    if v == rid:
                        break
                if rid in skip:
                    continue
                if not self.pool.stack:
                    plan.restricted = True
                    continue
                r.table.extend(self.pool.alloc(1))
            dec.append(rid)
        for rid in dec:
            r = self.reqs[rid]
            plan.decode.append(dict(id=rid, slot=r.slot, len=r.n, pos=r.seq,
                                    table=list(r.table)))
        # S6: admission
        while (not plan.restricted and self.waiting
               and len(self.running) < self.max_running):
            q = self.reqs[self.waiting[0]]
            length = q.prompt + q.generated
            shared = len(self.prefixes[q.group]) if q.group >= 0 else 0
            need = (length + b - 1) // b - shared
            gets_slot = len(self.running) < self.M
            if length >= self._slot_free_stop() and not gets_slot:
                break
            if need > len(self.pool.stack):
                break
            self.waiting.popleft()
            q.table = []
            for bid in (self.prefixes[q.group] if q.group >= 0 else []):
                self.pool.incref(bid)
                q.table.append(bid)
            q.table.extend(self.pool.alloc(need))
            q.n = q.seq = length
            self.running.append(q.rid)
            if gets_slot:
                q.slot = self._take_slot()
                q.captured = min(w, length)
                plan.new_slots.append(q.slot)
            else:
                q.slot, q.captured = -1, 0
            plan.admitted.append(dict(id=q.rid, len=length, slot=q.slot,
                                      table=list(q.table), shared=shared * b))
            self.stats["admitted"] += 1
        self.stats["steps"] += 1
        self.stats["restricted_steps"] += int(plan.restricted)
        self._pending = (plan, bm_plan)
        return plan

    def complete(self) -> None:
        plan, bm_plan = self._pending
        nmax, b = self.n_max, self.b
        if bm_plan is not None:
            self.pool.commit(bm_plan)
            for c in plan.compress:
                r = self.reqs[c["id"]]
                r.table = list(c["dst"])
                r.n = (nmax - 1) * b
                self.stats["compressions"] += 1
        for d in plan.decode:
            r = self.reqs[d["id"]]
            r.n += 1
            r.seq += 1
            r.generated += 1
            if r.slot >= 0:
                r.captured += 1
            self.stats["tokens"] += 1
            if r.generated >= r.gen:
                self._release(r.table)
                r.table = []
                if r.slot >= 0:
                    self.free_slots.add(r.slot)
                r.slot, r.captured = -1, 0
                self.running.remove(r.rid)
                self.stats["finished"] += 1
        self._pending = None
