"""Model-free engine loop around the library: hybrid scheduling driving the
compression and decode kernels on two streams.

Each step asks the native scheduler (``Scheduler``) for a plan and runs it:
  * admitted requests are prefilled: their K/V rows (and, for slot holders,
    the queries of their last prompt positions) are drawn at random, standing
    in for a model's prefill;
  * slots handed out this step get their query ring and global-score row
    cleared;
  * stream C compresses the plan's compress set (``zp_compress`` reading the
    query rings, with the global-score update in the same kernel);
  * stream D captures the decode set's new queries into the rings of slot
    holders (``zp_capture_queries``) and decodes one token per request with
    the new K/V row appended (``zp_paged_decode_append``);
  * both streams are joined and the scheduler commits the step.
The two streams touch disjoint blocks: compression writes only its own
requests' blocks and freshly popped targets, decode appends only into blocks
of the decode set, and blocks freed by a compression return to the free list
only when the step is committed ([zh] §2.1 asynchronous compression, [zh]
§2.2 hybrid scheduling).

All random inputs come from one seeded torch generator on the device. With
``record=True`` every step's inputs, plans and outputs are kept on the host,
so a test can replay the run.
"""

from __future__ import annotations

import time
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

from . import (ZP_BF16, ZP_OK, ZP_UPDATE_GLOBAL, ZP_WINDOW_RING, DeviceBatch, Scheduler,
               alloc_outputs, alloc_workspace, make_params, make_pool, zp_capture_queries,
               zp_compress, zp_paged_decode_append, zp_workspace_error)


@dataclass
class EngineConfig:
    layers: int
    kv_heads: int
    q_heads: int
    head_dim: int
    block_size: int
    n_max: int
    window: int
    num_blocks: int
    query_slots: int
    max_running: int
    max_blocks: int
    seed: int = 0
    # > 0: prefill copies rows from a bank of this many random blocks per
    # layer (fast set-up for long runs) instead of drawing every row
    prefill_bank_blocks: int = 0


@dataclass
class StepRecord:
    plan: object
    prefill: Dict[int, tuple] = field(default_factory=dict)   # id -> (k, v, q or None)
    q: Optional[np.ndarray] = None
    k_new: Optional[np.ndarray] = None
    v_new: Optional[np.ndarray] = None
    out: Optional[np.ndarray] = None
    keep: Optional[np.ndarray] = None
    attn: Optional[np.ndarray] = None
    glob_after: Optional[np.ndarray] = None


class Engine:
    def __init__(self, cfg: EngineConfig, device: str = "cuda", record: bool = False):
        import torch
        self.torch = torch
        self.cfg, self.dev, self.record = cfg, device, record
        c = cfg
        self.sched = Scheduler(c.num_blocks, c.block_size, c.n_max, c.window,
                               c.query_slots, c.max_running, c.max_blocks)
        shape = (c.layers, c.num_blocks, c.kv_heads, c.block_size, c.head_dim)
        self.k_pool = torch.zeros(shape, dtype=torch.bfloat16, device=device)
        self.v_pool = torch.zeros_like(self.k_pool)
        self.n_cap = c.max_blocks * c.block_size
        self.ring = torch.zeros((c.query_slots, c.layers, c.window, c.q_heads, c.head_dim),
                                dtype=torch.bfloat16, device=device)
        self.glob = torch.zeros((c.query_slots, c.layers, c.kv_heads, self.n_cap),
                                dtype=torch.float32, device=device)
        self.params = make_params(c.n_max, c.window, c.q_heads, ZP_BF16,
                                  flags=ZP_WINDOW_RING | ZP_UPDATE_GLOBAL)
        self.pool = make_pool(self.k_pool, self.v_pool)
        self.ws = alloc_workspace(self.pool, self.params, 1, device)
        self.gen = torch.Generator(device=device)
        self.gen.manual_seed(c.seed)
        self.sc, self.sd = torch.cuda.Stream(), torch.cuda.Stream()
        self.records: List[StepRecord] = []
        self.bank = None
        if c.prefill_bank_blocks > 0:
            self.bank = (self._randn((c.layers, c.prefill_bank_blocks, c.kv_heads,
                                      c.block_size, c.head_dim)),
                         self._randn((c.layers, c.prefill_bank_blocks, c.kv_heads,
                                      c.block_size, c.head_dim)))
        self.prefixes: List[np.ndarray] = []
        self.time = dict(compress_ms=0.0, decode_ms=0.0, step_ms=0.0)

    # ------------------------------------------------------------- inputs
    def _randn(self, shape):
        t = self.torch
        return t.randn(shape, generator=self.gen, device=self.dev).to(t.bfloat16)

    def add_prefix(self, blocks: int) -> int:
        """A cached shared prefix; its K/V rows are drawn now."""
        group, ids = self.sched.add_prefix(blocks)
        idx = self.torch.from_numpy(ids.astype(np.int64)).to(self.dev)
        c = self.cfg
        shape = (c.layers, blocks, c.kv_heads, c.block_size, c.head_dim)
        k, v = self._randn(shape), self._randn(shape)
        self.k_pool[:, idx] = k
        self.v_pool[:, idx] = v
        self.prefixes.append(ids)
        if self.record:
            self.prefix_rows = getattr(self, "prefix_rows", [])
            self.prefix_rows.append((ids.copy(), _raw(k), _raw(v)))
        return group

    def submit(self, req_id: int, prompt: int, gen: int, group: int = -1) -> None:
        self.sched.submit(req_id, prompt, gen, group)

    # --------------------------------------------------------------- step
    def step(self) -> object:
        t, c = self.torch, self.cfg
        t0 = time.perf_counter()
        plan = self.sched.step()
        rec = StepRecord(plan) if self.record else None
        cur = t.cuda.current_stream()
        for s in plan.new_slot.tolist():
            self.ring[s].zero_()
            self.glob[s].zero_()
        # prefill of admitted requests: K/V rows [shared, len), window queries
        for i, rid in enumerate(plan.admit_id.tolist()):
            length, shared, slot = (int(plan.admit_len[i]), int(plan.admit_shared[i]),
                                    int(plan.admit_slot[i]))
            nb = (length + c.block_size - 1) // c.block_size
            first = shared // c.block_size
            ids = plan.admit_table[i, first:nb].astype(np.int64)
            shape = (c.layers, nb - first, c.kv_heads, c.block_size, c.head_dim)
            if self.bank is not None and nb - first <= c.prefill_bank_blocks:
                off = int(t.randint(0, c.prefill_bank_blocks - (nb - first) + 1, (1,),
                                    generator=self.gen, device=self.dev).item())
                k = self.bank[0][:, off:off + nb - first]
                v = self.bank[1][:, off:off + nb - first]
            else:
                k, v = self._randn(shape), self._randn(shape)
            idx = t.from_numpy(ids).to(self.dev)
            self.k_pool[:, idx] = k
            self.v_pool[:, idx] = v
            qs = None
            if slot >= 0:
                cnt = min(c.window, length)
                qs = self._randn((cnt, 1, c.layers, c.q_heads, c.head_dim))
                slot_t = t.tensor([slot], dtype=t.int32, device=self.dev)
                for j in range(cnt):
                    pos = t.tensor([length - cnt + j], dtype=t.int32, device=self.dev)
                    zp_capture_queries(self.ring, qs[j], slot_t, pos, self.params, cur)
            if rec is not None:
                rec.prefill[rid] = (_raw(k), _raw(v), None if qs is None else _raw(qs))
        # everything the streams read is created on the current stream first
        e = [t.cuda.Event(enable_timing=True) for _ in range(4)]
        C, D = len(plan.compress_id), len(plan.decode_id)
        out_c = batch = None
        if C:
            U = C * c.layers * c.kv_heads
            k_keep = (c.n_max - 1) * c.block_size
            out_c = alloc_outputs(U, k_keep, self.n_cap, self.dev, debug=False)
            batch = DeviceBatch(
                slot=_dev(plan.compress_slot, self.dev), n_tokens=_dev(plan.compress_len, self.dev),
                src_table=_dev(plan.compress_src, self.dev),
                dst_table=_dev(plan.compress_dst, self.dev),
                n_pinned=_dev(plan.compress_pinned, self.dev), num_slots=c.query_slots,
                n_cap=self.n_cap, seq_pos=_dev(plan.compress_pos, self.dev))
        out_d = None
        if D:
            q = self._randn((D, c.layers, c.q_heads, c.head_dim))
            k_new = self._randn((D, c.layers, c.kv_heads, c.head_dim))
            v_new = self._randn((D, c.layers, c.kv_heads, c.head_dim))
            out_d = t.empty((D, c.layers, c.q_heads, c.head_dim), dtype=t.float32,
                            device=self.dev)
            d_slot, d_pos = _dev(plan.decode_slot, self.dev), _dev(plan.decode_pos, self.dev)
            d_tab, d_len = _dev(plan.decode_table, self.dev), _dev(plan.decode_len, self.dev)
            if rec is not None:
                rec.q, rec.k_new, rec.v_new = _raw(q), _raw(k_new), _raw(v_new)
        ready = t.cuda.Event()
        ready.record(cur)
        self.sc.wait_event(ready)
        self.sd.wait_event(ready)
        if C:
            e[0].record(self.sc)
            zp_compress(self.pool, batch, self.ring, self.glob, self.params, out_c, self.ws,
                        self.sc)
            e[1].record(self.sc)
        if D:
            e[2].record(self.sd)
            zp_capture_queries(self.ring, q, d_slot, d_pos, self.params, self.sd)
            zp_paged_decode_append(out_d, q, k_new, v_new, self.pool, d_tab, d_len,
                                   self.params, self.sd)
            e[3].record(self.sd)
        t.cuda.synchronize()
        if C:
            self.time["compress_ms"] += e[0].elapsed_time(e[1])
        if D:
            self.time["decode_ms"] += e[2].elapsed_time(e[3])
        if zp_workspace_error(self.ws) != ZP_OK:
            raise RuntimeError("device error in the engine step")
        if rec is not None:
            if D:
                rec.out = out_d.cpu().numpy()
            if C:
                rec.keep = out_c.keep_idx.cpu().numpy()
                rec.attn = out_c.attn.cpu().numpy()
                rec.glob_after = self.glob.cpu().numpy()
            self.records.append(rec)
        self.sched.complete()
        self.time["step_ms"] += (time.perf_counter() - t0) * 1e3
        return plan

    def run(self, max_steps: int, total: int) -> int:
        """Step until `total` requests finished (or max_steps); returns steps."""
        for i in range(max_steps):
            self.step()
            if self.sched.stats()["finished"] >= total:
                return i + 1
        return max_steps


def _dev(a: np.ndarray, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def _raw(t) -> np.ndarray:
    """Stored bits of a bf16 tensor as uint16 (host)."""
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
