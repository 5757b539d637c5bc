"""The engine loop (scheduler + capture + compression on one stream beside
decode with append on another) replayed step by step on the CPU oracle.

Every input the GPU run drew (prefill rows, window queries, decode queries
and new K/V rows) is recorded; the replay applies the same plans to host
copies of the pools, the query rings and the global scores with the oracle's
functions. At every compression the GPU keep set must agree with the oracle's
scores (exact outside the 1e-4 band around the k-th score) and the attention
within its tolerance; the compaction is then applied with the GPU keep set so
the host pools follow the GPU's bit for bit. Every decode output must match the
oracle's attention over the host cache within 1e-4 relative + 1e-5. At the
end both pools must be byte-identical.
"""

import sys

import numpy as np
import pytest
import torch

import oracle as O
from kv_cache_compression_paged_amd.sim import Engine, EngineConfig
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _row(t):
    return [int(x) for x in t if x >= 0]


def test_engine_loop_replays_on_the_oracle():
    cfg = EngineConfig(layers=2, kv_heads=2, q_heads=4, head_dim=128, block_size=16,
                       n_max=4, window=8, num_blocks=26, query_slots=3, max_running=8,
                       max_blocks=12, seed=5)
    eng = Engine(cfg, record=True)
    group = eng.add_prefix(1)
    rng = np.random.default_rng(3)
    nreq = 12
    for rid in range(nreq):
        prompt = int(rng.integers(5, 60))
        gen = int(rng.integers(20, 110))
        g = group if rid % 4 == 0 else -1
        if g >= 0:
            prompt = max(prompt, cfg.block_size + 1)
        eng.submit(rid, prompt, gen, g)
    steps = eng.run(2000, nreq)
    st = eng.sched.stats()
    _say(f"[engine] {steps} steps: {st}")
    assert st["finished"] == nreq
    assert st["compressions"] > 0 and st["preemptions"] > 0

    L, H, b, d = cfg.layers, cfg.kv_heads, cfg.block_size, cfg.head_dim
    w, nmax, M = cfg.window, cfg.n_max, cfg.query_slots
    G = cfg.q_heads // H
    k = (nmax - 1) * b
    n_cap = cfg.max_blocks * b
    hk = np.zeros((L, cfg.num_blocks, H, b, d), dtype=np.uint16)
    hv = np.zeros_like(hk)
    for ids, kk, vv in eng.prefix_rows:
        hk[:, ids] = kk
        hv[:, ids] = vv
    ring = np.zeros((M, L, w, cfg.q_heads, d), dtype=np.uint16)
    glob = np.zeros((M, L, H, n_cap))
    oparams = O.Params(n_max=nmax, block_size=b, window=w)
    checked = dict(compress_units=0, decode_pairs=0, pinned=0)
    for si, rec in enumerate(eng.records):
        plan = rec.plan
        for s in plan.new_slot.tolist():
            ring[s] = 0
            glob[s] = 0.0
        for i, rid in enumerate(plan.admit_id.tolist()):
            length, shared = int(plan.admit_len[i]), int(plan.admit_shared[i])
            nb = (length + b - 1) // b
            ids = plan.admit_table[i, shared // b:nb]
            kk, vv, qs = rec.prefill[rid]
            hk[:, ids] = kk
            hv[:, ids] = vv
            if qs is not None:
                cnt = qs.shape[0]
                for j in range(cnt):
                    O.capture_queries(ring, qs[j], [int(plan.admit_slot[i])],
                                      [length - cnt + j], w)
        # compressions: host pools are the GPU's as of the step start
        src_k, src_v = hk.copy(), hv.copy()
        for i, rid in enumerate(plan.compress_id.tolist()):
            n, pos = int(plan.compress_len[i]), int(plan.compress_pos[i])
            slot, pinned = int(plan.compress_slot[i]), int(plan.compress_pinned[i])
            src, dst = _row(plan.compress_src[i]), plan.compress_dst[i].tolist()
            checked["pinned"] += int(pinned > 0)
            for l in range(L):
                qwin = O.window_from_ring(ring[slot, l], pos, w)      # [w][Hq][d]
                for h in range(H):
                    u = (i * L + l) * H + h
                    keys = O.widen(O.gather_rows(src_k, src, l, h, n, b), "bf16")
                    ur = O.score_unit(O.widen(qwin[:, h * G:(h + 1) * G], "bf16"), keys,
                                      glob[slot, l, h], n, pinned, oparams)
                    ga = rec.attn[u, :n].astype(np.float64)
                    assert np.all(np.abs(ga - ur.attn) <= P.ATTN_RTOL * np.abs(ur.attn)
                                  + P.ATTN_ATOL), (si, rid, l, h)
                    gk = rec.keep[u]
                    fin = np.isfinite(ur.score)
                    tau = min(float(ur.score[t]) for t in ur.keep if fin[t])
                    for t in set(gk.tolist()) ^ set(ur.keep.tolist()):
                        assert abs(ur.score[t] - tau) <= P.BAND, (si, rid, l, h, t)
                    O.compact_unit(src_k, hk, src, dst, l, h, gk, b)
                    O.compact_unit(src_v, hv, src, dst, l, h, gk, b)
                    g_new = O.update_global(glob[slot, l, h], ur.attn, gk, k)
                    gg = rec.glob_after[slot, l, h].astype(np.float64)
                    assert np.all(np.abs(gg - g_new) <= 1e-4 * np.abs(g_new) + 1e-6)
                    glob[slot, l, h] = g_new
                    checked["compress_units"] += 1
        # decode with append
        D = len(plan.decode_id)
        if D:
            O.capture_queries(ring, rec.q, plan.decode_slot.tolist(),
                              plan.decode_pos.tolist(), w)
            tables = [_row(r) for r in plan.decode_table]
            ref, hk, hv = O.paged_decode_append(rec.q, "bf16", rec.k_new, rec.v_new, hk, hv,
                                                "bf16", tables, plan.decode_len.tolist())
            got = rec.out.astype(np.float64)
            for (r, l), want in ref.items():
                err = np.abs(got[r, l] - want)
                assert np.all(err <= 1e-4 * np.abs(want) + 1e-5), (si, r, l, err.max())
                checked["decode_pairs"] += 1
    _say(f"[engine] replay checked {checked}")
    assert checked["pinned"] > 0
    assert np.array_equal(hk, eng.k_pool.cpu().view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(hv, eng.v_pool.cpu().view(torch.int16).numpy().view(np.uint16))
