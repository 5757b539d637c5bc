"""GPU parity of query-window capture and of compression reading a ring window.

Capture is a byte copy, so it is compared bit for bit with the oracle's
ring after every decode step. A compression that reads its window through
the ring (ZP_WINDOW_RING) must give bit-identical outputs and pools to the
same compression handed the window in position order, which the parity
suite checks against the oracle.
"""

import sys

import numpy as np
import pytest
import torch

import oracle as O
import kv_cache_compression_paged_amd as Z
from kv_cache_compression_paged_amd import synth
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_capture_matches_oracle_over_decode_steps(dtype, d):
    dev = "cuda"
    R, L, Hq, w, S = 6, 3, 8, 5, 4
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    slot = np.array([0, 2, -1, 1, 7, 3], dtype=np.int32)   # -1: no slot, 7: out of range
    pos = np.array([0, 3, 4, 9, 1, 40], dtype=np.int32)
    ring = torch.zeros((S, L, w, Hq, d), dtype=tdt, device=dev)
    ring_ref = synth.raw_numpy(ring).copy()
    params = Z.make_params(4, w, Hq, Z.ZP_BF16 if dtype == "bf16" else Z.ZP_F32)
    gen = torch.Generator(device=dev)
    gen.manual_seed(21)
    for step in range(2 * w + 3):
        q = torch.randn((R, L, Hq, d), generator=gen, device=dev).to(tdt)
        p = pos + step
        p[5] = -1 if step == 2 else p[5]                    # a negative position
        Z.zp_capture_queries(ring, q, torch.from_numpy(slot).to(dev),
                             torch.from_numpy(p).to(dev), params)
        O.capture_queries(ring_ref, synth.raw_numpy(q), slot, p, w)
        torch.cuda.synchronize()
        assert synth.raw_numpy(ring).tobytes() == ring_ref.tobytes(), f"step {step}"
    _say(f"[capture] {dtype} d={d}: {2 * w + 3} steps bit-exact")


def _linear_to_ring(q_window, seq, slots, w):
    """Ring layout of a linear window: the query of sequence position
    P-w+i (P = seq[r], the next token's position) goes to row (P-w+i) mod w."""
    ring = torch.empty_like(q_window)
    for r, s in enumerate(slots):
        P = int(seq[r])
        idx = torch.tensor([(P - w + i) % w for i in range(w)], device=q_window.device)
        ring[s, :, idx] = q_window[s]
    return ring


@pytest.mark.parametrize("flags,shift", [(0, 0), (Z.ZP_NONCAUSAL, 0), (0, 16), (0, 37),
                                         (Z.ZP_SPLIT_UNITS, 0), (Z.ZP_SPLIT_UNITS, 37)])
def test_ring_window_compression_is_bit_identical(flags, shift):
    """shift > 0: the sequence is ahead of the cache (earlier compressions
    evicted tokens), so the ring is indexed by seq_pos, not n. With
    ZP_SPLIT_UNITS the units span 4 slices of 512 tokens, and every part
    reads the window rows out of the ring itself."""
    n_max = 100 if flags & Z.ZP_SPLIT_UNITS else 20
    spec = synth.scaled(synth.EIGHT_B, requests=3, layers=2, kv_heads=2, q_heads=8,
                        n_max=n_max, pool_blocks=3 * n_max + 3 * 3)
    n = spec.n_tokens
    case = P.Case(spec, n_tokens=[n, n + 7, n + 21], max_blocks=spec.n_max + 2)
    wl, glob, host, dev, tables, dst, pinned, n_tok, _ = P.build_inputs(case)
    zparams, _ = P._params_for(spec, flags)
    rparams, _ = P._params_for(spec, flags | Z.ZP_WINDOW_RING)
    R, L, H = spec.requests, spec.layers, spec.kv_heads
    U, k = R * L * H, spec.keep
    seq = np.asarray(n_tok) + shift
    ring = _linear_to_ring(wl.q_window, seq, wl.slots, spec.window)
    ring_batch = Z.DeviceBatch(slot=dev.slot, n_tokens=dev.n_tokens,
                               src_table=dev.src_table, dst_table=dev.dst_table,
                               n_pinned=dev.n_pinned, num_slots=dev.num_slots,
                               n_cap=dev.n_cap,
                               seq_pos=(torch.from_numpy(seq.astype(np.int32)).cuda()
                                        if shift else None))
    results = []
    for qw, prm, bt in ((wl.q_window, zparams, dev), (ring, rparams, ring_batch)):
        kp, vp, g = wl.k_pool.clone(), wl.v_pool.clone(), glob.clone()
        pool = Z.make_pool(kp, vp)
        out = Z.alloc_outputs(U, k, dev.n_cap, "cuda", debug=True)
        ws = Z.alloc_workspace(pool, prm, R, "cuda")
        Z.zp_compress(pool, bt, qw, g, prm, out, ws)
        Z.zp_update_global(g, pool, bt, out, prm)
        torch.cuda.synchronize()
        assert Z.zp_workspace_error(ws) == Z.ZP_OK
        results.append((kp, vp, g, out))
    (k1, v1, g1, o1), (k2, v2, g2, o2) = results
    assert torch.equal(k1, k2) and torch.equal(v1, v2) and torch.equal(g1, g2)
    assert torch.equal(o1.keep_idx, o2.keep_idx)
    assert torch.equal(o1.first_hole, o2.first_hole)
    for name in ("attn", "red", "score"):    # entries [0, n) of each unit are defined
        a, b = getattr(o1, name), getattr(o2, name)
        for u in range(U):
            nu = int(n_tok[u // (L * H)])
            assert torch.equal(a[u, :nu].view(torch.int32), b[u, :nu].view(torch.int32)), \
                (name, u)
    _say("[capture] ring window compression bit-identical to the linear window")


def test_capture_then_compress_end_to_end():
    """Queries captured step by step on the GPU feed a ring-window compression
    whose attention matches the oracle's over the same queries in order."""
    spec = synth.scaled(synth.EIGHT_B, requests=2, layers=2, kv_heads=2, q_heads=8,
                        n_max=12, pool_blocks=2 * 12)
    case = P.Case(spec)
    wl, glob, host, dev, tables, dst, pinned, n_tok, _ = P.build_inputs(case)
    R, L, H, b = spec.requests, spec.layers, spec.kv_heads, spec.block_size
    w, n, k = spec.window, spec.n_tokens, spec.keep
    G = spec.q_heads // H
    zparams, oparams = P._params_for(spec, Z.ZP_WINDOW_RING)
    ring = torch.zeros_like(wl.q_window)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    seq = []
    slots = torch.from_numpy(wl.slots).cuda()
    for p in range(n - w - 3, n):          # a few extra steps wrap the ring
        q = torch.randn((R, L, spec.q_heads, spec.head_dim), generator=gen,
                        device="cuda").to(torch.bfloat16)
        seq.append(synth.raw_numpy(q))
        Z.zp_capture_queries(ring, q, slots,
                             torch.full((R,), p, dtype=torch.int32, device="cuda"),
                             zparams)
    pool = Z.make_pool(wl.k_pool, wl.v_pool)
    U = R * L * H
    out = Z.alloc_outputs(U, k, dev.n_cap, "cuda", debug=True)
    ws = Z.alloc_workspace(pool, zparams, R, "cuda")
    Z.zp_compress(pool, dev, ring, glob, zparams, out, ws)
    torch.cuda.synchronize()
    assert Z.zp_workspace_error(ws) == Z.ZP_OK
    last_w = np.stack(seq[-w:])            # [w][R][L][Hq][d], positions n-w..n-1
    for r in range(R):
        for l in range(L):
            for h in range(H):
                u = (r * L + l) * H + h
                keys = O.widen(O.gather_rows(host["k"], tables[r], l, h, n, b), spec.dtype)
                q_lin = O.widen(last_w[:, r, l, h * G:(h + 1) * G], spec.dtype)
                ur = O.score_unit(q_lin, keys, host["g"][r, l, h].astype(np.float64),
                                  n, 0, oparams)
                ga = out.attn[u, :n].cpu().numpy().astype(np.float64)
                assert np.all(np.abs(ga - ur.attn) <= P.ATTN_RTOL * np.abs(ur.attn)
                              + P.ATTN_ATOL), (r, l, h)
