"""GPU parity of the split-unit schedule (ZP_SPLIT_UNITS), where one unit's
key slices are scored by up to 8 workgroups that exchange row normalisers and
eviction candidates, against the CPU oracle.

The cases are sized so that units really span several slices (512 tokens,
256 with 192 window rows): 8 parts, a ragged last part, E larger than a slice,
slices wholly pinned by a shared prefix, all tokens tied, evictions on slice
boundaries, and enough units that every group exchange slot is reused. Each
goes through tests/parity.py (every unit element by element, pools byte for
byte); a few run again without the flag, on the one-workgroup schedule.
"""

import sys

import numpy as np
import pytest
import torch

import kv_cache_compression_paged_amd as Z
from kv_cache_compression_paged_amd import synth
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


SPLIT = Z.ZP_SPLIT_UNITS


def _check(case, label):
    _say(f"[split] {label}: {case.spec} flags={case.flags}")
    res = P.run_case(case)
    _say(f"[split] {label}: ok={res.ok} stats={res.stats}")
    assert res.ok, "\n".join(res.failures)


# 8 parts of 512 tokens (w*G = 128)
FULL = synth.scaled(synth.EIGHT_B, requests=2, layers=1, kv_heads=2, q_heads=8,
                    n_max=256, pool_blocks=2 * 256 + 8)
# 192 window rows: 8 parts of 256 tokens
ROWS192 = synth.scaled(synth.SMALL, requests=1, layers=1, n_max=128,
                       pool_blocks=128 + 8)
D64 = synth.scaled(FULL, head_dim=64, near_dup=False)
PREFIX = synth.scaled(synth.PREFIX, requests=2, layers=1, kv_heads=2, q_heads=8,
                      n_max=256, groups=1, shared_blocks=40,
                      pool_blocks=40 + 2 * 216 + 2 * 215 + 5)
OVER = synth.scaled(FULL, n_max=200, pool_blocks=2 * 200 + 8 + 48)


def _forced_global(spec, positions):
    g = np.zeros((spec.requests, spec.layers, spec.kv_heads, spec.n_tokens))
    g[..., list(positions)] = -100.0
    return g


CASES = [
    ("8 parts", P.Case(FULL, flags=SPLIT)),
    ("4 parts, ragged last slice", P.Case(synth.scaled(FULL, n_max=100, pool_blocks=208),
                                          flags=SPLIT)),
    ("overshoot, E = 616 > slice", P.Case(OVER, flags=SPLIT,
                                          n_tokens=[OVER.n_tokens + 600, OVER.n_tokens + 37],
                                          max_blocks=OVER.n_max + 38)),
    ("overshoot, tail slice inside the causal window", P.Case(
        synth.scaled(synth.EIGHT_B, requests=3, layers=2, kv_heads=2, q_heads=8, n_max=32,
                     pool_blocks=112 + 12),
        flags=SPLIT, n_tokens=[512 + 5, 512 + 16, 512 + 37], max_blocks=35)),
    ("192 rows, 8 parts of 256", P.Case(ROWS192, flags=SPLIT)),
    ("head_dim 64, 8 parts", P.Case(D64, flags=SPLIT)),
    ("shared prefix over 1.25 slices", P.Case(PREFIX, flags=SPLIT, use_block_manager=True)),
    ("non-causal, protected window", P.Case(
        FULL, flags=SPLIT | Z.ZP_NONCAUSAL | Z.ZP_PROTECT_WINDOW)),
    ("evict block 0: every later row shifts",
     P.Case(FULL, flags=SPLIT, global_override=_forced_global(FULL, range(16)))),
    ("evictions on slice boundaries",
     P.Case(FULL, flags=SPLIT, global_override=_forced_global(
         FULL, [511, 512, 1023, 1024, 1535, 2047, 2048, 2559, 3071, 3072, 3583, 3584,
                4079, 4080, 4094, 4095]))),
    ("outlier key x100", P.Case(synth.scaled(FULL, requests=1), flags=SPLIT,
                                outlier=(700, 100.0))),
]


@pytest.mark.parametrize("label,case", CASES, ids=[c[0] for c in CASES])
def test_split_schedule(label, case):
    _check(case, label)


@pytest.mark.parametrize("label,case", [CASES[0], CASES[2], CASES[5]],
                         ids=[CASES[i][0] for i in (0, 2, 5)])
def test_single_workgroup_schedule(label, case):
    c = P.Case(**{**case.__dict__, "flags": case.flags & ~SPLIT})
    _check(c, label + " (one workgroup per unit)")


def test_all_tokens_tied():
    # identical keys, constant global scores, no mask: every score is equal,
    # every token of every slice is a candidate (the union holds all 4096),
    # and the first k positions are kept
    spec = synth.scaled(FULL, requests=1)
    g = np.full((1, 1, spec.kv_heads, spec.n_tokens), 0.25)
    case = P.Case(spec, flags=SPLIT | Z.ZP_NONCAUSAL, identical_keys=True, global_override=g)
    _check(case, "all tokens tied")


def test_exchange_slots_reused():
    # 320 units of 2 parts over at most 128 groups: every group's exchange
    # slot serves several units in a row
    spec = synth.scaled(synth.EIGHT_B, requests=10, layers=4, n_max=64,
                        pool_blocks=10 * 64 + 8)
    _check(P.Case(spec, flags=SPLIT), "320 units, exchange slots reused")


def test_fused_global_update_is_bit_identical_split():
    """ZP_UPDATE_GLOBAL in the split schedule: each part updates the global
    scores of its own kept tokens; the result equals zp_compress followed by
    zp_update_global bit for bit, and so do pools, keep sets and attention."""
    case = P.Case(OVER, flags=SPLIT, n_tokens=[OVER.n_tokens + 600, OVER.n_tokens + 37],
                  max_blocks=OVER.n_max + 38)
    spec = case.spec
    wl, glob, host, dev, tables, dst, pinned, n_tok, _ = P.build_inputs(case)
    R, L, H = spec.requests, spec.layers, spec.kv_heads
    U, k = R * L * H, spec.keep
    zparams, _ = P._params_for(spec, SPLIT)
    fparams, _ = P._params_for(spec, SPLIT | Z.ZP_UPDATE_GLOBAL)
    res = []
    for fused in (False, True):
        kp, vp, g = wl.k_pool.clone(), wl.v_pool.clone(), glob.clone()
        pool = Z.make_pool(kp, vp)
        out = Z.alloc_outputs(U, k, dev.n_cap, "cuda")
        ws = Z.alloc_workspace(pool, zparams, R, "cuda")
        if fused:
            Z.zp_compress(pool, dev, wl.q_window, g, fparams, out, ws)
        else:
            Z.zp_compress(pool, dev, wl.q_window, g, zparams, out, ws)
            Z.zp_update_global(g, pool, dev, out, zparams)
        torch.cuda.synchronize()
        assert Z.zp_workspace_error(ws) == Z.ZP_OK
        res.append((kp, vp, g, out))
    (k1, v1, g1, o1), (k2, v2, g2, o2) = res
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    assert torch.equal(g1.view(torch.int32), g2.view(torch.int32))
    assert torch.equal(o1.keep_idx, o2.keep_idx)
    for u in range(U):
        nu = int(n_tok[u // (L * H)])
        assert torch.equal(o1.attn[u, :nu].view(torch.int32), o2.attn[u, :nu].view(torch.int32))
    _say("[split] fused global update: bit-identical")


def test_small_workspace_takes_the_one_workgroup_schedule():
    """With ZP_SPLIT_UNITS a 256-byte workspace is still accepted: the call
    runs the one-workgroup schedule, with the same results."""
    case = P.Case(synth.scaled(FULL, requests=1))
    spec = case.spec
    wl, glob, host, dev, tables, dst, pinned, n_tok, _ = P.build_inputs(case)
    U, k = spec.layers * spec.kv_heads, spec.keep
    zparams, _ = P._params_for(spec, SPLIT)
    keeps = []
    for ws_bytes in (256, None):
        kp, vp, g = wl.k_pool.clone(), wl.v_pool.clone(), glob.clone()
        pool = Z.make_pool(kp, vp)
        out = Z.alloc_outputs(U, k, dev.n_cap, "cuda")
        ws = (torch.zeros(64, dtype=torch.int32, device="cuda") if ws_bytes
              else Z.alloc_workspace(pool, zparams, 1, "cuda"))
        Z.zp_compress(pool, dev, wl.q_window, g, zparams, out, ws)
        torch.cuda.synchronize()
        assert Z.zp_workspace_error(ws) == Z.ZP_OK
        keeps.append((out.keep_idx.clone(), kp, vp))
    # the two schedules sum attention in different orders; on this seeded
    # input no score lies near the threshold, so keep sets and bytes agree
    assert torch.equal(keeps[0][0], keeps[1][0])
    assert torch.equal(keeps[0][1], keeps[1][1]) and torch.equal(keeps[0][2], keeps[1][2])


def _random_split_case(seed):
    """Seeded random shapes for the split schedule: up to 8 slices per unit
    (n_max up to 256), 1 to 12 query heads per KV head, windows up to the
    192-row limit, head_dim 64 or 128, overshoot up to 90 tokens, either
    mask, the protected window and shared prefixes, all inside the split
    schedule's limits (n_cap <= 4096 for up to 128 window rows, else 2048)."""
    rng = np.random.default_rng(77_000 + seed)
    prefix = rng.random() < 0.3
    d = int(rng.choice([64, 128]))
    hkv = int(rng.integers(1, 3))
    G = int(rng.choice([1, 2, 4, 6, 8, 12]))
    w_cap = 192 // G
    w = int(rng.integers(1, min(64, w_cap) + 1))
    cap = 4096 if w * G <= 128 else 2048
    over_max = 90
    n_max = int(rng.integers(2, (cap - over_max) // 16 + 1))
    w = min(w, n_max * 16)
    flags = SPLIT | int(rng.choice([0, Z.ZP_NONCAUSAL]))
    protect = rng.random() < 0.3 and w <= (n_max - 1) * 16
    if prefix:
        groups = 1
        R = 2
        s_max = n_max - 1 - ((w + 15) // 16 if protect else 0)
        if s_max < 1:
            protect = False
            s_max = n_max - 1
        S = int(rng.integers(1, s_max + 1))
    else:
        groups, R, S = 1, int(rng.integers(1, 3)), 0
    if protect:
        flags |= Z.ZP_PROTECT_WINDOW
    over = [int(x) for x in rng.integers(0, over_max + 1, size=R)] if rng.random() < 0.4 else [0] * R
    extra = sum((n_max * 16 + e + 15) // 16 - n_max for e in over)
    if prefix:
        pool = groups * S + R * (n_max - S) + extra + R * (n_max - 1 - S) + 4
        base = synth.PREFIX
    else:
        pool = R * n_max + extra + 2
        base = synth.EIGHT_B
    spec = synth.scaled(base, name=f"split_{seed}", seed=7000 + seed, requests=R, layers=1,
                        kv_heads=hkv, q_heads=hkv * G, head_dim=d, n_max=n_max, window=w,
                        groups=groups, shared_blocks=S, pool_blocks=pool, permute=True,
                        near_dup=True)
    n = spec.n_tokens
    return P.Case(spec, flags=flags, n_tokens=[n + e for e in over],
                  max_blocks=n_max + 6, use_block_manager=prefix)


@pytest.mark.parametrize("seed", range(48))
def test_random_split_shapes(seed):
    case = _random_split_case(seed)
    s = case.spec
    _check(case, f"random split shape {seed}: n_max {s.n_max}, d {s.head_dim}, "
                 f"G {s.q_heads // s.kv_heads}, w {s.window}, S {s.shared_blocks}, "
                 f"n {case.n_tokens}")


def test_wait_limit_reports_esync_and_the_workspace_recovers(monkeypatch):
    """With the exchange waits limited to zero polls (ZP_SPLIT_SPIN_LIMIT=0,
    read by the host at each call), a workgroup that finds a partner's words
    missing gives up at once, raises the abort flag and returns; every other
    workgroup returns at its next unready wait. The call ends normally with
    ZP_ESYNC in the error word. The same workspace then serves a call at the
    default limit, whose results equal those of a fresh workspace bit for bit."""
    spec = synth.scaled(FULL, requests=4, layers=2, pool_blocks=4 * 256 + 8)
    case = P.Case(spec)
    wl, glob, host, dev, tables, dst, pinned, n_tok, _ = P.build_inputs(case)
    R, L, H = spec.requests, spec.layers, spec.kv_heads
    U, k = R * L * H, spec.keep
    zparams, _ = P._params_for(spec, SPLIT)
    shared_ws = None

    def run(limit, ws=None):
        kp, vp, g = wl.k_pool.clone(), wl.v_pool.clone(), glob.clone()
        pool = Z.make_pool(kp, vp)
        out = Z.alloc_outputs(U, k, dev.n_cap, "cuda")
        ws = ws if ws is not None else Z.alloc_workspace(pool, zparams, R, "cuda")
        if limit is None:
            monkeypatch.delenv("ZP_SPLIT_SPIN_LIMIT", raising=False)
        else:
            monkeypatch.setenv("ZP_SPLIT_SPIN_LIMIT", str(limit))
        Z.zp_compress(pool, dev, wl.q_window, g, zparams, out, ws)
        torch.cuda.synchronize()
        return Z.zp_workspace_error(ws), ws, (kp, vp, out.keep_idx)

    seen = []
    for attempt in range(3):
        err, shared_ws, _ = run(0, shared_ws)
        seen.append(err)
        _say(f"[split] zero-poll wait limit, attempt {attempt}: status {err}")
        assert err in (Z.ZP_ESYNC, Z.ZP_OK)
        if err == Z.ZP_ESYNC:
            break
    assert Z.ZP_ESYNC in seen, f"no wait gave up: {seen}"
    err1, _, (k1, v1, keep1) = run(None, shared_ws)
    err2, _, (k2, v2, keep2) = run(None)
    assert err1 == Z.ZP_OK and err2 == Z.ZP_OK
    assert torch.equal(keep1, keep2)
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    _say("[split] ZP_ESYNC reported; the workspace serves the next call unchanged")


def test_split_schedule_beside_decode_on_another_stream():
    """The two-stream case on the split-unit schedule: 8 query-slot holders
    (4 layers x 8 KV heads of the 8B-like layout) compress on stream C with
    ZP_SPLIT_UNITS and the global update fused, while the other 24 requests
    decode one token on stream D, so the persistent split grid shares the
    device with decode workgroups. Every compressed unit is checked (keep =
    top k of its own scores, rows against an untouched copy, global rows bit
    for bit), 6 of them against the oracle, and 16 decode pairs against the
    oracle's attention."""
    import oracle as O
    from tests import fullsize as F
    spec = synth.scaled(synth.OVERLAP, requests=32, layers=4, groups=4,
                        compress_groups=4, pool_blocks=32 * 256)
    dev = "cuda"
    per = 8
    wl = synth.make(spec, device=dev, slots=per)
    L, H, b = spec.layers, spec.kv_heads, spec.block_size
    n, k = spec.n_tokens, spec.keep
    G = spec.q_heads // H
    grp, rest = np.arange(per), np.arange(per, spec.requests)
    tab_c = torch.from_numpy(np.ascontiguousarray(wl.tables[grp])).to(dev)
    tab_d = torch.from_numpy(np.ascontiguousarray(wl.tables[rest])).to(dev)
    rng = np.random.default_rng(41)
    lens = rng.integers(k + 1, n, size=rest.size).astype(np.int32)
    q = synth.decode_queries(spec, rest.size, dev, 42)
    zparams, oparams = P._params_for(spec, SPLIT | Z.ZP_UPDATE_GLOBAL)
    pool = Z.make_pool(wl.k_pool, wl.v_pool)
    batch = Z.DeviceBatch(
        slot=torch.arange(per, dtype=torch.int32, device=dev),
        n_tokens=torch.full((per,), n, dtype=torch.int32, device=dev),
        src_table=tab_c, dst_table=tab_c.clone(),
        n_pinned=torch.zeros(per, dtype=torch.int32, device=dev),
        num_slots=per, n_cap=wl.n_cap)
    Uc = per * L * H
    out = Z.alloc_outputs(Uc, k, wl.n_cap, dev, debug=True)
    ws = Z.alloc_workspace(pool, zparams, per, dev)
    assert ws.numel() * ws.element_size() > 256          # the split schedule runs
    k0, v0, g0 = wl.k_pool.clone(), wl.v_pool.clone(), wl.global_scores.clone()
    qwin = synth.raw_numpy(wl.q_window)
    dec = torch.full((rest.size, L, spec.q_heads, spec.head_dim), float("nan"),
                     dtype=torch.float32, device=dev)
    sc, sd = torch.cuda.Stream(), torch.cuda.Stream()
    ready = torch.cuda.Event()
    ready.record(torch.cuda.current_stream())
    sc.wait_event(ready)
    sd.wait_event(ready)
    _say(f"[split] two streams: {Uc} units split on C, {rest.size} requests decode on D")
    Z.zp_compress(pool, batch, wl.q_window, wl.global_scores, zparams, out, ws, sc)
    Z.zp_paged_decode(dec, q, pool, tab_d, torch.from_numpy(lens).to(dev), zparams, sd)
    torch.cuda.synchronize()
    assert Z.zp_workspace_error(ws) == Z.ZP_OK
    F.check_keep_is_topk_of_own_scores(out.keep_idx, out.score, n)
    F.check_global_rows(wl.global_scores, g0, out.keep_idx, out.attn, range(per), L, H)
    F.check_rows_against_copy(wl.k_pool, k0, tab_c, batch.dst_table, out.keep_idx, n,
                              spec.n_max, in_place=True, what="K")
    F.check_rows_against_copy(wl.v_pool, v0, tab_c, batch.dst_table, out.keep_idx, n,
                              spec.n_max, in_place=True, what="V")
    hk = synth.raw_numpy(k0)
    for u in sorted(set(int(x) for x in rng.choice(Uc, 6, replace=False)) | {0, Uc - 1}):
        r, l, h = u // (L * H), (u // H) % L, u % H
        keys = O.widen(O.gather_rows(hk, wl.tables[r], l, h, n, b), spec.dtype)
        ur = O.score_unit(O.widen(qwin[r, l, :, h * G:(h + 1) * G], spec.dtype), keys,
                          g0[r, l, h].cpu().numpy().astype(np.float64), n, 0, oparams)
        ga = out.attn[u, :n].cpu().numpy().astype(np.float64)
        assert np.all(np.abs(ga - ur.attn) <= P.ATTN_RTOL * np.abs(ur.attn) + P.ATTN_ATOL)
        diff = set(out.keep_idx[u].cpu().numpy().tolist()) ^ set(ur.keep.tolist())
        fin = np.isfinite(ur.score)
        tau = min(float(ur.score[t]) for t in ur.keep if fin[t])
        assert all(abs(ur.score[t] - tau) <= P.BAND for t in diff)
    qh = synth.raw_numpy(q)
    got = dec.cpu().numpy().astype(np.float64)
    hv = synth.raw_numpy(v0)
    for i in rng.choice(rest.size, 4, replace=False):
        for l in range(L):
            r = int(rest[i])
            for h in range(H):
                kr = O.gather_rows(hk, wl.tables[r], l, h, int(lens[i]), b)
                vr = O.gather_rows(hv, wl.tables[r], l, h, int(lens[i]), b)
                want = O.decode_attention(O.widen(qh[i, l, h * G:(h + 1) * G], spec.dtype),
                                          O.widen(kr, spec.dtype), O.widen(vr, spec.dtype))
                err = np.abs(got[i, l, h * G:(h + 1) * G] - want)
                assert np.all(err <= 1e-4 * np.abs(want) + 1e-5), (r, l, h, err.max())
    _say("[split] two streams: compressed units and decode pairs match")
