"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small cases compare every unit element by element (see tests/parity.py for
the rules); the full-size cases run the exact launch configuration bench.py
times and compare a seeded sample of units one by one, plus properties that
hold for every unit.
"""

import sys

import numpy as np
import pytest
import torch

import oracle as O
import kv_cache_compression_paged_amd as Z
from kv_cache_compression_paged_amd import synth
from tests import fullsize as F
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check(case, label):
    _say(f"[parity] {label}: {case.spec}")
    res = P.run_case(case)
    _say(f"[parity] {label}: ok={res.ok} stats={res.stats}")
    assert res.ok, "\n".join(res.failures)


# ---------------------------------------------------------------- small ---

SMALL_MODEL = synth.scaled(synth.SMALL, requests=2, layers=2, n_max=16,
                           pool_blocks=48)
EIGHT_B = synth.scaled(synth.EIGHT_B, requests=3, layers=2, kv_heads=2,
                       q_heads=8, n_max=32, pool_blocks=112)
PREFIX = synth.scaled(synth.PREFIX, requests=4, layers=2, kv_heads=2,
                      q_heads=8, n_max=12, groups=2, shared_blocks=3,
                      pool_blocks=6 + 4 * 9 + 4 * 8 + 5)
D64 = synth.scaled(synth.EIGHT_B, requests=2, layers=1, kv_heads=2, q_heads=4,
                   head_dim=64, n_max=20, window=16, pool_blocks=48,
                   near_dup=False)
F32_D128 = synth.scaled(synth.TINY, requests=2, layers=1, kv_heads=1,
                        q_heads=2, head_dim=128, n_max=10, window=16,
                        pool_blocks=24, permute=True)


def test_tiny_fp32_full_config():
    _check(P.Case(synth.TINY), "tiny fp32 (d=64, G=2, w=8)")


def test_small_model_shape():
    _check(P.Case(SMALL_MODEL), "G=6, w=32 (192 window rows)")


def test_8b_shape_near_duplicates():
    _check(P.Case(EIGHT_B), "G=4, w=32, near-duplicate keys")


def test_noncausal():
    _check(P.Case(EIGHT_B, flags=Z.ZP_NONCAUSAL), "non-causal window")


def test_protect_window():
    _check(P.Case(EIGHT_B, flags=Z.ZP_PROTECT_WINDOW), "protected window")


def test_bf16_head_dim_64():
    _check(P.Case(D64), "bf16 d=64")


def test_fp32_head_dim_128():
    _check(P.Case(F32_D128), "fp32 d=128")


LONG = synth.scaled(synth.EIGHT_B, requests=1, layers=1, kv_heads=2,
                    q_heads=8, n_max=1024, pool_blocks=1024 + 8)


def test_long_context_takes_the_short_ring():
    # 16384 tokens: the token rows (64 KiB) no longer fit beside the default
    # 7-slot key ring in LDS, so the launcher picks the 5-slot ring
    _check(P.Case(LONG), "n = 16384 (5-slot ring)")


def test_long_context_fp32_d64():
    # fp32 rows of head_dim 64 are 4 KiB blocks as well: 16384 tokens take
    # the 5-slot ring in that element type too
    spec = synth.scaled(synth.TINY, requests=1, layers=1, kv_heads=2, q_heads=4,
                        n_max=1024, window=16, pool_blocks=1024 + 8, permute=True)
    _check(P.Case(spec), "fp32 d=64, n = 16384 (5-slot ring)")


def test_long_context_window_rows_192():
    # the largest window (w*G = 192) beside 16384 token rows: the 5-slot
    # ring's static LDS is largest here and must still fit
    spec = synth.scaled(synth.SMALL, requests=1, layers=1, n_max=1024,
                        pool_blocks=1024 + 8)
    _check(P.Case(spec), "192 window rows, n = 16384 (5-slot ring)")


def test_fp32_d128_n_cap_beyond_lds_is_rejected():
    # fp32 keys with head_dim 128 take 8 KiB per block: token rows of 8192
    # entries do not fit in LDS beside the ring; the call must refuse and
    # leave every buffer untouched
    spec = synth.scaled(F32_D128, requests=1, n_max=512, pool_blocks=512 + 4)
    wl = synth.make(spec, device="cuda")
    zparams, _ = P._params_for(spec, 0)
    pool = Z.make_pool(wl.k_pool, wl.v_pool)
    dev = "cuda"
    batch = Z.DeviceBatch(
        slot=torch.from_numpy(wl.slots).to(dev),
        n_tokens=torch.from_numpy(wl.n_tokens).to(dev),
        src_table=torch.from_numpy(wl.tables).to(dev),
        dst_table=torch.from_numpy(wl.tables).to(dev),
        n_pinned=torch.zeros(spec.requests, dtype=torch.int32, device=dev),
        num_slots=spec.requests, n_cap=wl.n_cap)
    U = spec.units
    out = Z.alloc_outputs(U, spec.keep, wl.n_cap, dev, debug=True)
    out.attn.fill_(7.0)
    ws = Z.alloc_workspace(pool, zparams, spec.requests, dev)
    k_before = wl.k_pool.clone()
    with pytest.raises(Z.ZipageError) as ei:
        Z.zp_compress(pool, batch, wl.q_window, wl.global_scores, zparams, out, ws)
    assert ei.value.status == Z.ZP_EUNSUPPORTED
    torch.cuda.synchronize()
    assert bool((out.attn == 7.0).all())
    assert torch.equal(k_before, wl.k_pool)


def test_prefill_overshoot_ragged_tail():
    spec = synth.scaled(EIGHT_B, requests=3, pool_blocks=112 + 12)
    n = spec.n_tokens
    _check(P.Case(spec, n_tokens=[n + 5, n + 16, n + 37], max_blocks=spec.n_max + 3),
           "overshoot n = N+5, N+16, N+37 (E > b, ragged last block)")


def test_prefix_targets_with_block_manager():
    _check(P.Case(PREFIX, use_block_manager=True),
           "shared prefix -> target blocks (plans from zp_bm)")


# The launcher runs units of at most 512 KiB of keys as two 4-wave
# workgroups per CU (2 key groups) and larger ones as one 8-wave workgroup
# (4 key groups); ZIPAGE_KEY_GROUPS forces either, so both workgroup shapes
# are compared with the oracle on the same inputs.
SHAPE_CASES = [
    ("tiny fp32", lambda: P.Case(synth.TINY)),
    ("192 window rows", lambda: P.Case(SMALL_MODEL)),
    ("near duplicates", lambda: P.Case(EIGHT_B)),
    ("non-causal", lambda: P.Case(EIGHT_B, flags=Z.ZP_NONCAUSAL)),
    ("protected window", lambda: P.Case(EIGHT_B, flags=Z.ZP_PROTECT_WINDOW)),
    ("bf16 d=64", lambda: P.Case(D64)),
    ("fp32 d=128", lambda: P.Case(F32_D128)),
    ("overshoot", lambda: P.Case(synth.scaled(EIGHT_B, requests=3, pool_blocks=112 + 12),
                                 n_tokens=[EIGHT_B.n_tokens + e for e in (5, 16, 37)],
                                 max_blocks=EIGHT_B.n_max + 3)),
    ("shared prefix", lambda: P.Case(PREFIX, use_block_manager=True)),
    ("fused update", lambda: P.Case(EIGHT_B, flags=Z.ZP_UPDATE_GLOBAL)),
    ("16384 tokens", lambda: P.Case(LONG)),
]


@pytest.mark.parametrize("kg", ["2", "4"], ids=["2-groups", "4-groups"])
@pytest.mark.parametrize("label,make", SHAPE_CASES, ids=[c[0] for c in SHAPE_CASES])
def test_both_workgroup_shapes(kg, label, make, monkeypatch):
    monkeypatch.setenv("ZIPAGE_KEY_GROUPS", kg)
    _check(make(), f"{label}, {kg} key groups")


@pytest.mark.parametrize("kg", ["2", "4"], ids=["2-groups", "4-groups"])
@pytest.mark.parametrize("seed", range(12))
def test_random_shapes_both_workgroup_shapes(kg, seed, monkeypatch):
    monkeypatch.setenv("ZIPAGE_KEY_GROUPS", kg)
    case = _random_case(100 + seed)
    _check(case, f"random shape {100 + seed}, flags {case.flags}, {kg} key groups")


@pytest.mark.parametrize("flags", [0, Z.ZP_SPLIT_UNITS], ids=["one-workgroup", "split-units"])
def test_device_table_errors_reject_only_their_units(flags):
    """A block id outside the pool (request 1) and a token count below the
    trigger (request 2) are caught by the kernel: those units write only
    their markers (keep row starting with -1, first hole -1), the error word
    reads ZP_EDEVICE, the global update skips them, and request 0 is
    compressed as usual. On the split-unit schedule every part of a unit
    checks the whole table, so all of them skip it without an exchange."""
    spec = synth.scaled(EIGHT_B, requests=3)
    case = P.Case(spec)
    wl, glob, host, dev, tables, dst, pinned, n_tok, _ = P.build_inputs(case)
    zparams, oparams = P._params_for(spec, flags)
    pool = Z.make_pool(wl.k_pool, wl.v_pool)
    R, L, H, b = spec.requests, spec.layers, spec.kv_heads, spec.block_size
    U, k, n = R * L * H, spec.keep, spec.n_tokens
    dev.src_table[1, 5] = spec.pool_blocks + 3
    dev.n_tokens[2] = spec.n_max * b - 1
    out = Z.alloc_outputs(U, k, dev.n_cap, "cuda", debug=True)
    out.keep_idx.fill_(-7)
    ws = Z.alloc_workspace(pool, zparams, R, "cuda")
    k_before = wl.k_pool.clone()
    v_before = wl.v_pool.clone()
    g_before = glob.clone()
    Z.zp_compress(pool, dev, wl.q_window, glob, zparams, out, ws)
    Z.zp_update_global(glob, pool, dev, out, zparams)
    torch.cuda.synchronize()
    assert Z.zp_workspace_error(ws) == Z.ZP_EDEVICE
    assert Z.zp_workspace_error(ws) == Z.ZP_OK  # reading clears the word
    per_req = L * H
    bad = slice(per_req, 3 * per_req)
    assert bool((out.keep_idx[bad, 0] == -1).all())
    assert bool((out.keep_idx[bad, 1:] == -7).all())
    assert bool((out.first_hole[bad] == -1).all())
    assert torch.equal(glob[1:3], g_before[1:3])
    for r in (1, 2):
        blocks = torch.from_numpy(tables[r]).cuda().long()
        assert torch.equal(wl.k_pool[:, blocks], k_before[:, blocks])
        assert torch.equal(wl.v_pool[:, blocks], v_before[:, blocks])
    # request 0 against the oracle
    keep = out.keep_idx.cpu().numpy()
    for u in range(per_req):
        l, h = u // H, u % H
        kr = O.gather_rows(host["k"], tables[0], l, h, n, b)
        vr = O.gather_rows(host["v"], tables[0], l, h, n, b)
        q = O.widen(host["q"][0, l, :, h * (spec.q_heads // H):(h + 1) * (spec.q_heads // H)],
                    spec.dtype)
        ur = O.score_unit(q, O.widen(kr, spec.dtype), host["g"][0, l, h].astype(np.float64),
                          n, 0, oparams)
        diff = set(keep[u].tolist()) ^ set(ur.keep.tolist())
        fin = np.isfinite(ur.score)
        tau = min(float(ur.score[t]) for t in ur.keep if fin[t])
        assert all(abs(ur.score[t] - tau) <= P.BAND for t in diff)
        blocks = torch.from_numpy(tables[0]).cuda().long()
        nk = synth.raw_numpy(wl.k_pool[l, blocks, h].reshape(n, -1))
        nv = synth.raw_numpy(wl.v_pool[l, blocks, h].reshape(n, -1))
        assert nk[:k].tobytes() == kr[keep[u]].tobytes()
        assert nv[:k].tobytes() == vr[keep[u]].tobytes()


@pytest.mark.parametrize("flags", [0, Z.ZP_SPLIT_UNITS, Z.ZP_UPDATE_GLOBAL,
                                   Z.ZP_SPLIT_UNITS | Z.ZP_UPDATE_GLOBAL],
                         ids=["one-workgroup", "split-units", "fused-update",
                              "split-fused-update"])
def test_duplicate_slots_are_rejected(flags):
    """Requests 1 and 3 name the same query slot, so both would rewrite one
    global-score row: every unit of both is rejected (markers only, error
    word ZP_EDEVICE, pools and global rows untouched, the separate global
    update skips them too), while requests 0 and 2 compress as usual."""
    spec = synth.scaled(EIGHT_B, requests=4, pool_blocks=4 * EIGHT_B.n_max + 8)
    case = P.Case(spec)
    wl, glob, host, dev, tables, dst, pinned, n_tok, _ = P.build_inputs(case)
    zparams, oparams = P._params_for(spec, flags)
    pool = Z.make_pool(wl.k_pool, wl.v_pool)
    R, L, H, b = spec.requests, spec.layers, spec.kv_heads, spec.block_size
    U, k, n = R * L * H, spec.keep, spec.n_tokens
    dev.slot[3] = dev.slot[1]
    out = Z.alloc_outputs(U, k, dev.n_cap, "cuda", debug=True)
    out.keep_idx.fill_(-7)
    ws = Z.alloc_workspace(pool, zparams, R, "cuda")
    k_before, v_before, g_before = wl.k_pool.clone(), wl.v_pool.clone(), glob.clone()
    Z.zp_compress(pool, dev, wl.q_window, glob, zparams, out, ws)
    if not flags & Z.ZP_UPDATE_GLOBAL:
        Z.zp_update_global(glob, pool, dev, out, zparams)
    torch.cuda.synchronize()
    assert Z.zp_workspace_error(ws) == Z.ZP_EDEVICE
    per_req = L * H
    for r in (1, 3):
        rows = slice(r * per_req, (r + 1) * per_req)
        assert bool((out.keep_idx[rows, 0] == -1).all())
        assert bool((out.keep_idx[rows, 1:] == -7).all())
        assert bool((out.first_hole[rows] == -1).all())
        blocks = torch.from_numpy(tables[r]).cuda().long()
        assert torch.equal(wl.k_pool[:, blocks], k_before[:, blocks])
        assert torch.equal(wl.v_pool[:, blocks], v_before[:, blocks])
    assert torch.equal(glob[1], g_before[1])   # the shared row (slot 1)
    assert torch.equal(glob[3], g_before[3])   # slot 3: named by no request now
    keep = out.keep_idx.cpu().numpy()
    attn = out.attn.cpu().numpy().astype(np.float64)
    g_now = glob.cpu().numpy()
    for r in (0, 2):
        blocks = torch.from_numpy(tables[r]).cuda().long()
        for l in range(L):
            for h in range(H):
                u = (r * L + l) * H + h
                kr = O.gather_rows(host["k"], tables[r], l, h, n, b)
                vr = O.gather_rows(host["v"], tables[r], l, h, n, b)
                G = spec.q_heads // H
                q = O.widen(host["q"][r, l, :, h * G:(h + 1) * G], spec.dtype)
                g0 = host["g"][r, l, h].astype(np.float64)
                ur = O.score_unit(q, O.widen(kr, spec.dtype), g0, n, 0, oparams)
                assert np.all(np.abs(attn[u, :n] - ur.attn) <=
                              P.ATTN_RTOL * np.abs(ur.attn) + P.ATTN_ATOL)
                diff = set(keep[u].tolist()) ^ set(ur.keep.tolist())
                fin = np.isfinite(ur.score)
                tau = min(float(ur.score[t]) for t in ur.keep if fin[t])
                assert all(abs(ur.score[t] - tau) <= P.BAND for t in diff)
                nk = synth.raw_numpy(wl.k_pool[l, blocks, h].reshape(n, -1))
                nv = synth.raw_numpy(wl.v_pool[l, blocks, h].reshape(n, -1))
                assert nk[:k].tobytes() == kr[keep[u]].tobytes()
                assert nv[:k].tobytes() == vr[keep[u]].tobytes()
                gref = O.update_global(host["g"][r, l, h], ur.attn, keep[u], k)
                assert np.all(np.abs(g_now[r, l, h] - gref) <= 1e-4 * np.abs(gref) + 1e-6)


SCHEDULES = pytest.mark.parametrize("flags", [0, Z.ZP_SPLIT_UNITS],
                                    ids=["one-workgroup", "split-units"])


@SCHEDULES
def test_non_default_weights_and_softmax_scale(flags):
    # s = 0.7 attn + 1.3 global - 0.2 red with an explicit scale 0.05: the
    # weights enter the kernels' fused score and the scale their exp2 domain
    _check(P.Case(EIGHT_B, flags=flags, weights=(0.7, 1.3, 0.2), sm_scale=0.05),
           "weights 0.7/1.3/0.2, sm_scale 0.05")


@SCHEDULES
@pytest.mark.parametrize("scale", [0.0, 1e-6], ids=["zero-norm", "tiny-norm"])
def test_small_norm_keys_hit_the_cosine_clamp(flags, scale):
    # zero keys (cosine 0 with every key) and keys of norm ~1e-5, whose
    # pairwise norm products fall below the 1e-8 clamp
    _check(P.Case(EIGHT_B, flags=flags, small_keys=scale,
                  weights=(1.0, 0.5, 2.0)), f"keys scaled by {scale}")


def _forced_global(spec, evict_positions):
    g = np.zeros((spec.requests, spec.layers, spec.kv_heads, spec.n_tokens))
    g[..., list(evict_positions)] = -100.0
    return g


@pytest.mark.parametrize("name,positions", [
    ("evict block 0 (every row shifts)", list(range(16))),
    ("evict the last block (nothing moves)", None),
    ("alternating holes", "alt"),
])
def test_adversarial_keep_sets(name, positions):
    spec = synth.scaled(EIGHT_B, requests=2)
    n = spec.n_tokens
    if positions is None:
        positions = list(range(n - 16, n))
    elif positions == "alt":
        positions = [17 * i + 3 for i in range(16)]
    _check(P.Case(spec, global_override=_forced_global(spec, positions)), name)


def test_outlier_key_takes_the_exact_softmax_pass():
    # logits of the scaled key exceed the first block's reference by far more
    # than 128 in the exp2 domain: the reference sums overflow and the unit is
    # re-scored with the exact online pass
    spec = synth.scaled(EIGHT_B, requests=2)
    _check(P.Case(spec, outlier=(100, 100.0)), "outlier key x100 at t=100")


def test_forced_ties_keep_prefix():
    spec = synth.scaled(EIGHT_B, requests=1, layers=1)
    g = np.full((1, 1, spec.kv_heads, spec.n_tokens), 0.25)
    case = P.Case(spec, flags=Z.ZP_NONCAUSAL, identical_keys=True,
                  global_override=g)
    res = P.run_case(case)
    assert res.ok, "\n".join(res.failures)


# ------------------------------------------------------------ full size ---

def _save_units(spec, wl, tab_dev, units, slot_of=lambda r: r):
    """Host copies of the sampled units' rows, window and global row."""
    L, H = spec.layers, spec.kv_heads
    n = spec.n_tokens
    G = spec.q_heads // H
    saved = {}
    for u in units:
        r, l, h = u // (L * H), (u // H) % L, u % H
        blocks = tab_dev[r].long()
        kr = wl.k_pool[l, blocks, h].reshape(n, -1)
        vr = wl.v_pool[l, blocks, h].reshape(n, -1)
        sl = slot_of(r)
        saved[u] = (synth.raw_numpy(kr), synth.raw_numpy(vr),
                    synth.raw_numpy(wl.q_window[sl, l, :, h * G:(h + 1) * G]),
                    wl.global_scores[sl, l, h].cpu().numpy().copy())
    return saved


def _check_all_units(spec, out, glob_rows, shared):
    """Properties that hold for every unit of the call."""
    b, k, n = spec.block_size, spec.keep, spec.n_tokens
    keep = out.keep_idx
    assert bool((keep[:, 1:] > keep[:, :-1]).all()), "keep rows not ascending"
    assert int(keep.min()) >= 0 and int(keep.max()) < n
    if not shared:
        ar = torch.arange(k, device=keep.device, dtype=torch.int32)
        hole_ref = torch.where(keep != ar, ar, torch.full_like(ar, k)).min(dim=1).values
        assert torch.equal(hole_ref, out.first_hole)
    else:
        assert bool((keep[:, :spec.shared_blocks * b] ==
                     torch.arange(spec.shared_blocks * b, device=keep.device,
                                  dtype=torch.int32)).all())
    tail = glob_rows[..., k:]
    assert bool((tail == 0).all()), "global tail not zeroed"


def _check_sampled_units(spec, wl, out, saved, pinned, dst_dev, unit_base=0,
                         slot_of=lambda r: r):
    """Sampled units one by one against the oracle. `saved` is keyed by the
    unit's index in the call; unit_base offsets the request index into the
    workload's tables and pools."""
    L, H, b = spec.layers, spec.kv_heads, spec.block_size
    k, n = spec.keep, spec.n_tokens
    _, oparams = P._params_for(spec, 0)
    keep = out.keep_idx
    for u, (kr, vr, q, g) in saved.items():
        r, l, h = u // (L * H), (u // H) % L, u % H
        keys = O.widen(kr, spec.dtype)
        ur = O.score_unit(O.widen(q, spec.dtype), keys, g.astype(np.float64), n,
                          int(pinned[r]), oparams)
        ga = out.attn[u, :n].cpu().numpy().astype(np.float64)
        gr = out.red[u, :n].cpu().numpy().astype(np.float64)
        gs = out.score[u, :n].cpu().numpy()
        assert np.all(np.abs(ga - ur.attn) <= P.ATTN_RTOL * np.abs(ur.attn) + P.ATTN_ATOL)
        assert np.all(np.abs(gr - ur.red) <= P.RED_RTOL * np.abs(ur.red) + P.RED_ATOL)
        fin = np.isfinite(ur.score)
        assert np.array_equal(fin, np.isfinite(gs))
        assert np.all(np.abs(gs[fin] - ur.score[fin]) <=
                      P.SCORE_RTOL * np.abs(ur.score[fin]) + P.SCORE_ATOL)
        gk = keep[u].cpu().numpy()
        assert np.array_equal(gk, O.select_keep(gs.astype(np.float64), k, ~fin))
        diff = set(gk.tolist()) ^ set(ur.keep.tolist())
        tau = min(float(ur.score[t]) for t in ur.keep if fin[t])
        assert all(abs(ur.score[t] - tau) <= P.BAND for t in diff)
        # compacted rows: logical rows [0, k) through the destination table
        blocks = dst_dev[r].long()
        nk = synth.raw_numpy(wl.k_pool[l, blocks, h].reshape(spec.n_max * b, -1))
        nv = synth.raw_numpy(wl.v_pool[l, blocks, h].reshape(spec.n_max * b, -1))
        assert nk[:k].tobytes() == kr[gk].tobytes(), f"K rows of unit {u}"
        assert nv[:k].tobytes() == vr[gk].tobytes(), f"V rows of unit {u}"
        if not spec.shared_blocks:  # the tail block keeps its old rows
            assert nk[k:].tobytes() == kr[k:n].tobytes()
        gn = wl.global_scores[slot_of(r), l, h].cpu().numpy().astype(np.float64)
        gref = O.update_global(g, ur.attn, gk, k)
        assert np.all(np.abs(gn - gref) <= 1e-4 * np.abs(gref) + 1e-6)


def _sample_units(R, L, H, n_samples, seed):
    """A seeded sample spread over requests, layers and heads (unit 0 and the
    last unit always included)."""
    rng = np.random.default_rng(seed)
    U = R * L * H
    units = {0, U - 1}
    i = 0
    while len(units) < min(U, n_samples + 2):
        r = int(rng.integers(R))
        l, h = i % L, (i + i // L) % H
        units.add((r * L + l) * H + h)
        i += 1
    return sorted(units)


def _full_size(spec, n_samples, seed, fused=False, flags=0):
    """Run the full call and check it. Every unit: keep = top k of its own
    scores, compacted K/V rows = the original rows through keep (against an
    untouched copy of the pool, or, with target blocks, against the sources,
    which are checked to be unchanged), global rows = g[keep] + attn[keep]
    bit for bit. A seeded sample of units: everything against the oracle.
    With fused=True the global update runs inside the compression kernel
    (ZP_UPDATE_GLOBAL), the launch configuration bench.py times; `flags`
    adds schedule bits (ZP_SPLIT_UNITS)."""
    dev = "cuda"
    _say(f"[full] generating {spec.name}")
    wl = synth.make(spec, device=dev)
    R, L, H, b = spec.requests, spec.layers, spec.kv_heads, spec.block_size
    U = R * L * H
    k, n = spec.keep, spec.n_tokens
    units = _sample_units(R, L, H, n_samples, seed)
    tables = wl.tables
    shared = bool(spec.shared_blocks)
    if shared:
        bm = Z.BlockManager(spec.pool_blocks)
        bm.alloc(spec.pool_blocks)
        for bid in range(spec.pool_blocks):
            c = int(wl.refcount[bid])
            if c == 0:
                bm.release([bid])
            for _ in range(c - 1):
                bm.incref(bid)
        plan = bm.plan_compress(tables, wl.n_tokens, spec.n_max, b)
        dst, pinned = plan.dst_tables, plan.n_pinned
    else:
        dst, pinned = tables.copy(), np.zeros(R, dtype=np.int32)
    tab_dev = torch.from_numpy(tables).to(dev)
    saved = _save_units(spec, wl, tab_dev, units)
    g0 = wl.global_scores.clone()
    hasher = F.RowHasher(spec.head_dim, dev)
    if shared:
        # the sources are never written with target blocks: their hashes now
        # and after the call show it, and they then serve as the original rows
        src_h = [F.hash_logical_rows(hasher, p_, tab_dev, spec.n_max)
                 for p_ in (wl.k_pool, wl.v_pool)]
        k0, v0 = wl.k_pool, wl.v_pool
    else:
        k0, v0 = wl.k_pool.clone(), wl.v_pool.clone()
    zparams, _ = P._params_for(spec, flags | (Z.ZP_UPDATE_GLOBAL if fused else 0))
    pool = Z.make_pool(wl.k_pool, wl.v_pool)
    batch = Z.DeviceBatch(
        slot=torch.from_numpy(wl.slots).to(dev),
        n_tokens=torch.from_numpy(wl.n_tokens).to(dev),
        src_table=tab_dev,
        dst_table=torch.from_numpy(np.ascontiguousarray(dst, dtype=np.int32)).to(dev),
        n_pinned=torch.from_numpy(np.ascontiguousarray(pinned, dtype=np.int32)).to(dev),
        num_slots=R, n_cap=wl.n_cap)
    out = Z.alloc_outputs(U, k, wl.n_cap, dev, debug=True)
    ws = Z.alloc_workspace(pool, zparams, R, dev)
    _say(f"[full] compress {spec.name}: U={U} flags={flags} workspace={ws.numel() * ws.element_size()} B")
    Z.zp_compress(pool, batch, wl.q_window, wl.global_scores, zparams, out, ws)
    if not fused:
        Z.zp_update_global(wl.global_scores, pool, batch, out, zparams)
    torch.cuda.synchronize()
    assert Z.zp_workspace_error(ws) == Z.ZP_OK
    _check_all_units(spec, out, wl.global_scores, shared)
    F.check_keep_is_topk_of_own_scores(out.keep_idx, out.score, n)
    F.check_global_rows(wl.global_scores, g0, out.keep_idx, out.attn, wl.slots, L, H)
    if shared:
        for p_, h0, what in ((wl.k_pool, src_h[0], "K"), (wl.v_pool, src_h[1], "V")):
            assert torch.equal(F.hash_logical_rows(hasher, p_, tab_dev, spec.n_max), h0), \
                f"{what} source rows changed"
        del src_h
    F.check_rows_against_copy(wl.k_pool, k0, tab_dev, batch.dst_table, out.keep_idx,
                              n, spec.n_max, in_place=not shared, what="K")
    F.check_rows_against_copy(wl.v_pool, v0, tab_dev, batch.dst_table, out.keep_idx,
                              n, spec.n_max, in_place=not shared, what="V")
    _say(f"[full] {spec.name}: all {U} units: keep = top-k of own scores, "
         "rows and global rows exact")
    del k0, v0, g0
    _check_sampled_units(spec, wl, out, saved, pinned, batch.dst_table)
    _say(f"[full] {spec.name}: {len(units)} sampled units match the oracle")
    del wl, out
    torch.cuda.empty_cache()


def test_full_size_small_model():
    _full_size(synth.SMALL, 64, 11)


def test_full_size_8b():
    # the timed launch: global update inside the compression kernel
    _full_size(synth.EIGHT_B, 64, 12, fused=True)


def test_full_size_8b_split():
    # the same batch on the split-unit schedule (bench.py --split-units)
    _full_size(synth.EIGHT_B, 64, 14, fused=True, flags=Z.ZP_SPLIT_UNITS)


def test_full_size_long_context():
    # 8 requests of 16384 tokens (2048 units): the 5-slot ring, launched as
    # the bench times it (fused update)
    _full_size(synth.LONG, 16, 15, fused=True)


def test_full_size_prefix():
    # 256 requests in 4 groups sharing 32 leading blocks each: the pinned
    # prefix stays in place and the kept private rows go to fresh targets
    _full_size(synth.PREFIX, 64, 13)


def test_full_size_overlap():
    """512 requests in 8 groups. Step 0: group 0 (64 requests, all 32 layers,
    holding the query slots) is compressed on one stream while the other 448
    requests decode on a second stream. Step 1: group 1 compresses while group
    0, now compacted to k tokens, decodes with the rest. Checked: every
    compressed unit of both steps (keep = top k of its own scores, global rows
    bit-exact; the compacted rows of step 0 against hashes of the original
    rows, since a 256 GiB pool leaves no room for a copy), 64 sampled
    compressed units against the oracle, sampled decode pairs of step 0, and
    sampled decode pairs of the compacted group (against the oracle's
    attention over the kept tokens of the original cache)."""
    spec = synth.OVERLAP
    dev = "cuda"
    per = spec.requests // spec.compress_groups
    _say(f"[full] generating {spec.name} ({per} query slots)")
    wl = synth.make(spec, device=dev, slots=per)
    L, H = spec.layers, spec.kv_heads
    n, k = spec.n_tokens, spec.keep
    tables = wl.tables
    grp = np.arange(per)
    rest = np.arange(per, spec.requests)
    tab_c = torch.from_numpy(np.ascontiguousarray(tables[grp])).to(dev)
    tab_d = torch.from_numpy(np.ascontiguousarray(tables[rest])).to(dev)
    Uc = per * L * H
    units = _sample_units(per, L, H, 64, 14)
    saved = _save_units(spec, wl, tab_c, units)
    hasher = F.RowHasher(spec.head_dim, dev)
    row_h = [F.hash_logical_rows(hasher, p_, tab_c, spec.n_max)
             for p_ in (wl.k_pool, wl.v_pool)]
    g0 = wl.global_scores.clone()
    rng = np.random.default_rng(spec.seed + 3)
    lens = rng.integers(k + 1, n, size=rest.size).astype(np.int32)  # U{k+1..N-1}
    q = synth.decode_queries(spec, rest.size, dev, spec.seed + 4)
    zparams, _ = P._params_for(spec, 0)
    pool = Z.make_pool(wl.k_pool, wl.v_pool)
    batch = Z.DeviceBatch(
        slot=torch.arange(per, dtype=torch.int32, device=dev),
        n_tokens=torch.full((per,), n, dtype=torch.int32, device=dev),
        src_table=tab_c, dst_table=tab_c.clone(),
        n_pinned=torch.zeros(per, dtype=torch.int32, device=dev),
        num_slots=per, n_cap=wl.n_cap)
    out = Z.alloc_outputs(Uc, k, wl.n_cap, dev, debug=True)
    ws = Z.alloc_workspace(pool, zparams, per, dev)
    dec = torch.full((rest.size, L, spec.q_heads, spec.head_dim), float("nan"),
                     dtype=torch.float32, device=dev)
    lens_dev = torch.from_numpy(lens).to(dev)
    sc, sd = torch.cuda.Stream(), torch.cuda.Stream()
    ready = torch.cuda.Event()
    ready.record(torch.cuda.current_stream())
    sc.wait_event(ready)
    sd.wait_event(ready)
    # original rows of a few (request, layer) pairs of group 0, for checking
    # their decode after compaction
    pairs0 = sorted(set((int(a), int(b)) for a, b in zip(
        rng.integers(0, per, 16), rng.integers(0, L, 16))))
    orig0 = {}
    for (r, l) in pairs0:
        blocks = tab_c[r].long()
        orig0[(r, l)] = [(synth.raw_numpy(wl.k_pool[l, blocks, h].reshape(n, -1)),
                          synth.raw_numpy(wl.v_pool[l, blocks, h].reshape(n, -1)))
                         for h in range(H)]
    _say(f"[full] compress {Uc} units on stream C, decode {rest.size} requests on stream D")
    Z.zp_compress(pool, batch, wl.q_window, wl.global_scores, zparams, out, ws, sc)
    Z.zp_update_global(wl.global_scores, pool, batch, out, zparams, sc)
    Z.zp_paged_decode(dec, q, pool, tab_d, lens_dev, zparams, sd)
    torch.cuda.synchronize()
    assert Z.zp_workspace_error(ws) == Z.ZP_OK
    _check_all_units(spec, out, wl.global_scores, False)
    F.check_keep_is_topk_of_own_scores(out.keep_idx, out.score, n)
    F.check_global_rows(wl.global_scores, g0, out.keep_idx, out.attn, range(per), L, H)
    for p_, h0, what in ((wl.k_pool, row_h[0], "K"), (wl.v_pool, row_h[1], "V")):
        F.check_rows_against_hashes(hasher, p_, h0, batch.dst_table, out.keep_idx,
                                    spec.n_max, in_place=True, what=what)
    del row_h
    _say(f"[full] {spec.name}: all {Uc} compressed units: keep = top-k of own "
         "scores, row hashes and global rows exact")
    _check_sampled_units(spec, wl, out, saved, np.zeros(per, dtype=np.int32),
                         batch.dst_table)
    _say(f"[full] {spec.name}: {len(units)} sampled compressed units match")
    # decode: 64 seeded (request, layer) pairs of the other groups
    pairs = sorted(set((int(a), int(b)) for a, b in zip(
        rng.integers(0, rest.size, 64), rng.integers(0, L, 64))))
    qh = synth.raw_numpy(q)
    got = dec.cpu().numpy().astype(np.float64)
    G = spec.q_heads // H
    for (i, l) in pairs:
        r = int(rest[i])
        blocks = torch.from_numpy(tables[r]).to(dev).long()
        for h in range(H):
            kr = synth.raw_numpy(wl.k_pool[l, blocks, h].reshape(n, -1))[:lens[i]]
            vr = synth.raw_numpy(wl.v_pool[l, blocks, h].reshape(n, -1))[:lens[i]]
            want = O.decode_attention(O.widen(qh[i, l, h * G:(h + 1) * G], spec.dtype),
                                      O.widen(kr, spec.dtype), O.widen(vr, spec.dtype))
            err = np.abs(got[i, l, h * G:(h + 1) * G] - want)
            assert np.all(err <= 1e-4 * np.abs(want) + 1e-5), (r, l, h, err.max())
    _say(f"[full] {spec.name}: {len(pairs)} sampled decode pairs match")

    # step 1: group 1 compresses; group 0 decodes its k kept tokens
    keep0 = out.keep_idx.cpu().numpy()
    grp1 = np.arange(per, 2 * per)
    dec_reqs = np.concatenate([grp, np.arange(2 * per, spec.requests)])
    lens1 = np.concatenate([np.full(per, k, dtype=np.int32),
                            rng.integers(k + 1, n, size=dec_reqs.size - per).astype(np.int32)])
    tab_c1 = torch.from_numpy(np.ascontiguousarray(tables[grp1])).to(dev)
    tab_d1 = torch.from_numpy(np.ascontiguousarray(tables[dec_reqs])).to(dev)
    batch1 = Z.DeviceBatch(
        slot=torch.arange(per, dtype=torch.int32, device=dev),
        n_tokens=torch.full((per,), n, dtype=torch.int32, device=dev),
        src_table=tab_c1, dst_table=tab_c1.clone(),
        n_pinned=torch.zeros(per, dtype=torch.int32, device=dev),
        num_slots=per, n_cap=wl.n_cap)
    q1 = synth.decode_queries(spec, dec_reqs.size, dev, spec.seed + 5)
    dec1 = torch.full((dec_reqs.size, L, spec.q_heads, spec.head_dim), float("nan"),
                      dtype=torch.float32, device=dev)
    lens1_dev = torch.from_numpy(lens1).to(dev)
    g0.copy_(wl.global_scores)
    ready.record(torch.cuda.current_stream())
    sc.wait_event(ready)
    sd.wait_event(ready)
    _say(f"[full] step 1: compress group 1, decode {dec_reqs.size} requests "
         f"(group 0 at k = {k})")
    Z.zp_compress(pool, batch1, wl.q_window, wl.global_scores, zparams, out, ws, sc)
    Z.zp_update_global(wl.global_scores, pool, batch1, out, zparams, sc)
    Z.zp_paged_decode(dec1, q1, pool, tab_d1, lens1_dev, zparams, sd)
    torch.cuda.synchronize()
    assert Z.zp_workspace_error(ws) == Z.ZP_OK
    _check_all_units(spec, out, wl.global_scores, False)
    F.check_keep_is_topk_of_own_scores(out.keep_idx, out.score, n)
    F.check_global_rows(wl.global_scores, g0, out.keep_idx, out.attn, range(per), L, H)
    q1h = synth.raw_numpy(q1)
    got1 = dec1.cpu().numpy().astype(np.float64)
    for (r, l) in pairs0:  # group 0 comes first in dec_reqs
        for h in range(H):
            u = (r * L + l) * H + h
            kr, vr = orig0[(r, l)][h]
            kk = keep0[u]
            want = O.decode_attention(O.widen(q1h[r, l, h * G:(h + 1) * G], spec.dtype),
                                      O.widen(kr[kk], spec.dtype), O.widen(vr[kk], spec.dtype))
            err = np.abs(got1[r, l, h * G:(h + 1) * G] - want)
            assert np.all(err <= 1e-4 * np.abs(want) + 1e-5), (r, l, h, err.max())
    _say(f"[full] {spec.name}: {len(pairs0)} decode pairs of the compacted group "
         f"match the oracle over their kept tokens")
    del wl, out, dec, dec1
    torch.cuda.empty_cache()


# ------------------------------------------------------------- edge shapes ---

EDGE_CASES = [
    # N_max = 2: one kept block, k = b
    ("n_max 2", P.Case(synth.scaled(EIGHT_B, requests=2, n_max=2, window=8,
                                    pool_blocks=8))),
    # G = 1 (no grouping) and a window as long as the kept part
    ("G 1, w = k", P.Case(synth.scaled(EIGHT_B, requests=2, kv_heads=2, q_heads=2,
                                       n_max=6, window=80, pool_blocks=16))),
    # the largest window: w*G = 192 rows with head_dim 64
    ("d64, 192 window rows", P.Case(synth.scaled(D64, q_heads=12, window=32,
                                                 n_max=20, pool_blocks=48))),
    # fp32 keys with head_dim 128 at the largest row count it supports (64)
    ("fp32 d128, 64 rows", P.Case(synth.scaled(F32_D128, q_heads=4, window=16))),
    # a shared prefix together with the protected window
    ("prefix + protected window", P.Case(PREFIX, flags=Z.ZP_PROTECT_WINDOW,
                                         use_block_manager=True)),
    # prefill overshoot on requests that share a prefix (freed tail blocks)
    ("prefix + overshoot", P.Case(
        synth.scaled(PREFIX, pool_blocks=PREFIX.pool_blocks + 16),
        n_tokens=[PREFIX.n_tokens + e for e in (3, 16, 17, 40)],
        max_blocks=PREFIX.n_max + 3, use_block_manager=True)),
]


@pytest.mark.parametrize("label,case", EDGE_CASES, ids=[c[0] for c in EDGE_CASES])
def test_edge_shapes(label, case):
    _check(case, label)


@pytest.mark.parametrize("label,case", [
    ("in place", P.Case(EIGHT_B)),
    ("overshoot", P.Case(synth.scaled(EIGHT_B, requests=3, pool_blocks=112 + 12),
                         n_tokens=[EIGHT_B.n_tokens + e for e in (5, 16, 37)],
                         max_blocks=EIGHT_B.n_max + 3)),
    ("shared prefix", P.Case(PREFIX, use_block_manager=True)),
], ids=["in place", "overshoot", "shared prefix"])
def test_fused_global_update_is_bit_identical(label, case):
    """ZP_UPDATE_GLOBAL applies the global-score update inside the
    compression kernel: pools, keep sets, attention and the updated global
    scores must equal those of zp_compress followed by zp_update_global, bit
    for bit (the update is the same single fp32 addition)."""
    spec = case.spec
    wl, glob, host, dev, tables, dst, pinned, n_tok, _ = P.build_inputs(case)
    R, L, H = spec.requests, spec.layers, spec.kv_heads
    U, k = R * L * H, spec.keep
    zparams, _ = P._params_for(spec, 0)
    fparams, _ = P._params_for(spec, Z.ZP_UPDATE_GLOBAL)
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
    _say(f"[parity] fused global update ({label}): bit-identical")


# ------------------------------------------------- seeded random shapes ---

def _random_case(seed):
    """A small random configuration inside the supported limits."""
    rng = np.random.default_rng(seed)
    dtype = "bf16" if rng.random() < 0.8 else "f32"
    d = int(rng.choice([64, 128]))
    hkv = int(rng.integers(1, 4))
    G = int(rng.choice([1, 2, 3, 4, 6, 8]))
    max_rows = 64 if (dtype == "f32" and d == 128) else 192
    n_max = int(rng.integers(2, 14))
    w = int(rng.integers(1, min(n_max * 16, max_rows // G) + 1))
    R = int(rng.integers(1, 4))
    L = int(rng.integers(1, 3))
    flags = int(rng.choice([0, Z.ZP_NONCAUSAL]))
    if w <= (n_max - 1) * 16 and rng.random() < 0.3:
        flags |= Z.ZP_PROTECT_WINDOW
    over = [int(x) for x in rng.integers(0, 40, size=R)] if rng.random() < 0.4 else [0] * R
    extra = sum((n_max * 16 + e + 15) // 16 - n_max for e in over)
    base = synth.TINY if dtype == "f32" else synth.EIGHT_B
    spec = synth.scaled(base, name=f"random_{seed}", seed=5000 + seed, requests=R,
                        layers=L, kv_heads=hkv, q_heads=hkv * G, head_dim=d,
                        n_max=n_max, window=w, pool_blocks=R * n_max + extra + 2,
                        permute=True, near_dup=(dtype == "bf16"))
    n = spec.n_tokens
    return P.Case(spec, flags=flags, n_tokens=[n + e for e in over],
                  max_blocks=n_max + 3)


@pytest.mark.parametrize("seed", range(48))
def test_random_shapes(seed):
    case = _random_case(seed)
    _check(case, f"random shape {seed}, flags {case.flags}")


def _random_prefix_case(seed):
    """A small random shared-prefix configuration: groups of 2-3 requests
    share their first S blocks; the block manager plans fresh targets."""
    rng = np.random.default_rng(10_000 + seed)
    d = int(rng.choice([64, 128]))
    hkv = int(rng.integers(1, 4))
    G = int(rng.choice([1, 2, 4, 6]))
    n_max = int(rng.integers(4, 14))
    w = int(rng.integers(1, min(n_max * 16, 192 // G) + 1))
    groups = int(rng.integers(1, 3))
    R = groups * int(rng.integers(2, 4))
    L = int(rng.integers(1, 3))
    flags = int(rng.choice([0, Z.ZP_NONCAUSAL]))
    protect = rng.random() < 0.3 and n_max - 1 - (w + 15) // 16 >= 1
    if protect:
        flags |= Z.ZP_PROTECT_WINDOW
    s_max = n_max - 1 - ((w + 15) // 16 if protect else 0)
    S = int(rng.integers(1, s_max + 1))
    over = [int(x) for x in rng.integers(0, 40, size=R)] if rng.random() < 0.4 else [0] * R
    extra = sum((n_max * 16 + e + 15) // 16 - n_max for e in over)
    pool = groups * S + R * (n_max - S) + extra + R * (n_max - 1 - S) + 4
    spec = synth.scaled(synth.PREFIX, name=f"random_prefix_{seed}", seed=7000 + seed,
                        requests=R, layers=L, kv_heads=hkv, q_heads=hkv * G, head_dim=d,
                        n_max=n_max, window=w, groups=groups, shared_blocks=S,
                        pool_blocks=pool, permute=True, near_dup=True)
    n = spec.n_tokens
    return P.Case(spec, flags=flags, n_tokens=[n + e for e in over],
                  max_blocks=n_max + 3, use_block_manager=True)


@pytest.mark.parametrize("seed", range(36))
def test_random_prefix_shapes(seed):
    case = _random_prefix_case(seed)
    s = case.spec
    _check(case, f"random prefix {seed}: R {s.requests} in {s.groups} groups, "
                 f"S {s.shared_blocks} of {s.n_max}, w {s.window}, flags {case.flags}")


def _random_wide_case(seed):
    """Wider random shapes: up to 64 blocks per request (many key tiles per
    quarter), 12 query heads per KV head, overshoot up to 89 tokens, with or
    without a shared prefix planned by the block manager."""
    rng = np.random.default_rng(90_000 + seed)
    prefix = rng.random() < 0.35
    dtype = "bf16" if (prefix or rng.random() < 0.8) else "f32"
    d = int(rng.choice([64, 128]))
    hkv = int(rng.integers(1, 5))
    G = int(rng.choice([1, 2, 3, 4, 6, 8, 12]))
    max_rows = 64 if (dtype == "f32" and d == 128) else 192
    n_max = int(rng.integers(2, 65))
    w = int(rng.integers(1, min(n_max * 16, max_rows // G) + 1))
    L = int(rng.integers(1, 4))
    flags = int(rng.choice([0, Z.ZP_NONCAUSAL]))
    protect = rng.random() < 0.3 and w <= (n_max - 1) * 16
    if prefix:
        groups = int(rng.integers(1, 3))
        R = groups * int(rng.integers(2, 4))
        s_max = n_max - 1 - ((w + 15) // 16 if protect else 0)
        if s_max < 1:
            protect = False
            s_max = n_max - 1
        S = int(rng.integers(1, s_max + 1)) if n_max >= 2 else 0
    else:
        groups, R, S = 1, int(rng.integers(1, 5)), 0
    if protect:
        flags |= Z.ZP_PROTECT_WINDOW
    over = [int(x) for x in rng.integers(0, 90, size=R)] if rng.random() < 0.4 else [0] * R
    extra = sum((n_max * 16 + e + 15) // 16 - n_max for e in over)
    if prefix:
        pool = groups * S + R * (n_max - S) + extra + R * (n_max - 1 - S) + 4
        base = synth.PREFIX
    else:
        pool = R * n_max + extra + 2
        base = synth.TINY if dtype == "f32" else synth.EIGHT_B
    spec = synth.scaled(base, name=f"wide_{seed}", seed=9000 + seed, requests=R, layers=L,
                        kv_heads=hkv, q_heads=hkv * G, head_dim=d, n_max=n_max, window=w,
                        groups=groups, shared_blocks=S, pool_blocks=pool, permute=True,
                        near_dup=(dtype == "bf16"))
    n = spec.n_tokens
    return P.Case(spec, flags=flags, n_tokens=[n + e for e in over],
                  max_blocks=n_max + 6, use_block_manager=prefix)


@pytest.mark.parametrize("seed", range(30))
def test_random_wide_shapes(seed):
    case = _random_wide_case(seed)
    s = case.spec
    _check(case, f"wide random {seed}: n_max {s.n_max}, w {s.window}, "
                 f"G {s.q_heads // s.kv_heads}, S {s.shared_blocks}, flags {case.flags}")


@pytest.mark.parametrize("seed", range(10))
def test_random_wide_shapes_on_eight_waves(seed, monkeypatch):
    # these sizes take the 4-wave workgroups by default; the same cases on
    # the 8-wave shape
    monkeypatch.setenv("ZIPAGE_KEY_GROUPS", "4")
    case = _random_wide_case(seed)
    s = case.spec
    _check(case, f"wide random {seed} on 8 waves: n_max {s.n_max}, w {s.window}, "
                 f"G {s.q_heads // s.kv_heads}, S {s.shared_blocks}, flags {case.flags}")
