"""Pins of the CPU oracle against things other than itself.

Each test checks one oracle function against a library routine, a closed
form, a brute force on tiny inputs or the hand-worked example in
tests/golden/hand_example.json. None of these tests re-types the oracle's own
formula. No GPU needed.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example.json")


def _ev(expr):
    return eval(expr, {"__builtins__": {}}, {"e": math.e, "sqrt": math.sqrt})


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ----------------------------------------------------------------- budget ---

def test_budget_formula_and_configs():
    # k = (N_max - 1) * b  -- [zh] section 2.1
    assert O.budget_tokens(8, 16) == 112
    assert O.budget_tokens(128, 16) == 2032
    assert O.budget_tokens(256, 16) == 4080
    assert O.budget_tokens(2, 2) == 2
    with pytest.raises(ValueError):
        O.budget_tokens(1, 16)


def test_widen_bf16_bit_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F80],
                    dtype=np.uint16)
    got = O.widen(bits, "bf16")
    assert list(got[:4]) == [1.0, -2.0, 1.0078125, 0.0]
    assert math.copysign(1.0, got[4]) == -1.0 and got[4] == 0.0
    assert math.isinf(got[5])
    # and against torch's own bf16 decoding
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    assert np.array_equal(got[:5], t.double().numpy()[:5])


def test_gather_rows_follows_block_table():
    L, NB, H, b, d = 2, 5, 3, 4, 2
    pool = np.zeros((L, NB, H, b, d), dtype=np.float32)
    for l, blk, h, s in itertools.product(range(L), range(NB), range(H), range(b)):
        pool[l, blk, h, s, 0] = 1000 * l + 100 * blk + 10 * h + s
    table = [3, 0, 4]
    rows = O.gather_rows(pool, table, 1, 2, 10, b)
    for t in range(10):
        assert rows[t, 0] == 1000 + 100 * table[t // b] + 20 + t % b


# -------------------------------------------------------- window attention ---

def test_attention_single_row_equals_scipy_softmax():
    rng = np.random.default_rng(1)
    n, d = 37, 16
    keys = rng.standard_normal((n, d))
    q = rng.standard_normal((1, 1, d))
    got = O.window_attention(q, keys, n, causal=False)
    want = scipy.special.softmax(keys @ q[0, 0] / math.sqrt(d))
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=0)


def _sdpa_probabilities(q_win, keys, n, causal):
    """Attention probabilities from torch's SDPA: with V = identity the output
    rows are the softmax rows themselves."""
    w, G, d = q_win.shape
    Q = torch.from_numpy(q_win.reshape(w * G, d)).unsqueeze(0)
    K = torch.from_numpy(keys).unsqueeze(0)
    V = torch.eye(n, dtype=torch.float64).unsqueeze(0)
    mask = None
    if causal:
        pos = torch.tensor([n - w + i for i in range(w) for _ in range(G)])
        mask = torch.arange(n).unsqueeze(0) <= pos.unsqueeze(1)
        mask = mask.unsqueeze(0)
    P = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask)
    return P[0].numpy()


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("w,G,n,d", [(8, 2, 128, 64), (4, 3, 33, 8), (1, 1, 5, 4),
                                     (5, 6, 5, 16)])
def test_attention_equals_torch_sdpa_row_mean(causal, w, G, n, d):
    rng = np.random.default_rng(w * 100 + G * 10 + n)
    keys = rng.standard_normal((n, d))
    q = rng.standard_normal((w, G, d))
    got = O.window_attention(q, keys, n, causal=causal)
    want = _sdpa_probabilities(q, keys, n, causal).mean(axis=0)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-300)
    assert abs(got.sum() - 1.0) < 1e-12


def test_attention_brute_force_python_loops():
    rng = np.random.default_rng(7)
    n, d, w, G = 6, 3, 3, 2
    keys = rng.standard_normal((n, d))
    q = rng.standard_normal((w, G, d))
    scale = 1 / math.sqrt(d)
    want = [0.0] * n
    for i in range(w):
        p = n - w + i
        for g in range(G):
            lg = [sum(q[i, g, c] * keys[t, c] for c in range(d)) * scale
                  for t in range(p + 1)]
            z = sum(math.exp(x) for x in lg)
            for t in range(p + 1):
                want[t] += math.exp(lg[t]) / z / (w * G)
    got = O.window_attention(q, keys, n, causal=True)
    np.testing.assert_allclose(got, want, rtol=1e-12)


@pytest.mark.parametrize("n,w", [(16, 4), (9, 9), (10, 1)])
def test_attention_identical_keys_closed_form(n, w):
    d, G = 8, 3
    keys = np.tile(np.arange(1.0, d + 1), (n, 1))
    q = np.random.default_rng(0).standard_normal((w, G, d))
    got = O.window_attention(q, keys, n, causal=True)
    pos = [n - w + i for i in range(w)]
    want = [sum(1.0 / (p + 1) for p in pos if p >= t) / w for t in range(n)]
    np.testing.assert_allclose(got, want, rtol=1e-12)
    got_nc = O.window_attention(q, keys, n, causal=False)
    np.testing.assert_allclose(got_nc, np.full(n, 1.0 / n), rtol=1e-12)


# ------------------------------------------------------------- redundancy ---

def _full_pairwise_same_block(keys, b):
    """The original O((N b)^2) redundancy: all-pairs cosine similarity (torch),
    then restricted to off-diagonal pairs of the same block."""
    K = torch.from_numpy(keys)
    n = K.shape[0]
    cos = torch.nn.functional.cosine_similarity(K.unsqueeze(1), K.unsqueeze(0),
                                                dim=-1, eps=1e-8)
    blk = torch.arange(n) // b
    same = (blk.unsqueeze(0) == blk.unsqueeze(1)) & ~torch.eye(n, dtype=torch.bool)
    cnt = same.sum(dim=1)
    tot = (cos * same).sum(dim=1)
    out = torch.where(cnt > 0, tot / cnt.clamp(min=1), torch.zeros_like(tot))
    return out.numpy()


@pytest.mark.parametrize("n,b,d", [(64, 16, 32), (50, 16, 8), (7, 2, 3),
                                   (33, 4, 128), (17, 16, 4)])
def test_lightning_equals_full_pairwise_restricted(n, b, d):
    rng = np.random.default_rng(n + b + d)
    keys = rng.standard_normal((n, d))
    got = O.lightning_redundancy(keys, b, n)
    want = _full_pairwise_same_block(keys, b)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


def test_redundancy_closed_forms():
    d, b = 16, 4
    same = np.tile(np.linspace(-1, 2, d), (8, 1))
    np.testing.assert_allclose(O.lightning_redundancy(same, b, 8), 1.0, rtol=1e-12)
    ortho = np.eye(d)[:8] * np.arange(1, 9)[:, None]  # scaled basis vectors
    np.testing.assert_allclose(O.lightning_redundancy(ortho, b, 8), 0.0, atol=1e-15)
    a, c = np.array([1.0, 2.0, 0.5]), np.array([-0.3, 1.0, 4.0])
    pair = O.lightning_redundancy(np.stack([a, c]), 2, 2)
    cosac = a @ c / (np.linalg.norm(a) * np.linalg.norm(c))
    np.testing.assert_allclose(pair, [cosac, cosac], rtol=1e-14)
    # a trailing block with one token has no partner: 0
    rng = np.random.default_rng(3)
    keys = rng.standard_normal((9, 5))
    assert O.lightning_redundancy(keys, 4, 9)[8] == 0.0


def test_redundancy_is_scale_invariant_per_token():
    rng = np.random.default_rng(11)
    keys = rng.standard_normal((32, 8))
    scales = rng.uniform(0.1, 10.0, size=(32, 1))
    np.testing.assert_allclose(O.lightning_redundancy(keys * scales, 16, 32),
                               O.lightning_redundancy(keys, 16, 32), rtol=1e-12)


def test_redundancy_against_sklearn():
    from sklearn.metrics.pairwise import cosine_similarity
    rng = np.random.default_rng(5)
    keys = rng.standard_normal((16, 12))
    c = cosine_similarity(keys)
    want = (c.sum(axis=1) - np.diag(c)) / 15
    np.testing.assert_allclose(O.lightning_redundancy(keys, 16, 16), want,
                               rtol=1e-12)


# ------------------------------------------------------ hand-worked example ---

def _hand_params(g, causal=True, protect=False):
    return O.Params(n_max=g["n_max"], block_size=g["block_size"],
                    window=g["window"], causal=causal, protect_window=protect)


def test_hand_example_causal():
    g = _golden()
    p = _hand_params(g)
    q = np.asarray(g["q_window"], dtype=np.float64)
    keys = np.asarray(g["keys"], dtype=np.float64)
    glob = np.asarray(g["global"], dtype=np.float64)
    res = O.score_unit(q, keys, glob, 4, 0, p)
    exp = g["expect_causal"]
    np.testing.assert_allclose(res.attn, [_ev(x) for x in exp["attn"]], rtol=1e-14)
    np.testing.assert_allclose(res.red, [_ev(x) for x in exp["red"]], atol=1e-15)
    np.testing.assert_allclose(res.score, [_ev(x) for x in exp["score"]],
                               rtol=1e-13)
    assert list(res.keep) == exp["keep"]
    assert res.hole == exp["hole"]
    gn = O.update_global(glob, res.attn, res.keep, p.keep_tokens)
    np.testing.assert_allclose(gn, [_ev(x) for x in exp["global_new"]],
                               rtol=1e-14)


def test_hand_example_noncausal_and_protected():
    g = _golden()
    q = np.asarray(g["q_window"], dtype=np.float64)
    keys = np.asarray(g["keys"], dtype=np.float64)
    glob = np.asarray(g["global"], dtype=np.float64)
    res = O.score_unit(q, keys, glob, 4, 0, _hand_params(g, causal=False))
    np.testing.assert_allclose(
        res.attn, [_ev(x) for x in g["expect_noncausal"]["attn"]], rtol=1e-14)
    res = O.score_unit(q, keys, glob, 4, 0, _hand_params(g, protect=True))
    assert list(res.keep) == g["expect_protect_window"]["keep"]


def test_hand_example_compaction_bytes():
    g = _golden()
    keys = np.asarray(g["keys"], dtype=np.float32)
    pool = keys.reshape(1, 2, 1, 2, 4).copy()       # 1 layer, blocks [0, 1]
    out = pool.copy()
    O.compact_unit(pool, out, [0, 1], [0, 1], 0, 0, np.array([1, 2]), 2)
    assert out[0, 0, 0, 0].tobytes() == keys[1].tobytes()
    assert out[0, 0, 0, 1].tobytes() == keys[2].tobytes()
    assert out[0, 1].tobytes() == pool[0, 1].tobytes()   # tail block untouched


# --------------------------------------------------------------- selection ---

def _valid_topk(s, k, pinned, keep):
    """Definition of the selected set: |keep| = k, pinned inside, and every
    kept free token ranks above every evicted one under (s desc, pos asc)."""
    keep = set(int(x) for x in keep)
    if len(keep) != k or not all(t in keep for t in range(len(s)) if pinned[t]):
        return False
    kept = [t for t in keep if not pinned[t]]
    gone = [t for t in range(len(s)) if t not in keep]
    rank = lambda t: (-s[t], t)  # noqa: E731
    return all(rank(a) < rank(b) for a in kept for b in gone)


def test_select_exhaustive_subsets():
    rng = np.random.default_rng(2)
    for trial in range(40):
        n = int(rng.integers(3, 10))
        k = int(rng.integers(1, n))
        s = rng.integers(0, 4, size=n).astype(np.float64)   # many ties
        pinned = rng.random(n) < 0.2
        if pinned.sum() > k:
            pinned[:] = False
        keep = O.select_keep(s, k, pinned)
        assert list(keep) == sorted(keep)
        valid = [c for c in itertools.combinations(range(n), k)
                 if _valid_topk(s, k, pinned, c)]
        assert valid == [tuple(int(x) for x in keep)]


def test_select_forced_ties_keep_prefix():
    n, k = 128, 112
    keep = O.select_keep(np.full(n, 0.25), k, np.zeros(n, dtype=bool))
    assert list(keep) == list(range(k))


def test_select_negative_zero_equals_zero():
    s = np.array([0.0, -0.0, 0.0, -0.0, 1.0])
    keep = O.select_keep(s, 3, np.zeros(5, dtype=bool))
    assert list(keep) == [0, 1, 4]


def test_pinned_mask_and_hole():
    m = O.pinned_mask(10, 2, 2, 3, True)
    assert list(np.flatnonzero(m)) == [0, 1, 2, 3, 7, 8, 9]
    assert O.first_hole(np.array([0, 1, 3, 4])) == 2
    assert O.first_hole(np.array([0, 1, 2])) == 3
    assert O.first_hole(np.array([5, 6])) == 0


# -------------------------------------------------------- global update ---

def test_update_global_identities():
    rng = np.random.default_rng(4)
    n, k, cap = 64, 48, 80
    g = rng.random(cap)
    attn = rng.random(n)
    keep = np.sort(rng.choice(n, size=k, replace=False))
    out = O.update_global(g, attn, keep, k)
    assert np.all(out[k:] == 0.0)
    np.testing.assert_allclose(out[:k].sum(), g[keep].sum() + attn[keep].sum(),
                               rtol=1e-13)
    # identity keep: the scores just grow by this round's attention
    ident = O.update_global(g, attn, np.arange(k), k)
    np.testing.assert_allclose(ident[:k], g[:k] + attn[:k], rtol=1e-15)


# ------------------------------------------------------------ whole batch ---

def _tiny_batch(rng, R=2, L=2, H=2, G=2, d=8, b=4, n_max=4, w=3, extra=0):
    nb = R * (n_max + extra) + 3
    pool_k = rng.standard_normal((L, nb, H, b, d)).astype(np.float32)
    pool_v = rng.standard_normal((L, nb, H, b, d)).astype(np.float32)
    perm = rng.permutation(nb)
    per = n_max + extra
    tables = np.stack([perm[r * per:(r + 1) * per] for r in range(R)])
    q = rng.standard_normal((R, L, w, H * G, d)).astype(np.float32)
    glob = rng.random((R, L, H, n_max * b + extra * b)).astype(np.float32)
    n_tok = np.full(R, (n_max + extra) * b)
    batch = O.Batch(slots=np.arange(R), n_tokens=n_tok, src_tables=tables,
                    dst_tables=tables[:, :n_max].copy(),
                    n_pinned=np.zeros(R, dtype=np.int64))
    return pool_k, pool_v, q, glob, batch, O.Params(n_max=n_max, block_size=b,
                                                    window=w)


@pytest.mark.parametrize("extra", [0, 2])
def test_compress_moves_exact_bytes_in_place(extra):
    rng = np.random.default_rng(9 + extra)
    pool_k, pool_v, q, glob, batch, p = _tiny_batch(rng, extra=extra)
    out = O.compress(pool_k, pool_v, "f32", q, "f32", glob, batch, p)
    k = p.keep_tokens
    b = p.block_size
    touched = set()
    for (r, l, h), res in out["units"].items():
        assert len(res.keep) == k
        src = batch.src_tables[r]
        for t in range(k):
            sblk, sslot = src[res.keep[t] // b], res.keep[t] % b
            dblk, dslot = batch.dst_tables[r][t // b], t % b
            assert out["pool_k"][l, dblk, h, dslot].tobytes() == \
                pool_k[l, sblk, h, sslot].tobytes()
            assert out["pool_v"][l, dblk, h, dslot].tobytes() == \
                pool_v[l, sblk, h, sslot].tobytes()
            touched.add((l, dblk, h, dslot))
        # rows before the first hole are their own source
        for t in range(res.hole):
            assert res.keep[t] == t
    # every row not written as a destination keeps its bytes
    L, NB, H, B, _ = pool_k.shape
    for idx in itertools.product(range(L), range(NB), range(H), range(B)):
        if idx not in touched:
            assert out["pool_k"][idx].tobytes() == pool_k[idx].tobytes()



def test_compress_into_target_blocks_after_a_shared_prefix():
    """With S leading shared blocks the kept private rows go, in order, to
    fresh target blocks listed after the prefix in the destination table
    ([zh §2.2]): each target row is a byte copy of its source row read through
    the source table, the shared blocks and every source block keep their
    bytes, and the S*b prefix tokens are kept where they are."""
    rng = np.random.default_rng(31)
    R, L, H, G, d, b, n_max, w, S = 2, 2, 2, 2, 8, 4, 5, 3, 2
    private = n_max - S
    nb = S + R * private + R * (n_max - 1 - S) + 2
    pool_k = rng.standard_normal((L, nb, H, b, d)).astype(np.float32)
    pool_v = rng.standard_normal((L, nb, H, b, d)).astype(np.float32)
    perm = rng.permutation(nb)
    shared = perm[:S]
    src = np.stack([np.concatenate([shared, perm[S + r * private:S + (r + 1) * private]])
                    for r in range(R)])
    base = S + R * private
    fresh = [perm[base + r * (n_max - 1 - S):base + (r + 1) * (n_max - 1 - S)]
             for r in range(R)]
    dst = np.stack([np.concatenate([shared, fresh[r], [shared[0]]]) for r in range(R)])
    q = rng.standard_normal((R, L, w, H * G, d)).astype(np.float32)
    glob = rng.random((R, L, H, n_max * b)).astype(np.float32)
    batch = O.Batch(slots=np.arange(R), n_tokens=np.full(R, n_max * b), src_tables=src,
                    dst_tables=dst, n_pinned=np.full(R, S))
    p = O.Params(n_max=n_max, block_size=b, window=w)
    out = O.compress(pool_k, pool_v, "f32", q, "f32", glob, batch, p)
    k = p.keep_tokens
    targets = set()
    for (r, l, h), res in out["units"].items():
        assert len(res.keep) == k
        assert list(res.keep[:S * b]) == list(range(S * b))
        for t in range(S * b, k):
            sblk, sslot = src[r][res.keep[t] // b], res.keep[t] % b
            dblk, dslot = dst[r][t // b], t % b
            assert dblk in fresh[r]
            assert out["pool_k"][l, dblk, h, dslot].tobytes() == \
                pool_k[l, sblk, h, sslot].tobytes()
            assert out["pool_v"][l, dblk, h, dslot].tobytes() == \
                pool_v[l, sblk, h, sslot].tobytes()
        targets.update(int(x) for x in fresh[r])
    for blk in range(nb):
        if blk not in targets:
            assert out["pool_k"][:, blk].tobytes() == pool_k[:, blk].tobytes()
            assert out["pool_v"][:, blk].tobytes() == pool_v[:, blk].tobytes()

# ----------------------------------------------------------- bookkeeping ---

def test_block_pool_lifo_and_plans():
    bp = O.BlockPool(12)
    a = bp.alloc(4)
    assert a == [0, 1, 2, 3]                      # id 0 pops first
    shared = bp.alloc(2)
    for bid in shared:
        bp.incref(bid)                             # shared by two requests
    r0 = shared + bp.alloc(2)                      # [4, 5, 6, 7]
    r1 = shared + bp.alloc(2)                      # [4, 5, 8, 9]
    before = list(bp.refcount)
    plan = bp.plan_compress([r0, r1], [8, 8], n_max=4, b=2)
    assert list(plan.n_pinned) == [2, 2]
    # each request pops n_max - 1 - S = 1 target: 10 then 11
    assert plan.popped == [10, 11]
    assert [list(x) for x in plan.dst_tables] == [[4, 5, 10, 7], [4, 5, 11, 9]]
    assert plan.to_free == [6, 8]
    bp.commit(plan)
    assert bp.refcount[4] == before[4] == 2 and bp.refcount[5] == 2
    assert bp.refcount[10] == 1 and bp.refcount[6] == 0
    # free list + held blocks = the pool, no duplicates
    held = {b for b in range(12) if bp.refcount[b] > 0}
    assert sorted(bp.stack + sorted(held)) == list(range(12))
    assert bp.stack[-2:] == [6, 8]                 # pushed in plan order


def test_block_pool_in_place_and_overshoot():
    bp = O.BlockPool(10)
    t = bp.alloc(6)
    plan = bp.plan_compress([t], [11], n_max=4, b=2)   # 6 blocks, overshoot
    assert list(plan.dst_tables[0]) == t[:4]
    assert plan.to_free == t[4:] and plan.popped == []
    with pytest.raises(ValueError):
        bp.plan_compress([t], [7], n_max=4, b=2)       # below trigger


def test_block_pool_exhausted_changes_nothing():
    bp = O.BlockPool(8)
    sh = bp.alloc(1)
    bp.incref(sh[0])
    r = sh + bp.alloc(3)
    r2 = sh + bp.alloc(3)
    bp.alloc(1)
    stack, refs = list(bp.stack), list(bp.refcount)
    with pytest.raises(MemoryError):
        bp.plan_compress([r, r2], [8, 8], n_max=4, b=2)  # needs 4 targets, 0 free
    assert bp.stack == stack and bp.refcount == refs


def test_block_pool_rejects_shared_or_repeated_private_blocks():
    """Blocks after the shared run are written, kept as the tail or freed:
    a block with another holder, or one listed twice in the call, must make
    the plan fail and leave the pool as it was ([de §2], [zh §2.2])."""
    bp = O.BlockPool(16)
    sh = bp.alloc(2)
    for x in sh:
        bp.incref(x)
    r0 = bp.alloc(4)                       # private: [2, 3, 4, 5]
    r1 = sh + bp.alloc(2)                  # shared prefix of 2, then private
    state = (list(bp.stack), list(bp.refcount))
    bad_tables = [
        [[r0[0], sh[1], r0[2], r0[3]]],    # a shared block after a private one
        [r0, [r0[0]] + r1[1:]],            # r0[0] held by two requests (S = 0)
        [r1, [r1[0], r1[1], r1[2], r0[3]], r0],  # r0[3] listed twice
        [[r0[0], r0[1], r0[2], r0[3], sh[0]]],   # overshoot block is shared
    ]
    ntok = [[8], [8, 8], [8, 8, 8], [9]]
    for tabs, n in zip(bad_tables, ntok):
        with pytest.raises(ValueError):
            bp.plan_compress(tabs, n, n_max=4, b=2)
        assert (list(bp.stack), list(bp.refcount)) == state
    # the same requests, well formed, plan fine
    plan = bp.plan_compress([r0, r1], [8, 8], n_max=4, b=2)
    assert list(plan.n_pinned) == [0, 2]


# ---------------------------------------------------------------- decode ---

def test_decode_attention_equals_torch_sdpa():
    rng = np.random.default_rng(8)
    n, d, G = 50, 16, 4
    q = rng.standard_normal((G, d))
    keys = rng.standard_normal((n, d))
    vals = rng.standard_normal((n, d))
    got = O.decode_attention(q, keys, vals)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(keys)[None],
        torch.from_numpy(vals)[None])[0].numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# query-window capture ([zh] §2.2 query slots; [zh] §2.1 last w queries)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("w,P", [(1, 5), (4, 4), (4, 11), (8, 37), (32, 100)])
def test_capture_ring_holds_the_last_w_queries(w, P):
    """Capturing positions 0..P-1 one decode step at a time leaves, read in
    position order, exactly the queries of the last w positions (a plain
    slice of the sequence)."""
    rng = np.random.default_rng(w * 1000 + P)
    L, Hq, d = 2, 3, 4
    seq = rng.standard_normal((P, L, Hq, d))      # queries of positions 0..P-1
    ring = np.zeros((2, L, w, Hq, d))
    for p in range(P):
        O.capture_queries(ring, seq[p][None], [1], [p], w)
    for layer in range(L):
        got = O.window_from_ring(ring[1, layer], P, w)
        assert np.array_equal(got, seq[P - w:P, layer])
    assert not ring[0].any()                       # the other slot untouched


def test_capture_skips_requests_without_a_slot():
    rng = np.random.default_rng(3)
    w, L, Hq, d = 4, 1, 2, 4
    ring = np.full((2, L, w, Hq, d), 7.0)
    q = rng.standard_normal((4, L, Hq, d))
    O.capture_queries(ring, q, [-1, 2, 0, 1], [5, 6, -1, 9], w)
    # request 0: no slot; 1: slot 2 out of range; 2: negative position
    assert np.array_equal(ring[0], np.full((L, w, Hq, d), 7.0))
    expect = np.full((L, w, Hq, d), 7.0)
    expect[:, 9 % w] = q[3]
    assert np.array_equal(ring[1], expect)


def test_ring_window_scores_like_the_linear_window():
    """A compression that reads its window through the ring gives the same
    attention as one handed the last w queries in order (closed ring walk
    against a direct slice)."""
    rng = np.random.default_rng(11)
    n, w, G, d = 40, 6, 2, 8
    keys = rng.standard_normal((n, d))
    seq = rng.standard_normal((n, 1, G, d))
    ring = np.zeros((1, 1, w, G, d))
    for p in range(n):
        O.capture_queries(ring, seq[p][None], [0], [p], w)
    lin = seq[n - w:, 0]
    a1 = O.window_attention(lin, keys, n, True)
    a2 = O.window_attention(O.window_from_ring(ring[0, 0], n, w), keys, n, True)
    assert np.array_equal(a1, a2)


# ---------------------------------------------------------------------------
# decode with an appended token ([zh] §2.3)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("lens", [[0, 5, 16, 31], [15, 1, 32, 47]])
def test_decode_append_equals_sdpa_over_cache_plus_new_token(lens):
    """The appended token lands in the slot its position names, nothing else
    in the pools changes, and each head's output is torch SDPA over the cached
    rows followed by the new one."""
    rng = np.random.default_rng(sum(lens))
    R, L, Hkv, G, b, d, nb = len(lens), 2, 2, 2, 16, 8, 3
    Hq = Hkv * G
    pool_k = rng.standard_normal((L, R * nb, Hkv, b, d))
    pool_v = rng.standard_normal((L, R * nb, Hkv, b, d))
    tables = rng.permutation(R * nb).reshape(R, nb)
    q = rng.standard_normal((R, L, Hq, d))
    k_new = rng.standard_normal((R, L, Hkv, d))
    v_new = rng.standard_normal((R, L, Hkv, d))
    out, pk, pv = O.paged_decode_append(q, "f64", k_new, v_new, pool_k, pool_v,
                                        "f64", tables, lens)
    mask = np.ones(pk.shape, dtype=bool)
    for r, n in enumerate(lens):
        mask[:, tables[r, n // b], :, n % b] = False
    assert np.array_equal(pk[mask], pool_k[mask])       # every other row unchanged
    assert np.array_equal(pv[mask], pool_v[mask])
    for r, n in enumerate(lens):
        blk, slot = tables[r, n // b], n % b
        assert np.array_equal(pk[:, blk, :, slot], k_new[r])
        assert np.array_equal(pv[:, blk, :, slot], v_new[r])
        for layer in range(L):
            for h in range(Hkv):
                rows = [pool_k[layer, tables[r, t // b], h, t % b] for t in range(n)]
                vrows = [pool_v[layer, tables[r, t // b], h, t % b] for t in range(n)]
                keys = np.array(rows + [k_new[r, layer, h]])
                vals = np.array(vrows + [v_new[r, layer, h]])
                want = torch.nn.functional.scaled_dot_product_attention(
                    torch.from_numpy(q[r, layer, h * G:(h + 1) * G])[None],
                    torch.from_numpy(keys)[None], torch.from_numpy(vals)[None])[0].numpy()
                np.testing.assert_allclose(out[(r, layer)][h * G:(h + 1) * G], want,
                                           rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# the all-pairs redundancy kept as an ablation ([zh] §2.1, [fr] §2.E)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,b,d", [(64, 16, 32), (50, 16, 8), (33, 4, 128), (17, 16, 4)])
def test_all_pairs_redundancy_pins(n, b, d):
    rng = np.random.default_rng(7 * n + d)
    keys = rng.standard_normal((n, d))
    red_block, red_all = O.redundancy_all_pairs(keys, b, n)
    # the same-block restriction is the lightning score (loops, per block)
    np.testing.assert_allclose(red_block, O.lightning_redundancy(keys, b, n),
                               rtol=1e-12, atol=1e-14)
    # the all-token mean against torch's pairwise cosine similarity
    t = torch.from_numpy(keys)
    cos = torch.nn.functional.cosine_similarity(t[:, None, :], t[None, :, :], dim=-1,
                                                eps=0.0).numpy()
    want = (cos.sum(axis=1) - np.diag(cos)) / (n - 1)
    np.testing.assert_allclose(red_all, want, rtol=1e-10, atol=1e-12)
