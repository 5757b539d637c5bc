"""Property-based pins of the oracle (hypothesis; CPU only).

Shapes are drawn over N_max in [2, 6], b in {1, 2, 4, 16}, head_dim in
{4, 8, 16}, window w in [1, N_max*b] and GQA group G in [1, 4], with ragged
token counts (a partial last block) and random values, including exact ties
and zero keys. Every property is checked against something other than the
oracle's own formula: a library routine (scipy's softmax, torch's cosine
matrix, numpy's lexsort), brute force over subsets, or an invariant the
pages' definitions imply ([zh] §2.1: softmax attention from the window,
intra-block redundancy, keep the k best; [de] §2: shared blocks intact).
"""

import itertools

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st
from scipy.special import softmax

import oracle as O

SETTINGS = settings(max_examples=60, deadline=None,
                    suppress_health_check=[HealthCheck.too_slow])


@st.composite
def unit_shapes(draw):
    n_max = draw(st.integers(2, 6))
    b = draw(st.sampled_from([1, 2, 4, 16]))
    d = draw(st.sampled_from([4, 8, 16]))
    G = draw(st.integers(1, 4))
    full = n_max * b
    n = draw(st.integers(max(1, full - b + 1), full))    # ragged last block
    w = draw(st.integers(1, n))
    seed = draw(st.integers(0, 2**31 - 1))
    ties = draw(st.booleans())
    return n_max, b, d, G, n, w, seed, ties


def _keys(n, d, rng, ties):
    keys = rng.standard_normal((n, d))
    if ties and n > 2:
        keys[1] = keys[0]                       # an exact duplicate
        keys[-1] = 0.0                          # a zero key (norm clamp)
    return keys


@SETTINGS
@given(unit_shapes(), st.booleans())
def test_attention_is_a_mean_of_softmax_rows(shape, causal):
    n_max, b, d, G, n, w, seed, ties = shape
    rng = np.random.default_rng(seed)
    keys = _keys(n, d, rng, ties)
    q = rng.standard_normal((w, G, d))
    attn = O.window_attention(q, keys, n, causal=causal)
    # the mean of w*G probability rows sums to one and is non-negative
    assert abs(attn.sum() - 1.0) < 1e-12
    assert np.all(attn >= 0)
    # against scipy's softmax, one row at a time (causal rows see t <= n-w+i)
    want = np.zeros(n)
    for i in range(w):
        vis = n - w + i + 1 if causal else n
        for g in range(G):
            want[:vis] += softmax(keys[:vis] @ q[i, g] / np.sqrt(d))
    np.testing.assert_allclose(attn, want / (w * G), rtol=1e-12, atol=1e-15)
    if causal and w >= 1:
        # the last token is seen only by the newest window row
        assert attn[n - 1] > 0


@SETTINGS
@given(unit_shapes())
def test_lightning_equals_the_full_cosine_matrix_inside_blocks(shape):
    n_max, b, d, G, n, w, seed, ties = shape
    rng = np.random.default_rng(seed)
    keys = _keys(n, d, rng, ties)
    red = O.lightning_redundancy(keys, b, n)
    kt = torch.from_numpy(keys)
    norms = kt.norm(dim=1)
    cos = (kt @ kt.T) / torch.clamp(norms[:, None] * norms[None, :], min=1e-8)
    blk = torch.arange(n) // b
    same = (blk[:, None] == blk[None, :]) & ~torch.eye(n, dtype=torch.bool)
    cnt = same.sum(dim=1)
    want = torch.where(cnt > 0, (cos * same).sum(dim=1) / cnt.clamp(min=1),
                       torch.zeros(n, dtype=torch.float64))
    np.testing.assert_allclose(red, want.numpy(), rtol=1e-12, atol=1e-12)
    assert np.all(np.abs(red) <= 1 + 1e-12)


@SETTINGS
@given(unit_shapes(), st.integers(0, 3), st.booleans())
def test_selection_keeps_the_k_best_under_the_total_order(shape, pinned_blocks, protect):
    n_max, b, d, G, n, w, seed, ties = shape
    k = (n_max - 1) * b
    rng = np.random.default_rng(seed)
    s = np.round(rng.standard_normal(n), 1 if ties else 12)   # rounding makes ties
    S = min(pinned_blocks, n_max - 1)
    pin = O.pinned_mask(n, S, b, w, protect)
    if pin.sum() > k:
        with pytest.raises(ValueError):
            O.select_keep(s, k, pin)
        return
    keep = O.select_keep(s, k, pin)
    assert len(keep) == k and np.all(np.diff(keep) > 0)
    assert set(np.flatnonzero(pin)) <= set(keep.tolist())
    # numpy's lexsort: pinned first, then score descending, then position
    order = np.lexsort((np.arange(n), -s, ~pin))
    assert sorted(order[:k].tolist()) == keep.tolist()
    # brute force on small units: no other k-subset holding P beats it
    free = [t for t in range(n) if not pin[t]]
    if len(free) <= 12:
        best = None
        for sub in itertools.combinations(free, k - int(pin.sum())):
            key = sorted(((-s[t], t) for t in sub))
            if best is None or key < best[0]:
                best = (key, sub)
        assert sorted(list(best[1]) + list(np.flatnonzero(pin))) == keep.tolist()


@SETTINGS
@given(unit_shapes())
def test_compaction_moves_byte_copies_and_the_global_row_follows(shape):
    n_max, b, d, G, n, w, seed, ties = shape
    if n < n_max * b:
        n = n_max * b                           # compaction needs the trigger
    k = (n_max - 1) * b
    rng = np.random.default_rng(seed)
    nb = n_max + 3
    table = list(rng.permutation(nb)[:n_max])
    pool = rng.integers(0, 2**16, size=(1, nb, 1, b, d), dtype=np.uint16)
    out = pool.copy()
    s = rng.standard_normal(n)
    keep = O.select_keep(s, k, np.zeros(n, dtype=bool))
    O.compact_unit(pool, out, table, table, 0, 0, keep, b)
    before = O.gather_rows(pool, table, 0, 0, n, b)
    after = O.gather_rows(out, table, 0, 0, n, b)
    assert after[:k].tobytes() == before[keep].tobytes()
    h = O.first_hole(keep)
    assert after[:h].tobytes() == before[:h].tobytes()       # rows below the hole
    assert after[k:].tobytes() == before[k:n].tobytes()       # the tail block
    other = [x for x in range(nb) if x not in table]
    assert out[:, other].tobytes() == pool[:, other].tobytes()
    # the global row moves with its tokens: sums and the zero tail
    g = rng.random(n)
    attn = rng.random(n)
    gn = O.update_global(g, attn, keep, k)
    assert abs(gn.sum() - (g[keep] + attn[keep]).sum()) < 1e-9
    assert np.all(gn[k:] == 0)


@settings(max_examples=40, deadline=None)
@given(st.integers(0, 2**31 - 1), st.integers(2, 5), st.sampled_from([1, 2, 4]))
def test_block_pool_conserves_blocks_over_random_histories(seed, n_max, b):
    rng = np.random.default_rng(seed)
    nb = 40
    bp = O.BlockPool(nb)
    for _ in range(6):
        s = int(rng.integers(0, n_max))
        members = int(rng.integers(1, 3))
        if len(bp.stack) < s + members * (n_max - s + 1):
            break
        shared = bp.alloc(s)
        tables = []
        for m in range(members):
            if m:
                for x in shared:
                    bp.incref(x)
            tables.append(shared + bp.alloc(n_max - s))
        stack, refs = list(bp.stack), list(bp.refcount)
        try:
            plan = bp.plan_compress(tables, [n_max * b] * members, n_max, b)
        except MemoryError:
            assert bp.stack == stack and bp.refcount == refs
            continue
        popped = len(plan.popped)
        bp.commit(plan)
        # pushes and pops balance for shared prefixes, shared counts unchanged
        assert len(plan.to_free) == popped
        for x in shared:
            assert bp.refcount[x] == refs[x]
        held = {x for x in range(nb) if bp.refcount[x] > 0}
        assert sorted(bp.stack + sorted(held)) == list(range(nb))
        assert len(set(bp.stack)) == len(bp.stack)
