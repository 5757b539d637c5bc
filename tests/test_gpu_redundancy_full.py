"""GPU parity of the all-pairs redundancy ablation ([zh] §2.1, [fr] §2.E).

The kernel forms every cosine of a unit's keys, each pair of tiles once; its
same-block mean must equal the oracle's (and the compression kernel's
lightning score), its all-token mean the oracle's full-matrix mean. fp32
sums of cosines (the all-token sums are added atomically, in any order): the
bound is 1e-4 relative plus 1e-6 absolute (means near zero). Cases span one
to five panels of row tiles per unit, ragged last blocks, and keys of zero
or tiny norm, where the clamp of the norm product binds across tiles.
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

RTOL, ATOL = 1e-4, 1e-6


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CASES = [
    ("bf16 d128 near-duplicates", synth.scaled(synth.EIGHT_B, requests=2, layers=2,
                                               kv_heads=2, q_heads=8, n_max=24,
                                               pool_blocks=2 * 24 + 4), [0, 9]),
    ("bf16 d128 five panels", synth.scaled(synth.EIGHT_B, requests=2, layers=1,
                                           kv_heads=2, q_heads=8, n_max=72,
                                           pool_blocks=2 * 72 + 8), [0, 21]),
    ("fp32 d64", synth.TINY, [0]),
    ("bf16 d64", synth.scaled(synth.EIGHT_B, requests=2, layers=1, kv_heads=2,
                              q_heads=4, head_dim=64, n_max=10, pool_blocks=2 * 10 + 4,
                              near_dup=False), [1, 33]),
]


SMALL_NORMS = synth.scaled(synth.EIGHT_B, requests=2, layers=1, kv_heads=2, q_heads=8,
                           n_max=40, pool_blocks=2 * 40 + 8, near_dup=False)
CASES += [
    ("tiny-norm keys", SMALL_NORMS, [0, 5], 1e-6),
    ("zero-norm keys", SMALL_NORMS, [3, 0], 0.0),
]


@pytest.mark.parametrize("label,spec,extra,scale",
                         [c if len(c) == 4 else (*c, None) for c in CASES],
                         ids=[c[0] for c in CASES])
def test_all_pairs_redundancy_matches_oracle(label, spec, extra, scale):
    _say(f"[ablation] {label}")
    n = spec.n_tokens
    R = spec.requests
    n_tok = [n + extra[r % len(extra)] for r in range(R)]   # ragged last block
    case = P.Case(spec, n_tokens=n_tok, max_blocks=spec.n_max + 3, small_keys=scale)
    wl, glob, host, dev, tables, dst, pinned, n_arr, _ = P.build_inputs(case)
    zparams, _ = P._params_for(spec, 0)
    pool = Z.make_pool(wl.k_pool, wl.v_pool)
    L, H, b = spec.layers, spec.kv_heads, spec.block_size
    U = R * L * H
    red_b = torch.full((U, dev.n_cap), float("nan"), device="cuda")
    red_a = torch.full((U, dev.n_cap), float("nan"), device="cuda")
    ws = Z.alloc_workspace(pool, zparams, R, "cuda")
    Z.zp_redundancy_full(red_b, pool, dev, zparams, ws, red_all=red_a)
    # the compression kernel's lightning score on the same keys
    out = Z.alloc_outputs(U, spec.keep, dev.n_cap, "cuda", debug=True)
    Z.zp_compress(pool, dev, wl.q_window, glob, zparams, out, ws)
    torch.cuda.synchronize()
    assert Z.zp_workspace_error(ws) == Z.ZP_OK
    gb, ga, gl = red_b.cpu().numpy(), red_a.cpu().numpy(), out.red.cpu().numpy()
    for u in range(U):
        r, l, h = u // (L * H), (u // H) % L, u % H
        nu = int(n_arr[r])
        keys = O.widen(O.gather_rows(host["k"], tables[r], l, h, nu, b), spec.dtype)
        want_b, want_a = O.redundancy_all_pairs(keys, b, nu)
        assert np.all(np.abs(gb[u, :nu] - want_b) <= RTOL * np.abs(want_b) + ATOL), u
        assert np.all(np.abs(ga[u, :nu] - want_a) <= RTOL * np.abs(want_a) + ATOL), u
        assert np.all(np.abs(gb[u, :nu] - gl[u, :nu]) <= 2 * (RTOL * np.abs(want_b) + ATOL)), u
    _say(f"[ablation] {label}: {U} units match")


def test_same_block_mean_alone():
    """Without red_all only the diagonal tiles are formed: red_block must not
    change, and every other output row stays as it was."""
    spec = CASES[1][1]
    n = spec.n_tokens
    case = P.Case(spec, n_tokens=[n + 3, n], max_blocks=spec.n_max + 3)
    wl, glob, host, dev, tables, dst, pinned, n_arr, _ = P.build_inputs(case)
    zparams, _ = P._params_for(spec, 0)
    pool = Z.make_pool(wl.k_pool, wl.v_pool)
    U = spec.requests * spec.layers * spec.kv_heads
    red_b = torch.full((U, dev.n_cap), float("nan"), device="cuda")
    red_b2 = torch.full((U, dev.n_cap), float("nan"), device="cuda")
    red_a = torch.full((U, dev.n_cap), float("nan"), device="cuda")
    ws = Z.alloc_workspace(pool, zparams, spec.requests, "cuda")
    Z.zp_redundancy_full(red_b, pool, dev, zparams, ws, red_all=red_a)
    Z.zp_redundancy_full(red_b2, pool, dev, zparams, ws)
    torch.cuda.synchronize()
    assert Z.zp_workspace_error(ws) == Z.ZP_OK
    for u in range(U):
        nu = int(n_arr[u // (spec.layers * spec.kv_heads)])
        assert torch.equal(red_b[u, :nu], red_b2[u, :nu]), u
        assert bool(torch.isnan(red_b2[u, nu:]).all()), u
        assert bool(torch.isnan(red_a[u, nu:]).all()), u
    _say(f"[ablation] same-block mean alone: {U} units bit-identical")
