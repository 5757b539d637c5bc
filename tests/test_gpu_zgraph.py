"""HIP-graph capture of the library's calls.

The entry points allocate nothing and synchronise nothing, so a caller can
record them into a graph (a serving loop replays one per step). The calls are
captured once into a torch CUDAGraph (a hipGraph on ROCm) and replayed several
times. Between replays, eager work on the same stream restores the in-place
state (pools, global scores), fills the static inputs with new values and
poisons the outputs. Every replay must be bit-identical to an eager call on
the same inputs.
"""

import sys

import numpy as np
import pytest
import torch

import kv_cache_compression_paged_amd as Z
from kv_cache_compression_paged_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("schedule", [0, Z.ZP_SPLIT_UNITS], ids=["one-workgroup", "split-units"])
def test_compress_graph_replays_match_eager(schedule):
    # the split-unit schedule records two kernel nodes: the fill kernel that
    # clears the exchange area, then the persistent kernel (3 slices a unit)
    n_max = 96 if schedule else 16
    spec = synth.scaled(synth.EIGHT_B, requests=3, layers=2, kv_heads=2, q_heads=8,
                        n_max=n_max, pool_blocks=3 * n_max + 16)
    _say(f"[graph] compress {spec.name} (scaled), flags {schedule}")
    wl = synth.make(spec, device=DEV)
    R, L, H = spec.requests, spec.layers, spec.kv_heads
    U = R * L * H
    params = Z.make_params(spec.n_max, spec.window, spec.q_heads, Z.ZP_BF16,
                           flags=Z.ZP_UPDATE_GLOBAL | schedule)
    pool = Z.make_pool(wl.k_pool, wl.v_pool)
    tables = torch.from_numpy(wl.tables).to(DEV)
    batch = Z.DeviceBatch(slot=torch.from_numpy(wl.slots).to(DEV),
                          n_tokens=torch.from_numpy(wl.n_tokens).to(DEV),
                          src_table=tables, dst_table=tables.clone(),
                          n_pinned=torch.zeros(R, dtype=torch.int32, device=DEV),
                          num_slots=wl.global_scores.shape[0], n_cap=wl.n_cap)
    out = Z.alloc_outputs(U, spec.keep, wl.n_cap, DEV)
    ws = Z.alloc_workspace(pool, params, R, DEV)
    k0, v0 = wl.k_pool.clone(), wl.v_pool.clone()
    gen = torch.Generator(device=DEV)
    gen.manual_seed(spec.seed + 77)
    globs = [torch.rand(wl.global_scores.shape, generator=gen, device=DEV)
             for _ in range(3)]
    qwins = [wl.q_window.clone()] + [
        torch.randn(wl.q_window.shape, generator=gen, device=DEV).to(torch.bfloat16)
        for _ in range(2)]
    q_static = wl.q_window  # the captured call reads this buffer

    def restore(j):
        wl.k_pool.copy_(k0)
        wl.v_pool.copy_(v0)
        wl.global_scores.copy_(globs[j])
        q_static.copy_(qwins[j])
        out.keep_idx.fill_(-7)
        out.attn.fill_(float("nan"))
        out.first_hole.fill_(-7)

    def call():
        Z.zp_compress(pool, batch, q_static, wl.global_scores, params, out, ws)

    def snapshot():
        return [t.clone() for t in (out.keep_idx, out.attn, out.first_hole,
                                    wl.k_pool, wl.v_pool, wl.global_scores)]

    ref = []
    for j in range(3):
        restore(j)
        call()
        torch.cuda.synchronize()
        ref.append(snapshot())
    assert Z.zp_workspace_error(ws) == Z.ZP_OK
    # the three inputs give different results (the check below is not vacuous)
    assert not torch.equal(ref[0][0], ref[1][0]) or not torch.equal(ref[0][1], ref[1][1])

    restore(0)
    graph = _capture(call)
    names = ("keep_idx", "attn", "first_hole", "k_pool", "v_pool", "global")
    for rep in range(2):
        for j in (2, 0, 1):
            restore(j)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for name, got, want in zip(names, snapshot(), ref[j]):
                assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), \
                    f"replay {rep}/{j}: {name} differs from the eager call"
            _say(f"[graph] compress replay {rep}/{j} bit-identical to eager")
    assert Z.zp_workspace_error(ws) == Z.ZP_OK


def test_decode_append_graph_replays_match_eager():
    spec = synth.scaled(synth.EIGHT_B, requests=4, layers=2, kv_heads=2, q_heads=8,
                        n_max=8, pool_blocks=40)
    _say(f"[graph] decode with append {spec.name} (scaled)")
    wl = synth.make(spec, device=DEV)
    R, L, H, d = spec.requests, spec.layers, spec.kv_heads, spec.head_dim
    params = Z.make_params(spec.n_max, spec.window, spec.q_heads, Z.ZP_BF16)
    pool = Z.make_pool(wl.k_pool, wl.v_pool)
    # room for the appended token: lengths end inside the last block
    tables = torch.from_numpy(wl.tables).to(DEV)
    lens = torch.tensor([spec.n_tokens - 1 - 3 * r for r in range(R)], dtype=torch.int32,
                        device=DEV)
    k0, v0 = wl.k_pool.clone(), wl.v_pool.clone()
    gen = torch.Generator(device=DEV)
    gen.manual_seed(spec.seed + 78)
    draws = [tuple(torch.randn(shape, generator=gen, device=DEV).to(torch.bfloat16)
                   for shape in ((R, L, spec.q_heads, d), (R, L, H, d), (R, L, H, d)))
             for _ in range(3)]
    q, k_new, v_new = (torch.empty_like(t) for t in draws[0])
    out = torch.empty((R, L, spec.q_heads, d), dtype=torch.float32, device=DEV)

    def restore(j):
        wl.k_pool.copy_(k0)
        wl.v_pool.copy_(v0)
        for dst, src in zip((q, k_new, v_new), draws[j]):
            dst.copy_(src)
        out.fill_(float("nan"))

    def call():
        Z.zp_paged_decode_append(out, q, k_new, v_new, pool, tables, lens, params)

    ref = []
    for j in range(3):
        restore(j)
        call()
        torch.cuda.synchronize()
        ref.append((out.clone(), wl.k_pool.clone(), wl.v_pool.clone()))
    assert not torch.equal(ref[0][0], ref[1][0])

    restore(0)
    graph = _capture(call)
    for rep in range(2):
        for j in (1, 2, 0):
            restore(j)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for name, got, want in zip(("out", "k_pool", "v_pool"),
                                       (out, wl.k_pool, wl.v_pool), ref[j]):
                assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), \
                    f"replay {rep}/{j}: {name} differs from the eager call"
            _say(f"[graph] decode replay {rep}/{j} bit-identical to eager")
