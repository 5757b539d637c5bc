"""The allocation-free split-K decode (zp_paged_decode_split_static) against
the workspace one (zp_paged_decode_split), through the C ABI.

Both run the same kernels; the static entry point keeps the split partials
in the library's own device array instead of a caller workspace. Two calls
in a row on the static path (the second with fewer requests, fewer splits
and an appended token) must give bit-identical outputs and pool bytes to
the workspace path on the same inputs, and a call whose partials exceed the
static array must be refused before anything is enqueued.
"""

import sys

import numpy as np
import pytest
import torch

import kv_cache_compression_paged_amd as Z
from kv_cache_compression_paged_amd import synth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(spec, R, seed):
    dev = "cuda"
    wl = synth.make(spec, device=dev)
    rng = np.random.default_rng(seed)
    n = spec.n_tokens
    lens = np.asarray([n - 1, 1, 17, n - 16, 200, 33][:R], dtype=np.int32)
    lens = np.minimum(lens, n - 1)
    q = synth.decode_queries(spec, R, dev, seed)
    tables = torch.from_numpy(np.ascontiguousarray(wl.tables[:R])).to(dev)
    return wl, q, tables, torch.from_numpy(lens).to(dev), rng


def _run_pair(wl, q, tables, lens, params, splits, append, seed):
    """The static call and the workspace call on identical pools."""
    dev = "cuda"
    R, L = q.shape[0], q.shape[1]
    H = wl.k_pool.shape[2]
    d = q.shape[-1]
    k_new = v_new = None
    if append:
        g = torch.Generator(device=dev).manual_seed(seed)
        k_new = torch.randn((R, L, H, d), generator=g, device=dev).to(q.dtype)
        v_new = torch.randn((R, L, H, d), generator=g, device=dev).to(q.dtype)
    k_ref, v_ref = wl.k_pool.clone(), wl.v_pool.clone()
    out_s = torch.full((R, L, q.shape[2], d), float("nan"), dtype=torch.float32, device=dev)
    out_w = out_s.clone()
    pool_s = Z.make_pool(wl.k_pool, wl.v_pool)
    pool_w = Z.make_pool(k_ref, v_ref)
    nbytes = Z.zp_decode_workspace_bytes(pool_w, params, R, splits)
    assert nbytes <= Z.ZP_DECODE_STATIC_BYTES
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    _say(f"[no-alloc] R={R} splits={splits} append={append} partials={nbytes} B")
    Z.zp_paged_decode_split_static(out_s, q, pool_s, tables, lens, params, splits,
                                   k_new=k_new, v_new=v_new)
    Z.zp_paged_decode_split(out_w, q, pool_w, tables, lens, params, splits, ws,
                            k_new=k_new, v_new=v_new)
    torch.cuda.synchronize()
    assert not torch.isnan(out_s).any()
    assert torch.equal(out_s.view(torch.int32), out_w.view(torch.int32))
    assert torch.equal(wl.k_pool.view(torch.int16), k_ref.view(torch.int16))
    assert torch.equal(wl.v_pool.view(torch.int16), v_ref.view(torch.int16))


def test_static_split_decode_matches_the_workspace_call_twice():
    spec = synth.scaled(synth.EIGHT_B, requests=6, layers=3, kv_heads=2, q_heads=8,
                        n_max=40, pool_blocks=6 * 40 + 4)
    wl, q, tables, lens, _ = _inputs(spec, 6, 31)
    params = Z.make_params(spec.n_max, spec.window, spec.q_heads, Z.ZP_BF16)
    _run_pair(wl, q, tables, lens, params, splits=8, append=False, seed=1)
    # second call: smaller (3 requests, 4 splits) and with an appended token;
    # the scratch still holds the first call's partials
    _run_pair(wl, q[:3].contiguous(), tables[:3].contiguous(), lens[:3].contiguous(),
              params, splits=4, append=True, seed=2)


def test_static_split_decode_refuses_partials_beyond_the_array():
    spec = synth.scaled(synth.EIGHT_B, requests=2, layers=1, kv_heads=2, q_heads=8,
                        n_max=8, pool_blocks=16)
    wl = synth.make(spec, device="cuda")
    params = Z.make_params(spec.n_max, spec.window, spec.q_heads, Z.ZP_BF16)
    pool = Z.make_pool(wl.k_pool, wl.v_pool)
    # 4096 requests x 1 layer x 8 heads x 256 splits x 130 x 4 bytes > 64 MiB
    R = 4096
    tables = torch.zeros((R, spec.n_max), dtype=torch.int32, device="cuda")
    lens = torch.ones(R, dtype=torch.int32, device="cuda")
    q = torch.zeros((R, 1, spec.q_heads, spec.head_dim), dtype=torch.bfloat16, device="cuda")
    out = torch.full((R, 1, spec.q_heads, spec.head_dim), 7.0, dtype=torch.float32,
                     device="cuda")
    with pytest.raises(Z.ZipageError) as ei:
        Z.zp_paged_decode_split_static(out, q, pool, tables, lens, params, 256)
    assert ei.value.status == Z.ZP_EWORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
