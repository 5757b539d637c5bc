"""Host-side checks of the C ABI that need no GPU.

* libzipage.so loads and exports every function include/zipage.h declares;
* the C++ block manager (zp_bm_*) matches the oracle's bookkeeping exactly on
  random histories (pops, pushes, plans, commits, aborts);
* argument errors are reported with the documented status before anything
  is enqueued (so these calls never touch a device).
"""

import ctypes
import os
import re
import subprocess
from pathlib import Path

import numpy as np
import pytest

import oracle as O
import kv_cache_compression_paged_amd as Z

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zipage.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(zp_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = Z.lib()
    declared = _declared()
    assert len(declared) >= 20
    for name in declared:
        assert hasattr(lib, name), f"{name} not exported"
    nm = subprocess.run(["nm", "-D", "--defined-only", Z.LIB_PATH],
                        capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (zp_\w+)", nm))
    assert set(declared) <= exported
    assert set(Z.EXPORTED) == set(declared)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built library every entry point raises before doing any
    work: there is no fallback path."""
    monkeypatch.setattr(Z, "_lib", None)
    monkeypatch.setattr(Z, "LIB_PATH", str(tmp_path / "libzipage.so"))
    with pytest.raises(Z.ZipageError) as ei:
        Z.lib()
    assert ei.value.status == Z.ZP_EHIP and "not built" in str(ei.value)
    with pytest.raises(Z.ZipageError):
        Z.zp_compress_workspace_bytes(Z.KVPool(), Z.Params(), 1)
    with pytest.raises(Z.ZipageError):
        Z.BlockManager(8)

def test_status_strings():
    lib = Z.lib()
    for code, name in [(0, "ZP_OK"), (-1, "ZP_EINVAL"), (-2, "ZP_EUNSUPPORTED"),
                       (-3, "ZP_EWORKSPACE"), (-4, "ZP_ENOSPACE"), (-5, "ZP_EHIP"),
                       (-6, "ZP_EDEVICE"), (-7, "ZP_ESYNC")]:
        assert lib.zp_status_str(code).decode() == name
    assert lib.zp_status_str(-99).decode() == "ZP_UNKNOWN"


def test_every_declared_status_has_its_name_everywhere():
    """Each ZP_OK / ZP_E* code the header defines is named by zp_status_str
    and by the binding, and the binding's constant has the header's value."""
    header = (Path(__file__).resolve().parents[1] / "include" / "zipage.h").read_text()
    codes = {m.group(1): int(m.group(2)) for m in
             re.finditer(r"#define (ZP_(?:OK|E[A-Z]+))\s+(-?\d+)", header)}
    assert len(codes) >= 8 and codes["ZP_OK"] == 0
    lib = Z.lib()
    for name, code in codes.items():
        assert lib.zp_status_str(code).decode() == name
        assert getattr(Z, name) == code
        assert Z._status_name(code) == name


# ------------------------------------------------------- block manager ---

def _same_state(bm, bp):
    assert bm.free_list() == bp.stack
    assert [bm.refcount(i) for i in range(bm.num_blocks)] == bp.refcount


def test_block_manager_matches_oracle_random_histories():
    rng = np.random.default_rng(123)
    for trial in range(30):
        nb = int(rng.integers(20, 80))
        bm, bp = Z.BlockManager(nb), O.BlockPool(nb)
        n_max, b = int(rng.integers(2, 6)), int(rng.choice([1, 2, 4, 16]))
        reqs = []
        for _ in range(int(rng.integers(1, 4))):
            # a group sharing s leading blocks, then private blocks
            s = int(rng.integers(0, n_max))
            members = int(rng.integers(1, 4))
            if bm.free_count() < s + members * (n_max - s + 2):
                break
            shared = bm.alloc(s)
            assert shared == bp.alloc(s)
            for m in range(members):
                if m:
                    for x in shared:
                        bm.incref(x)
                        bp.incref(x)
                extra = int(rng.integers(0, 3))
                priv = bm.alloc(n_max - s + extra)
                assert priv == bp.alloc(n_max - s + extra)
                ntok = (n_max + extra) * b - int(rng.integers(0, b)) * (extra > 0)
                reqs.append((shared + priv, max(ntok, n_max * b)))
        _same_state(bm, bp)
        if not reqs:
            continue
        mb = max(len(t) for t, _ in reqs)
        tables = np.zeros((len(reqs), mb), dtype=np.int32)
        for i, (t, _) in enumerate(reqs):
            tables[i, :len(t)] = t
        ntoks = [n for _, n in reqs]
        try:
            oplan = bp.plan_compress([list(t) for t in tables], ntoks, n_max, b)
        except MemoryError:
            with pytest.raises(Z.ZipageError) as ei:
                bm.plan_compress(tables, ntoks, n_max, b)
            assert ei.value.status == Z.ZP_ENOSPACE
            _same_state(bm, bp)
            continue
        plan = bm.plan_compress(tables, ntoks, n_max, b)
        assert plan.dst_tables.tolist() == [list(x) for x in oplan.dst_tables]
        assert plan.n_pinned.tolist() == list(oplan.n_pinned)
        assert plan.targets() == oplan.popped
        assert plan.freed() == oplan.to_free
        if rng.random() < 0.3:
            bm.abort(plan)
            bp.stack.extend(reversed(oplan.popped))
        else:
            bm.commit(plan)
            bp.commit(oplan)
        _same_state(bm, bp)
        # conservation: every block is either free or held, exactly once
        free = bm.free_list()
        held = [i for i in range(nb) if bm.refcount(i) > 0]
        assert sorted(free + held) == list(range(nb))


def test_block_manager_errors_change_nothing():
    bm = Z.BlockManager(6)
    ids = bm.alloc(4)
    with pytest.raises(Z.ZipageError) as ei:
        bm.alloc(3)
    assert ei.value.status == Z.ZP_ENOSPACE
    assert bm.free_count() == 2
    with pytest.raises(Z.ZipageError):
        bm.incref(5)                      # free block
    with pytest.raises(Z.ZipageError):
        bm.release([ids[0], ids[0]])      # released twice: nothing changes
    assert bm.refcount(ids[0]) == 1
    with pytest.raises(Z.ZipageError):
        bm.plan_compress(np.array([ids]), [3], 4, 1)   # below trigger
    with pytest.raises(Z.ZipageError):
        bm.plan_compress(np.array([[0, 1, 2, 99]]), [4], 4, 1)  # bad id
    bm.release(ids)
    assert bm.free_count() == 6


def test_block_manager_rejects_shared_or_repeated_private_blocks():
    """The library planner refuses what the oracle's refuses (a block after
    the shared run with another holder, or listed twice in the call), with
    ZP_EINVAL and no state change."""
    bm, bp = Z.BlockManager(16), O.BlockPool(16)
    sh = bm.alloc(2)
    assert sh == bp.alloc(2)
    for x in sh:
        bm.incref(x)
        bp.incref(x)
    r0 = bm.alloc(4)
    assert r0 == bp.alloc(4)
    r1 = sh + bm.alloc(2)
    assert r1[2:] == bp.alloc(2)
    cases = [
        ([[r0[0], sh[1], r0[2], r0[3]]], [8]),
        ([r0, [r0[0]] + r1[1:]], [8, 8]),
        ([r1, [r1[0], r1[1], r1[2], r0[3]], r0], [8, 8, 8]),
        ([r0 + [sh[0]]], [9]),
    ]
    for tabs, ntok in cases:
        width = max(len(t) for t in tabs)
        arr = np.array([t + [0] * (width - len(t)) for t in tabs], dtype=np.int32)
        with pytest.raises(ValueError):
            bp.plan_compress(tabs, ntok, n_max=4, b=2)
        with pytest.raises(Z.ZipageError) as ei:
            bm.plan_compress(arr, ntok, 4, 2)
        assert ei.value.status == Z.ZP_EINVAL
        _same_state(bm, bp)
    plan = bm.plan_compress(np.array([r0, r1], dtype=np.int32), [8, 8], 4, 2)
    assert plan.n_pinned.tolist() == [0, 2]
    bm.abort(plan)


# ------------------------------------------------ argument validation ---

FAKE = 0x10000  # never dereferenced: every call below fails validation first


def _pool(**kw):
    d = dict(k=FAKE, v=FAKE, num_blocks=64, layers=2, kv_heads=2, block_size=16,
             head_dim=128, dtype=Z.ZP_BF16)
    d.update(kw)
    return Z.KVPool(**d)


def _params(**kw):
    d = dict(n_max=4, window=8, q_heads=8, q_dtype=Z.ZP_BF16, w_attn=1.0,
             w_global=0.5, w_red=0.5, sm_scale=0.0, flags=0)
    d.update(kw)
    return Z.Params(**d)


def _batch(**kw):
    d = dict(num_reqs=2, max_blocks=4, num_slots=2, n_cap=64, slot=FAKE,
             n_tokens=FAKE, src_table=FAKE, dst_table=FAKE, n_pinned=FAKE)
    d.update(kw)
    return Z.BatchStruct(**d)


def _compress(pool=None, batch=None, params=None, ws_bytes=1 << 20,
              q=FAKE, keep=FAKE, attn=FAKE, ws=0x100000):
    out = Z.CompressOut(keep, attn, None, None, None)
    return Z.lib().zp_compress(ctypes.byref(pool or _pool()),
                               ctypes.byref(batch or _batch()), q, FAKE,
                               ctypes.byref(params or _params()),
                               ctypes.byref(out), ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(pool=_pool(block_size=8)), Z.ZP_EUNSUPPORTED),
    (dict(pool=_pool(head_dim=96)), Z.ZP_EUNSUPPORTED),
    (dict(pool=_pool(dtype=7)), Z.ZP_EINVAL),
    (dict(pool=_pool(k=FAKE + 4)), Z.ZP_EINVAL),
    (dict(params=_params(q_heads=7)), Z.ZP_EINVAL),
    (dict(params=_params(q_dtype=Z.ZP_F32)), Z.ZP_EUNSUPPORTED),
    (dict(params=_params(n_max=1)), Z.ZP_EINVAL),
    (dict(params=_params(n_max=1025)), Z.ZP_EUNSUPPORTED),  # n_max * b > 16384
    (dict(params=_params(n_max=(1 << 31) - 1)), Z.ZP_EUNSUPPORTED),  # no int overflow
    (dict(params=_params(window=0)), Z.ZP_EINVAL),
    (dict(params=_params(flags=1 << 7)), Z.ZP_EINVAL),
    (dict(params=_params(window=49, flags=Z.ZP_PROTECT_WINDOW)), Z.ZP_EINVAL),
    (dict(params=_params(w_red=float("nan"))), Z.ZP_EINVAL),
    (dict(params=_params(window=64, q_heads=8)), Z.ZP_EUNSUPPORTED),  # w*G=256
    (dict(batch=_batch(max_blocks=3)), Z.ZP_EINVAL),
    (dict(batch=_batch(n_cap=32)), Z.ZP_EINVAL),
    (dict(batch=_batch(n_cap=20000)), Z.ZP_EUNSUPPORTED),
    (dict(batch=_batch(n_pinned=None)), Z.ZP_EINVAL),
    (dict(q=None), Z.ZP_EINVAL),
    (dict(keep=None), Z.ZP_EINVAL),
    (dict(ws_bytes=16), Z.ZP_EWORKSPACE),
    (dict(ws=0x100010), Z.ZP_EWORKSPACE),
])
def test_compress_rejects_bad_arguments_before_enqueue(kw, status):
    assert _compress(**kw) == status
    assert Z.last_error()


def test_compress_empty_batch_is_a_no_op():
    assert _compress(batch=_batch(num_reqs=0)) == Z.ZP_OK


def test_workspace_size_formula():
    # the error word only (compaction runs inside the scoring kernel, so no
    # per-unit hand-over array is needed); with ZP_SPLIT_UNITS on bf16, the
    # split-unit schedule's error word, ticket and abort flag, and 256 group
    # exchange slots of 8 parts x (192 rows + 512 candidates) 64-bit words,
    # whatever the batch
    assert Z.zp_compress_workspace_bytes(_pool(), _params(), 2) == 256
    assert Z.zp_compress_workspace_bytes(_pool(), _params(), 100) == 256
    split = 512 + 256 * (8 * 192 * 8 + 8 * 512 * 8)
    sp = _params(flags=Z.ZP_SPLIT_UNITS)
    assert Z.zp_compress_workspace_bytes(_pool(), sp, 2) == split
    assert Z.zp_compress_workspace_bytes(_pool(), sp, 100) == split
    f32 = _pool(dtype=Z.ZP_F32)
    assert Z.zp_compress_workspace_bytes(
        f32, _params(q_dtype=Z.ZP_F32, flags=Z.ZP_SPLIT_UNITS), 2) == 256


def test_split_flag_is_accepted_and_other_bits_are_not():
    assert _compress(params=_params(flags=Z.ZP_SPLIT_UNITS),
                     batch=_batch(num_reqs=0)) == Z.ZP_OK
    assert _compress(params=_params(flags=1 << 5), batch=_batch(num_reqs=0)) == Z.ZP_EINVAL


def test_decode_rejects_bad_arguments():
    lib = Z.lib()
    r = lib.zp_paged_decode(FAKE, FAKE, ctypes.byref(_pool(head_dim=80)), FAKE,
                            4, FAKE, 2, ctypes.byref(_params()), None)
    assert r == Z.ZP_EUNSUPPORTED
    r = lib.zp_paged_decode(FAKE, FAKE, ctypes.byref(_pool()), FAKE, 4, FAKE, 2,
                            ctypes.byref(_params(q_heads=3)), None)
    assert r == Z.ZP_EINVAL
    r = lib.zp_paged_decode(FAKE, FAKE, ctypes.byref(_pool()), FAKE, 4, FAKE, 0,
                            ctypes.byref(_params()), None)
    assert r == Z.ZP_OK


def test_capture_rejects_bad_arguments():
    lib = Z.lib()
    P = ctypes.byref

    def cap(q_window=FAKE, q=FAKE, slot=FAKE, pos=FAKE, R=2, L=2, S=4, d=128,
            params=None):
        return lib.zp_capture_queries(q_window, q, slot, pos, R, L, S, d,
                                      P(params or _params()), None)
    assert cap(d=80) == Z.ZP_EUNSUPPORTED
    assert cap(L=0) == Z.ZP_EINVAL
    assert cap(S=0) == Z.ZP_EINVAL
    assert cap(R=-1) == Z.ZP_EINVAL
    assert cap(params=_params(window=0)) == Z.ZP_EINVAL
    assert cap(params=_params(q_dtype=7)) == Z.ZP_EINVAL
    assert cap(slot=None) == Z.ZP_EINVAL
    assert cap(q=FAKE + 4) == Z.ZP_EINVAL           # misaligned
    assert cap(R=0, q=None, slot=None) == Z.ZP_OK   # empty batch: nothing to do


def test_window_ring_flag_is_accepted_by_validation():
    # an unknown flag bit is rejected; ZP_WINDOW_RING is known
    b = _batch(num_reqs=0)
    assert _compress(params=_params(flags=Z.ZP_WINDOW_RING), batch=b) == Z.ZP_OK
    assert _compress(params=_params(flags=1 << 7), batch=b) == Z.ZP_EINVAL


def test_decode_append_and_split_reject_bad_arguments():
    lib = Z.lib()
    P = ctypes.byref
    pool, prm = _pool(), _params()
    # append needs both new rows
    assert lib.zp_paged_decode_append(FAKE, FAKE, None, None, P(pool), FAKE, 4, FAKE, 2,
                                      P(prm), None) == Z.ZP_EINVAL
    assert lib.zp_paged_decode_append(FAKE, FAKE, FAKE, FAKE + 8, P(pool), FAKE, 4, FAKE,
                                      2, P(prm), None) == Z.ZP_EINVAL   # misaligned
    assert lib.zp_paged_decode_append(FAKE, FAKE, FAKE, FAKE, P(pool), FAKE, 4, FAKE, 0,
                                      P(prm), None) == Z.ZP_OK          # empty batch

    def split(splits, ws=0x100000, nbytes=1 << 30, k_new=None, v_new=None, R=2):
        return lib.zp_paged_decode_split(FAKE, FAKE, k_new, v_new, P(pool), FAKE, 4, FAKE,
                                         R, P(prm), splits, ws, nbytes, None)
    assert split(0) == Z.ZP_EINVAL
    assert split(257) == Z.ZP_EINVAL
    assert split(4, ws=None) == Z.ZP_EWORKSPACE
    assert split(4, ws=0x100010) == Z.ZP_EWORKSPACE                    # not 256-aligned
    assert split(4, nbytes=100) == Z.ZP_EWORKSPACE
    assert split(4, k_new=FAKE) == Z.ZP_EINVAL                          # k_new without v_new
    assert split(4, R=0) == Z.ZP_OK


def test_static_split_decode_refuses_oversized_partials_before_any_gpu_call():
    """The allocation-free split-K decode checks its partials against the
    library's static array first: beyond it the call fails with
    ZP_EWORKSPACE and touches nothing (so it runs without a GPU here)."""
    pool = Z.KVPool(FAKE, FAKE, 16, 32, 8, 16, 128, Z.ZP_BF16)
    params = Z.make_params(8, 32, 32, Z.ZP_BF16)
    lib = Z.lib()
    # 128 requests x 32 layers x 32 heads x 64 splits x 130 x 4 B > 64 MiB
    st = lib.zp_paged_decode_split_static(FAKE, FAKE, None, None, ctypes.byref(pool),
                                          FAKE, 8, FAKE, 128, ctypes.byref(params),
                                          64, None)
    assert st == Z.ZP_EWORKSPACE
    assert "static scratch" in Z.last_error()


def test_decode_workspace_formula():
    pool, prm = _pool(), _params()
    # R * layers * q_heads * splits * (head_dim + 2) floats; none for one split
    assert Z.zp_decode_workspace_bytes(pool, prm, 3, 1) == 0
    assert Z.zp_decode_workspace_bytes(pool, prm, 3, 5) == 3 * 2 * 8 * 5 * 130 * 4
