"""GPU-vs-oracle parity harness (used by the GPU tests and by smoke()).

Runs the HIP path through the C ABI on a seeded workload, runs the CPU oracle
on host copies of the very same inputs and compares, unit by unit:

  attn   |gpu - ref| <= 1e-4 |ref| + 1e-12         (softmax column means)
  red    |gpu - ref| <= 1e-4 |ref| + 1e-6          (mean cosine, may be ~0)
  score  |gpu - ref| <= 1e-4 |ref| + 1e-6, and +inf exactly where pinned
  keep   (a) bit-exact equal to the oracle's top-k applied to the GPU's own
             fp32 scores (same precision takes the same decision);
         (b) differs from the oracle's own keep set only in tokens whose
             oracle score lies within 1e-4 of the oracle's k-th threshold;
  hole   equal to the first evicted position of the GPU keep set;
  pools  K and V byte-identical to the oracle's compaction with the GPU keep
         set (whole pools: untouched rows must keep their bytes too);
  global |gpu - ref| <= 1e-4 |ref| + 1e-6 with ref = g[keep] + attn_ref[keep].

The 1e-4 relative bound is the stated target for scores (fp32 accumulation
against a float64 reference); the absolute floors cover values that are
legitimately ~0 (a redundancy or a score that cancels).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

import oracle as O
import kv_cache_compression_paged_amd as Z
from kv_cache_compression_paged_amd import synth

ATTN_RTOL, ATTN_ATOL = 1e-4, 1e-12
RED_RTOL, RED_ATOL = 1e-4, 1e-6
SCORE_RTOL, SCORE_ATOL = 1e-4, 1e-6
BAND = 1e-4


@dataclass
class Case:
    spec: synth.Spec
    flags: int = 0
    n_tokens: Optional[Sequence[int]] = None      # default: n_max * b each
    max_blocks: Optional[int] = None
    global_override: Optional[np.ndarray] = None  # [R][L][Hkv][n_cap] or None
    identical_keys: bool = False
    use_block_manager: bool = False               # prefix plans from zp_bm
    outlier: Optional[Tuple[int, float]] = None   # (logical position, scale)
    weights: Optional[Tuple[float, float, float]] = None  # w_attn, w_global, w_red
    sm_scale: Optional[float] = None              # None: 1/sqrt(d)
    small_keys: Optional[float] = None            # scale of 6 rows per 3rd block


@dataclass
class Result:
    ok: bool
    failures: List[str] = field(default_factory=list)
    stats: Dict[str, float] = field(default_factory=dict)

    def fail(self, msg: str) -> None:
        self.ok = False
        if len(self.failures) < 20:
            self.failures.append(msg)


def _params_for(spec: synth.Spec, flags: int,
                weights: Optional[Tuple[float, float, float]] = None,
                sm_scale: Optional[float] = None) -> Tuple[Z.Params, O.Params]:
    dt = Z.ZP_BF16 if spec.dtype == "bf16" else Z.ZP_F32
    # the library receives the weights and the scale as fp32 fields: the
    # oracle is given those same values
    wa, wg, wr = (float(np.float32(x)) for x in (weights or (1.0, 0.5, 0.5)))
    sc = None if sm_scale is None else float(np.float32(sm_scale))
    zp = Z.make_params(spec.n_max, spec.window, spec.q_heads, dt, w_attn=wa,
                       w_global=wg, w_red=wr, sm_scale=sc or 0.0, flags=flags)
    op = O.Params(n_max=spec.n_max, block_size=spec.block_size,
                  window=spec.window, w_attn=wa, w_global=wg, w_red=wr,
                  sm_scale=sc,
                  causal=not (flags & Z.ZP_NONCAUSAL),
                  protect_window=bool(flags & Z.ZP_PROTECT_WINDOW))
    return zp, op


def build_inputs(case: Case, device: str = "cuda"):
    """Workload + host copies + device batch for a case."""
    spec = case.spec
    wl = synth.make(spec, device=device)
    R = spec.requests
    b = spec.block_size
    n_tok = np.asarray(case.n_tokens if case.n_tokens is not None
                       else [spec.n_tokens] * R, dtype=np.int32)
    max_blocks = case.max_blocks or spec.n_max
    need_blocks = int(np.max((n_tok + b - 1) // b))
    if need_blocks > max_blocks:
        raise ValueError("max_blocks too small for n_tokens")
    n_cap = max(wl.n_cap, int(n_tok.max()))
    tables = np.zeros((R, max_blocks), dtype=np.int32)
    base = wl.tables
    extra_pool = []
    if max_blocks > spec.n_max:
        # overshoot requests hold extra blocks taken from the unused pool tail
        used = set(base.reshape(-1).tolist())
        free = [x for x in range(spec.pool_blocks) if x not in used]
        extra_pool = free
    nxt = 0
    refc = wl.refcount.copy()
    for r in range(R):
        tables[r, :spec.n_max] = base[r]
        nb = (int(n_tok[r]) + b - 1) // b
        for j in range(spec.n_max, nb):
            tables[r, j] = extra_pool[nxt]
            refc[extra_pool[nxt]] += 1        # held by the request from now on
            nxt += 1
    wl.refcount = refc
    if case.identical_keys:
        wl.k_pool[:] = wl.k_pool[0, 0, 0, 0].clone()
    if case.outlier is not None:
        # one key per unit scaled up: its logits dwarf everything before it
        pos, scale = case.outlier
        for r in range(R):
            blk = int(tables[r, pos // b])
            wl.k_pool[:, blk, :, pos % b, :] *= scale
    if case.small_keys is not None:
        # rows 0..5 of every third block (all layers and heads) scaled down:
        # pairs of such keys have |a||c| below the 1e-8 clamp of the cosine
        # (scale 1e-6), or are zero vectors (scale 0)
        blocks = sorted(set(int(x) for x in tables.reshape(-1)[::3]))
        sel = torch.as_tensor(blocks, device=wl.k_pool.device)
        wl.k_pool[:, sel, :, 0:6, :] *= case.small_keys
    glob = wl.global_scores
    if n_cap != wl.n_cap:
        g2 = torch.rand((glob.shape[0], glob.shape[1], glob.shape[2], n_cap),
                        generator=torch.Generator(device=device).manual_seed(spec.seed + 7),
                        device=device, dtype=torch.float32)
        glob = g2
    if case.global_override is not None:
        glob = torch.from_numpy(np.ascontiguousarray(
            case.global_override.astype(np.float32))).to(device)
    # plan: block manager of the library (checked against the oracle's)
    bm_plan = None
    if case.use_block_manager:
        bm = Z.BlockManager(spec.pool_blocks)
        # replay the workload's ownership into the manager
        held = {}
        ids = bm.alloc(spec.pool_blocks)
        assert ids == list(range(spec.pool_blocks))
        for bid in range(spec.pool_blocks):
            c = int(refc[bid])
            if c == 0:
                bm.release([bid])
            else:
                for _ in range(c - 1):
                    bm.incref(bid)
        bm_plan = (bm, bm.plan_compress(tables, n_tok, spec.n_max, b))
        dst = bm_plan[1].dst_tables
        pinned = bm_plan[1].n_pinned
    else:
        dst = tables[:, :spec.n_max].copy()
        pinned = np.zeros(R, dtype=np.int32)
    host = {
        "k": synth.raw_numpy(wl.k_pool), "v": synth.raw_numpy(wl.v_pool),
        "q": synth.raw_numpy(wl.q_window), "g": glob.detach().cpu().numpy(),
    }
    dev = Z.DeviceBatch(
        slot=torch.from_numpy(wl.slots).to(device),
        n_tokens=torch.from_numpy(n_tok).to(device),
        src_table=torch.from_numpy(tables).to(device),
        dst_table=torch.from_numpy(np.ascontiguousarray(dst, dtype=np.int32)).to(device),
        n_pinned=torch.from_numpy(np.ascontiguousarray(pinned, dtype=np.int32)).to(device),
        num_slots=wl.q_window.shape[0], n_cap=n_cap)
    return wl, glob, host, dev, tables, dst, pinned, n_tok, bm_plan


def oracle_bookkeeping(spec, tables, n_tok, refcount):
    """The oracle's own plan for the same pool state."""
    bp = O.BlockPool(spec.pool_blocks)
    bp.alloc(spec.pool_blocks)
    # rebuild the stack exactly as the library replay did: release in id order
    for bid in range(spec.pool_blocks):
        bp.refcount[bid] = int(refcount[bid])
        if refcount[bid] == 0:
            bp.stack.append(bid)
    return bp, bp.plan_compress(tables.tolist(), n_tok.tolist(), spec.n_max,
                                spec.block_size)


def run_case(case: Case, device: str = "cuda") -> Result:
    spec = case.spec
    res = Result(ok=True)
    wl, glob, host, dev, tables, dst, pinned, n_tok, bm_plan = build_inputs(case, device)
    zparams, oparams = _params_for(spec, case.flags, case.weights, case.sm_scale)
    pool = Z.make_pool(wl.k_pool, wl.v_pool)
    R, L, H = spec.requests, spec.layers, spec.kv_heads
    U = R * L * H
    k = spec.keep
    out = Z.alloc_outputs(U, k, dev.n_cap, device, debug=True)
    ws = Z.alloc_workspace(pool, zparams, R, device)
    Z.zp_compress(pool, dev, wl.q_window, glob, zparams, out, ws)
    if not (case.flags & Z.ZP_UPDATE_GLOBAL):   # else the kernel updated the rows
        Z.zp_update_global(glob, pool, dev, out, zparams)
    torch.cuda.synchronize()
    err = Z.zp_workspace_error(ws)
    if err != Z.ZP_OK:
        res.fail(f"device error word {err}")
        return res
    g_keep = out.keep_idx.cpu().numpy()
    g_attn = out.attn.cpu().numpy()
    g_red = out.red.cpu().numpy()
    g_score = out.score.cpu().numpy()
    g_hole = out.first_hole.cpu().numpy()
    g_k = synth.raw_numpy(wl.k_pool)
    g_v = synth.raw_numpy(wl.v_pool)
    g_glob = glob.cpu().numpy()

    # bookkeeping: the library's plan must equal the oracle's plan
    if bm_plan is not None:
        bp, oplan = oracle_bookkeeping(spec, tables, n_tok, wl.refcount)
        bm, plan = bm_plan
        if not np.array_equal(np.asarray(oplan.dst_tables), plan.dst_tables):
            res.fail("dst tables differ from the oracle's plan")
        if list(oplan.n_pinned) != plan.n_pinned.tolist():
            res.fail("n_pinned differs from the oracle's plan")
        if oplan.popped != plan.targets() or oplan.to_free != plan.freed():
            res.fail("popped/freed blocks differ from the oracle's plan")
        bm.commit(plan)
        bp.commit(oplan)
        if bm.free_list() != bp.stack:
            res.fail("free list after commit differs from the oracle's")
        for bid in range(spec.pool_blocks):
            if bm.refcount(bid) != bp.refcount[bid]:
                res.fail(f"refcount of block {bid} differs")
                break

    batch = O.Batch(slots=np.arange(R), n_tokens=n_tok, src_tables=tables,
                    dst_tables=np.asarray(dst), n_pinned=np.asarray(pinned))
    elem = spec.dtype
    ref = O.compress(host["k"], host["v"], elem, host["q"], elem, host["g"],
                     batch, oparams)
    exp_k, exp_v = host["k"].copy(), host["v"].copy()
    exp_g = host["g"].astype(np.float64)
    worst = {"attn": 0.0, "red": 0.0, "score": 0.0, "global": 0.0}
    band_diffs = 0
    for (r, l, h), ur in ref["units"].items():
        u = (r * L + l) * H + h
        n = int(n_tok[r])
        ga, gr, gs = g_attn[u, :n], g_red[u, :n], g_score[u, :n]
        for name, gv, rv, rt, at in (("attn", ga, ur.attn, ATTN_RTOL, ATTN_ATOL),
                                     ("red", gr, ur.red, RED_RTOL, RED_ATOL)):
            err_ = np.abs(gv.astype(np.float64) - rv)
            tol = rt * np.abs(rv) + at
            worst[name] = max(worst[name], float(np.max(err_ / tol)))
            if np.any(err_ > tol):
                t = int(np.argmax(err_ - tol))
                res.fail(f"{name} unit {(r, l, h)} t={t}: gpu {gv[t]!r} ref {rv[t]!r}")
        fin = np.isfinite(ur.score)
        if not np.array_equal(fin, np.isfinite(gs)):
            res.fail(f"pinned set differs in unit {(r, l, h)}")
        else:
            err_ = np.abs(gs[fin].astype(np.float64) - ur.score[fin])
            tol = SCORE_RTOL * np.abs(ur.score[fin]) + SCORE_ATOL
            if err_.size:
                worst["score"] = max(worst["score"], float(np.max(err_ / tol)))
            if np.any(err_ > tol):
                res.fail(f"score unit {(r, l, h)} exceeds tolerance")
        keep = g_keep[u]
        pin = ~fin
        same_prec = O.select_keep(gs.astype(np.float64), k, pin)
        if not np.array_equal(keep, same_prec):
            res.fail(f"keep set of unit {(r, l, h)} is not the top-k of its own "
                     f"fp32 scores")
        diff = set(keep.tolist()) ^ set(ur.keep.tolist())
        if diff:
            free_kept = [float(ur.score[t]) for t in ur.keep if fin[t]]
            tau = min(free_kept) if free_kept else np.inf
            for t in diff:
                if abs(ur.score[t] - tau) > BAND:
                    res.fail(f"unit {(r, l, h)} token {t} outside the band "
                             f"differs (s={ur.score[t]}, tau={tau})")
            band_diffs += len(diff)
        if int(g_hole[u]) != O.first_hole(keep):
            res.fail(f"first hole of unit {(r, l, h)}")
        O.compact_unit(host["k"], exp_k, tables[r], dst[r], l, h, keep,
                       spec.block_size)
        O.compact_unit(host["v"], exp_v, tables[r], dst[r], l, h, keep,
                       spec.block_size)
        gref = O.update_global(host["g"][r, l, h], ur.attn, keep, k)
        gv = g_glob[r, l, h].astype(np.float64)
        err_ = np.abs(gv - gref)
        tol = 1e-4 * np.abs(gref) + 1e-6
        worst["global"] = max(worst["global"], float(np.max(err_ / tol)))
        if np.any(err_ > tol):
            res.fail(f"global scores of unit {(r, l, h)}")
        exp_g[r, l, h] = gref
    if g_k.tobytes() != exp_k.tobytes():
        bad = np.argwhere((g_k != exp_k).reshape(g_k.shape[:4] + (-1,)).any(-1))
        res.fail(f"K pool bytes differ at {bad[:5].tolist()}")
    if g_v.tobytes() != exp_v.tobytes():
        res.fail("V pool bytes differ")
    res.stats = dict(worst)
    res.stats["band_diffs"] = band_diffs
    return res
