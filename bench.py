"""Throughput of the Compressed-PagedAttention compression step on one GPU.

A step is one whole compression pass over the batch: zp_compress (score,
select, K/V compaction and, with ZP_UPDATE_GLOBAL, the global-score update in
one kernel; --separate-update runs zp_update_global as its own launch), for every
(request, layer, KV head) unit of the workload. The default workload is the
8B-like shape: 128 requests x 32 layers x 8 KV heads (32 query heads),
head_dim 128, b = 16, N_max = 256 (4096 tokens, keep 4080), w = 32, bf16
K/V/Q with near-duplicate keys, shuffled block tables. Inputs are resident in
HBM before timing starts; the pools are compacted in place, so each step
compresses the previous step's output (same shape, same trigger point).

Prints one JSON line: tokens compressed per second (value), algorithmic HBM
GB/s of the whole step, a roofline entry for the dominant kernel (kernel
durations from HIP events recorded on the launch stream during the timed
steps) and the CPU oracle timed on a bounded sample of the same workload.

After that line's timed steps, the same run times the tiny, small-model,
shared-prefix, long-context (8 requests of 16384 tokens) and overlap workloads
and reports them under "other_workloads".

With --workload overlap_512req_8grp the step is the two-stream case: 512
requests in 8 groups, one group (64 requests, the query-slot holders) is
compressed on stream C while the other 448 requests decode one token over all
32 layers on stream D. Each step times C alone, D alone and both together;
the line reports compressed tokens/s under overlap plus the three times.

With --workload capture_8b_32L_32q it times query-window capture alone (128
slot-holding requests x 32 layers x 32 query heads of 128, w = 32); with
--workload decode_8b_32L_8kv_32q the decode consumer (plain, with append, and
split-K on a long-context small batch); with --workload redundancy_ablation_8b
the all-pairs redundancy against the whole compression step on 1024 units;
with --workload engine_8b the model-free engine loop (scheduler, capture,
compression beside decode) at the 8B-like layout.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       [--cpu-seconds S] [--no-cpu]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "KV tokens compressed/sec + achieved HBM GB/s (frac of peak), 1 MI355X"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-seconds", type=float, default=0.0,
                    help="after the --warmup steps, keep taking untimed steps until "
                         "this many seconds of warm-up have passed (compression "
                         "workloads; 0: exactly --warmup steps)")
    ap.add_argument("--workload", default="8b_32L_8kv_32q_N4096")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--variant", choices=("causal", "noncausal", "protect"),
                    default="causal", help="window mask / protection variant")
    ap.add_argument("--separate-update", action="store_true",
                    help="run the global-score update as its own launch")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device copy first (counter scaling)")
    ap.add_argument("--headline-only", action="store_true",
                    help="time the 8B-like workload alone (skip the other workloads)")
    ap.add_argument("--split-units", action="store_true",
                    help="time the split-unit schedule (ZP_SPLIT_UNITS) instead of one "
                         "workgroup per unit")
    return ap.parse_args()


def unit_bytes(spec, M: np.ndarray) -> dict:
    """Algorithmic bytes per unit, summed over units, for one step.

    whole step: B_alg = s*d*(N + 4M) + s_q*w*G*d + 12*N_cap -- keys read once,
    the M moved K and V rows read and written, the window, the global row read
    for scoring plus read and written by the update. The kernels split it:
      compress:      s*d*(N + 4M) + s_q*w*G*d + 4*N_cap (global read)
      global_update: 8*N_cap (row read and written)
    so with the update inside the compression kernel (ZP_UPDATE_GLOBAL) the
    kernel's bytes are the step's B_alg. Outputs the method does not need in
    HBM to be consumed later (attention row, keep row) are not counted.
    """
    s = 2 if spec.dtype == "bf16" else 4
    d, N = spec.head_dim, spec.n_tokens
    G = spec.q_heads // spec.kv_heads
    wGd = spec.window * G * d * s
    U = M.size
    n_cap = N
    Msum = float(M.sum())
    return {
        "step": U * (s * d * N + wGd + 12 * n_cap) + 4.0 * s * d * Msum,
        "compress": U * (s * d * N + wGd + 4 * n_cap) + 4.0 * s * d * Msum,
        "global_update": U * (8 * n_cap),
    }


KERNEL_SOURCES = {
    "compress": ["compress.hip", "zp_device.h"],
    "compress_split": ["compress_split.hip", "zp_device.h"],
    "global_update": ["global_update.hip", "zp_device.h"],
    "paged_decode": ["decode.hip", "zp_device.h"],
    "capture": ["capture.hip", "zp_device.h"],
    "redundancy_full": ["redundancy_full.hip", "zp_device.h"],
}


def traffic_from_profile(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary of `kernel` on
    this workload, or None when there is none or the kernel's sources changed
    since the counters were taken (the summary records their hash)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"hbm_{kernel}_{workload}.txt")
    if not os.path.exists(path) or kernel not in KERNEL_SOURCES:
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            key, val = line.split(":", 1)
            fields[key.strip()] = val.split()[0] if val.split() else ""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "kv_cache_compression_paged_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if fields.get("source_sha256_16") != h.hexdigest()[:16]:
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(spec, wl, seconds: float) -> dict:
    """The oracle, unchanged, on a bounded seeded sample of units."""
    import oracle as O
    import torch
    from threadpoolctl import threadpool_info
    from kv_cache_compression_paged_amd import synth
    R, L, H, b = spec.requests, spec.layers, spec.kv_heads, spec.block_size
    n, k = spec.n_tokens, spec.keep
    G = spec.q_heads // H
    rng = np.random.default_rng(spec.seed + 99)
    order = rng.permutation(R * L * H)
    p = O.Params(n_max=spec.n_max, block_size=b, window=spec.window)
    tab = torch.from_numpy(wl.tables).to(wl.k_pool.device)
    done, t_cpu = 0, 0.0
    # the oracle as it stands: numpy's BLAS with its own default thread pool
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    blas_threads = max([i.get("num_threads", 1) for i in blas] or [1])
    blas_name = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in blas) or "none"
    for u in order:
        if t_cpu >= seconds and done >= 2:
            break
        u = int(u)
        r, l, h = u // (L * H), (u // H) % L, u % H
        blocks = tab[r].long()
        kr = synth.raw_numpy(wl.k_pool[l, blocks, h].reshape(n, -1))
        vr = synth.raw_numpy(wl.v_pool[l, blocks, h].reshape(n, -1))
        q = synth.raw_numpy(wl.q_window[r, l, :, h * G:(h + 1) * G])
        g = wl.global_scores[r, l, h].cpu().numpy()
        pk = kr.reshape(1, spec.n_max, 1, b, -1)
        pv = vr.reshape(1, spec.n_max, 1, b, -1)
        t0 = time.perf_counter()
        res = O.score_unit(O.widen(q, spec.dtype), O.widen(kr, spec.dtype),
                           g.astype(np.float64), n, 0, p)
        nk, nv = pk.copy(), pv.copy()
        table = list(range(spec.n_max))
        O.compact_unit(pk, nk, table, table, 0, 0, res.keep, b)
        O.compact_unit(pv, nv, table, table, 0, 0, res.keep, b)
        O.update_global(g, res.attn, res.keep, k)
        t_cpu += time.perf_counter() - t0
        done += 1
    tokens_per_s = done * n / (L * H) / t_cpu
    return {"value": tokens_per_s, "unit": "tokens/s", "cores": blas_threads,
            "kind": "oracle", "cpu": _cpu_model(), "host_cpus": os.cpu_count(),
            "blas": blas_name, "extrapolated": done < R * L * H,
            "units_timed": done, "units_in_workload": R * L * H,
            "sample": f"extrapolated linearly from {done} of {R * L * H} seeded "
                      f"(request, layer, kv_head) units of this workload: full "
                      f"oracle chain (score, select, K/V compaction, global "
                      f"update) in {t_cpu:.1f} s; numpy's BLAS on up to "
                      f"{blas_threads} threads, the rest of the oracle on one; "
                      f"a token covers {L * H} units"}


def decode_bytes(spec, lens: np.ndarray) -> float:
    """Algorithmic bytes of one decode call: K and V rows of every (request,
    layer, KV head) read once, the query read and the fp32 output written."""
    s = 2 if spec.dtype == "bf16" else 4
    d, L, H, Hq = spec.head_dim, spec.layers, spec.kv_heads, spec.q_heads
    R = lens.size
    return (2.0 * s * d * float(lens.sum()) * L * H
            + R * L * Hq * d * (s + 4))


def run_overlap(args, spec, steps: int, warm: int) -> dict:
    """Compression of one group overlapped with decoding of the others."""
    import torch
    import kv_cache_compression_paged_amd as Z
    from kv_cache_compression_paged_amd import synth
    dev = "cuda"
    groups = spec.compress_groups
    per = spec.requests // groups
    L, H = spec.layers, spec.kv_heads
    n, k = spec.n_tokens, spec.keep
    print(f"[bench] generating {spec.name} ({per} query slots)", file=sys.stderr,
          flush=True)
    t_gen = time.perf_counter()
    wl = synth.make(spec, device=dev, slots=per)
    torch.cuda.synchronize()
    print(f"[bench] generated in {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)
    dt = Z.ZP_BF16 if spec.dtype == "bf16" else Z.ZP_F32
    params = Z.make_params(spec.n_max, spec.window, spec.q_heads, dt)
    pool = Z.make_pool(wl.k_pool, wl.v_pool)
    Uc = per * L * H
    out = Z.alloc_outputs(Uc, k, wl.n_cap, dev)
    ws = Z.alloc_workspace(pool, params, per, dev)
    R_d = spec.requests - per
    q = torch.empty((R_d, L, spec.q_heads, spec.head_dim), dtype=wl.k_pool.dtype,
                    device=dev)
    dec = torch.empty((R_d, L, spec.q_heads, spec.head_dim), dtype=torch.float32,
                      device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(spec.seed + 500)
    rng = np.random.default_rng(spec.seed + 501)
    sc, sd = torch.cuda.Stream(), torch.cuda.Stream()
    compressed = set()
    rec = {"C": [], "D": [], "CD": [], "bytes_C": [], "bytes_D": []}

    def elapsed(a, b):
        return a.elapsed_time(b)

    for i in range(warm + steps):
        s = i % groups
        grp = np.arange(s * per, (s + 1) * per)
        rest = np.setdiff1d(np.arange(spec.requests), grp)
        # A-23 lengths: groups compressed earlier decode at k, others at
        # seeded lengths in [k+1, N-1]
        lens = np.where(np.isin(rest // per, list(compressed)), k,
                        rng.integers(k + 1, n, size=rest.size)).astype(np.int32)
        tab_c = torch.from_numpy(np.ascontiguousarray(wl.tables[grp])).to(dev)
        tab_d = torch.from_numpy(np.ascontiguousarray(wl.tables[rest])).to(dev)
        lens_dev = torch.from_numpy(lens).to(dev)
        batch = Z.DeviceBatch(
            slot=torch.arange(per, dtype=torch.int32, device=dev),
            n_tokens=torch.full((per,), n, dtype=torch.int32, device=dev),
            src_table=tab_c, dst_table=tab_c.clone(),
            n_pinned=torch.zeros(per, dtype=torch.int32, device=dev),
            num_slots=per, n_cap=wl.n_cap)
        holes = torch.empty((2, Uc), dtype=torch.int32, device=dev)
        q.copy_(torch.randn(q.shape, generator=gen, device=dev))
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(7)]

        def fresh_global(j):
            # each compression of the group sees fresh U[0,1) global scores
            wl.global_scores.copy_(torch.rand(wl.global_scores.shape, generator=gen,
                                              device=dev))
            torch.cuda.synchronize()
            out.first_hole = holes[j]

        # C alone
        fresh_global(0)
        ev[0].record(sc)
        Z.zp_compress(pool, batch, wl.q_window, wl.global_scores, params, out, ws, sc)
        Z.zp_update_global(wl.global_scores, pool, batch, out, params, sc)
        ev[1].record(sc)
        torch.cuda.synchronize()
        # D alone
        ev[2].record(sd)
        Z.zp_paged_decode(dec, q, pool, tab_d, lens_dev, params, sd)
        ev[3].record(sd)
        torch.cuda.synchronize()
        # both: D waits for C's start event, then the two run side by side
        fresh_global(1)
        ev[4].record(sc)
        sd.wait_event(ev[4])
        Z.zp_compress(pool, batch, wl.q_window, wl.global_scores, params, out, ws, sc)
        Z.zp_update_global(wl.global_scores, pool, batch, out, params, sc)
        Z.zp_paged_decode(dec, q, pool, tab_d, lens_dev, params, sd)
        ev[5].record(sc)
        ev[6].record(sd)
        torch.cuda.synchronize()
        if Z.zp_workspace_error(ws) != Z.ZP_OK:
            raise RuntimeError("device error in the overlap step")
        compressed.add(s)
        if i < warm:
            continue
        hole_np = holes.cpu().numpy().astype(np.int64)
        M = (k - hole_np).clip(min=0)
        rec["C"].append(elapsed(ev[0], ev[1]))
        rec["D"].append(elapsed(ev[2], ev[3]))
        rec["CD"].append(max(elapsed(ev[4], ev[5]), elapsed(ev[4], ev[6])))
        rec["bytes_C"].append(unit_bytes(spec, M[1])["step"])
        rec["bytes_D"].append(decode_bytes(spec, lens))
        print(f"[bench] step {i}: group {s} C {rec['C'][-1]:.2f} ms, D "
              f"{rec['D'][-1]:.2f} ms, C||D {rec['CD'][-1]:.2f} ms",
              file=sys.stderr, flush=True)
    t_c, t_d, t_cd = (float(np.median(rec[x])) for x in ("C", "D", "CD"))
    b_c, b_d = float(np.mean(rec["bytes_C"])), float(np.mean(rec["bytes_D"]))
    ach = (b_c + b_d) / (t_cd * 1e-3) / 1e9
    tokens = per * n
    result = {
        "metric": METRIC, "value": round(tokens / (t_cd * 1e-3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": round(t_cd, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": spec.dtype,
        "data": "synthetic",
        "config": {"workload": spec.name, "requests": spec.requests,
                   "groups": groups, "compressed_per_step": per,
                   "decoded_per_step": spec.requests - per, "layers": L,
                   "kv_heads": H, "q_heads": spec.q_heads,
                   "head_dim": spec.head_dim, "n_max": spec.n_max,
                   "tokens_per_request": n, "keep": k, "window": spec.window,
                   "parallelism": "single GPU, two streams"},
        "overlap": {"t_C_ms": round(t_c, 3), "t_D_ms": round(t_d, 3),
                    "t_CD_ms": round(t_cd, 3),
                    "gain": round((t_c + t_d) / t_cd, 3),
                    "compress_GBps_alone": round(b_c / (t_c * 1e-3) / 1e9, 1),
                    "decode_GBps_alone": round(b_d / (t_d * 1e-3) / 1e9, 1)},
        "achieved_GBps": round(ach, 1),
        "frac_of_peak": round(ach / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "kernel": "compress || decode",
                     "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                     "traffic": None,
                     "alg_bytes_per_launch": round(b_c + b_d)},
    }
    del wl, out, ws, q, dec
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return result


def run_capture(args):
    """Query-window capture at the 8B-like shape: 128 slot-holding requests,
    32 layers, 32 query heads of 128 (bf16), w = 32. One call moves each
    request's new-token queries of all layers into its ring rows."""
    import torch
    import kv_cache_compression_paged_amd as Z
    dev = "cuda"
    R, L, Hq, d, w = 128, 32, 32, 128, 32
    ring = torch.zeros((R, L, w, Hq, d), dtype=torch.bfloat16, device=dev)
    q = torch.randn((R, L, Hq, d), device=dev).to(torch.bfloat16)
    slot = torch.arange(R, dtype=torch.int32, device=dev)
    params = Z.make_params(256, w, Hq, Z.ZP_BF16)
    calls = max(args.steps, 1) * 20
    poss = [torch.full((R,), 4000 + i, dtype=torch.int32, device=dev)
            for i in range(calls + args.warmup)]
    for i in range(args.warmup):
        Z.zp_capture_queries(ring, q, slot, poss[i], params)
    torch.cuda.synchronize()
    Z.timing_read()
    Z.timing_enable(True)
    t0 = time.perf_counter()
    for i in range(calls):
        Z.zp_capture_queries(ring, q, slot, poss[args.warmup + i], params)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    Z.timing_enable(False)
    cnt, tot = Z.timing_read()["capture"]
    avg_ms = tot / cnt
    nbytes = 2.0 * R * L * Hq * d * 2
    ach = nbytes / (avg_ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "query rows captured/sec (query-window capture)",
        "value": round(R * L / (avg_ms * 1e-3), 1), "unit": "rows/s",
        "n_gpus": 1, "steps": calls, "warmup": args.warmup,
        "ms_per_step": round(avg_ms, 5), "wall_ms_per_call": round(elapsed * 1e3 / calls, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "capture_8b_32L_32q", "requests": R, "layers": L,
                   "q_heads": Hq, "head_dim": d, "window": w},
        "roofline": {"bound": "hbm", "kernel": "capture", "achieved": round(ach, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_from_profile("capture", "capture_8b_32L_32q"),
                     "alg_bytes_per_launch": round(nbytes)},
    }), flush=True)


def run_decode(args):
    """Decode consumer on the 8B-like pool: (a) 128 requests x 32 layers at the
    compressed length k = 4080, plain and with the new token appended; (b) a
    long-context, small batch (4 requests of 16384 tokens) with one wave per
    unit against split-K."""
    import torch
    import kv_cache_compression_paged_amd as Z
    from kv_cache_compression_paged_amd import synth
    spec = synth.EIGHT_B
    dev = "cuda"
    wl = synth.make(spec, device=dev)
    R, L, H, d = spec.requests, spec.layers, spec.kv_heads, spec.head_dim
    params = Z.make_params(spec.n_max, spec.window, spec.q_heads, Z.ZP_BF16)
    pool = Z.make_pool(wl.k_pool, wl.v_pool)
    reps = max(args.steps, 1)

    def timed(fn):
        for _ in range(max(args.warmup, 1)):
            fn()
        torch.cuda.synchronize()
        Z.timing_read()
        Z.timing_enable(True)
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        Z.timing_enable(False)
        cnt, tot = Z.timing_read()["paged_decode"]
        return tot / cnt

    def kv_bytes(lens, reqs):
        return 2.0 * 2 * d * float(np.sum(lens)) * L * H + reqs * L * spec.q_heads * d * (2 + 4)

    res = {}
    tab = torch.from_numpy(wl.tables).to(dev)
    lens = np.full(R, spec.keep, dtype=np.int32)
    lens_dev = torch.from_numpy(lens).to(dev)
    q = synth.decode_queries(spec, R, dev, spec.seed + 7)
    out = torch.empty((R, L, spec.q_heads, d), dtype=torch.float32, device=dev)
    k_new = torch.randn((R, L, H, d), device=dev).to(torch.bfloat16)
    v_new = torch.randn((R, L, H, d), device=dev).to(torch.bfloat16)
    b_plain = kv_bytes(lens, R)
    t = timed(lambda: Z.zp_paged_decode(out, q, pool, tab, lens_dev, params))
    res["plain_128req_len4080"] = {"ms": round(t, 4), "GBps": round(b_plain / (t * 1e-3) / 1e9, 1)}
    b_app = kv_bytes(lens + 1, R) + 2.0 * R * L * H * d * 2
    t = timed(lambda: Z.zp_paged_decode_append(out, q, k_new, v_new, pool, tab, lens_dev,
                                               params))
    res["append_128req_len4080"] = {"ms": round(t, 4), "GBps": round(b_app / (t * 1e-3) / 1e9, 1)}
    # long context: 4 requests of 1024 blocks each, tables from the same pool
    RL, nb = 4, 1024
    tl = torch.from_numpy(np.ascontiguousarray(
        wl.tables.reshape(-1)[:RL * nb].reshape(RL, nb))).to(dev)
    ll = np.full(RL, nb * 16, dtype=np.int32)
    ll_dev = torch.from_numpy(ll).to(dev)
    ql = synth.decode_queries(spec, RL, dev, spec.seed + 8)
    ol = torch.empty((RL, L, spec.q_heads, d), dtype=torch.float32, device=dev)
    b_long = kv_bytes(ll, RL)
    for splits in (1, 4, 16, 64):
        nbytes = Z.zp_decode_workspace_bytes(pool, params, RL, splits)
        ws = torch.empty(max(nbytes, 256) // 4 + 64, dtype=torch.int32, device=dev)
        t = timed(lambda: Z.zp_paged_decode_split(ol, ql, pool, tl, ll_dev, params, splits,
                                                  ws if splits > 1 else None))
        res[f"long_4req_len16384_splits{splits}"] = {
            "ms": round(t, 4), "GBps": round(b_long / (t * 1e-3) / 1e9, 1)}
    best = res["plain_128req_len4080"]
    print(json.dumps({
        "metric": "paged decode KV GB/s (consumer of the compressed cache)",
        "value": best["GBps"], "unit": "GB/s", "n_gpus": 1, "steps": reps,
        "warmup": args.warmup, "ms_per_step": best["ms"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode_8b_32L_8kv_32q", "layers": L, "kv_heads": H,
                   "q_heads": spec.q_heads, "head_dim": d},
        "roofline": {"bound": "hbm", "kernel": "paged_decode", "achieved": best["GBps"],
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(best["GBps"] / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_from_profile("paged_decode", "decode_8b_32L_8kv_32q"),
                     "alg_bytes_per_launch": round(b_plain)},
        "cases": res,
    }), flush=True)


def all_pairs_flops(units: int, n: int, d: int, b: int = 16) -> float:
    """MFMA work of the all-pairs cosine matrix as the kernel forms it: every
    pair of b-row key tiles once (the matrix is symmetric), nt (nt + 1) / 2
    tile products of 2 b^2 d flops per unit, nt = ceil(n / b)."""
    nt = (n + b - 1) // b
    return units * (nt * (nt + 1) / 2) * 2.0 * b * b * d


def run_redundancy_ablation(args):
    """All-pairs redundancy (the score lightning replaces) against the whole
    compression step on the same units: 4 requests x 32 layers x 8 KV heads of
    the 8B-like workload, N = 4096."""
    import torch
    import kv_cache_compression_paged_amd as Z
    from kv_cache_compression_paged_amd import synth
    spec = synth.scaled(synth.EIGHT_B, requests=4, pool_blocks=4 * 256)
    dev = "cuda"
    wl = synth.make(spec, device=dev)
    R, L, H, d, n = spec.requests, spec.layers, spec.kv_heads, spec.head_dim, spec.n_tokens
    U = R * L * H
    params = Z.make_params(spec.n_max, spec.window, spec.q_heads, Z.ZP_BF16)
    pool = Z.make_pool(wl.k_pool, wl.v_pool)
    tab = torch.from_numpy(wl.tables).to(dev)
    batch = Z.DeviceBatch(slot=torch.arange(R, dtype=torch.int32, device=dev),
                          n_tokens=torch.full((R,), n, dtype=torch.int32, device=dev),
                          src_table=tab, dst_table=tab.clone(),
                          n_pinned=torch.zeros(R, dtype=torch.int32, device=dev),
                          num_slots=R, n_cap=n)
    ws = Z.alloc_workspace(pool, params, R, dev)
    red_b = torch.empty((U, n), device=dev)
    red_a = torch.empty((U, n), device=dev)
    out = Z.alloc_outputs(U, spec.keep, n, dev)
    reps = max(args.steps, 1)

    def timed(fn, kind):
        fn()
        torch.cuda.synchronize()
        Z.timing_read()
        Z.timing_enable(True)
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        Z.timing_enable(False)
        cnt, tot = Z.timing_read()[kind]
        return tot / cnt

    t_full = timed(lambda: Z.zp_redundancy_full(red_b, pool, batch, params, ws, red_all=red_a),
                   "redundancy_full")
    t_comp = timed(lambda: Z.zp_compress(pool, batch, wl.q_window, wl.global_scores, params,
                                         out, ws), "compress")
    if Z.zp_workspace_error(ws) != Z.ZP_OK:
        raise RuntimeError("device error in the ablation run")
    flops_full = all_pairs_flops(U, n, d)
    print(json.dumps({
        "metric": "all-pairs redundancy vs lightning (whole compression step), same units",
        "value": round(t_full / t_comp, 2), "unit": "x slower than the full compression",
        "n_gpus": 1, "steps": reps, "warmup": 1, "ms_per_step": round(t_full, 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "redundancy_ablation_8b", "units": U, "tokens": n,
                   "head_dim": d},
        "all_pairs_ms": round(t_full, 4), "compress_ms": round(t_comp, 4),
        "all_pairs_TFLOPs": round(flops_full / (t_full * 1e-3) / 1e12, 1),
        "roofline": {"bound": "mfma", "kernel": "redundancy_full",
                     "achieved": round(flops_full / (t_full * 1e-3) / 1e12, 1),
                     "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(flops_full / (t_full * 1e-3) / 1e12 / 2500.0, 4),
                     "traffic": traffic_from_profile("redundancy_full", "redundancy_ablation_8b"),
                     "alg_flops_per_launch": flops_full},
    }), flush=True)


def run_redundancy_sweep(args):
    """Time against N_max of the all-pairs redundancy and of the whole
    lightning compression step (score, select, compaction; the lightning
    score is fused into its key sweep) on the same units: 4 requests x 32
    layers x 8 KV heads (1024 units) of the 8B-like layout, b = 16, N_max in
    {64, ..., 1024}. Fits t ~ N_max^p by least squares in log-log space: the
    pages' claim is O(N^2 b^2) for the all-pairs score against O(N b^2) for
    the lightning one ([zh] §2.1)."""
    import torch
    import kv_cache_compression_paged_amd as Z
    from kv_cache_compression_paged_amd import synth
    dev = "cuda"
    reps = max(args.steps, 1)
    rows = []
    for n_max in (64, 128, 256, 512, 1024):
        spec = synth.scaled(synth.EIGHT_B, requests=4, n_max=n_max, pool_blocks=4 * n_max)
        wl = synth.make(spec, device=dev)
        R, L, H, d, n = spec.requests, spec.layers, spec.kv_heads, spec.head_dim, spec.n_tokens
        U = R * L * H
        params = Z.make_params(spec.n_max, spec.window, spec.q_heads, Z.ZP_BF16)
        pool = Z.make_pool(wl.k_pool, wl.v_pool)
        tab = torch.from_numpy(wl.tables).to(dev)
        batch = Z.DeviceBatch(slot=torch.arange(R, dtype=torch.int32, device=dev),
                              n_tokens=torch.full((R,), n, dtype=torch.int32, device=dev),
                              src_table=tab, dst_table=tab.clone(),
                              n_pinned=torch.zeros(R, dtype=torch.int32, device=dev),
                              num_slots=R, n_cap=n)
        ws = Z.alloc_workspace(pool, params, R, dev)
        red_b = torch.empty((U, n), device=dev)
        red_a = torch.empty((U, n), device=dev)
        out = Z.alloc_outputs(U, spec.keep, n, dev)

        def timed(fn, kind):
            fn()
            torch.cuda.synchronize()
            Z.timing_read()
            Z.timing_enable(True)
            for _ in range(reps):
                fn()
            torch.cuda.synchronize()
            Z.timing_enable(False)
            cnt, tot = Z.timing_read()[kind]
            return tot / cnt

        t_all = timed(lambda: Z.zp_redundancy_full(red_b, pool, batch, params, ws,
                                                   red_all=red_a), "redundancy_full")
        t_comp = timed(lambda: Z.zp_compress(pool, batch, wl.q_window, wl.global_scores,
                                             params, out, ws), "compress")
        if Z.zp_workspace_error(ws) != Z.ZP_OK:
            raise RuntimeError("device error in the sweep")
        flops = all_pairs_flops(U, n, d)
        rows.append({"n_max": n_max, "tokens": n, "all_pairs_ms": round(t_all, 4),
                     "compress_ms": round(t_comp, 4),
                     "all_pairs_TFLOPs": round(flops / (t_all * 1e-3) / 1e12, 1),
                     "ratio": round(t_all / t_comp, 2)})
        print(f"[bench] sweep N_max {n_max}: all-pairs {t_all:.3f} ms, compress "
              f"{t_comp:.3f} ms", file=sys.stderr, flush=True)
        del wl, out, red_b, red_a, batch, pool
        torch.cuda.empty_cache()
    x = np.log([r["n_max"] for r in rows])
    p_all = float(np.polyfit(x, np.log([r["all_pairs_ms"] for r in rows]), 1)[0])
    p_comp = float(np.polyfit(x, np.log([r["compress_ms"] for r in rows]), 1)[0])
    best = max(r["all_pairs_TFLOPs"] for r in rows)
    print(json.dumps({
        "metric": "time against N_max: all-pairs redundancy vs the lightning compression step",
        "value": round(p_all, 3), "unit": "fitted exponent of the all-pairs time",
        "n_gpus": 1, "steps": reps, "warmup": 1, "ms_per_step": rows[-1]["all_pairs_ms"],
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "redundancy_sweep_1024units", "units": 1024,
                   "block_size": 16, "head_dim": 128, "n_max": [r["n_max"] for r in rows]},
        "exponent_all_pairs": round(p_all, 3), "exponent_compress": round(p_comp, 3),
        "rows": rows,
        "roofline": {"bound": "mfma", "kernel": "redundancy_full", "achieved": best,
                     "peak": 2500.0, "unit": "TFLOP/s", "frac": round(best / 2500.0, 4),
                     "traffic": None, "alg_bytes_per_launch": None},
    }), flush=True)


def run_engine(args):
    """The engine loop at the 8B-like layout (32 layers, 8 KV heads, 32 query
    heads of 128, b = 16, N_max = 256, w = 32): 96 running requests, each
    holding one of 96 query slots, prompts U[3800, 4064) tokens (just under
    the slot threshold) and generations U[200, 1200): after the warm-up every
    request compresses each time it fills its tail block, beside the decode of
    the others. Random K/V rows and queries stand in for a model. Timed over
    K steps after W warm-up steps; reports decode tokens/s, compressed tokens/s
    and the time of each stream."""
    import torch
    from kv_cache_compression_paged_amd.sim import Engine, EngineConfig
    cfg = EngineConfig(layers=32, kv_heads=8, q_heads=32, head_dim=128, block_size=16,
                       n_max=256, window=32, num_blocks=96 * 256 + 2048, query_slots=96,
                       max_running=96, max_blocks=340, seed=2024,
                       prefill_bank_blocks=320)
    eng = Engine(cfg)
    rng = np.random.default_rng(7)
    nreq = 2048
    for rid in range(nreq):
        eng.submit(rid, int(rng.integers(3800, 4064)), int(rng.integers(200, 1200)))
    warm, steps = max(args.warmup, 1) * 150, max(args.steps, 1) * 12
    t_w = time.perf_counter()
    for i in range(warm):
        eng.step()
        if i % 50 == 49:
            print(f"[bench] engine warm-up step {i + 1}: {eng.sched.stats()}",
                  file=sys.stderr, flush=True)
    print(f"[bench] engine warm-up {warm} steps in {time.perf_counter() - t_w:.1f} s",
          file=sys.stderr, flush=True)
    s0 = eng.sched.stats()
    for key in eng.time:
        eng.time[key] = 0.0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        eng.step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    s1 = eng.sched.stats()
    d = {k: s1[k] - s0[k] for k in ("tokens", "compressions", "preemptions",
                                   "restricted_steps", "admitted", "finished")}
    print(json.dumps({
        "metric": "engine loop: decode tokens/s with compression beside decoding",
        "value": round(d["tokens"] / el, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warm, "ms_per_step": round(el * 1e3 / steps, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "engine_8b_96run_96slots", "layers": 32, "kv_heads": 8,
                   "q_heads": 32, "head_dim": 128, "n_max": 256, "window": 32,
                   "query_slots": 96, "max_running": 96},
        "per_step": {k: round(v / steps, 3) for k, v in d.items()},
        "stream_ms_per_step": {k: round(v / steps, 3) for k, v in eng.time.items()},
        "compressed_tokens_per_s": round(d["compressions"] * 4096 / el, 1),
    }), flush=True)


def measure_compress(spec, args, steps: int, warm: int, with_cpu: bool,
                     with_copy: bool = True, warm_min_s: float = 0.0) -> dict:
    """Times `steps` compression steps of one workload and returns its JSON
    record (the device memory of the workload is released on return).
    After the `warm` warm-up steps, more untimed steps run until `warm_min_s`
    seconds of warm-up have passed (0: exactly `warm`): the device takes a
    few hundred milliseconds of this load to reach its steady clocks."""
    import torch
    import kv_cache_compression_paged_amd as Z
    from kv_cache_compression_paged_amd import synth
    dev = "cuda"
    print(f"[bench] generating {spec.name}", file=sys.stderr, flush=True)
    t_gen = time.perf_counter()
    wl = synth.make(spec, device=dev)
    torch.cuda.synchronize()
    print(f"[bench] generated in {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)
    R, L, H = spec.requests, spec.layers, spec.kv_heads
    U = R * L * H
    k, n = spec.keep, spec.n_tokens
    dt = Z.ZP_BF16 if spec.dtype == "bf16" else Z.ZP_F32
    # the step's global-score update runs inside the compression kernel
    # (ZP_UPDATE_GLOBAL: the same update zp_update_global applies)
    vflags = {"causal": 0, "noncausal": Z.ZP_NONCAUSAL,
              "protect": Z.ZP_PROTECT_WINDOW}[args.variant]
    vflags |= Z.ZP_SPLIT_UNITS if args.split_units else 0
    params = Z.make_params(spec.n_max, spec.window, spec.q_heads, dt,
                           flags=vflags | (0 if args.separate_update else Z.ZP_UPDATE_GLOBAL))
    pool = Z.make_pool(wl.k_pool, wl.v_pool)
    tables = torch.from_numpy(wl.tables).to(dev)
    if spec.shared_blocks:
        # shared prefixes: the library's block manager plans the targets once;
        # sources are never written in this mode, so every step repeats the
        # same compression into the same targets
        bm = Z.BlockManager(spec.pool_blocks)
        bm.alloc(spec.pool_blocks)
        for bid in range(spec.pool_blocks):
            c = int(wl.refcount[bid])
            if c == 0:
                bm.release([bid])
            for _ in range(c - 1):
                bm.incref(bid)
        plan = bm.plan_compress(wl.tables, wl.n_tokens, spec.n_max, spec.block_size)
        dst_table = torch.from_numpy(np.ascontiguousarray(plan.dst_tables, dtype=np.int32)).to(dev)
        n_pinned = torch.from_numpy(np.ascontiguousarray(plan.n_pinned, dtype=np.int32)).to(dev)
    else:
        dst_table = tables.clone()
        n_pinned = torch.zeros(R, dtype=torch.int32, device=dev)
    batch = Z.DeviceBatch(
        slot=torch.from_numpy(wl.slots).to(dev),
        n_tokens=torch.from_numpy(wl.n_tokens).to(dev),
        src_table=tables, dst_table=dst_table, n_pinned=n_pinned,
        num_slots=R, n_cap=wl.n_cap)
    out = Z.alloc_outputs(U, k, wl.n_cap, dev)
    ws = Z.alloc_workspace(pool, params, R, dev)
    holes = torch.empty((warm + steps, U), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    # Every step gets its own global-score rows drawn U[0,1) like the
    # workload's first step (resident before timing). K/V stay in place, so a
    # step compresses the previous step's compacted pools at the same trigger
    # point; fresh global scores keep the eviction pattern of a fresh batch.
    gen = torch.Generator(device=dev)
    gen.manual_seed(spec.seed + 500)
    globs = [wl.global_scores]
    for _ in range(warm + steps - 1):
        globs.append(torch.rand(wl.global_scores.shape, generator=gen,
                                device=dev, dtype=torch.float32))
    copy_gbps = None
    if with_copy:
        # the device's copy rate as torch's own device-to-device copy gives
        # it (2 GiB); this is not a peak: the step's traffic mix runs faster
        csrc = torch.empty(1 << 29, dtype=torch.float32, device=dev).fill_(1.0)
        cdst = torch.empty_like(csrc)
        cdst.copy_(csrc)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            cdst.copy_(csrc)
        e1.record()
        torch.cuda.synchronize()
        copy_gbps = 5 * 2 * csrc.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del csrc, cdst
    if args.copy_calibration:
        # a plain copy of known size, for scaling the HBM byte counters
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(i, glob=None):
        glob = globs[i] if glob is None else glob
        out.first_hole = holes[i]
        Z.zp_compress(pool, batch, wl.q_window, glob, params, out, ws,
                      stream)
        if args.separate_update:
            Z.zp_update_global(glob, pool, batch, out, params, stream)

    t_w = time.perf_counter()
    for i in range(warm):
        step(i)
    torch.cuda.synchronize()
    extra = 0
    if warm_min_s > 0:
        # Extra warm-up steps must leave the pool as the timed steps expect
        # it (in place, every step compacts the previous step's result, and
        # hundreds of them would pile up stale tail copies and shift the
        # holes): global rows of 1e6 below k and 0 from k on make every unit
        # evict exactly its tail, so it sweeps and selects but moves no row.
        # (The update keeps that pattern: 1e6 + attn below k, 0 after.)
        g_warm = torch.zeros_like(globs[0])
        g_warm[..., :k] = 1e6
        while time.perf_counter() - t_w < warm_min_s and extra < 1000:
            step(0, g_warm)
            torch.cuda.synchronize()
            extra += 1
        del g_warm
    if Z.zp_workspace_error(ws) != Z.ZP_OK:
        raise RuntimeError("device error during warm-up")
    Z.timing_read()  # drop anything recorded before
    Z.timing_enable(True)
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    marks[0].record(stream)
    for i in range(warm, warm + steps):
        step(i)
        marks[i - warm + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = np.array([marks[j].elapsed_time(marks[j + 1]) for j in range(steps)])
    Z.timing_enable(False)
    kern = Z.timing_read()
    if Z.zp_workspace_error(ws) != Z.ZP_OK:
        raise RuntimeError("device error during the timed steps")
    print(f"[bench] {spec.name}: {steps} steps in {elapsed:.3f} s", file=sys.stderr,
          flush=True)

    hole_np = holes[warm:].cpu().numpy().astype(np.int64)
    M = (k - hole_np).clip(min=0)                      # moved rows per unit
    if spec.shared_blocks:   # rows [S*b, k) go to the targets
        pin = np.repeat(batch.n_pinned.cpu().numpy().astype(np.int64), L * H)
        M = np.broadcast_to(k - pin * spec.block_size, hole_np.shape).copy()
    per_step = [unit_bytes(spec, M[i]) for i in range(steps)]
    if not args.separate_update:   # the update's bytes are the compression kernel's
        for p in per_step:
            p["compress"] += p.pop("global_update")
    alg = {key: float(np.mean([p[key] for p in per_step])) for key in per_step[0]}
    ms_step = elapsed * 1e3 / steps
    tokens_step = float(np.sum(wl.n_tokens))
    value = tokens_step * steps / elapsed
    gbps = alg["step"] / (ms_step * 1e-3) / 1e9

    kernels = {}
    for name, (cnt, tot) in kern.items():
        if cnt == 0:
            continue
        avg = tot / cnt
        b = alg.get(name)
        kernels[name] = {"launches": cnt, "avg_ms": round(avg, 4),
                         "alg_GBps": round(b / (avg * 1e-3) / 1e9, 1) if b else None}
    dom = max(kernels, key=lambda x: kernels[x]["avg_ms"] * kernels[x]["launches"])
    dom_ach = kernels[dom]["alg_GBps"]
    # counter summaries are per kernel: the split schedule's launch is its own
    prof_kernel = "compress_split" if (args.split_units and dom == "compress") else dom
    traffic = traffic_from_profile(prof_kernel, spec.name)
    roofline = {"bound": "hbm", "kernel": prof_kernel, "achieved": dom_ach,
                "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(dom_ach / HBM_PEAK_GBPS, 4),
                "traffic": traffic,
                "alg_bytes_per_launch": round(alg[dom]),
                "traffic_GBps": (round(traffic / (kernels[dom]["avg_ms"] * 1e-3) / 1e9, 1)
                                 if traffic else None)}
    # MFMA work of the scoring (window logits + block Grams, counted once):
    # 2*w*G*d*N + 2*b*d*N flops per unit
    G = spec.q_heads // spec.kv_heads
    flops = U * (2.0 * spec.window * G * spec.head_dim * n
                 + 2.0 * spec.block_size * spec.head_dim * n)
    t_c = kernels["compress"]["avg_ms"] * 1e-3
    peak_tf = 2500.0 if spec.dtype == "bf16" else 157.3
    mfma = {"alg_TFLOPs": round(flops / t_c / 1e12, 1), "peak_TFLOPs": peak_tf,
            "frac": round(flops / t_c / 1e12 / peak_tf, 4)}
    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warm + extra,
        "ms_per_step": round(ms_step, 3),
        "ms_step_median": round(float(np.median(step_ms)), 3),
        "ms_step_min": round(float(step_ms.min()), 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": spec.dtype,
        "data": "synthetic",
        "config": {"workload": spec.name, "requests": R, "layers": L,
                   "kv_heads": H, "q_heads": spec.q_heads,
                   "head_dim": spec.head_dim, "block_size": spec.block_size,
                   "n_max": spec.n_max, "tokens_per_request": n,
                   "keep": k, "window": spec.window, "units": U,
                   "variant": args.variant,
                   "schedule": "split units" if args.split_units else "one workgroup per unit",
                   "parallelism": "single GPU"},
        "achieved_GBps": round(gbps, 1),
        "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "moved_rows_mean": round(float(M.mean()), 1),
        "roofline": roofline,
        "mfma": mfma,
        "kernels": kernels,
        # inputs come from torch's device Philox generator: record its build
        "software": {"torch": torch.__version__, "hip": torch.version.hip},
    }
    if copy_gbps is not None:
        result["torch_copy_GBps"] = round(copy_gbps, 1)
        result["frac_of_torch_copy"] = round(gbps / copy_gbps, 4)
    if with_cpu:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(spec, wl, args.cpu_seconds)
    del wl, globs, out, holes, batch, tables, dst_table, pool
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return result


def _brief(res: dict) -> dict:
    """The per-config entry of the headline line."""
    r = res["roofline"]
    return {"ms_per_step": res["ms_per_step"], "ms_step_median": res["ms_step_median"],
            "tokens_per_s": res["value"], "steps": res["steps"], "warmup": res["warmup"],
            "achieved_GBps": res["achieved_GBps"], "frac_of_peak": res["frac_of_peak"],
            "kernel_avg_ms": res["kernels"]["compress"]["avg_ms"],
            "kernel_frac": r["frac"], "alg_bytes_per_launch": r["alg_bytes_per_launch"],
            "moved_rows_mean": res["moved_rows_mean"]}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the "
              "compression path needs no collective, see the design notes on "
              "sharding.", file=sys.stderr)
        sys.exit(2)
    import torch
    import kv_cache_compression_paged_amd as Z
    from kv_cache_compression_paged_amd import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    Z.lib()
    if args.workload == "capture_8b_32L_32q":
        run_capture(args)
        return
    if args.workload == "decode_8b_32L_8kv_32q":
        run_decode(args)
        return
    if args.workload == "redundancy_ablation_8b":
        run_redundancy_ablation(args)
        return
    if args.workload == "redundancy_sweep":
        run_redundancy_sweep(args)
        return
    if args.workload == "engine_8b":
        run_engine(args)
        return
    spec = synth.SPECS[args.workload]
    if spec.compress_groups > 1:
        print(json.dumps(run_overlap(args, spec, args.steps, args.warmup)), flush=True)
        return
    result = measure_compress(spec, args, args.steps, args.warmup, not args.no_cpu,
                              warm_min_s=args.warmup_seconds)
    if args.workload == synth.EIGHT_B.name and not args.headline_only:
        # the other workloads, timed in the same run: up to 20 steps
        # each after at least 0.3 s of their own warm-up steps, one at a time
        # (the largest pools need most of the device)
        ks, kw = min(args.steps, 20), min(args.warmup, 5)
        others = {}
        for other in (synth.TINY, synth.SMALL, synth.PREFIX, synth.LONG):
            others[other.name] = _brief(measure_compress(other, args, ks, kw, False,
                                                         with_copy=False, warm_min_s=0.3))
        ov = run_overlap(args, synth.OVERLAP, min(args.steps, 8), min(args.warmup, 2))
        others[synth.OVERLAP.name] = {
            "tokens_per_s": ov["value"], "steps": ov["steps"], **ov["overlap"],
            "achieved_GBps_CD": ov["achieved_GBps"], "frac_of_peak_CD": ov["frac_of_peak"]}
        result["other_workloads"] = others
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
