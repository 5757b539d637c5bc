"""Seeded synthetic workloads for the compression step.

This module only draws inputs: pools of keys and values, query windows, global
scores and block tables. It holds none of the method's arithmetic and imports
nothing from the library or from the oracle; both the tests and bench.py feed
its tensors to either side.

Recipe (per workload; see each spec):
  * bulk tensors from a torch.Generator on the target device seeded with the
    workload seed (Philox on the GPU, the CPU generator on the host), so a
    workload is fixed by (seed, device);
  * K, V and Q ~ N(0, 1) drawn in fp32 and rounded to the storage type (RNE);
  * global scores ~ U[0, 1) in fp32;
  * the physical block order is a numpy PCG64 permutation of the pool
    (contiguous for the tiny workload);
  * near-duplicate keys (the 8B-like workload and the ones built on it): in
    every (layer, block, head) tile exactly 5 of the 16 rows are replaced by
    bf16(k_src + 0.01 z), z ~ N(0, 1), where src is drawn uniformly from the
    tile's 11 rows that are not replaced.

Pool layout: [layer][block][kv_head][slot][head_dim] for K and for V.
Query windows: [slot][layer][w][q_head][head_dim]. Global scores:
[slot][layer][kv_head][n_cap] fp32.
"""

from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Spec:
    name: str
    seed: int
    requests: int
    layers: int
    kv_heads: int
    q_heads: int
    head_dim: int
    block_size: int
    n_max: int
    window: int
    dtype: str                 # 'f32' or 'bf16' for K, V and Q
    pool_blocks: int
    permute: bool = True
    near_dup: bool = False
    groups: int = 1            # shared-prefix groups (requests split evenly)
    shared_blocks: int = 0     # leading blocks shared inside a group
    compress_groups: int = 1   # overlap workload: groups that rotate

    @property
    def n_tokens(self) -> int:
        return self.n_max * self.block_size

    @property
    def keep(self) -> int:
        return (self.n_max - 1) * self.block_size

    @property
    def units(self) -> int:
        return self.requests * self.layers * self.kv_heads

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


# The workloads (sizes follow the 2048- and 4096-token KV budgets and an
# 8B-class GQA layout; the last one is a 16384-token budget, whose token rows
# no longer fit in LDS beside the default key ring).
TINY = Spec("tiny_fp32_1req", 1000, 1, 1, 2, 4, 64, 16, 8, 8, "f32", 8,
            permute=False)
SMALL = Spec("small_28L_2kv_12q_N2048", 1001, 64, 28, 2, 12, 128, 16, 128, 32,
             "bf16", 8192)
EIGHT_B = Spec("8b_32L_8kv_32q_N4096", 1002, 128, 32, 8, 32, 128, 16, 256, 32,
               "bf16", 32768, near_dup=True)
PREFIX = Spec("prefix_256req_4grp_32shared", 1003, 256, 32, 8, 32, 128, 16, 256,
              32, "bf16", 114560, near_dup=True, groups=4, shared_blocks=32)
OVERLAP = Spec("overlap_512req_8grp", 1004, 512, 32, 8, 32, 128, 16, 256, 32,
               "bf16", 131072, near_dup=True, groups=8, compress_groups=8)
LONG = Spec("long_8req_32L_8kv_N16384", 1005, 8, 32, 8, 32, 128, 16, 1024, 32,
            "bf16", 8192, near_dup=True)

SPECS: Dict[str, Spec] = {s.name: s for s in (TINY, SMALL, EIGHT_B, PREFIX,
                                              OVERLAP, LONG)}


def scaled(spec: Spec, **kw) -> Spec:
    """A smaller variant with the same structure (for parity runs the oracle
    finishes in seconds)."""
    return replace(spec, **kw)


@dataclass
class Workload:
    spec: Spec
    k_pool: torch.Tensor       # [L][blocks][Hkv][b][d]
    v_pool: torch.Tensor
    q_window: torch.Tensor     # [slots][L][w][Hq][d]
    global_scores: torch.Tensor  # [slots][L][Hkv][n_cap] fp32
    tables: np.ndarray         # [R][blocks per request] int32 (host)
    slots: np.ndarray          # [R] int32
    n_tokens: np.ndarray       # [R] int32
    refcount: np.ndarray       # [blocks] int32: users of each block
    n_cap: int


def _normal_into(t: torch.Tensor, gen: torch.Generator, chunk_rows: int = 1
                 ) -> None:
    """Fill t (any float dtype) with N(0,1) drawn in fp32, one leading index
    at a time to bound the fp32 temporary."""
    for i in range(0, t.shape[0], chunk_rows):
        tmp = torch.randn(t[i:i + chunk_rows].shape, generator=gen,
                          device=t.device, dtype=torch.float32)
        t[i:i + chunk_rows].copy_(tmp)


def _near_duplicates(k_layer: torch.Tensor, gen: torch.Generator,
                     chunk: int = 1 << 17) -> None:
    """In every tile [block][head] of one layer, replace 5 of the b rows by a
    noisy copy of another row of the same tile (the 11 others are sources).
    Tiles are processed `chunk` at a time to bound the temporaries."""
    nb, hkv, b, d = k_layer.shape
    if b != 16:
        raise ValueError("near-duplicate recipe is defined for b = 16")
    all_tiles = k_layer.view(nb * hkv, b, d)
    for c0 in range(0, nb * hkv, chunk):
        tiles = all_tiles[c0:c0 + chunk]
        nt = tiles.shape[0]
        order = torch.argsort(torch.rand((nt, b), generator=gen,
                                         device=k_layer.device), dim=1)
        dst = order[:, :5]
        pick = torch.randint(0, 11, (nt, 5), generator=gen,
                             device=k_layer.device)
        src = torch.gather(order[:, 5:], 1, pick)
        rows = torch.arange(nt, device=k_layer.device).unsqueeze(1)
        noise = torch.randn((nt, 5, d), generator=gen,
                            device=k_layer.device, dtype=torch.float32)
        copies = tiles[rows, src].float() + 0.01 * noise
        tiles[rows, dst] = copies.to(tiles.dtype)


def block_tables(spec: Spec) -> (np.ndarray, np.ndarray):
    """Per-request block tables and per-block user counts.

    Plain workloads: request r owns n_max blocks. Shared-prefix workloads:
    requests are split into `groups`; a group's first `shared_blocks` logical
    blocks are one set of physical blocks used by every request of the group,
    the rest are private. Physical ids come from a PCG64 permutation.
    """
    R, nm = spec.requests, spec.n_max
    rng = np.random.Generator(np.random.PCG64(spec.seed))
    if spec.permute:
        perm = rng.permutation(spec.pool_blocks).astype(np.int32)
    else:
        perm = np.arange(spec.pool_blocks, dtype=np.int32)
    refcount = np.zeros(spec.pool_blocks, dtype=np.int32)
    tables = np.zeros((R, nm), dtype=np.int32)
    nxt = 0
    if spec.shared_blocks:
        per_group = R // spec.groups
        for grp in range(spec.groups):
            shared = perm[nxt:nxt + spec.shared_blocks]
            nxt += spec.shared_blocks
            for j in range(per_group):
                r = grp * per_group + j
                tables[r, :spec.shared_blocks] = shared
        for r in range(R):
            priv = nm - spec.shared_blocks
            tables[r, spec.shared_blocks:] = perm[nxt:nxt + priv]
            nxt += priv
    else:
        for r in range(R):
            tables[r] = perm[nxt:nxt + nm]
            nxt += nm
    if nxt > spec.pool_blocks:
        raise ValueError("pool too small for the tables")
    np.add.at(refcount, tables.reshape(-1), 1)
    return tables, refcount


def make(spec: Spec, device: str = "cpu", slots: Optional[int] = None
         ) -> Workload:
    """Draw a whole workload on `device`. Every request holds exactly
    n_max*b tokens (the trigger point) and owns query slot r."""
    gen = torch.Generator(device=device)
    gen.manual_seed(spec.seed)
    L, nb, hkv, b, d = (spec.layers, spec.pool_blocks, spec.kv_heads,
                        spec.block_size, spec.head_dim)
    k_pool = torch.empty((L, nb, hkv, b, d), dtype=spec.torch_dtype,
                         device=device)
    v_pool = torch.empty_like(k_pool)
    for layer in range(L):
        _normal_into(k_pool[layer], gen, chunk_rows=max(1, nb // 4))
        if spec.near_dup:
            _near_duplicates(k_pool[layer], gen)
    for layer in range(L):
        _normal_into(v_pool[layer], gen, chunk_rows=max(1, nb // 4))
    n_slots = spec.requests if slots is None else slots
    q = torch.empty((n_slots, L, spec.window, spec.q_heads, d),
                    dtype=spec.torch_dtype, device=device)
    _normal_into(q, gen)
    n_cap = spec.n_tokens
    glob = torch.rand((n_slots, L, hkv, n_cap), generator=gen, device=device,
                      dtype=torch.float32)
    tables, refcount = block_tables(spec)
    return Workload(spec=spec, k_pool=k_pool, v_pool=v_pool, q_window=q,
                    global_scores=glob, tables=tables,
                    slots=np.arange(spec.requests, dtype=np.int32),
                    n_tokens=np.full(spec.requests, spec.n_tokens,
                                     dtype=np.int32),
                    refcount=refcount, n_cap=n_cap)


def raw_numpy(t: torch.Tensor) -> np.ndarray:
    """Host copy of a tensor in its stored bits: uint16 for bf16, float32 for
    fp32, int32 for int32."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def decode_queries(spec: Spec, requests: int, device: str, seed: int
                   ) -> torch.Tensor:
    """Fresh decode queries q ~ N(0,1), [R][L][Hq][d] in the storage type."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    q = torch.randn((requests, spec.layers, spec.q_heads, spec.head_dim),
                    generator=gen, device=device, dtype=torch.float32)
    return q.to(spec.torch_dtype)

