"""Checks of every unit of a full-size compression launch, run on the GPU with
plain torch ops (the oracle scores a seeded sample of units one by one; these
hold for all of them):

  keep    each keep row is the top k of the unit's own fp32 score row under
          (score descending, position ascending), written ascending -- the
          selection rule of [zh] §2.1 (keep the k = (N_max-1)*b best) with the
          lower-position tie rule, taken in the kernel's precision;
  rows    the compacted K and V rows of logical rows [0, k), read through the
          destination table, equal the original rows keep[0..k) read through
          the source table, bit for bit ([zh] §2.1 re-packing into the first
          N_max-1 blocks; [zh] §2.2 target blocks), and in place the tail
          rows [k, N) keep their bytes;
  global  the updated global row equals fp32 g[keep] + attn[keep] bit for bit
          (one IEEE addition, the same on both sides) with a +0 tail.

Row identity is checked on the raw bits (int16 for bf16). Where the device
cannot hold an untouched copy of the pool beside it, rows are compared by an
exact float64 hash instead: each row's bit patterns, read as int16, dotted with
random integer weights below 2^30 in float64 (every partial sum is an integer
below 2^53, so the hash is exact); two different rows agree with probability
about 2^-30.
"""

from __future__ import annotations

import torch


def bits(x: torch.Tensor) -> torch.Tensor:
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16)
    if x.dtype == torch.float32:
        return x.view(torch.int32)
    return x


def logical_rows(pool: torch.Tensor, tables: torch.Tensor, r0: int, r1: int,
                 nblk: int) -> torch.Tensor:
    """[r1-r0][L][H][nblk*b][d]: the rows of requests r0..r1-1 in logical
    order, read through their tables (pool layout [L][block][H][b][d])."""
    t = tables[r0:r1, :nblk].long()
    x = pool[:, t]                                  # [L, R', nblk, H, b, d]
    L, Rr, _, H, b, d = x.shape
    return x.permute(1, 0, 3, 2, 4, 5).reshape(Rr, L, H, nblk * b, d)


def check_keep_is_topk_of_own_scores(keep: torch.Tensor, score: torch.Tensor,
                                     n: int, chunk: int = 2048) -> None:
    U, k = keep.shape
    for u0 in range(0, U, chunk):
        sc = score[u0:u0 + chunk, :n]
        top = torch.sort(sc, dim=1, descending=True, stable=True).indices[:, :k]
        want = torch.sort(top, dim=1).values.to(torch.int32)
        got = keep[u0:u0 + chunk]
        if not torch.equal(want, got):
            bad = (want != got).any(dim=1).nonzero()[:5].flatten().tolist()
            raise AssertionError(f"keep rows of units {[u0 + x for x in bad]} are "
                                 "not the top k of their own scores")


def check_global_rows(glob_after: torch.Tensor, glob_before: torch.Tensor,
                      keep: torch.Tensor, attn: torch.Tensor, slots,
                      L: int, H: int, req_chunk: int = 16) -> None:
    """glob_*: [slots][L][H][n_cap] fp32; rows of request r live at slots[r]."""
    U, k = keep.shape
    R = U // (L * H)
    for r0 in range(0, R, req_chunk):
        r1 = min(R, r0 + req_chunk)
        sl = torch.as_tensor(list(slots[r0:r1]), device=glob_after.device).long()
        u0, u1 = r0 * L * H, r1 * L * H
        g0 = glob_before[sl].reshape(u1 - u0, -1)
        g1 = glob_after[sl].reshape(u1 - u0, -1)
        kk = keep[u0:u1].long()
        want = torch.gather(g0, 1, kk) + torch.gather(attn[u0:u1], 1, kk)
        if not torch.equal(bits(g1[:, :k]), bits(want)):
            bad = (bits(g1[:, :k]) != bits(want)).any(dim=1).nonzero()[:5]
            raise AssertionError(f"global rows of units {(bad + u0).flatten().tolist()}"
                                 " differ from g[keep] + attn[keep]")
        if not bool((bits(g1[:, k:]) == 0).all()):
            raise AssertionError(f"global tail not +0 in requests {r0}..{r1 - 1}")


def check_rows_against_copy(pool_after: torch.Tensor, pool_before: torch.Tensor,
                            src_tab: torch.Tensor, dst_tab: torch.Tensor,
                            keep: torch.Tensor, n: int, n_max: int,
                            in_place: bool, req_chunk: int = 4,
                            what: str = "K") -> None:
    """Compacted rows through dst_tab against the untouched rows through
    src_tab of `pool_before` (a copy taken before the call, or the pool
    itself when the sources are never written)."""
    R = src_tab.shape[0]
    b = pool_after.shape[3]
    L, H = pool_after.shape[0], pool_after.shape[2]
    U, k = keep.shape
    nblk = (n + b - 1) // b
    for r0 in range(0, R, req_chunk):
        r1 = min(R, r0 + req_chunk)
        old = bits(logical_rows(pool_before, src_tab, r0, r1, nblk))
        new = bits(logical_rows(pool_after, dst_tab, r0, r1, n_max))
        kk = keep[r0 * L * H:r1 * L * H].view(r1 - r0, L, H, k).long()
        want = torch.gather(old, 3, kk[..., None].expand(-1, -1, -1, -1, old.shape[-1]))
        if not torch.equal(new[..., :k, :], want):
            bad = (new[..., :k, :] != want).any(-1).nonzero()[:3].tolist()
            raise AssertionError(f"{what} rows differ (request offset {r0}): "
                                 f"[r, l, h, t] = {bad}")
        if in_place and not torch.equal(new[..., k:, :], old[..., k:n_max * b, :]):
            raise AssertionError(f"{what} tail rows changed in requests {r0}..{r1 - 1}")


class RowHasher:
    """Exact float64 hash of 16-bit rows (see the module docstring)."""

    def __init__(self, d: int, device, seed: int = 77):
        g = torch.Generator(device="cpu").manual_seed(seed)
        w = torch.randint(1, 1 << 30, (d,), generator=g, dtype=torch.int64)
        self.w = w.to(torch.float64).to(device)

    def __call__(self, rows: torch.Tensor, piece: int = 1 << 16) -> torch.Tensor:
        x = bits(rows)
        flat = x.reshape(-1, x.shape[-1])
        out = torch.empty(flat.shape[0], dtype=torch.float64, device=flat.device)
        for i in range(0, flat.shape[0], piece):
            out[i:i + piece] = flat[i:i + piece].to(torch.float64) @ self.w
        return out.view(x.shape[:-1])


def hash_logical_rows(hasher: RowHasher, pool: torch.Tensor, tables: torch.Tensor,
                      nblk: int, req_chunk: int = 1) -> torch.Tensor:
    """[R][L][H][nblk*b] hashes of every request's rows through `tables`."""
    R = tables.shape[0]
    parts = []
    for r0 in range(0, R, req_chunk):
        r1 = min(R, r0 + req_chunk)
        parts.append(hasher(logical_rows(pool, tables, r0, r1, nblk)))
    return torch.cat(parts, 0)


def check_rows_against_hashes(hasher: RowHasher, pool_after: torch.Tensor,
                              before: torch.Tensor, dst_tab: torch.Tensor,
                              keep: torch.Tensor, n_max: int, in_place: bool,
                              what: str = "K") -> None:
    """`before`: [R][L][H][N] hashes of the original rows (through the source
    tables), taken before the call."""
    R, L, H, _ = before.shape
    U, k = keep.shape
    nk = n_max * pool_after.shape[3]
    kk = keep.view(R, L, H, k).long()
    for r in range(R):
        after = hasher(logical_rows(pool_after, dst_tab, r, r + 1, n_max))[0]
        want = torch.gather(before[r], 2, kk[r])
        if not torch.equal(after[..., :k], want):
            bad = (after[..., :k] != want).nonzero()[:3].tolist()
            raise AssertionError(f"{what} row hashes of request {r} differ at "
                                 f"[l, h, t] = {bad}")
        if in_place and not torch.equal(after[..., k:], before[r, ..., k:nk]):
            raise AssertionError(f"{what} tail rows of request {r} changed")
