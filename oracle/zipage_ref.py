"""CPU oracle for one Compressed-PagedAttention compression step (float64).

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or run
this module: only the tests, the smoke check in ``__graft_entry__.smoke`` and
the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code, header,
table or helper with the HIP library and imports nothing from it.

What it computes is the compression step of Zipage ("Zipage: Maintain High
Request Concurrency for LLM Reasoning through Compressed PagedAttention",
arXiv 2603.08743) as described by four summary pages of that paper, cited here
as follows (each page has a technical summary with numbered sections):

  [zh] gist.science/zh/paper/2603.08743  -- 技术总结, sections 1-5 (2.1, 2.2, 2.3)
  [de] gist.science/de/paper/2603.08743  -- Zusammenfassung, sections 1-5
  [es] gist.science/es/paper/2603.08743  -- Resumen Técnico, sections 1-5
  [fr] gist.science/fr/paper/2603.08743  -- sections 1-5 (2.A .. 2.E)

Every floating-point step runs in float64 on inputs widened exactly from their
stored type (bf16 or fp32). Loops are plain; the only library primitives are
numpy dot products, exp, sqrt and a Python sort.

Where the pages leave a step open, the reading taken is stated in the docstring
of the function that implements it (e.g. how the three scores combine, the
causal mask, tie breaking, the shared-prefix policy, the free-list order).

Pins: every function here is checked by ``tests/test_oracle_pins.py`` against
something other than itself (a library routine, a closed form, a brute force
on tiny inputs or a hand-worked example under ``tests/golden/``). One thing is
not pinnable from the pages: whether this reading matches the authors' exact
scoring code -- the pages print no listing, no worked example and no values.
That part is "parity unpinned" against the paper itself; only the reading
fixed below is pinned.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

# --------------------------------------------------------------------------
# parameters
# --------------------------------------------------------------------------


@dataclass
class Params:
    """Parameters of one compression call.

    n_max  -- per-request block cap N_max; b -- block size; window -- w, the
    number of most recent query states in the observation window
    ([zh §2.1], [de §2], [es §2]). w_attn, w_global, w_red are the weights of
    the three score parts. The pages list the parts (attention, redundancy and
    a global score built from past attention, [zh §2.1]) without a formula;
    the reading taken is s = 1*attn + 0.5*global - 0.5*red: redundant tokens
    are penalised, historically attended tokens rewarded.
    sm_scale defaults to 1/sqrt(d) (the usual attention scale; pages silent).
    causal: a window query at position p attends keys at positions <= p
    (a decoder query never saw later keys; pages silent). protect_window pins
    the last w tokens (only [fr §2.A] says the window is always kept; the other
    pages do not, so it is an option, off by default).
    """

    n_max: int
    block_size: int
    window: int
    w_attn: float = 1.0
    w_global: float = 0.5
    w_red: float = 0.5
    sm_scale: Optional[float] = None
    causal: bool = True
    protect_window: bool = False

    @property
    def keep_tokens(self) -> int:
        return budget_tokens(self.n_max, self.block_size)


def budget_tokens(n_max: int, b: int) -> int:
    """Number of tokens kept by one compression: k = (N_max - 1) * b.

    [zh §2.1] keeps the k best tokens with k = (N_max - 1) * b and re-packs them
    into the first N_max - 1 blocks; [de §2] reserves the N_max-th block for
    the tokens decoded next.
    """
    if n_max < 2 or b < 1:
        raise ValueError("need n_max >= 2 and b >= 1")
    return (n_max - 1) * b


# --------------------------------------------------------------------------
# storage helpers: exact widening and paged gathers
# --------------------------------------------------------------------------


def widen(raw: np.ndarray, elem: str) -> np.ndarray:
    """Exact float64 value of stored elements.

    elem 'bf16': raw holds the 16-bit patterns (uint16); a bf16 value is the
    fp32 value whose upper 16 bits are that pattern. elem 'f32': raw is float32.
    """
    if elem == "bf16":
        bits = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if elem == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if elem == "f64":  # float64 test inputs, already exact
        return np.asarray(raw, dtype=np.float64)
    raise ValueError(f"unknown element type {elem!r}")


def row_location(table: Sequence[int], t: int, b: int) -> Tuple[int, int]:
    """(physical block, slot in block) of logical token t through a block table.

    PagedAttention maps a request's logical token t to block table[t // b],
    slot t % b ([zh §2], [de §2]: the method builds on PagedAttention).
    """
    return int(table[t // b]), t % b


def gather_rows(pool: np.ndarray, table: Sequence[int], layer: int, head: int,
                n: int, b: int) -> np.ndarray:
    """Logical rows 0..n-1 of one (layer, KV head) from a pool laid out
    [layer][block][kv_head][slot][d], returned in logical order (raw dtype)."""
    d = pool.shape[-1]
    out = np.empty((n, d), dtype=pool.dtype)
    for t in range(n):
        blk, slot = row_location(table, t, b)
        out[t] = pool[layer, blk, head, slot]
    return out


# --------------------------------------------------------------------------
# the three score parts
# --------------------------------------------------------------------------


def window_positions(n: int, w: int) -> List[int]:
    """Positions of the observation window: window slot i holds the query state
    of token n - w + i, i = 0..w-1 (the last w tokens, [zh §2.1], [de §2])."""
    if not 1 <= w <= n:
        raise ValueError("window must satisfy 1 <= w <= n")
    return [n - w + i for i in range(w)]


def capture_queries(q_window: np.ndarray, q: np.ndarray, slot: Sequence[int],
                    pos: Sequence[int], w: int) -> None:
    """Query slots ([zh] §2.2, [de] §2): only requests holding a slot keep
    their recent query states, and the last w of them score the cache
    ([zh] §2.1). Reading: each slot keeps, per layer, a ring of w rows; the
    queries (all query heads) of the token at position p go to row p mod w.
    q_window: raw [slots][L][w][Hq][d], updated in place; q: raw
    [R][L][Hq][d]. A request with slot < 0 (no slot), a slot out of range or
    a negative position writes nothing."""
    S = q_window.shape[0]
    for r in range(q.shape[0]):
        s, p = int(slot[r]), int(pos[r])
        if s < 0 or s >= S or p < 0:
            continue
        for layer in range(q.shape[1]):
            q_window[s, layer, p % w] = q[r, layer]


def window_from_ring(ring: np.ndarray, n: int, w: int) -> np.ndarray:
    """The w rows of one (slot, layer) ring in position order n-w .. n-1."""
    return np.stack([ring[(n - w + i) % w] for i in range(w)])


def window_attention(q_win: np.ndarray, keys: np.ndarray, n: int,
                     causal: bool = True,
                     sm_scale: Optional[float] = None) -> np.ndarray:
    """Attention score of every cached token from the observation window.

    q_win: [w, G, d] float64, the query states of the last w tokens for the G
    query heads that share this KV head (query head h*G+g reads KV head h;
    pages silent, the usual contiguous grouping). keys: [n, d] float64.

    Each window row (i, g) takes a softmax over the keys it may see (all n, or
    t <= n - w + i when causal) of q.k * sm_scale; attn_t is the mean over the
    w*G rows of that row's probability of t, with a masked entry counting as 0
    and the divisor always w*G. Token importance from window attention:
    [zh §2.1], [de §2], [es §2], [fr §2.A].
    """
    w, G, d = q_win.shape
    if keys.shape != (n, d):
        raise ValueError("keys must be [n, d]")
    scale = (1.0 / math.sqrt(d)) if sm_scale is None else float(sm_scale)
    pos = window_positions(n, w)
    attn = np.zeros(n, dtype=np.float64)
    for i in range(w):
        visible = pos[i] + 1 if causal else n
        for g in range(G):
            logits = keys[:visible] @ q_win[i, g] * scale
            m = logits.max()
            e = np.exp(logits - m)
            attn[:visible] += e / e.sum()
    return attn / (w * G)


def lightning_redundancy(keys: np.ndarray, b: int, n: int) -> np.ndarray:
    """Intra-block ("lightning") redundancy of every token.

    The lightning score looks only at similarity inside a block, one block at
    a time, instead of the all-pairs key similarity, cutting O(N^2 b^2) to
    O(N b^2) for N blocks ([zh §2.1], [de §2], [es §2], [fr §2.E]).

    red_t = mean over the other valid tokens j of t's block of
    cos(k_t, k_j) = k_t.k_j / max(|k_t| |k_j|, 1e-8); red_t = 0 when t is
    alone in its block (a partial last block of one token).
    """
    if keys.shape[0] != n:
        raise ValueError("keys must hold n rows")
    red = np.zeros(n, dtype=np.float64)
    nblocks = (n + b - 1) // b
    for beta in range(nblocks):
        lo, hi = beta * b, min(n, (beta + 1) * b)
        cnt = hi - lo
        if cnt < 2:
            continue
        blk = keys[lo:hi]
        norms = np.sqrt((blk * blk).sum(axis=1))
        for a in range(cnt):
            acc = 0.0
            for c in range(cnt):
                if c == a:
                    continue
                denom = max(norms[a] * norms[c], 1e-8)
                acc += float(blk[a] @ blk[c]) / denom
            red[lo + a] = acc / (cnt - 1)
    return red


def redundancy_all_pairs(keys: np.ndarray, b: int, n: int
                         ) -> Tuple[np.ndarray, np.ndarray]:
    """The all-pairs key similarity that the lightning score replaces
    ([zh §2.1], [fr §2.E]: the original score was O(N^2 b^2) for N blocks of
    b tokens). The full n x n cosine matrix is formed, the diagonal dropped,
    and two means taken per token: over the other tokens of its block (this
    equals the lightning score, the reading that makes lightning an exact
    speed-up) and over all other tokens. Same clamp as lightning: the norm
    product is taken at least 1e-8; a lone token scores 0."""
    if keys.shape[0] != n:
        raise ValueError("keys must hold n rows")
    norms = np.sqrt((keys * keys).sum(axis=1))
    cos = (keys @ keys.T) / np.maximum(np.outer(norms, norms), 1e-8)
    np.fill_diagonal(cos, 0.0)
    blk = np.arange(n) // b
    same = blk[:, None] == blk[None, :]
    cnt = np.bincount(blk)[blk]
    red_block = np.where(cnt >= 2, (cos * same).sum(axis=1) / np.maximum(cnt - 1, 1), 0.0)
    red_all = cos.sum(axis=1) / (n - 1) if n >= 2 else np.zeros(n)
    return red_block, red_all


def combine_scores(attn: np.ndarray, glob: np.ndarray, red: np.ndarray,
                   p: Params) -> np.ndarray:
    """s_t = w_attn*attn_t + w_global*global_t - w_red*red_t.

    The pages name the three parts and say they are combined ([zh §2.1],
    [es §2]); the weights (1, 0.5, 0.5) are this reading's choice.
    """
    return p.w_attn * attn + p.w_global * glob - p.w_red * red


# --------------------------------------------------------------------------
# selection, compaction, global-score update
# --------------------------------------------------------------------------


def pinned_mask(n: int, n_pinned_blocks: int, b: int, w: int,
                protect_window: bool) -> np.ndarray:
    """Tokens that must be kept whatever their score.

    Tokens of the leading shared blocks stay where they are: compression does
    not move data of shared-prefix blocks ([zh §2.2], [de §2], [fr §2.C]);
    this reading keeps them whole and counts them in k. With protect_window,
    the last w tokens are pinned too ([fr §2.A]).
    """
    m = np.zeros(n, dtype=bool)
    m[: n_pinned_blocks * b] = True
    if protect_window:
        m[n - w:] = True
    return m


def select_keep(s: np.ndarray, k: int, pinned: np.ndarray) -> np.ndarray:
    """Token-level selection: keep the pinned tokens plus the best k - |P| others.

    Eviction is per token, not per page ([zh §2.1], [de §2], [fr §2.A]), keeping
    the k highest scores ([zh §2.1]). Order: higher score first; equal scores
    rank the lower position first. Returns the kept positions ascending (kept
    tokens keep their relative order when re-packed, [zh §2.1]).
    """
    n = len(s)
    pin = [t for t in range(n) if pinned[t]]
    if len(pin) > k:
        raise ValueError("more pinned tokens than the budget k")
    free = [t for t in range(n) if not pinned[t]]
    ranked = sorted(free, key=lambda t: (-float(s[t]), t))
    keep = sorted(pin + ranked[: k - len(pin)])
    return np.asarray(keep, dtype=np.int64)


def first_hole(keep: np.ndarray) -> int:
    """First evicted position h: keep[t] == t for all t < h."""
    for t, src in enumerate(keep):
        if src != t:
            return t
    return len(keep)


def compact_unit(src_pool: np.ndarray, dst_pool: np.ndarray,
                 src_table: Sequence[int], dst_table: Sequence[int],
                 layer: int, head: int, keep: np.ndarray, b: int) -> None:
    """Re-pack the kept rows of one (layer, KV head) into logical rows 0..k-1.

    Kept tokens are moved, in order, into the first N_max - 1 blocks
    ([zh §2.1], [de §2], [es §2]). Rows are read through src_table from
    src_pool, the pool as it was before the call, and written through
    dst_table into dst_pool; a row whose destination is its own source is
    left alone, any other is copied byte for byte. With a shared prefix the
    destination blocks past the prefix are freshly allocated targets
    ([zh §2.2], [de §2], [fr §2.C]).
    """
    for t, src in enumerate(keep):
        sb, ss = row_location(src_table, int(src), b)
        db, ds = row_location(dst_table, t, b)
        if (sb, ss) == (db, ds):
            continue
        dst_pool[layer, db, head, ds] = src_pool[layer, sb, head, ss]


def update_global(g: np.ndarray, attn: np.ndarray, keep: np.ndarray,
                  k: int) -> np.ndarray:
    """New global scores in logical order after compaction.

    The global score accumulates past attention over the whole sequence
    ([zh §2.1], [de §2], [fr §2.E]); the pages name a kernel that updates it
    ([zh §2.3]). Reading: g'_t = g_{keep[t]} + attn_{keep[t]} for t < k (this
    round's attention is added and the score moves with its token); the freed
    tail [k, len(g)) is zeroed.
    """
    out = np.zeros_like(np.asarray(g, dtype=np.float64))
    for t in range(k):
        out[t] = float(g[keep[t]]) + float(attn[keep[t]])
    return out


# --------------------------------------------------------------------------
# one unit and a whole batch
# --------------------------------------------------------------------------


@dataclass
class UnitResult:
    attn: np.ndarray
    red: np.ndarray
    score: np.ndarray
    keep: np.ndarray
    hole: int


def score_unit(q_win: np.ndarray, keys: np.ndarray, glob: np.ndarray, n: int,
               n_pinned_blocks: int, p: Params) -> UnitResult:
    """Score and select one (request, layer, KV head): steps in page order --
    window attention, lightning redundancy, global score, combination, pinning,
    top-k ([zh §2.1])."""
    attn = window_attention(q_win, keys, n, p.causal, p.sm_scale)
    red = lightning_redundancy(keys, p.block_size, n)
    s = combine_scores(attn, glob[:n], red, p)
    pin = pinned_mask(n, n_pinned_blocks, p.block_size, p.window,
                      p.protect_window)
    s = np.where(pin, np.inf, s)
    keep = select_keep(s, p.keep_tokens, pin)
    return UnitResult(attn=attn, red=red, score=s, keep=keep,
                      hole=first_hole(keep))


@dataclass
class Batch:
    """One compression call. src_tables [R][>=ceil(n/b)] (logical block ->
    physical block), dst_tables [R][n_max] (where compacted rows go),
    n_pinned [R] (leading blocks pinned), slots [R] (query-slot / global-score
    row of the request), n_tokens [R]."""

    slots: np.ndarray
    n_tokens: np.ndarray
    src_tables: np.ndarray
    dst_tables: np.ndarray
    n_pinned: np.ndarray


def compress(pool_k: np.ndarray, pool_v: np.ndarray, elem: str,
             q_window: np.ndarray, q_elem: str, global_scores: np.ndarray,
             batch: Batch, p: Params,
             units: Optional[Sequence[Tuple[int, int, int]]] = None
             ) -> Dict[str, object]:
    """Whole compression call on copies of the pools.

    pool_k / pool_v: [L][blocks][Hkv][b][d] raw (uint16 bf16 bits or float32);
    q_window: [slots][L][w][Hq][d] raw; global_scores: [slots][L][Hkv][N_cap]
    float32. units: the (r, l, h) to process (default: all).

    Returns the new pools (copies), new global scores (copy, float64) and per
    unit results keyed by (r, l, h).
    """
    L, _, Hkv, b, d = pool_k.shape
    Hq = q_window.shape[3]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if b != p.block_size:
        raise ValueError("pool block size differs from params")
    R = len(batch.slots)
    if units is None:
        units = [(r, l, h) for r in range(R) for l in range(L) for h in range(Hkv)]
    new_k, new_v = pool_k.copy(), pool_v.copy()
    new_g = global_scores.astype(np.float64)
    results: Dict[Tuple[int, int, int], UnitResult] = {}
    k = p.keep_tokens
    for (r, l, h) in units:
        n = int(batch.n_tokens[r])
        slot = int(batch.slots[r])
        src = batch.src_tables[r]
        keys = widen(gather_rows(pool_k, src, l, h, n, b), elem)
        q = widen(q_window[slot, l], q_elem)[:, h * G:(h + 1) * G, :]
        glob = global_scores[slot, l, h].astype(np.float64)
        res = score_unit(q, keys, glob, n, int(batch.n_pinned[r]), p)
        results[(r, l, h)] = res
        compact_unit(pool_k, new_k, src, batch.dst_tables[r], l, h, res.keep, b)
        compact_unit(pool_v, new_v, src, batch.dst_tables[r], l, h, res.keep, b)
        new_g[slot, l, h] = update_global(global_scores[slot, l, h], res.attn,
                                          res.keep, k)
    return {"pool_k": new_k, "pool_v": new_v, "global": new_g,
            "units": results}


# --------------------------------------------------------------------------
# block bookkeeping (host side)
# --------------------------------------------------------------------------


@dataclass
class Plan:
    dst_tables: np.ndarray            # [R][n_max]
    n_pinned: np.ndarray              # [R]
    popped: List[int] = field(default_factory=list)
    to_free: List[int] = field(default_factory=list)
    new_tables: List[List[int]] = field(default_factory=list)


class BlockPool:
    """Free list and reference counts of a paged KV pool.

    Requests hold blocks of b tokens and give them back when done
    ([zh §2], [es §2]); blocks of a shared prefix carry a reference count and
    those with a count above one stay untouched by compression ([de §2]).
    Free-list reading (pages silent): a LIFO stack; a fresh pool holds ids
    0..n-1 with id 0 popped first; pops take the top, pushes go on top.
    """

    def __init__(self, num_blocks: int):
        self.refcount = [0] * num_blocks
        self.stack = list(range(num_blocks - 1, -1, -1))

    def alloc(self, n: int) -> List[int]:
        if n > len(self.stack):
            raise MemoryError("free list exhausted")
        out = [self.stack.pop() for _ in range(n)]
        for bid in out:
            self.refcount[bid] = 1
        return out

    def incref(self, bid: int) -> None:
        if self.refcount[bid] < 1:
            raise ValueError("incref of a free block")
        self.refcount[bid] += 1

    def shared_prefix(self, table: Sequence[int], n_max: int) -> int:
        """S: length of the leading run of blocks whose count exceeds one."""
        s = 0
        while s < n_max - 1 and self.refcount[table[s]] > 1:
            s += 1
        return s

    def check_private(self, tables, n_tokens, shared, b: int) -> None:
        """Blocks a request holds after its shared run are rewritten in place,
        kept as its tail or freed, so no other request may hold them: each
        must have a count of one and appear once in the call ([de §2]: blocks
        with a count above one stay intact; [zh §2.2]: shared data is never
        moved)."""
        private = set()
        for r in range(len(tables)):
            held = (int(n_tokens[r]) + b - 1) // b
            for bid in tables[r][shared[r]:held]:
                bid = int(bid)
                if self.refcount[bid] != 1 or bid in private:
                    raise ValueError(f"block {bid} after the shared prefix is "
                                     "shared or listed twice")
                private.add(bid)

    def plan_compress(self, tables: Sequence[Sequence[int]],
                      n_tokens: Sequence[int], n_max: int, b: int) -> Plan:
        """Plan one compression call; no state changes until commit, except
        that target blocks are popped here (they are written by the kernels).

        Trigger: a request compresses once it holds N_max blocks and its last
        block is full, n_tokens == N_max*b ([zh §2.1], [de §2]); a request that
        overshot during prefill (n_tokens > N_max*b) is accepted too.
        No shared prefix (S = 0): in place; dst table = first N_max entries of
        the table, and blocks past N_max (overshoot) are freed in logical order.
        Shared prefix (S > 0): the S shared blocks stay, N_max-1-S fresh targets
        are popped in logical order, the old block N_max-1 becomes the tail,
        and old private blocks S..N_max-2 (then any past N_max) are freed in
        logical order ([zh §2.2], [de §2], [fr §2.C]).
        """
        R = len(tables)
        dst = np.zeros((R, n_max), dtype=np.int64)
        pinned = np.zeros(R, dtype=np.int64)
        need = 0
        shared = []
        for r in range(R):
            n = int(n_tokens[r])
            if n < n_max * b:
                raise ValueError("request below the trigger point")
            sb = self.shared_prefix(tables[r], n_max)
            shared.append(sb)
            if sb > 0:
                need += n_max - 1 - sb
        self.check_private(tables, n_tokens, shared, b)
        if need > len(self.stack):
            raise MemoryError("free list exhausted")
        plan = Plan(dst_tables=dst, n_pinned=pinned)
        for r in range(R):
            n = int(n_tokens[r])
            nb = (n + b - 1) // b
            table = [int(x) for x in tables[r][:nb]]
            sb = shared[r]
            pinned[r] = sb
            if sb == 0:
                new = table[:n_max]
                freed = table[n_max:]
            else:
                targets = [self.stack.pop() for _ in range(n_max - 1 - sb)]
                plan.popped.extend(targets)
                new = table[:sb] + targets + [table[n_max - 1]]
                freed = table[sb:n_max - 1] + table[n_max:]
            dst[r] = new
            plan.new_tables.append(new)
            plan.to_free.extend(freed)
        return plan

    def commit(self, plan: Plan) -> None:
        """After the compression kernels finished: targets count one user,
        freed blocks go back on the stack in plan order, shared counts stay."""
        for bid in plan.popped:
            self.refcount[bid] = 1
        for bid in plan.to_free:
            self.refcount[bid] = 0
            self.stack.append(bid)


# --------------------------------------------------------------------------
# consumer: decode attention over the compressed cache
# --------------------------------------------------------------------------


def decode_attention(q: np.ndarray, keys: np.ndarray, values: np.ndarray,
                     sm_scale: Optional[float] = None) -> np.ndarray:
    """One new query token per query head over the cached keys/values:
    softmax(q.K^T * scale) V, all float64. q: [G, d]; keys, values: [n, d].
    Decoding reads the paged cache as PagedAttention does ([zh §2.3])."""
    d = q.shape[-1]
    scale = (1.0 / math.sqrt(d)) if sm_scale is None else float(sm_scale)
    out = np.zeros((q.shape[0], values.shape[1]), dtype=np.float64)
    for g in range(q.shape[0]):
        logits = keys @ q[g] * scale
        e = np.exp(logits - logits.max())
        out[g] = (e / e.sum()) @ values
    return out


def paged_decode(q: np.ndarray, q_elem: str, pool_k: np.ndarray,
                 pool_v: np.ndarray, elem: str, tables: np.ndarray,
                 seq_lens: Sequence[int],
                 pairs: Optional[Sequence[Tuple[int, int]]] = None
                 ) -> Dict[Tuple[int, int], np.ndarray]:
    """Decode attention for (request, layer) pairs. q: [R][L][Hq][d] raw.
    Returns {(r, l): [Hq, d] float64}."""
    L, _, Hkv, b, d = pool_k.shape
    R, _, Hq, _ = q.shape
    G = Hq // Hkv
    if pairs is None:
        pairs = [(r, l) for r in range(R) for l in range(L)]
    out = {}
    for (r, l) in pairs:
        n = int(seq_lens[r])
        res = np.zeros((Hq, d), dtype=np.float64)
        for h in range(Hkv):
            keys = widen(gather_rows(pool_k, tables[r], l, h, n, b), elem)
            vals = widen(gather_rows(pool_v, tables[r], l, h, n, b), elem)
            qh = widen(q[r, l, h * G:(h + 1) * G], q_elem)
            res[h * G:(h + 1) * G] = decode_attention(qh, keys, vals)
        out[(r, l)] = res
    return out


def paged_decode_append(q: np.ndarray, q_elem: str, k_new: np.ndarray,
                        v_new: np.ndarray, pool_k: np.ndarray, pool_v: np.ndarray,
                        elem: str, tables: np.ndarray, seq_lens: Sequence[int]
                        ) -> Tuple[Dict[Tuple[int, int], np.ndarray], np.ndarray, np.ndarray]:
    """A decode step that appends its token ([zh] §2.3: decoding extends the
    request's tail block and attends over the paged cache). For every request
    r the new rows k_new[r][l][h], v_new[r][l][h] (raw) are stored at logical
    position seq_lens[r] of the block table in copies of the pools, then each
    query head attends over the seq_lens[r] + 1 tokens. Returns the outputs
    {(r, l): [Hq, d] float64} and the two updated pools (raw)."""
    pk, pv = pool_k.copy(), pool_v.copy()
    L, _, Hkv, b, _ = pool_k.shape
    for r in range(q.shape[0]):
        blk, slot = row_location(tables[r], int(seq_lens[r]), b)
        for layer in range(L):
            for h in range(Hkv):
                pk[layer, blk, h, slot] = k_new[r, layer, h]
                pv[layer, blk, h, slot] = v_new[r, layer, h]
    out = paged_decode(q, q_elem, pk, pv, elem, tables, [int(x) + 1 for x in seq_lens])
    return out, pk, pv
