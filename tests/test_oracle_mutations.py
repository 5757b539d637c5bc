"""Planted mistakes in the oracle must be caught by the pins.

Each case swaps one oracle function for a copy with a plausible bug (a dropped
term, a wrong sign, an off-by-one, a wrong divisor, a reversed tie break) and
checks that at least one pin in test_oracle_pins.py then fails. CPU only.
"""

import contextlib
import math
from unittest import mock

import numpy as np
import pytest

import oracle as O
import oracle.zipage_ref as Z
from tests import test_oracle_pins as P


@contextlib.contextmanager
def planted(name, fn):
    with mock.patch.object(Z, name, fn), mock.patch.object(O, name, fn):
        yield


def _fails(test, *args):
    try:
        test(*args)
    except AssertionError:
        return True
    return False


def combine_red_sign(attn, glob, red, p):
    return p.w_attn * attn + p.w_global * glob + p.w_red * red


def combine_no_global(attn, glob, red, p):
    return p.w_attn * attn - p.w_red * red


def attention_off_by_one(q_win, keys, n, causal=True, sm_scale=None):
    w, G, d = q_win.shape
    scale = 1.0 / math.sqrt(d) if sm_scale is None else sm_scale
    attn = np.zeros(n)
    for i in range(w):
        visible = (n - w + i) if causal else n      # should be n - w + i + 1
        for g in range(G):
            lg = keys[:visible] @ q_win[i, g] * scale
            e = np.exp(lg - lg.max())
            attn[:visible] += e / e.sum()
    return attn / (w * G)


def attention_wrong_divisor(q_win, keys, n, causal=True, sm_scale=None):
    w, G, d = q_win.shape
    return Z.__dict__["_orig_window_attention"](q_win, keys, n, causal,
                                                sm_scale) * G


def attention_transposed_group(q_win, keys, n, causal=True, sm_scale=None):
    # uses the first query head for every head of the group
    q = np.repeat(q_win[:, :1, :], q_win.shape[1], axis=1)
    return Z.__dict__["_orig_window_attention"](q, keys, n, causal, sm_scale)


def redundancy_divisor(keys, b, n):
    red = Z.__dict__["_orig_lightning_redundancy"](keys, b, n)
    out = red.copy()
    for beta in range((n + b - 1) // b):
        cnt = min(n, (beta + 1) * b) - beta * b
        out[beta * b:beta * b + cnt] *= (cnt - 1) / cnt
    return out


def redundancy_unnormalised(keys, b, n):
    red = np.zeros(n)
    for beta in range((n + b - 1) // b):
        lo, hi = beta * b, min(n, (beta + 1) * b)
        for a in range(lo, hi):
            others = [keys[a] @ keys[c] for c in range(lo, hi) if c != a]
            red[a] = np.mean(others) if others else 0.0
    return red


def select_ties_reversed(s, k, pinned):
    n = len(s)
    pin = [t for t in range(n) if pinned[t]]
    free = [t for t in range(n) if not pinned[t]]
    ranked = sorted(free, key=lambda t: (-float(s[t]), -t))
    return np.asarray(sorted(pin + ranked[:k - len(pin)]))


def global_without_attention(g, attn, keep, k):
    out = np.zeros(len(g))
    out[:k] = np.asarray(g)[keep[:k]]
    return out


def row_location_ignores_table(table, t, b):
    return t // b, t % b                  # logical block used as the physical one


def pinned_without_prefix(n, n_pinned_blocks, b, w, protect_window):
    m = np.zeros(n, dtype=bool)
    if protect_window:
        m[n - w:] = True
    return m


def pinned_window_one_short(n, n_pinned_blocks, b, w, protect_window):
    m = np.zeros(n, dtype=bool)
    m[: n_pinned_blocks * b] = True
    if protect_window:
        m[n - w + 1:] = True
    return m


def first_hole_one_late(keep):
    for t, src in enumerate(keep):
        if src != t:
            return t + 1
    return len(keep)


def compact_reversed(src_pool, dst_pool, src_table, dst_table, layer, head, keep, b):
    k = len(keep)
    for t, src in enumerate(keep):
        sb, ss = Z.row_location(src_table, int(src), b)
        db, ds = Z.row_location(dst_table, k - 1 - t, b)
        dst_pool[layer, db, head, ds] = src_pool[layer, sb, head, ss]


def compact_reads_through_dst_table(src_pool, dst_pool, src_table, dst_table, layer, head,
                                    keep, b):
    for t, src in enumerate(keep):
        sb, ss = Z.row_location(dst_table, int(src) % (len(dst_table) * b), b)
        db, ds = Z.row_location(dst_table, t, b)
        if (sb, ss) != (db, ds):
            dst_pool[layer, db, head, ds] = src_pool[layer, sb, head, ss]


@pytest.fixture(autouse=True)
def _keep_originals():
    Z._orig_window_attention = Z.window_attention
    Z._orig_lightning_redundancy = Z.lightning_redundancy
    yield


CASES = [
    ("combine_scores", combine_red_sign, P.test_hand_example_causal, ()),
    ("combine_scores", combine_no_global, P.test_hand_example_causal, ()),
    ("window_attention", attention_off_by_one,
     P.test_attention_equals_torch_sdpa_row_mean, (True, 8, 2, 128, 64)),
    ("window_attention", attention_wrong_divisor,
     P.test_attention_equals_torch_sdpa_row_mean, (True, 4, 3, 33, 8)),
    ("window_attention", attention_transposed_group,
     P.test_attention_equals_torch_sdpa_row_mean, (False, 4, 3, 33, 8)),
    ("lightning_redundancy", redundancy_divisor,
     P.test_lightning_equals_full_pairwise_restricted, (64, 16, 32)),
    ("lightning_redundancy", redundancy_unnormalised,
     P.test_redundancy_is_scale_invariant_per_token, ()),
    ("select_keep", select_ties_reversed, P.test_select_forced_ties_keep_prefix,
     ()),
    ("update_global", global_without_attention, P.test_hand_example_causal, ()),
    ("row_location", row_location_ignores_table, P.test_gather_rows_follows_block_table, ()),
    ("pinned_mask", pinned_without_prefix, P.test_pinned_mask_and_hole, ()),
    ("pinned_mask", pinned_window_one_short, P.test_pinned_mask_and_hole, ()),
    ("first_hole", first_hole_one_late, P.test_pinned_mask_and_hole, ()),
    ("compact_unit", compact_reversed, P.test_hand_example_compaction_bytes, ()),
    ("compact_unit", compact_reads_through_dst_table,
     P.test_compress_into_target_blocks_after_a_shared_prefix, ()),
]


@pytest.mark.parametrize("name,mutant,pin,args", CASES,
                         ids=[f"{c[0]}:{c[1].__name__}" for c in CASES])
def test_planted_mistake_is_caught(name, mutant, pin, args):
    assert not _fails(pin, *args), "pin must pass on the real oracle"
    with planted(name, mutant):
        assert _fails(pin, *args), f"{mutant.__name__} slipped past {pin.__name__}"


def test_block_pool_without_private_check_is_caught():
    """A planner that lets a shared or repeated block through after the
    shared run (it would compact into, or free, another request's block)."""
    pin = P.test_block_pool_rejects_shared_or_repeated_private_blocks

    def fails():
        try:
            pin()
        except (AssertionError, pytest.fail.Exception):
            return True
        return False

    assert not fails()
    with mock.patch.object(Z.BlockPool, "check_private", lambda *a, **k: None):
        assert fails()


def capture_row_off_by_one(q_window, q, slot, pos, w):
    S = q_window.shape[0]
    for r in range(q.shape[0]):
        s, p = int(slot[r]), int(pos[r])
        if s < 0 or s >= S or p < 0:
            continue
        for layer in range(q.shape[1]):
            q_window[s, layer, (p + 1) % w] = q[r, layer]   # should be p % w


def capture_ignores_slot(q_window, q, slot, pos, w):
    for r in range(q.shape[0]):
        p = int(pos[r])
        s = max(int(slot[r]), 0) % q_window.shape[0]          # no skip
        for layer in range(q.shape[1]):
            q_window[s, layer, p % w] = q[r, layer]


@pytest.mark.parametrize("fn", [capture_row_off_by_one, capture_ignores_slot])
def test_capture_mistakes_are_caught(fn):
    with planted("capture_queries", fn):
        caught = (_fails(P.test_capture_ring_holds_the_last_w_queries, 4, 11)
                  or _fails(P.test_capture_skips_requests_without_a_slot))
    assert caught
