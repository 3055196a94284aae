"""Pins for the oracle's visibility rule and cache accounting (CPU only).

The EXCLUSIVE rule is pinned by the figures the mSeek page prints ("Results"
table and the bullets under it), stored in tests/golden/kv_accounting.json:
they reproduce exactly under EXCLUSIVE and not under the alternatives.
"""
import json
import os

import pytest

from oracle import brute
from oracle import lbca_oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kv_accounting.json")))
GIB = 1 << 30


def _bytes(L, m, mode=O.EXCLUSIVE):
    g = GOLD["model"]
    return O.kv_cache_bytes(L, g["layers"] - g["lbca_layers"], g["lbca_layers"],
                            g["kv_heads"], g["head_dim"], 2, m, GOLD["window"], mode)


def _dense(L):
    g = GOLD["model"]
    return O.kv_cache_bytes(L, g["layers"], 0, g["kv_heads"], g["head_dim"], 2, 64,
                            GOLD["window"])


@pytest.mark.parametrize("mode", [O.EXCLUSIVE, O.OVERLAP])
def test_closed_form_matches_enumeration(mode):
    for m in (1, 2, 3, 4, 7, 16):
        for W in (1, 2, 5, 8, 16, 33):
            for t in range(0, 90):
                n_p, rb = O.visible_range(t, m, W, mode)
                pooled, raw = brute.visible_sets(t, m, W, exclusive=(mode == O.EXCLUSIVE))
                assert pooled == list(range(n_p)), (t, m, W)
                assert raw == list(range(rb, t + 1)), (t, m, W)


def test_exclusive_raw_span_width():
    # the raw span always holds the window and at most m-1 extra tokens
    for m in (4, 16, 64):
        for W in (8, 128):
            for t in range(W, W + 5 * m):
                n_p, rb = O.visible_range(t, m, W, O.EXCLUSIVE)
                assert W <= t - rb + 1 <= W + m - 1


def test_128k_cache_sizes():
    L = 128 * 1024
    gold = GOLD["analytic_kv_128k_gib"]
    assert round(_dense(L) / GIB, 3) == gold["dense"]
    assert round(_bytes(L, 64) / GIB, 3) == gold["lbca"]


def test_reduction_percentages():
    red = lambda L, m: 100.0 * (1 - _bytes(L, m) / _dense(L))
    assert round(red(4096, GOLD["block_schedule"]["initial"])) == GOLD["reduction_percent"]["at_4k"]
    for L in (16384, 32768, 65536, 131072):
        assert round(red(L, GOLD["block_schedule"]["from_16k"])) == \
            GOLD["reduction_percent"]["from_16k_onward_approx"]


def _capacity(budget, m, mode):
    lo, hi = 1, 10_000_000
    while lo < hi:  # largest L with bytes(L) <= budget
        mid = (lo + hi + 1) // 2
        if _bytes(mid, m, mode) <= budget:
            lo = mid
        else:
            hi = mid - 1
    return lo


def test_capacity_in_budget_pins_exclusive_rule():
    cap = GOLD["capacity_tokens"]
    budget = _dense(cap["dense"])
    assert _dense(cap["dense"] + 1) > budget
    assert _capacity(budget, 64, O.EXCLUSIVE) == cap["lbca"]
    assert round(cap["lbca"] / cap["dense"], 2) == cap["ratio_printed"]
    # the overlapping rule does not reproduce the printed capacity
    assert _capacity(budget, 64, O.OVERLAP) != cap["lbca"]


def test_workload_entry_counts():
    # 32K LBCA decode: 510 pooled + 128 raw
    assert O.visible_range(32767, 64, 128, O.EXCLUSIVE) == (510, 32640)
    # tiny layer decode at position 1024, m=16, W=128: 56 pooled + 129 raw
    assert O.visible_range(1024, 16, 128, O.EXCLUSIVE) == (56, 896)
    # HCA 1M context, m'=128: 8192 entries plus the 128-token window
    assert O.visible_range(2 ** 20 - 1, 128, 128, O.OVERLAP) == (8192, 2 ** 20 - 128)
    # CSA 128K context, m=4: 32768 candidate entries
    assert O.visible_range(2 ** 17 - 1, 4, 128, O.OVERLAP)[0] == 32768


def test_invalid_arguments_rejected():
    for args in [(-1, 4, 8, 0), (3, 0, 8, 0), (3, 4, 0, 0), (3, 4, 8, 7)]:
        with pytest.raises(ValueError):
            O.visible_range(*args)
