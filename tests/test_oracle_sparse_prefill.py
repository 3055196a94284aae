"""Pins for the oracle's CSA sparse prefill (csa_sparse_prefill) on the CPU.

Brute force on tiny sizes: every score summed head by head in plain Python,
the selection by sorting (score descending, then index), the attention by an
explicit softmax over the selected entries and the raw window.  With k at
least the number of visible entries the selection is every visible entry, and
the result is the plain OVERLAP prefill (attend_prefill).  Causality: entries
and indexer keys past the last query's visibility, and raw rows after a
query's position, change nothing for that query.
"""
import math

import numpy as np

from oracle import lbca_oracle as O

RNG = np.random.default_rng(2468)


def _case(B=1, Tq=5, HI=3, dI=4, Hq=2, d=6, m=2, R=12, N=8):
    return dict(qi=RNG.standard_normal((B, Tq, HI, dI)), w=RNG.uniform(size=(B, Tq, HI)),
                ki=RNG.standard_normal((B, N, dI)), q=RNG.standard_normal((B, Tq, Hq, d)),
                entries=RNG.standard_normal((B, N, d)), raw=RNG.standard_normal((B, R, d)))


def test_brute_force_tiny():
    c = _case()
    m, W, k, base, p0, scale = 2, 3, 3, 2, 9, 0.4
    idx, o, lse = O.csa_sparse_prefill(c["qi"], c["w"], c["ki"], c["q"], c["entries"], c["raw"], base, p0,
                                       m, W, k, scale)
    for i in range(c["q"].shape[1]):
        t = p0 + i
        n_vis = (t + 1) // m
        sc = []
        for j in range(n_vis):
            tot = 0.0
            for h in range(c["qi"].shape[2]):
                dot = sum(c["qi"][0, i, h, e] * c["ki"][0, j, e] for e in range(c["qi"].shape[3]))
                tot += c["w"][0, i, h] * max(dot, 0.0)
            sc.append((tot, j))
        chosen = sorted(j for _, j in sorted(sc, key=lambda x: (-x[0], x[1]))[:k])
        assert list(idx[0, i][idx[0, i] >= 0]) == chosen
        rows = [c["entries"][0, j] for j in chosen] + [c["raw"][0, s - base] for s in range(max(0, t - W + 1), t + 1)]
        for h in range(c["q"].shape[2]):
            logits = [scale * float(np.dot(c["q"][0, i, h], r)) for r in rows]
            mx = max(logits)
            ex = [math.exp(x - mx) for x in logits]
            ref = sum(e * r for e, r in zip(ex, rows)) / sum(ex)
            np.testing.assert_allclose(o[0, i, h], ref, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse[0, i, h], mx + math.log(sum(ex)), rtol=1e-12)


def test_k_covering_every_visible_entry_is_dense_overlap_prefill():
    c = _case(B=2, Tq=4, N=10, R=16)
    m, W, base, p0, scale = 2, 4, 3, 15, 0.3
    idx, o, lse = O.csa_sparse_prefill(c["qi"], c["w"], c["ki"], c["q"], c["entries"], c["raw"], base, p0,
                                       m, W, 10, scale)
    ro, rl = O.attend_prefill(c["q"], p0, c["entries"][:, None], None, c["raw"][:, None], None, base, m, W,
                              O.OVERLAP, scale)
    np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=1e-12)
    # query t sees (t + 1) // m entries; the rest of its row is -1 padding
    for i in range(4):
        n_vis = (p0 + i + 1) // m
        assert list(idx[0, i]) == list(range(n_vis)) + [-1] * (10 - n_vis)


def test_causality():
    c = _case(Tq=4, N=10, R=14)
    m, W, k, base, p0, scale = 2, 3, 2, 0, 8, 0.5
    args = lambda cc: O.csa_sparse_prefill(cc["qi"], cc["w"], cc["ki"], cc["q"], cc["entries"], cc["raw"],
                                           base, p0, m, W, k, scale)
    idx, o, lse = args(c)
    d = {n: a.copy() for n, a in c.items()}
    last_vis = (p0 + 3 + 1) // m
    d["entries"][:, last_vis:] = 100.0
    d["ki"][:, last_vis:] = 100.0
    d["raw"][:, p0 + 2 - base:] = -50.0   # rows from position p0 + 2 on
    idx2, o2, lse2 = args(d)
    np.testing.assert_array_equal(idx, idx2)
    np.testing.assert_array_equal(o[:, :2], o2[:, :2])   # queries at p0, p0 + 1 see none of the changes
    assert not np.allclose(o[:, 2:], o2[:, 2:])


def test_treated_chunk_matches_decode_at_each_position():
    c = _case(Tq=3, d=8, N=8, R=16)
    m, W, k, base, p0, scale = 2, 4, 3, 1, 10, 0.35
    tr = dict(sink=np.array([0.2, -0.4]), rmsnorm_eps=1e-6, rope_dims=4, rope_base=100.0)
    idx, o, lse = O.csa_sparse_prefill(c["qi"], c["w"], c["ki"], c["q"], c["entries"], c["raw"], base, p0,
                                       m, W, k, scale, **tr)
    t = [p0, p0 + 1, p0 + 2]
    ro, rl = O.attend_decode(c["q"][0], np.repeat(c["entries"], 3, 0)[:, None], None,
                             np.repeat(c["raw"], 3, 0)[:, None], None, t, m, W, O.OVERLAP, scale,
                             raw_pos_base=[base] * 3, sel_idx=idx[0], **tr)
    np.testing.assert_allclose(o[0], ro, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[0], rl, rtol=1e-12)
