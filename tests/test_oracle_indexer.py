"""Pins for the oracle's lightning-indexer scores and top-k selection (CPU only).

Brute force (a full sort of every visible entry by (score desc, index asc)), the
k >= visible case, a one-hot head weight reducing to single-head ReLU ranking,
non-negative scores for non-negative weights, and a planted tie that must go to
the lower index.
"""
import numpy as np
import torch

from block_compressed_kv_amd import synth
from oracle import brute
from oracle import lbca_oracle as O


def _inputs(tag, B=2, N=48, HI=4, dI=8):
    g = lambda n, shape, **kw: synth.normal(shape, synth.seed_of(tag, n), **kw).double().numpy()
    qi = g("qi", (B, HI, dI))
    ki = g("ki", (B, N, dI))
    w = synth.uniform((B, HI), synth.seed_of(tag, "w")).double().numpy()
    return qi, w, ki


def test_brute_force_agreement():
    qi, w, ki = _inputs("idx-brute")
    m, k = 4, 5
    for t in (0, 2, 3, 17, 100, 191):
        idx, sc = O.csa_index_topk(qi, w, ki, [t, t], m, k)
        for b in range(2):
            ref, scores = brute.indexer_topk(qi[b], w[b], ki[b], t, m, k)
            assert list(idx[b]) == ref
            n_vis = min((t + 1) // m, ki.shape[1])
            np.testing.assert_allclose(O.index_scores(qi[b], w[b], ki[b], n_vis), scores, atol=1e-13)


def test_fewer_visible_than_k_returns_all_padded():
    qi, w, ki = _inputs("idx-few")
    idx, sc = O.csa_index_topk(qi, w, ki, [10, 10], 4, 8)      # 2 visible
    assert list(idx[0]) == [0, 1, -1, -1, -1, -1, -1, -1]
    assert np.isnan(sc[0, 2:]).all() and not np.isnan(sc[0, :2]).any()


def test_one_hot_weight_is_single_head_relu_ranking():
    qi, w, ki = _inputs("idx-onehot")
    w1 = np.zeros_like(w[0])
    w1[2] = 1.0
    s = O.index_scores(qi[0], w1, ki[0], 48)
    np.testing.assert_allclose(s, np.maximum(ki[0] @ qi[0, 2], 0.0), atol=1e-15)


def test_scores_non_negative_for_non_negative_weights():
    qi, w, ki = _inputs("idx-nonneg")
    assert (O.index_scores(qi[0], w[0], ki[0], 48) >= 0).all()


def test_planted_tie_goes_to_lower_index():
    scores = np.array([0.5, 2.0, 1.0, 2.0, 0.1, 1.0, 3.0])
    assert list(O.topk_select(scores, 2)) == [1, 6]
    assert list(O.topk_select(scores, 3)) == [1, 3, 6]
    assert list(O.topk_select(scores, 4)) == [1, 2, 3, 6]       # 1.0 tie: index 2 before 5
    assert O.topk_margin(scores, 4) == 0.0
    # zero scores (all relu-clipped) tie too: lowest indices win
    assert list(O.topk_select(np.zeros(6), 3)) == [0, 1, 2]


def test_selection_is_the_top_set():
    rng = np.random.default_rng(5)
    s = rng.standard_normal(1000)
    sel = O.topk_select(s, 37)
    assert (np.diff(sel) > 0).all()
    thr = np.sort(s)[::-1][36]
    assert (s[sel] >= thr).all() and (np.delete(s, sel) < thr).all()
