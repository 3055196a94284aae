"""Pins of the oracle's projections around the path (oracle.lbca_oracle:
grouped_projection, indexer_queries, output_projection), read from "CSA:
Compressed Sparse Attention (toy implementation)", "What is implemented"
(low-rank indexer queries, grouped output projection) and "HCA: Heavily
Compressed Attention (toy implementation)", "What is implemented"."""
import numpy as np

from oracle import lbca_oracle as O

rng = np.random.default_rng(7)


def test_grouped_projection_brute_force():
    g, N, K, T = 3, 4, 5, 2
    x = rng.standard_normal((T, g * K))
    w = rng.standard_normal((g, N, K))
    got = O.grouped_projection(x, w)
    for t in range(T):
        for i in range(g):
            for j in range(N):
                s = 0.0
                for l in range(K):
                    s += x[t, i * K + l] * w[i, j, l]
                assert abs(got[t, i * N + j] - s) < 1e-12


def test_grouped_equals_dense_block_diagonal():
    g, N, K = 4, 6, 8
    x = rng.standard_normal((7, g * K))
    w = rng.standard_normal((g, N, K))
    dense = np.zeros((g * N, g * K))
    for i in range(g):
        dense[i * N:(i + 1) * N, i * K:(i + 1) * K] = w[i]
    np.testing.assert_allclose(O.grouped_projection(x, w), x @ dense.T, rtol=1e-12, atol=1e-12)


def test_identity_groups_and_linearity():
    g, K = 2, 5
    x = rng.standard_normal((3, g * K))
    eye = np.stack([np.eye(K)] * g)
    np.testing.assert_array_equal(O.grouped_projection(x, eye), x)
    w = rng.standard_normal((g, 3, K))
    y = rng.standard_normal((3, g * K))
    np.testing.assert_allclose(O.grouped_projection(2 * x - 3 * y, w),
                               2 * O.grouped_projection(x, w) - 3 * O.grouped_projection(y, w), atol=1e-12)


def test_output_projection_is_one_dense_map():
    # W_O after the block-diagonal group maps equals one dense projection W_O B
    H, c, g, dg, dm = 8, 4, 2, 3, 5
    o = rng.standard_normal((6, H, c))
    wg = rng.standard_normal((g, dg, H // g * c))
    wo = rng.standard_normal((dm, g * dg))
    bd = np.zeros((g * dg, H * c))
    for i in range(g):
        bd[i * dg:(i + 1) * dg, i * (H // g) * c:(i + 1) * (H // g) * c] = wg[i]
    np.testing.assert_allclose(O.output_projection(o, wg, wo), o.reshape(6, H * c) @ (wo @ bd).T, atol=1e-12)
    # one group reduces to two plain projections
    wg1, wo1 = rng.standard_normal((1, dg, H * c)), rng.standard_normal((dm, dg))
    np.testing.assert_allclose(O.output_projection(o, wg1, wo1), (o.reshape(6, H * c) @ wg1[0].T) @ wo1.T,
                               atol=1e-12)


def test_indexer_queries_split_into_heads():
    dc, HI, dI = 12, 3, 4
    c = rng.standard_normal((2, 5, dc))
    w = rng.standard_normal((HI * dI, dc))
    q = O.indexer_queries(c, w, HI)
    assert q.shape == (2, 5, HI, dI)
    for h in range(HI):
        np.testing.assert_allclose(q[:, :, h], c @ w[h * dI:(h + 1) * dI].T, atol=1e-12)


def test_pooling_logits_closed_forms():
    # a one-hot hidden state returns one column of W^Z, split into the series;
    # a stacked pair of maps is the pair of single maps
    dm, dim = 10, 4
    w = rng.standard_normal((2 * dim, dm))
    h = np.zeros((3, dm))
    for i, c in enumerate((0, 4, 9)):
        h[i, c] = 1.0
    z = O.pooling_logits(h, w, dim)
    assert z.shape == (3, 2, dim)
    for i, c in enumerate((0, 4, 9)):
        np.testing.assert_array_equal(z[i, 0], w[:dim, c])
        np.testing.assert_array_equal(z[i, 1], w[dim:, c])
    h2 = rng.standard_normal((5, dm))
    za = O.pooling_logits(h2, w[:dim], dim)[:, 0]
    zb = O.pooling_logits(h2, w[dim:], dim)[:, 0]
    np.testing.assert_allclose(O.pooling_logits(h2, w, dim), np.stack([za, zb], axis=1), atol=1e-12)
