"""Pins for the oracle's pooling gradients (pool_single_backward) on the CPU.

The gradients are pinned against numbers the oracle's formula does not
produce: central finite differences of the forward pooling (a plausible slip in
the backward, a dropped term, a wrong sign or index, a bias summed over the
wrong axis, fails them), plus invariants of a per-channel softmax: the logit
gradients of a block sum to zero per channel, the series gradients of a block
sum to the upstream gradient, uniform logits spread it evenly, and a block
size of one passes it straight through with zero logit gradient.
"""
import numpy as np
import pytest

from oracle import lbca_oracle as O

RNG = np.random.default_rng(4321)


def _rand(*shape, std=1.0):
    return RNG.standard_normal(shape) * std


def _loss(x, z, bias, m, b0, b1, g, v=None, gv=None):
    out = O.pool_single(x, z, bias, m, b0, b1, values=v)
    if v is None:
        return float((out * g).sum())
    return float((out[0] * g).sum() + (out[1] * gv).sum())


def _numeric(f, a, eps=1e-6):
    grad = np.zeros_like(a)
    it = np.nditer(a, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        keep = a[i]
        a[i] = keep + eps
        hi = f()
        a[i] = keep - eps
        lo = f()
        a[i] = keep
        grad[i] = (hi - lo) / (2 * eps)
    return grad


@pytest.mark.parametrize("with_values", [False, True])
def test_gradients_match_finite_differences(with_values):
    B, H, m, d, n_blk, b0, b1 = 2, 2, 4, 3, 4, 1, 3
    T = n_blk * m
    x, z = _rand(B, H, T, d), _rand(B, H, T, d)
    bias = _rand(H, m, d, std=0.3)
    v = _rand(B, H, T, d) if with_values else None
    g = _rand(B, H, b1 - b0, d)
    gv = _rand(B, H, b1 - b0, d) if with_values else None
    dx, dv, dz, db = O.pool_single_backward(x, z, bias, m, b0, b1, g, values=v, grad_values=gv)
    f = lambda: _loss(x, z, bias, m, b0, b1, g, v, gv)
    np.testing.assert_allclose(dx, _numeric(f, x), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dz, _numeric(f, z), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(db, _numeric(f, bias), rtol=1e-6, atol=1e-8)
    if with_values:
        np.testing.assert_allclose(dv, _numeric(f, v), rtol=1e-6, atol=1e-8)
    # rows outside the pooled blocks carry no gradient
    assert not dx[..., : b0 * m, :].any() and not dz[..., b1 * m:, :].any()


def test_bias_without_head_axis_sums_over_heads_too():
    B, H, m, d = 2, 3, 4, 2
    x, z = _rand(B, H, 3 * m, d), _rand(B, H, 3 * m, d)
    bias = _rand(m, d)
    g = _rand(B, H, 3, d)
    _, _, _, db = O.pool_single_backward(x, z, bias, m, 0, 3, g)
    np.testing.assert_allclose(db, _numeric(lambda: _loss(x, z, bias, m, 0, 3, g), bias), rtol=1e-6,
                               atol=1e-8)


def test_block_invariants():
    B, H, m, d, n = 1, 2, 8, 5, 3
    x, z, v = _rand(B, H, n * m, d), _rand(B, H, n * m, d), _rand(B, H, n * m, d)
    bias = _rand(H, m, d)
    g, gv = _rand(B, H, n, d), _rand(B, H, n, d)
    dx, dv, dz, _ = O.pool_single_backward(x, z, bias, m, 0, n, g, values=v, grad_values=gv)
    blocks = lambda a: a.reshape(B, H, n, m, d)
    # softmax gradients sum to zero over the block, per channel
    np.testing.assert_allclose(blocks(dz).sum(axis=3), 0.0, atol=1e-12)
    # the weights sum to one, so the series gradients of a block sum to g
    np.testing.assert_allclose(blocks(dx).sum(axis=3), g, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(blocks(dv).sum(axis=3), gv, rtol=1e-12, atol=1e-12)


def test_uniform_logits_and_block_size_one():
    B, H, m, d = 1, 1, 6, 4
    x = _rand(B, H, 2 * m, d)
    z = np.zeros((B, H, 2 * m, d))
    g = _rand(B, H, 2, d)
    dx, _, dz, _ = O.pool_single_backward(x, z, np.zeros((H, m, d)), m, 0, 2, g)
    np.testing.assert_allclose(dx.reshape(B, H, 2, m, d), np.repeat(g[:, :, :, None] / m, m, axis=3),
                               rtol=1e-14)
    xb = x.reshape(B, H, 2, m, d)
    np.testing.assert_allclose(dz.reshape(B, H, 2, m, d), (g[:, :, :, None] / m) * (xb - xb.mean(axis=3, keepdims=True)),
                               rtol=1e-12, atol=1e-14)
    # m = 1: the entry is the token, its gradient passes through, the logit gets none
    x1, z1 = _rand(B, H, 5, d), _rand(B, H, 5, d)
    g1 = _rand(B, H, 5, d)
    dx1, _, dz1, db1 = O.pool_single_backward(x1, z1, _rand(H, 1, d), 1, 0, 5, g1)
    np.testing.assert_allclose(dx1, g1, rtol=1e-14)
    assert np.abs(dz1).max() < 1e-14 and np.abs(db1).max() < 1e-14


def test_empty_range():
    x = _rand(1, 1, 8, 2)
    dx, dv, dz, db = O.pool_single_backward(x, x, _rand(1, 4, 2), 4, 1, 1, np.zeros((1, 1, 0, 2)))
    assert dv is None and not dx.any() and not dz.any() and not db.any()
