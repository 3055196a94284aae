"""Pins for the oracle's pooling gradients (pool_single_backward,
pool_dual_backward, treat_backward) on the CPU.

The gradients are pinned against numbers the oracle's formula does not
produce: central finite differences of the forward pooling (a plausible slip in
the backward, a dropped term, a wrong sign or index, a bias summed over the
wrong axis, fails them), plus invariants of a per-channel softmax: the logit
gradients of a block sum to zero per channel, the series gradients of a block
sum to the upstream gradient, uniform logits spread it evenly, and a block
size of one passes it straight through with zero logit gradient.  The entry
treatment's gradient (RMSNorm, then partial RoPE) and the dual gradients are
pinned by finite differences too; the RMSNorm gradient is orthogonal to its
input row, and dual pooling with an absent b-part reduces to the single form.
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


@pytest.mark.parametrize("eps,r", [(1e-6, 0), (-1.0, 8), (1e-3, 8)])
def test_treatment_gradient_matches_finite_differences(eps, r):
    d, pos = 16, np.array([[3.0], [17.0]])
    x = _rand(2, 2, d)
    g = _rand(2, 2, d)
    treat = lambda: O.rope(O.rmsnorm(x, eps) if eps >= 0 else x, pos, r, 10000.0)
    dx = O.treat_backward(x, g, eps, r, 10000.0, pos)
    np.testing.assert_allclose(dx, _numeric(lambda: float((treat() * g).sum()), x), rtol=1e-6, atol=1e-8)


def test_treatment_gradient_is_orthogonal_to_the_row():
    # RMSNorm output is invariant to scaling its input row, so the gradient has no
    # component along x (after undoing the rotation, which keeps x fixed here: r = 0)
    x, g = _rand(3, 32), _rand(3, 32)
    dx = O.treat_backward(x, g, 0.0, 0, 10000.0, np.zeros((3, 1)))
    np.testing.assert_allclose((dx * x).sum(axis=-1), 0.0, atol=1e-12)


def test_dual_gradients_match_finite_differences():
    B, H, m, d, n = 1, 2, 3, 2, 4
    T = n * m
    ca, za, cb, zb = _rand(B, H, T, d), _rand(B, H, T, d), _rand(B, H, T, d), _rand(B, H, T, d)
    ba, bb = _rand(m, d, std=0.3), _rand(m, d, std=0.3)
    e0, e1 = 0, n
    g = _rand(B, H, e1 - e0, d)
    f = lambda: float((O.pool_dual(ca, za, ba, cb, zb, bb, m, e0, e1) * g).sum())
    dca, dza, dba, dcb, dzb, dbb = O.pool_dual_backward(ca, za, ba, cb, zb, bb, m, e0, e1, g)
    for got, arr in ((dca, ca), (dza, za), (dba, ba), (dcb, cb), (dzb, zb), (dbb, bb)):
        np.testing.assert_allclose(got, _numeric(f, arr), rtol=1e-6, atol=1e-8)
    # the b-series block after the last entry's is unused
    assert not dcb[..., (n - 1) * m:, :].any()


def test_dual_with_absent_b_part_equals_single():
    B, H, m, d, n = 1, 1, 4, 3, 3
    x, z = _rand(B, H, n * m, d), _rand(B, H, n * m, d)
    bias = _rand(m, d)
    g = _rand(B, H, n, d)
    dca, dza, dba, dcb, _, _ = O.pool_dual_backward(x, z, bias, x, np.full_like(z, -1e300), bias, m, 0, n, g)
    sx, _, sz, sb = O.pool_single_backward(x, z, bias, m, 0, n, g)
    np.testing.assert_allclose(dca, sx, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dza, sz, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dba, sb, rtol=1e-12, atol=1e-14)
    assert np.abs(dcb).max() < 1e-300
