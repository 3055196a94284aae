"""Pins for the oracle's pooling (single, shared and dual) on the CPU.

Closed forms and invariants fixed by the definition (per-channel softmax over a
block of logit+bias, then a weighted sum): weights sum to one, uniform logits
give the block mean, m=1 is the identity, a per-(block, channel) shift of the
logits changes nothing, one dominant logit selects its token, dual pooling with
an absent b-part equals single pooling, and the brute-force twin agrees.
"""
import numpy as np
import pytest
import torch

from block_compressed_kv_amd import synth
from oracle import brute
from oracle import lbca_oracle as O

RNG = np.random.default_rng(1234)


def _rand(*shape, std=1.0):
    return RNG.standard_normal(shape) * std


def test_weights_sum_to_one_per_channel():
    w = O.pool_weights(_rand(3, 16, 8), _rand(16, 8, std=0.1))
    assert w.shape == (3, 16, 8)
    np.testing.assert_allclose(w.sum(axis=-2), 1.0, atol=1e-14)
    assert (w > 0).all()


def test_uniform_logits_give_block_mean():
    x = _rand(2, 3, 64, 8)
    z = np.full_like(x, 0.37)
    bias = np.zeros((3, 16, 8))
    pk, pv = O.pool_single(x, z, bias, 16, 0, 4, values=2 * x)
    mean = x.reshape(2, 3, 4, 16, 8).mean(axis=-2)
    np.testing.assert_allclose(pk, mean, atol=1e-14)
    np.testing.assert_allclose(pv, 2 * mean, atol=1e-14)


def test_block_size_one_is_identity():
    x = _rand(2, 10, 4)
    out = O.pool_single(x, _rand(2, 10, 4), _rand(1, 4), 1, 0, 10)
    np.testing.assert_allclose(out, x, atol=0)


def test_logit_shift_per_block_channel_is_invariant():
    x, z = _rand(1, 2, 32, 4), _rand(1, 2, 32, 4)
    bias = _rand(2, 8, 4)
    shift = np.repeat(_rand(1, 2, 4, 1, 4) * 5, 8, axis=3).reshape(1, 2, 32, 4)
    a = O.pool_single(x, z, bias, 8, 0, 4)
    b = O.pool_single(x, z + shift, bias, 8, 0, 4)
    np.testing.assert_allclose(a, b, atol=1e-13)


def test_dominant_logit_selects_token():
    x, z = _rand(24, 3), _rand(24, 3) * 0.1
    z[8 + 5, 1] += 60.0          # block 1, offset 5, channel 1
    out = O.pool_single(x, z, np.zeros((8, 3)), 8, 0, 3)
    assert abs(out[1, 1] - x[13, 1]) < 1e-20
    assert not np.isclose(out[1, 0], x[13, 0])


def test_bias_is_indexed_by_offset_and_head():
    # a huge bias at offset 3 of head 1 selects token j*m+3 in every block of head 1 only
    x, z = _rand(1, 2, 40, 4), _rand(1, 2, 40, 4) * 0.01
    bias = np.zeros((2, 8, 4))
    bias[1, 3, :] = 80.0
    out = O.pool_single(x, z, bias, 8, 0, 5)
    np.testing.assert_allclose(out[0, 1], x[0, 1, 3::8], rtol=1e-15, atol=1e-30)
    assert not np.allclose(out[0, 0], x[0, 0, 3::8])


def test_dual_without_b_part_equals_single():
    T, m, d = 32, 4, 6
    ca, za, cb = _rand(T, d), _rand(T, d), _rand(T, d)
    ba, bb = _rand(m, d, std=0.1), _rand(m, d, std=0.1)
    zb = np.full((T, d), -np.inf)
    dual = O.pool_dual(ca, za, ba, cb, zb, bb, m, 0, T // m)
    single = O.pool_single(ca, za, ba, m, 0, T // m)
    np.testing.assert_allclose(dual, single, atol=1e-15)


def test_dual_entry_zero_uses_only_its_block():
    T, m, d = 16, 4, 3
    ca, za, cb, zb = _rand(T, d), _rand(T, d), _rand(T, d), _rand(T, d)
    ba, bb = _rand(m, d), _rand(m, d)
    e0 = O.pool_dual(ca, za, ba, cb, zb, bb, m, 0, 1)[0]
    np.testing.assert_allclose(e0, O.pool_single(ca, za, ba, m, 0, 1)[0], atol=1e-15)
    # changing the b-series of block 0 moves entry 1, not entry 0
    cb2 = cb.copy()
    cb2[:m] += 1.0
    a = O.pool_dual(ca, za, ba, cb, zb, bb, m, 0, 2)
    b = O.pool_dual(ca, za, ba, cb2, zb, bb, m, 0, 2)
    assert np.array_equal(a[0], b[0]) and not np.allclose(a[1], b[1])


def test_brute_force_agrees_single_and_shared():
    T, m, d = 40, 8, 5
    inp = synth.lbca_layer("pool-brute", 1, 2, 2, T, d, m, "f32", "f32")
    k, v, z, bias = (inp[n].numpy().astype(np.float64) for n in ("k", "v", "z", "bias"))
    pk, pv = O.pool_single(k, z, bias, m, 1, 5, values=v)
    for h in range(2):
        for j in range(1, 5):
            np.testing.assert_allclose(pk[0, h, j - 1], brute.pool_block(k[0, h], z[0, h], bias[h], j, m), atol=1e-13)
            np.testing.assert_allclose(pv[0, h, j - 1], brute.pool_block(v[0, h], z[0, h], bias[h], j, m), atol=1e-13)


def test_brute_force_agrees_dual():
    T, m, d = 24, 4, 6
    inp = synth.csa_layer("dual-brute", 1, 2, T, d, m, 2, 4, dtype="bf16")
    f = lambda n: inp[n][0, 0].to(torch.float64).numpy()
    ca, za, cb, zb = f("ca"), f("za"), f("cb"), f("zb")
    ba, bb = inp["bias_a"][0].double().numpy(), inp["bias_b"][0].double().numpy()
    out = O.pool_dual(ca, za, ba, cb, zb, bb, m, 0, T // m)
    for i in range(T // m):
        np.testing.assert_allclose(out[i], brute.pool_dual_entry(ca, za, ba, cb, zb, bb, i, m), atol=1e-13)


def test_pool_matches_library_softmax():
    # scipy's softmax over the token axis as an independent library routine
    from scipy.special import softmax

    x, z, bias = _rand(3, 64, 8), _rand(3, 64, 8), _rand(16, 8, std=0.1)
    w = softmax(z.reshape(3, 4, 16, 8) + bias, axis=2)
    ref = (w * x.reshape(3, 4, 16, 8)).sum(axis=2)
    np.testing.assert_allclose(O.pool_single(x, z, bias, 16, 0, 4), ref, atol=1e-14)


@pytest.mark.parametrize("blocks", [(0, 0), (2, 2)])
def test_empty_block_range(blocks):
    out = O.pool_single(_rand(1, 16, 4), _rand(1, 16, 4), _rand(4, 4), 4, *blocks)
    assert out.shape == (1, 0, 4)
