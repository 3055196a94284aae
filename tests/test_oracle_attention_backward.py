"""Pins of the oracle's attention backward (oracle.lbca_oracle.attend_prefill_backward),
the gradients of attention over the visible pooled entries plus the raw window
("mSeek: learned KV-cache compression in a 3B model", "How LBCA works", steps
4-5; trained end to end, "Experiment at a glance"):
* central finite differences of the forward oracle (attend_prefill) along
  random directions, for every input, both visibility rules, with and without
  a sink;
* without a sink the logit gradients of each query sum to zero, so the key
  gradients of a KV head sum to zero and its value gradients sum to the
  upstream gradients;
* with a window covering the context (or m = 1) it is dense causal attention:
  equal to the autograd gradients of torch's scaled_dot_product_attention in fp64;
* the chain into the pooling gradients (pool_single_backward) equals finite
  differences of the pooled-then-attended loss with respect to the raw history.
"""
import math

import numpy as np
import pytest
import torch

from oracle import lbca_oracle as O

rng = np.random.default_rng(11)


def _case(B=1, Tq=9, q_pos0=21, Hq=4, Hkv=2, d=8, m=4, W=6, mode=O.EXCLUSIVE):
    T = q_pos0 + Tq
    n_last, _ = O.visible_range(T - 1, m, W, mode)
    N = n_last + 1
    return dict(q=rng.standard_normal((B, Tq, Hq, d)), pk=rng.standard_normal((B, Hkv, N, d)),
                pv=rng.standard_normal((B, Hkv, N, d)), rk=rng.standard_normal((B, Hkv, T, d)),
                rv=rng.standard_normal((B, Hkv, T, d)), g=rng.standard_normal((B, Tq, Hq, d)),
                q_pos0=q_pos0, m=m, W=W, mode=mode)


def _loss(c, sink, **over):
    x = dict(c, **over)
    o, _ = O.attend_prefill(x["q"], c["q_pos0"], x["pk"], x["pv"], x["rk"], x["rv"], 0, c["m"], c["W"], c["mode"],
                            0.35, sink=sink)
    return float((o * c["g"]).sum())


@pytest.mark.parametrize("mode", [O.EXCLUSIVE, O.OVERLAP])
@pytest.mark.parametrize("with_sink", [False, True])
def test_finite_differences(mode, with_sink):
    c = _case(mode=mode)
    sink = rng.standard_normal(4) if with_sink else None
    dq, dpk, dpv, drk, drv, ds = O.attend_prefill_backward(c["q"], c["q_pos0"], c["pk"], c["pv"], c["rk"], c["rv"],
                                                          0, c["m"], c["W"], mode, 0.35, c["g"], sink=sink)
    eps = 1e-6
    for name, grad in (("q", dq), ("pk", dpk), ("pv", dpv), ("rk", drk), ("rv", drv)):
        for _ in range(3):
            dirn = rng.standard_normal(c[name].shape)
            num = (_loss(c, sink, **{name: c[name] + eps * dirn}) - _loss(c, sink, **{name: c[name] - eps * dirn})) / (2 * eps)
            assert abs(num - (grad * dirn).sum()) < 1e-6 * max(1.0, abs(num)), name
    if with_sink:
        dirn = rng.standard_normal(4)
        num = (_loss(c, sink + eps * dirn) - _loss(c, sink - eps * dirn)) / (2 * eps)
        assert abs(num - (ds * dirn).sum()) < 1e-6 * max(1.0, abs(num))
    else:
        assert ds is None


def test_key_gradients_sum_to_zero_value_gradients_to_upstream():
    c = _case(B=2, Tq=12, q_pos0=30)
    dq, dpk, dpv, drk, drv, _ = O.attend_prefill_backward(c["q"], c["q_pos0"], c["pk"], c["pv"], c["rk"], c["rv"],
                                                         0, c["m"], c["W"], c["mode"], 0.35, c["g"])
    G = 2
    for b in range(2):
        for kh in range(2):
            np.testing.assert_allclose(dpk[b, kh].sum(0) + drk[b, kh].sum(0), 0, atol=1e-12)
            np.testing.assert_allclose(dpv[b, kh].sum(0) + drv[b, kh].sum(0),
                                       c["g"][b, :, kh * G:(kh + 1) * G].sum((0, 1)), atol=1e-12)


@pytest.mark.parametrize("m,W", [(1, 3), (4, 64)])
def test_dense_limit_matches_torch_autograd(m, W):
    # m = 1 pools single tokens (entries equal the raw rows); a window covering the
    # context pools nothing visible: both are dense causal attention over positions
    B, T, Hq, Hkv, d = 1, 12, 2, 1, 8
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    q = rng.standard_normal((B, T, Hq, d))
    g = rng.standard_normal((B, T, Hq, d))
    dq, dpk, dpv, drk, drv, _ = O.attend_prefill_backward(q, 0, k, v, k, v, 0, m, W, O.EXCLUSIVE, 0.3, g)
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    vt = torch.tensor(v, requires_grad=True)
    ot = torch.nn.functional.scaled_dot_product_attention(qt.transpose(1, 2), kt.expand(B, Hq, T, d),
                                                          vt.expand(B, Hq, T, d), is_causal=True, scale=0.3)
    (ot.transpose(1, 2) * torch.tensor(g)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dpk + drk, kt.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dpv + drv, vt.grad.numpy(), atol=1e-10)


def test_chain_through_pooling_matches_finite_differences():
    # history -> pooled entries (pool_single) -> attention; the history gradient is
    # the raw-row gradient plus the pooling gradient of the entry gradients
    B, Hq, Hkv, d, m, W, Tq, q0 = 1, 2, 1, 8, 4, 6, 8, 20
    T = q0 + Tq
    x = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    z = rng.standard_normal((B, Hkv, T, d))
    bias = rng.standard_normal((Hkv, m, d)) * 0.1
    q = rng.standard_normal((B, Tq, Hq, d))
    g = rng.standard_normal((B, Tq, Hq, d))
    N = O.visible_range(T - 1, m, W, O.EXCLUSIVE)[0]

    def loss(xx, vv, zz):
        pk, pv = O.pool_single(xx, zz, bias, m, 0, N, values=vv)
        o, _ = O.attend_prefill(q, q0, pk, pv, xx, vv, 0, m, W, O.EXCLUSIVE, 0.4)
        return float((o * g).sum())

    pk, pv = O.pool_single(x, z, bias, m, 0, N, values=v)
    _, dpk, dpv, drk, drv, _ = O.attend_prefill_backward(q, q0, pk, pv, x, v, 0, m, W, O.EXCLUSIVE, 0.4, g)
    dx, dv, dz, _ = O.pool_single_backward(x, z, bias, m, 0, N, dpk, values=v, grad_values=dpv)
    gx, gv = dx + drk, dv + drv
    eps = 1e-6
    for name, grad in (("x", gx), ("v", gv), ("z", dz)):
        dirn = rng.standard_normal(x.shape)
        args = {"x": x, "v": v, "z": z}
        plus = dict(args, **{name: args[name] + eps * dirn})
        minus = dict(args, **{name: args[name] - eps * dirn})
        num = (loss(plus["x"], plus["v"], plus["z"]) - loss(minus["x"], minus["v"], minus["z"])) / (2 * eps)
        assert abs(num - (grad * dirn).sum()) < 1e-6 * max(1.0, abs(num)), name
