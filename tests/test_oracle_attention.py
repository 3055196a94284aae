"""Pins for the oracle's attention (LBCA GQA, HCA/CSA shared-KV MQA) on the CPU.

* dense limit: block size 1, or a window covering the whole context, is exact
  dense causal attention -> torch's scaled_dot_product_attention in fp64;
* causality: inputs at positions > t never change output t;
* chunked prefill equals one-shot prefill equals per-token decode;
* GQA equals MHA with every KV head repeated for its G query heads;
* sink: closed form o_sink = o * sigmoid(lse - sigma);
* RoPE: shifting every position by the same amount leaves the output unchanged
  (relative-position property; pins the -t output rotation);
* RMSNorm: rescaling q or one entry by a positive factor leaves it unchanged;
* brute-force twin agreement for LBCA and for HCA with the full treatment.
"""
import math

import numpy as np
import pytest
import torch

from block_compressed_kv_amd import synth
from oracle import brute
from oracle import lbca_oracle as O


def _np(x):
    return x.to(torch.float64).numpy()


def _layer(tag, T, Hq=2, Hkv=1, d=8, m=4):
    inp = synth.lbca_layer(tag, 1, Hq, Hkv, T, d, m, "f32", "f32", q_len=T)
    return {k: _np(v) for k, v in inp.items()}


def _sdpa_causal(q, k, v, scale):
    # q [B,T,Hq,d]; k,v [B,Hkv,T,d] -> repeat KV heads, library attention in fp64
    G = q.shape[2] // k.shape[1]
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("m,W", [(1, 4), (1, 1), (4, 64), (16, 200)])
def test_dense_limit(m, W):
    T = 48
    L = _layer(f"dense-{m}-{W}", T, Hq=4, Hkv=2, d=8, m=m)
    scale = 1 / math.sqrt(8)
    o, _ = O.prefill_chunked(L["q"], L["k"], L["v"], L["z"], L["bias"], m, W, 16, scale)
    np.testing.assert_allclose(o, _sdpa_causal(L["q"], L["k"], L["v"], scale), atol=1e-13)


def test_textbook_dense_formula_small():
    # the same limit checked against softmax(QK^T/sqrt(d))V written out with a mask
    T, d = 9, 4
    L = _layer("textbook", T, Hq=1, Hkv=1, d=d, m=1)
    q, k, v = L["q"][0, :, 0], L["k"][0, 0], L["v"][0, 0]
    s = q @ k.T / math.sqrt(d)
    s[np.triu_indices(T, 1)] = -np.inf
    p = np.exp(s - s.max(axis=1, keepdims=True))
    ref = (p / p.sum(axis=1, keepdims=True)) @ v
    o, _ = O.prefill_chunked(L["q"], L["k"], L["v"], L["z"], L["bias"], 1, 3, 4, 0.5)
    np.testing.assert_allclose(o[0, :, 0], ref, atol=1e-14)


def test_causality_future_inputs_do_not_leak():
    T, m, W = 60, 4, 8
    L = _layer("causal", T, Hq=2, Hkv=1, d=8, m=m)
    o1, _ = O.prefill_chunked(L["q"], L["k"], L["v"], L["z"], L["bias"], m, W, 60, 0.3)
    t = 37
    L2 = {k: v.copy() for k, v in L.items()}
    for n in ("k", "v", "z"):
        L2[n][:, :, t + 1:] += 3.0
    L2["q"][:, t + 1:] -= 2.0
    o2, _ = O.prefill_chunked(L2["q"], L2["k"], L2["v"], L2["z"], L2["bias"], m, W, 60, 0.3)
    assert np.array_equal(o1[:, :t + 1], o2[:, :t + 1])
    assert not np.allclose(o1[:, t + 1:], o2[:, t + 1:])


def test_chunk_invariance_and_decode_equivalence():
    T, m, W = 64, 4, 8
    L = _layer("chunks", T, Hq=3, Hkv=1, d=8, m=m)
    ref, ref_lse = O.prefill_chunked(L["q"], L["k"], L["v"], L["z"], L["bias"], m, W, T, 0.35)
    for chunk in (1, 7, 16):
        o, lse = O.prefill_chunked(L["q"], L["k"], L["v"], L["z"], L["bias"], m, W, chunk, 0.35)
        np.testing.assert_allclose(o, ref, atol=1e-12, rtol=1e-12)
        np.testing.assert_allclose(lse, ref_lse, atol=1e-12, rtol=1e-12)
    # decode of the last position through a pooled cache equals the prefill row
    t = T - 1
    n_p, _ = O.visible_range(t, m, W, O.EXCLUSIVE)
    pk, pv = O.pool_single(L["k"], L["z"], L["bias"], m, 0, n_p, values=L["v"])
    o, lse = O.attend_decode(L["q"][:, t], pk, pv, L["k"], L["v"], [t], m, W, O.EXCLUSIVE, 0.35)
    np.testing.assert_allclose(o, ref[:, t], atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse[:, t], atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    T, m, W, G = 40, 4, 8, 3
    L = _layer("gqa", T, Hq=2 * G, Hkv=2, d=8, m=m)
    t = T - 1
    n_p, _ = O.visible_range(t, m, W, O.EXCLUSIVE)
    pk, pv = O.pool_single(L["k"], L["z"], L["bias"], m, 0, n_p, values=L["v"])
    o, _ = O.attend_decode(L["q"][:, t], pk, pv, L["k"], L["v"], [t], m, W, O.EXCLUSIVE, 0.3)
    rep = lambda x: np.repeat(x, G, axis=1)
    o2, _ = O.attend_decode(L["q"][:, t], rep(pk), rep(pv), rep(L["k"]), rep(L["v"]), [t], m, W,
                            O.EXCLUSIVE, 0.3)
    np.testing.assert_allclose(o, o2, atol=1e-15)
    # and the mapping is h // G: swapping KV heads changes heads 0..G-1 only by that swap
    o3, _ = O.attend_decode(L["q"][:, t], pk[:, ::-1], pv[:, ::-1], L["k"][:, ::-1],
                            L["v"][:, ::-1], [t], m, W, O.EXCLUSIVE, 0.3)
    assert not np.allclose(o3[:, :G], o[:, :G])


def test_sink_closed_form():
    T, m, W = 50, 4, 8
    L = _layer("sink", T, Hq=2, Hkv=1, d=8, m=m)
    t = T - 1
    n_p, _ = O.visible_range(t, m, W, O.EXCLUSIVE)
    pk, pv = O.pool_single(L["k"], L["z"], L["bias"], m, 0, n_p, values=L["v"])
    args = (L["q"][:, t], pk, pv, L["k"], L["v"], [t], m, W, O.EXCLUSIVE, 0.4)
    o, lse = O.attend_decode(*args)
    sink = np.array([0.7, -1.3])
    o_s, lse_s = O.attend_decode(*args, sink=sink)
    sig = 1 / (1 + np.exp(-(lse - sink)))
    np.testing.assert_allclose(o_s, o * sig[..., None], atol=1e-14)
    np.testing.assert_allclose(lse_s, np.logaddexp(lse, sink), atol=1e-14)
    o_n, _ = O.attend_decode(*args, sink=np.array([-800.0, -800.0]))
    np.testing.assert_allclose(o_n, o, atol=1e-300)


def test_brute_force_lbca():
    T, m, W, d = 45, 4, 8, 6
    L = _layer("brute-lbca", T, Hq=2, Hkv=1, d=d, m=m)
    sink = [0.2, -0.4]
    o, lse = O.prefill_chunked(L["q"], L["k"], L["v"], L["z"], L["bias"], m, W, 11, 0.4,
                               sink=np.array(sink))
    for t in (0, 3, 8, 11, 12, 13, 27, 44):
        res = brute.lbca_query(L["q"][0, t], L["k"][0, 0], L["v"][0, 0], L["z"][0, 0],
                               L["bias"][0], t, m, W, 0.4, sink)
        for g in range(2):
            np.testing.assert_allclose(o[0, t, g], res[g][0], atol=1e-13)
            assert abs(lse[0, t, g] - res[g][1]) < 1e-13


def _hca(tag, T=48, Hq=3, d=16, m=4):
    inp = synth.hca_layer(tag, 1, Hq, T, d, m, dtype="f32")
    return {k: _np(v) for k, v in inp.items()}


def _hca_decode(H, t, m, W, **kw):
    n_p, _ = O.visible_range(t, m, W, O.OVERLAP)
    pooled = O.pool_single(H["c"], H["z"], H["bias"], m, 0, n_p)
    return O.attend_decode(H["q"], pooled, None, H["c"], None, [t], m, W, O.OVERLAP,
                           1 / math.sqrt(H["c"].shape[-1]), **kw)


def test_brute_force_hca_with_treatment():
    T, m, W = 48, 4, 8
    H = _hca("brute-hca", T=T)
    for t in (5, 20, 47):
        o, lse = _hca_decode(H, t, m, W, sink=H["sink"], rmsnorm_eps=1e-6, rope_dims=8,
                             rope_base=10000.0)
        res = brute.hca_query(H["q"][0], H["c"][0, 0], H["z"][0, 0], H["bias"][0], t, m, W,
                              1 / 4, list(H["sink"]), 1e-6, 8, 10000.0)
        for g in range(3):
            np.testing.assert_allclose(o[0, g], res[g][0], atol=1e-12)
            assert abs(lse[0, g] - res[g][1]) < 1e-12


def test_treatment_off_is_plain_mqa():
    T, m, W = 40, 4, 8
    H = _hca("plain", T=T)
    t = T - 1
    o, _ = _hca_decode(H, t, m, W)
    n_p, rb = O.visible_range(t, m, W, O.OVERLAP)
    rows = np.concatenate([O.pool_single(H["c"], H["z"], H["bias"], m, 0, n_p)[0, 0],
                           H["c"][0, 0, rb:t + 1]])
    q = torch.from_numpy(H["q"][0])[:, None]                        # [Hq,1,d]
    kv = torch.from_numpy(rows)[None].expand(3, -1, -1)             # [Hq,n,d]
    ref = torch.nn.functional.scaled_dot_product_attention(q, kv, kv, scale=0.25)[:, 0]
    np.testing.assert_allclose(o[0], ref.numpy(), atol=1e-14)


def test_rope_shift_invariance():
    # same rows at positions shifted by D (a multiple of m): pooled entries re-indexed
    # through selection, raw window through raw_pos_base.
    T, m, W, d = 40, 4, 8, 16
    H = _hca("shift", T=T, d=d)
    t = T - 1
    n_p, rb = O.visible_range(t, m, W, O.OVERLAP)
    pooled = O.pool_single(H["c"], H["z"], H["bias"], m, 0, n_p)
    kw = dict(sink=H["sink"], rmsnorm_eps=1e-6, rope_dims=8, rope_base=10000.0)
    sel = np.arange(n_p)[None]
    o0, l0 = O.attend_decode(H["q"], pooled, None, H["c"], None, [t], m, W, O.OVERLAP, 0.25,
                             sel_idx=sel, **kw)
    for D in (4, 1000, 123456 * m):
        junk = np.full((1, 1, D // m, d), 7.0)
        shifted = np.concatenate([junk, pooled], axis=2)
        o1, l1 = O.attend_decode(H["q"], shifted, None, H["c"], None, [t + D], m, W, O.OVERLAP,
                                 0.25, raw_pos_base=[D], sel_idx=sel + D // m, **kw)
        np.testing.assert_allclose(o1, o0, atol=1e-9)
        np.testing.assert_allclose(l1, l0, atol=1e-9)
    # without the -t output rotation the shift would show: rotating back by a
    # different angle changes the output
    assert not np.allclose(O.rope(o0, 5.0, 8, 10000.0), o0)


def test_rmsnorm_scale_invariance():
    # t=41, m=4: tokens 40 and 41 are raw only; block 2 (tokens 8..11) is pooled only.
    # Pooling is linear in the series, so scaling a whole block scales its entry.
    T, m, W = 42, 4, 8
    H = _hca("rms", T=T)
    t = T - 1
    kw = dict(rmsnorm_eps=0.0, rope_dims=8, rope_base=10000.0, sink=H["sink"])
    o0, _ = _hca_decode(H, t, m, W, **kw)
    H2 = {k: v.copy() for k, v in H.items()}
    H2["q"][0, 1] *= 5.0
    H2["c"][0, 0, 40] *= 0.125
    H2["c"][0, 0, 8:12] *= 3.0
    o1, _ = _hca_decode(H2, t, m, W, **kw)
    np.testing.assert_allclose(o1, o0, atol=1e-13)
    # without the norm the same rescaling does change the output
    o2, _ = _hca_decode(H2, t, m, W, rope_dims=8, rope_base=10000.0)
    o3, _ = _hca_decode(H, t, m, W, rope_dims=8, rope_base=10000.0)
    assert not np.allclose(o2, o3)


def test_rope_zero_dims_is_identity_and_pairing():
    x = np.arange(8.0)
    assert np.array_equal(O.rope(x, 3.0, 0, 10000.0), x)
    # r=4: dims 4..7 rotate; pair (4,6) turns by pos*1, pair (5,7) by pos*0.01
    y = O.rope(x, math.pi / 2, 4, 10000.0)
    np.testing.assert_allclose(y[:4], x[:4])
    np.testing.assert_allclose([y[4], y[6]], [-x[6], x[4]], atol=1e-15)
    a = math.pi / 2 * 0.01
    np.testing.assert_allclose([y[5], y[7]], [x[5] * math.cos(a) - x[7] * math.sin(a),
                                              x[7] * math.cos(a) + x[5] * math.sin(a)])


def test_selection_restricts_pooled_entries():
    T, m, W = 40, 4, 8
    H = _hca("sel", T=T)
    t = T - 1
    n_p, rb = O.visible_range(t, m, W, O.OVERLAP)
    pooled = O.pool_single(H["c"], H["z"], H["bias"], m, 0, n_p)
    sel = np.array([[1, 5, -1, 7, n_p + 3]])          # -1 and invisible ids are skipped
    o, _ = O.attend_decode(H["q"], pooled, None, H["c"], None, [t], m, W, O.OVERLAP, 0.25,
                           sel_idx=sel)
    rows = np.concatenate([pooled[0, 0, [1, 5, 7]], H["c"][0, 0, rb:t + 1]])
    for g in range(3):
        ref, _ = O.attend_rows(H["q"][0, g], rows, rows, 0.25)
        np.testing.assert_allclose(o[0, g], ref, atol=1e-15)
