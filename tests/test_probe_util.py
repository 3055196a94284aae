"""The expected results of the exact indexing probes (tests/probe_util.py) agree
with the oracle's attention (oracle.lbca_oracle.attend_decode / attend_prefill)
on small cases of every probe form: uniform and spike, both visibility rules,
separate and shared series, selected entries, a sink."""
import math

import numpy as np
import pytest

from oracle import lbca_oracle as O
from probe_util import SPIKE, codes, expect


@pytest.mark.parametrize("mode", [O.EXCLUSIVE, O.OVERLAP])
@pytest.mark.parametrize("shared", [False, True])
def test_expect_matches_oracle_decode(mode, shared):
    d, m, W, N, R, rpb = 16, 4, 6, 12, 40, 3
    P = codes(np.arange(N), 0, 0, 0, d)
    Rw = codes(rpb + np.arange(R), 1, 0, 0, d)
    scale = 1 / math.sqrt(d)
    rng = np.random.default_rng(0)
    for t in [9, 10, 11, 20, 33, 41]:
        n_p, rb = O.visible_range(t, m, W, mode)
        for sel in [None, np.array([2, -1, 0, n_p, 5, 1])]:
            for sink in [None, 0.0, 1.5]:
                spikes = [None, ("pool", 0), ("pool", max(n_p - 1, 0)), ("pool", n_p), ("raw", rb), ("raw", rb - 1),
                          ("raw", t), ("raw", t + 1)]
                for sp in spikes:
                    if sp is not None and sp[0] == "pool" and sp[1] >= N:
                        continue
                    Kp, Kr = (P.copy(), Rw.copy()) if shared else (np.zeros_like(P), np.zeros_like(Rw))
                    q = np.zeros(d)
                    row = None
                    if sp is not None:
                        q[0] = SPIKE
                        if sp[0] == "pool":
                            Kp[sp[1], 0] = SPIKE
                            row = (Kp if shared else P)[sp[1]]
                        else:
                            Kr[sp[1] - rpb, 0] = SPIKE
                            row = (Kr if shared else Rw)[sp[1] - rpb]
                    Pv, Rv = (Kp, Kr) if shared else (P, Rw)
                    got_o, got_l = expect(Pv, Rv, rpb, [t], m, W, mode, scale, sel=sel, sink=sink, spike=sp,
                                          spike_row=row)
                    ro, rl = O.attend_decode(q[None, None], Kp[None, None], None if shared else P[None, None],
                                             Kr[None, None], None if shared else Rw[None, None], [t], m, W, mode,
                                             scale, raw_pos_base=[rpb], sel_idx=None if sel is None else sel[None],
                                             sink=None if sink is None else np.array([sink]))
                    np.testing.assert_allclose(got_o[0], ro[0, 0], rtol=1e-12, atol=1e-12)
                    np.testing.assert_allclose(got_l[0], rl[0, 0], rtol=1e-12, atol=1e-12)


def test_expect_matches_oracle_prefill():
    d, m, W, q_pos0, Tq = 16, 4, 6, 5, 30
    n_last, _ = O.visible_range(q_pos0 + Tq - 1, m, W, O.EXCLUSIVE)
    _, rb0 = O.visible_range(q_pos0, m, W, O.EXCLUSIVE)
    P = codes(np.arange(n_last), 0, 0, 0, d)
    Rw = codes(rb0 + np.arange(q_pos0 + Tq - rb0), 1, 0, 0, d)
    scale = 1 / math.sqrt(d)
    ts = q_pos0 + np.arange(Tq)
    for sp in [None, ("pool", 3), ("raw", 20), ("raw", rb0)]:
        Kp, Kr = np.zeros_like(P), np.zeros_like(Rw)
        q = np.zeros((1, Tq, 1, d))
        row = None
        if sp is not None:
            q[..., 0] = SPIKE
            if sp[0] == "pool":
                Kp[sp[1], 0] = SPIKE
                row = P[sp[1]]
            else:
                Kr[sp[1] - rb0, 0] = SPIKE
                row = Rw[sp[1] - rb0]
        got_o, got_l = expect(P, Rw, rb0, ts, m, W, O.EXCLUSIVE, scale, spike=sp, spike_row=row)
        ro, rl = O.attend_prefill(q, q_pos0, Kp[None, None], P[None, None], Kr[None, None], Rw[None, None], rb0, m,
                                  W, O.EXCLUSIVE, scale)
        np.testing.assert_allclose(got_o, ro[0, :, 0], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(got_l, rl[0, :, 0], rtol=1e-12, atol=1e-12)


def test_codes_name_rows():
    c = codes(np.arange(300000), 1, 3, 5, 16)
    digits = c[:, 1:8].astype(np.int64)
    ids = (digits * (8 ** np.arange(7))).sum(axis=1)
    assert (ids == np.arange(300000)).all()
    assert (c[:, 0] == 0).all() and (c[:, 8] == 1).all() and (c[:, 9] == 3).all() and (c[:, 10] == 5).all()


def test_topk_tie_band_fails_unless_allowed():
    """The selection check: a clear margin demands the exact set; a k-th/(k+1)-th
    pair closer than its fp32 bounds fails unless the test opts in, and then only
    a top-k of scores within the bounds passes."""
    from parity_util import topk_matches
    s = np.array([5.0, 1.0, 3.0, 2.0, 4.0])
    err = np.full(5, 1e-3)
    margin, band = topk_matches(np.array([0, 2, 4, -1]), s, 3, "clear", err)
    assert not band and margin == pytest.approx(1.0)
    with pytest.raises(AssertionError):
        topk_matches(np.array([0, 3, 4]), s, 3, "wrong set", err)
    s2 = np.array([5.0, 3.0004, 3.0, 2.0, 4.0])  # 2nd and 3rd of the top-3 within 2e-3
    with pytest.raises(AssertionError, match="tie band"):
        topk_matches(np.array([0, 1, 4]), s2, 3, "band", err)
    _, band = topk_matches(np.array([0, 2, 4]), s2, 3, "band", err, allow_band=True)  # the other tie order
    assert band
    with pytest.raises(AssertionError):
        topk_matches(np.array([0, 3, 4]), s2, 3, "band", err, allow_band=True)  # 2.0 is not within the bounds
    # with the kernel's own fp32 scores the band case is exact: those scores within
    # their bounds, and the set their top-k (ties to the lower index)
    own = np.array([5.0, 2.9999, 3.0, 2.0, 4.0], dtype=np.float32)
    assert topk_matches(np.array([0, 2, 4]), s2, 3, "band", err, gpu_scores=own)[1]
    with pytest.raises(AssertionError, match="own fp32 scores"):
        topk_matches(np.array([0, 1, 4]), s2, 3, "band", err, gpu_scores=own)
    with pytest.raises(AssertionError, match="outside their fp32 bound"):
        topk_matches(np.array([0, 2, 4]), s2, 3, "band", err, gpu_scores=own + np.float32(0.01))
