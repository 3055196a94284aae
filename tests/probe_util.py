"""Inputs and expected results of the exact indexing probes (tests/test_gpu_probes.py).

Two probe inputs make every attention result exact in fp32:
* uniform: q = 0, so every logit is 0 and the output is the plain mean of the
  visible value rows, lse = ln(count);
* spike: q = (SPIKE, 0, ...) and one chosen row with SPIKE in channel 0 of its
  key (every other key row 0 there), so that row's logit is SPIKE^2 * scale and
  all other weights vanish in fp32: the output is that row if it is visible,
  the uniform mean otherwise.
Value rows name themselves (``codes``).  ``expect`` gives the exact fp64 result
from the visibility rule of the oracle (``oracle.lbca_oracle.visible_range``);
tests/test_probe_util.py pins it against the oracle's attention on small cases.
"""
import math

import numpy as np

from oracle import lbca_oracle as O

SPIKE = 64.0


def codes(ids, flag, kvh, seq, d):
    """Self-naming rows [..., d]: channel 0 free for a spike, channels 1-7 the base-8
    digits of the id (entry index or position), 8 a raw (1) / pooled (0) flag, 9 the
    KV head, 10 the sequence.  Small integers: exact in bf16 and in fp32 sums."""
    ids = np.asarray(ids, dtype=np.int64)
    shape = np.broadcast_shapes(ids.shape, np.shape(flag), np.shape(kvh), np.shape(seq))
    c = np.zeros(shape + (d,))
    for i in range(7):
        c[..., 1 + i] = (ids >> (3 * i)) & 7
    c[..., 8] = flag
    c[..., 9] = kvh
    c[..., 10] = seq
    return c


def _softmax_two_level(n_rest, spike_logit, vrow, rest_sum, sink):
    """One row with logit s, n_rest rows with logit 0 and value sum rest_sum, an
    optional sink logit: exact fp64 output and lse."""
    terms_max = max(spike_logit, 0.0 if n_rest else -math.inf, -math.inf if sink is None else sink)
    den = math.exp(spike_logit - terms_max) + n_rest * math.exp(-terms_max)
    if sink is not None:
        den += math.exp(sink - terms_max)
    out = (math.exp(spike_logit - terms_max) * vrow + math.exp(-terms_max) * rest_sum) / den
    return out, terms_max + math.log(den)


def expect(P, Rw, rpb, ts, m, W, mode, scale, sel=None, sink=None, spike=None, spike_row=None):
    """Exact probe result for one (sequence, KV head) at each query position in ts.

    P [N, d] pooled value rows (entry j = row j); Rw [R, d] raw value rows (row r =
    position rpb + r); sel: selected entry ids (-1 and ids not visible skipped) or
    None for every visible entry; sink: one sink logit or None; spike: None (uniform
    probe) or ("pool", j) / ("raw", position) with spike_row its value row.
    Returns out [len(ts), d] and lse [len(ts)].
    """
    Pc = np.vstack([np.zeros((1, P.shape[1])), np.cumsum(P, axis=0)])
    Rc = np.vstack([np.zeros((1, Rw.shape[1])), np.cumsum(Rw, axis=0)])
    out = np.zeros((len(ts), P.shape[1]))
    lse = np.zeros(len(ts))
    for i, t in enumerate(ts):
        n_p, rb = O.visible_range(int(t), m, W, mode)
        if sel is None:
            ids = None
            psum, n_pool = Pc[n_p], n_p
        else:
            s = np.asarray(sel)
            ids = s[(s >= 0) & (s < n_p)]
            psum, n_pool = P[ids].sum(axis=0), ids.size
        lo, hi = rb - rpb, t - rpb + 1
        assert lo >= 0 and hi <= Rw.shape[0] and n_p <= P.shape[0], "probe buffers do not cover the query"
        total = psum + Rc[hi] - Rc[lo]
        n = n_pool + hi - lo
        seen = False
        if spike is not None:
            where, idx = spike
            if where == "pool":
                seen = (idx < n_p) if ids is None else bool(np.isin(idx, ids))
            else:
                seen = rb <= idx <= t
        if seen:
            s_logit = SPIKE * SPIKE * scale
            out[i], lse[i] = _softmax_two_level(n - 1, s_logit, spike_row, total - spike_row, sink)
        else:
            out[i], lse[i] = _softmax_two_level(n, -math.inf, np.zeros_like(total), total, sink) \
                if n else (np.zeros_like(total), -math.inf)
    return out, lse
