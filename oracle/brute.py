"""Pure-Python brute-force twin of ``lbca_oracle`` for tiny inputs.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Written separately from
``lbca_oracle``: visibility is found by enumerating blocks and tokens one by one
and testing the pages' membership conditions, and every sum, softmax and dot
product is an explicit loop over Python floats (IEEE double).  Inputs are nested
lists or anything convertible with ``float``.  Intended for T up to ~64.

Pages cited as in ``lbca_oracle``: [mSeek] "mSeek: learned KV-cache compression
in a 3B model"; [HCA] "HCA: Heavily Compressed Attention (toy implementation)";
[CSA] "CSA: Compressed Sparse Attention (toy implementation)".
"""
from __future__ import annotations

import math


def visible_sets(t, m, W, exclusive):
    """Enumerate (pooled block ids, raw token positions) a query at t sees.

    LBCA ([mSeek] "How LBCA works", steps 4-5): a block is a summary once all its
    m tokens exist AND its last token precedes the window [t-W+1, t]; every
    token up to t that is not inside such a block stays raw.
    HCA/CSA ([HCA]/[CSA] "What is implemented"): every complete block is a
    summary and, separately, the last W tokens are raw.
    """
    pooled = []
    j = 0
    while (j + 1) * m - 1 <= t:                # block j complete by t
        last = (j + 1) * m - 1
        if not exclusive or last < t - W + 1:  # wholly older than the window
            pooled.append(j)
        j += 1
    if exclusive:
        covered = set()
        for jj in pooled:
            covered.update(range(jj * m, (jj + 1) * m))
        raw = [s for s in range(t + 1) if s not in covered]
    else:
        raw = [s for s in range(t + 1) if s >= t - W + 1]
    return pooled, raw


def pool_block(xs, zs, bias, j, m):
    """One pooled row: per channel c, softmax over s in block j of
    (zs[s][c] + bias[s - j*m][c]), then the weighted sum of xs[s][c]
    ([mSeek] "How LBCA works", steps 2-3)."""
    d = len(xs[0])
    out = []
    for c in range(d):
        logits = [float(zs[j * m + i][c]) + float(bias[i][c]) for i in range(m)]
        top = max(logits)
        ws = [math.exp(a - top) for a in logits]
        tot = sum(ws)
        out.append(sum(ws[i] / tot * float(xs[j * m + i][c]) for i in range(m)))
    return out


def pool_dual_entry(ca, za, ba, cb, zb, bb, i, m):
    """Entry i of dual pooling: one softmax per channel over block i of the
    a-series and block i-1 of the b-series ([CSA] "What is implemented")."""
    d = len(ca[0])
    out = []
    for c in range(d):
        terms = [(float(za[i * m + s][c]) + float(ba[s][c]), float(ca[i * m + s][c]))
                 for s in range(m)]
        if i > 0:
            terms += [(float(zb[(i - 1) * m + s][c]) + float(bb[s][c]),
                       float(cb[(i - 1) * m + s][c])) for s in range(m)]
        top = max(a for a, _ in terms)
        ws = [math.exp(a - top) for a, _ in terms]
        tot = sum(ws)
        out.append(sum(w * x for w, (_, x) in zip(ws, terms)) / tot)
    return out


def dot(a, b):
    acc = 0.0
    for x, y in zip(a, b):
        acc += float(x) * float(y)
    return acc


def rms_normalise(v, eps):
    ms = sum(float(x) * float(x) for x in v) / len(v)
    r = 1.0 / math.sqrt(ms + eps)
    return [float(x) * r for x in v]


def rotate(v, pos, r, base):
    """Turn pairs (k, k + r/2) of the last r dims by pos * base^(-2k/r)."""
    v = [float(x) for x in v]
    d = len(v)
    half = r // 2
    out = list(v)
    for k in range(half):
        ang = pos * base ** (-2.0 * k / r)
        a, b = v[d - r + k], v[d - half + k]
        out[d - r + k] = a * math.cos(ang) - b * math.sin(ang)
        out[d - half + k] = b * math.cos(ang) + a * math.sin(ang)
    return out


def attend(q, rows_k, rows_v, scale, sink=None):
    """softmax over scale*q.k (plus an optional sink in the denominator), then
    the weighted sum of the value rows; returns (o, lse)."""
    logits = [scale * dot(q, k) for k in rows_k]
    top = max(logits + ([sink] if sink is not None else []))
    ws = [math.exp(a - top) for a in logits]
    den = sum(ws) + (math.exp(sink - top) if sink is not None else 0.0)
    d = len(rows_v[0])
    o = [sum(ws[j] * float(rows_v[j][c]) for j in range(len(ws))) / den for c in range(d)]
    return o, top + math.log(den)


def lbca_query(q_heads, keys, values, logits, bias, t, m, W, scale, sink=None):
    """One LBCA layer for a single KV head and its G query heads at position t,
    computed from the raw history: pool the visible blocks, gather the raw span,
    attend.  keys/values/logits [T][d], bias [m][d], q_heads [G][d]."""
    pooled, raw = visible_sets(t, m, W, exclusive=True)
    rk = [pool_block(keys, logits, bias, j, m) for j in pooled]
    rv = [pool_block(values, logits, bias, j, m) for j in pooled]
    rk += [keys[s] for s in raw]
    rv += [values[s] for s in raw]
    return [attend(qh, rk, rv, scale, None if sink is None else sink[g])
            for g, qh in enumerate(q_heads)]


def hca_query(q_heads, series, logits, bias, t, m, W, scale, sink, eps, r, base):
    """One HCA query (shared K=V series, OVERLAP visibility) with RMSNorm,
    partial RoPE, sink and the -t output rotation ([HCA] "What is implemented")."""
    pooled, raw = visible_sets(t, m, W, exclusive=False)
    rows, pos = [], []
    for j in pooled:
        rows.append(pool_block(series, logits, bias, j, m))
        pos.append(j * m)
    for s in raw:
        rows.append([float(x) for x in series[s]])
        pos.append(s)
    rows = [rotate(rms_normalise(v, eps), p, r, base) for v, p in zip(rows, pos)]
    outs = []
    for g, qh in enumerate(q_heads):
        qv = rotate(rms_normalise(qh, eps), t, r, base)
        o, lse = attend(qv, rows, rows, scale, sink[g])
        outs.append((rotate(o, -t, r, base), lse))
    return outs


def indexer_topk(qi, w, ki, t, m, k):
    """Scores sum_h w_h*relu(q_h.k_j) over visible j (complete blocks), then the
    k best by (score desc, index asc), returned ascending and padded with -1."""
    n_vis = 0
    while (n_vis + 1) * m - 1 <= t and n_vis < len(ki):
        n_vis += 1
    scores = []
    for j in range(n_vis):
        acc = 0.0
        for h in range(len(qi)):
            acc += float(w[h]) * max(0.0, dot(qi[h], ki[j]))
        scores.append(acc)
    best = sorted(range(n_vis), key=lambda j: (-scores[j], j))[:k]
    best.sort()
    return best + [-1] * (k - len(best)), scores
