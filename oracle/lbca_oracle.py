"""fp64 CPU oracle: learned block pooling + attention over pooled entries and a raw window.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Every array is upcast
exactly to float64 on entry; every step is written in the order the pages state
it, with no blocking, fusion or reordering beyond a library matmul, exp or sort.

Pages cited (title, then section):
  [mSeek] "mSeek: learned KV-cache compression in a 3B model"
          (github.dongbeiw.com/mattdani21/mseek-lbca)
  [HCA]   "HCA: Heavily Compressed Attention (toy implementation)"
          (mailtotanvir.github.io/mastering-deepseek-v4-architecture/architecture/hca/)
  [CSA]   "CSA: Compressed Sparse Attention (toy implementation)"
          (mailtotanvir.github.io/mastering-deepseek-v4-architecture/architecture/csa/)

Readings where the pages are silent or garbled:
  * Two visibility rules.  LBCA ([mSeek] "How LBCA works", steps 4-5, and the
    "Results" table) pools a block only once it is complete AND wholly older
    than the W-token window; the raw span runs from the first unpooled block to
    the query (EXCLUSIVE).  HCA/CSA ([HCA] and [CSA] "What is implemented") see
    every causally complete compressed entry plus a separate W-token sliding
    window, which may overlap (OVERLAP).  The published cache figures pin
    EXCLUSIVE exactly (tests/test_oracle_visibility.py).
  * The query's own key/value is in the cache before it attends; position t is
    0-based.
  * Pooling weights are per channel; one logit tensor z serves both K and V;
    the bias is indexed by (head, offset inside the block, channel).
  * Softmax scale is supplied by the caller (1/sqrt(d) by default in tests).
  * GQA: query head h reads KV head h // G.
  * Sink: one logit per query head, in scaled-score units, adding exp(sigma)
    to the softmax denominator only.
  * RMSNorm: x / sqrt(mean(x^2) + eps), unit weight, over the whole head dim.
  * Partial RoPE: the last r dims, rotate-half pairing (k, k + r/2),
    theta_k = base^(-2k/r); a pooled entry sits at its block start j*m, a raw
    token at its own position, the query at t; outputs rotated by -t.
  * Indexer score: I_j = sum_h w_h * relu(q_h . k_j), no scale.
  * Top-k: ties go to the lower index; fewer than k visible -> all visible,
    padded with -1; indices returned in ascending order.
  * Attention backward: the pages train the layer end to end ([mSeek]
    "Experiment at a glance") without writing its gradients out; the oracle
    differentiates the forward above exactly (softmax-attention backward with
    per-query visibility and the sink), pinned by finite differences
    (tests/test_oracle_attention_backward.py).
"""
from __future__ import annotations

import numpy as np

EXCLUSIVE = 0
OVERLAP = 1


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor (CPU): exact upcast
        import torch

        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------------------------
# a1. Visibility
# ----------------------------------------------------------------------------
def visible_range(t: int, m: int, W: int, mode: int) -> tuple[int, int]:
    """Return (number of visible pooled entries, first raw position) for query t.

    EXCLUSIVE ([mSeek] "How LBCA works", steps 4-5): block j (tokens
    [j*m, (j+1)*m)) is a visible summary once it is complete and every token of
    it lies before the W-token window [t-W+1, t]; everything from the first
    unpooled block up to t stays raw.
    OVERLAP ([HCA]/[CSA] "What is implemented"): every block complete by t is
    visible, and the window is exactly the last W tokens [max(0, t-W+1), t].
    """
    if m < 1 or W < 1 or t < 0:
        raise ValueError("need m >= 1, W >= 1, t >= 0")
    if mode == EXCLUSIVE:
        n_pooled = max(0, t + 1 - W) // m
        raw_begin = n_pooled * m
    elif mode == OVERLAP:
        n_pooled = (t + 1) // m
        raw_begin = max(0, t - W + 1)
    else:
        raise ValueError("mode must be EXCLUSIVE or OVERLAP")
    return n_pooled, raw_begin


def cache_entries(L: int, m: int, W: int, mode: int = EXCLUSIVE) -> int:
    """Cache rows per KV head of one compressed layer holding a context of L tokens.

    The last token sits at t = L-1 and its own K/V is cached; the cache keeps the
    visible pooled entries plus the raw span ([mSeek] "How LBCA works").
    """
    n_pooled, raw_begin = visible_range(L - 1, m, W, mode)
    return n_pooled + (L - raw_begin)


def kv_cache_bytes(L: int, n_dense_layers: int, n_lbca_layers: int, kv_heads: int,
                   head_dim: int, elem_bytes: int, m: int, W: int,
                   mode: int = EXCLUSIVE) -> int:
    """Analytic KV bytes of a model whose dense layers keep L rows and whose
    compressed layers keep ``cache_entries`` rows; K and V per row per KV head
    ([mSeek] "Results" table and the bullet list under it)."""
    per_row = kv_heads * head_dim * 2 * elem_bytes
    return per_row * (n_dense_layers * L + n_lbca_layers * cache_entries(L, m, W, mode))


# ----------------------------------------------------------------------------
# a2-a4. Pooling
# ----------------------------------------------------------------------------
def _softmax_over_axis(a, axis):
    a = a - a.max(axis=axis, keepdims=True)
    e = np.exp(a)
    return e / e.sum(axis=axis, keepdims=True)


def pool_weights(z_block, bias):
    """Per-channel softmax over the block's tokens of (content logit + bias).

    ``z_block`` [..., m, d] and ``bias`` [..., m, d] (broadcastable); the softmax
    runs over the token axis (-2) separately for every channel
    ([mSeek] "How LBCA works", steps 2-3; [HCA] "What is implemented", first item).
    """
    return _softmax_over_axis(_f64(z_block) + _f64(bias), axis=-2)


def pool_single(series, logits, bias, m, block_begin, block_end, values=None):
    """LBCA / HCA single-series pooling of blocks [block_begin, block_end).

    ``series``, ``logits`` (and ``values``) are [..., T, d] with token index =
    position.  ``bias`` is [m, d] or [H, m, d]; it broadcasts against the
    series' leading dims from the right, so [H, m, d] pairs with a head axis
    just before T (series [B, H, T, d]).  Block j covers tokens
    [j*m, (j+1)*m).  Returns the pooled keys [..., n, d] (and pooled values when
    ``values`` is given; with ``values`` None the single series is the shared
    K=V entry of HCA).
    """
    x = _f64(series)
    z = _f64(logits)
    b = _f64(bias)
    n = block_end - block_begin
    lead = x.shape[:-2]
    d = x.shape[-1]
    if n <= 0:
        out = np.zeros(lead + (0, d))
        return (out, out.copy()) if values is not None else out
    lo, hi = block_begin * m, block_end * m
    xb = x[..., lo:hi, :].reshape(lead + (n, m, d))
    zb = z[..., lo:hi, :].reshape(lead + (n, m, d))
    w = pool_weights(zb, b[..., None, :, :])           # bias broadcast over blocks
    pk = (w * xb).sum(axis=-2)
    if values is None:
        return pk
    vb = _f64(values)[..., lo:hi, :].reshape(lead + (n, m, d))
    return pk, (w * vb).sum(axis=-2)


def pool_single_backward(series, logits, bias, m, block_begin, block_end, grad_out, values=None,
                         grad_values=None):
    """Gradients of single-series pooling (``pool_single``) of blocks
    [block_begin, block_end) for upstream gradients ``grad_out`` (and
    ``grad_values``) of the pooled rows, [..., n, d].

    The chain rule through the definition ([mSeek] "How LBCA works", steps 2-3:
    a = z + bias, w = softmax over the block's tokens per channel, out = sum w x):
      d series[s] = w[s] * g                              (s in block j, g = grad_out[j])
      d values[s] = w[s] * gv
      d logits[s] = w[s] * (g * (x[s] - out[j]) + gv * (v[s] - vout[j]))
      d bias[i]   = d logits of token j*m + i, summed over blocks and over the
                    leading axes the bias broadcasts along.
    Token rows outside the blocks get zero gradient.  Returns (d_series,
    d_values or None, d_logits, d_bias) in float64, shaped like the inputs.
    """
    x, z, b = _f64(series), _f64(logits), _f64(bias)
    g = _f64(grad_out)
    n = block_end - block_begin
    lead, d = x.shape[:-2], x.shape[-1]
    dx, dz = np.zeros_like(x), np.zeros_like(z)
    v = None if values is None else _f64(values)
    dv = None if values is None else np.zeros_like(v)
    if n <= 0:
        return dx, dv, dz, np.zeros_like(b)
    lo, hi = block_begin * m, block_end * m
    xb = x[..., lo:hi, :].reshape(lead + (n, m, d))
    w = pool_weights(z[..., lo:hi, :].reshape(lead + (n, m, d)), b[..., None, :, :])
    out = (w * xb).sum(axis=-2)                          # [..., n, d]
    gb = g[..., None, :]                                 # one upstream row per block
    dx[..., lo:hi, :] = (w * gb).reshape(lead + (n * m, d))
    da = w * gb * (xb - out[..., None, :])
    if v is not None:
        vb = v[..., lo:hi, :].reshape(lead + (n, m, d))
        vout = (w * vb).sum(axis=-2)
        gvb = _f64(grad_values)[..., None, :]
        dv[..., lo:hi, :] = (w * gvb).reshape(lead + (n * m, d))
        da = da + w * gvb * (vb - vout[..., None, :])
    dz[..., lo:hi, :] = da.reshape(lead + (n * m, d))
    db = da.sum(axis=-3)                                 # over blocks: [..., m, d]
    while db.ndim > b.ndim:                              # over axes the bias broadcasts along
        db = db.sum(axis=0)
    return dx, dv, dz, db


def pool_dual(ca, za, bias_a, cb, zb, bias_b, m, entry_begin, entry_end):
    """CSA dual overlapped pooling ([CSA] "What is implemented", first item).

    Entry i pools its own block i of the a-series (C^a, logits Z^a, bias B^a)
    together with block i-1 of the b-series (C^b, Z^b, B^b) under ONE softmax
    per channel over the 2m logits; entry 0 has no preceding block, so its
    softmax runs over the a-part alone.  Series are [..., T, d]; biases [m, d].
    """
    ca, za, cb, zb = _f64(ca), _f64(za), _f64(cb), _f64(zb)
    ba, bb = _f64(bias_a), _f64(bias_b)
    lead = ca.shape[:-2]
    d = ca.shape[-1]
    out = np.zeros(lead + (entry_end - entry_begin, d))
    for i in range(entry_begin, entry_end):
        la = za[..., i * m:(i + 1) * m, :] + ba            # [..., m, d]
        xa = ca[..., i * m:(i + 1) * m, :]
        if i == 0:
            logits, rows = la, xa
        else:
            lb = zb[..., (i - 1) * m:i * m, :] + bb
            xb = cb[..., (i - 1) * m:i * m, :]
            logits = np.concatenate([la, lb], axis=-2)
            rows = np.concatenate([xa, xb], axis=-2)
        w = _softmax_over_axis(logits, axis=-2)
        out[..., i - entry_begin, :] = (w * rows).sum(axis=-2)
    return out


# ----------------------------------------------------------------------------
# Entry treatment used by HCA / CSA core attention
# ----------------------------------------------------------------------------
def rmsnorm(x, eps):
    """Unit-weight RMSNorm over the last axis ([HCA]/[CSA] "What is implemented")."""
    x = _f64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rope(x, pos, rope_dims, base):
    """Rotate the last ``rope_dims`` dims of x at position(s) ``pos``.

    Rotate-half pairing inside the rotated slice: dim k pairs with k + r/2 and
    turns by angle pos * base^(-2k/r) ([CSA] "What is implemented", third item:
    partial RoPE on the last dims).  ``pos`` broadcasts against x[..., 0];
    a negative pos rotates backwards (used for the -t output rotation).
    """
    x = _f64(x).copy()
    r = int(rope_dims)
    if r == 0:
        return x
    d = x.shape[-1]
    half = r // 2
    k = np.arange(half, dtype=np.float64)
    theta = base ** (-2.0 * k / r)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    x1 = x[..., d - r:d - half].copy()
    x2 = x[..., d - half:].copy()
    x[..., d - r:d - half] = x1 * c - x2 * s
    x[..., d - half:] = x2 * c + x1 * s
    return x


def treat_backward(x, grad_y, eps, rope_dims, base, pos):
    """Gradient with respect to x of y = rope(rmsnorm(x, eps), pos, rope_dims,
    base) for an upstream gradient ``grad_y`` (the chain rule through the
    treatment of ``rmsnorm`` and ``rope`` above; eps < 0 means no RMSNorm,
    rope_dims 0 no RoPE).

    RoPE is a rotation, so its gradient turns grad_y back by the same angle; for
    u = x / r, r = sqrt(mean(x^2) + eps), the gradient is
    (g_u - u * mean(g_u * u)) / r.
    """
    x, g = _f64(x), _f64(grad_y)
    if rope_dims:
        g = rope(g, -np.asarray(pos, dtype=np.float64), rope_dims, base)
    if eps is None or eps < 0:
        return g
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    u = x / r
    return (g - u * np.mean(g * u, axis=-1, keepdims=True)) / r


def pool_dual_backward(ca, za, bias_a, cb, zb, bias_b, m, entry_begin, entry_end, grad_out):
    """Gradients of ``pool_dual`` for upstream gradients ``grad_out`` [..., n, d]
    of entries [entry_begin, entry_end): the single-series formulas of
    ``pool_single_backward`` over the joint 2m-token softmax of each entry
    (block i of the a-series, block i-1 of the b-series; block i alone for
    i = 0).  Returns (d ca, d za, d bias_a, d cb, d zb, d bias_b); the biases
    are [m, d] and sum over blocks and leading axes.
    """
    ca, za, cb, zb = _f64(ca), _f64(za), _f64(cb), _f64(zb)
    ba, bb = _f64(bias_a), _f64(bias_b)
    g = _f64(grad_out)
    dca, dza, dcb, dzb = (np.zeros_like(a) for a in (ca, za, cb, zb))
    dba, dbb = np.zeros(ca.shape[:-2] + ba.shape), np.zeros(ca.shape[:-2] + bb.shape)
    for i in range(entry_begin, entry_end):
        gi = g[..., i - entry_begin, None, :]                  # [..., 1, d]
        la = za[..., i * m:(i + 1) * m, :] + ba
        xa = ca[..., i * m:(i + 1) * m, :]
        if i == 0:
            logits, rows = la, xa
        else:
            logits = np.concatenate([la, zb[..., (i - 1) * m:i * m, :] + bb], axis=-2)
            rows = np.concatenate([xa, cb[..., (i - 1) * m:i * m, :]], axis=-2)
        w = _softmax_over_axis(logits, axis=-2)
        out = (w * rows).sum(axis=-2, keepdims=True)
        dx = w * gi
        da = w * gi * (rows - out)
        dca[..., i * m:(i + 1) * m, :] += dx[..., :m, :]
        dza[..., i * m:(i + 1) * m, :] += da[..., :m, :]
        dba += da[..., :m, :]
        if i > 0:
            dcb[..., (i - 1) * m:i * m, :] += dx[..., m:, :]
            dzb[..., (i - 1) * m:i * m, :] += da[..., m:, :]
            dbb += da[..., m:, :]
    while dba.ndim > ba.ndim:
        dba, dbb = dba.sum(axis=0), dbb.sum(axis=0)
    return dca, dza, dba, dcb, dzb, dbb


# ----------------------------------------------------------------------------
# a5-a7, a10. Attention
# ----------------------------------------------------------------------------
def attend_rows(q, keys, values, scale, sink=None):
    """One query vector against a list of rows under a single softmax.

    logits_j = scale * q.k_j; an optional sink logit sigma adds exp(sigma) to the
    denominator only ([HCA]/[CSA] "What is implemented": attention sink).
    Returns (o, lse) with lse = log(sum_j exp(logit_j) [+ exp(sigma)]).
    """
    q = _f64(q)
    keys = _f64(keys)
    values = _f64(values)
    s = scale * (keys @ q)
    mx = s.max()
    if sink is not None:
        mx = max(mx, float(sink))
    p = np.exp(s - mx)
    den = p.sum()
    if sink is not None:
        den += np.exp(float(sink) - mx)
    o = (p @ values) / den
    return o, mx + np.log(den)


def _rows_for_query(t, m, W, mode, pooled_k, pooled_v, raw_k, raw_v, raw_pos_base,
                    sel):
    """Gather the (positions, K rows, V rows) a query at t sees.

    Pooled entries first (all j < n_pooled, or the selected ones), then the raw
    span [raw_begin, t] read from the raw buffer (row r = position raw_pos_base + r).
    """
    n_pooled, raw_begin = visible_range(t, m, W, mode)
    if sel is None:
        idx = np.arange(n_pooled)
    else:
        sel = np.asarray(sel)
        idx = sel[(sel >= 0) & (sel < n_pooled)]
    rows = np.arange(raw_begin, t + 1) - raw_pos_base
    if rows.size and (rows[0] < 0 or rows[-1] >= raw_k.shape[-2]):
        raise ValueError("raw buffer does not cover the raw span")
    if idx.size and idx.max() >= pooled_k.shape[-2]:
        raise ValueError("pooled buffer does not hold every visible entry")
    pos = np.concatenate([idx * m, np.arange(raw_begin, t + 1)]).astype(np.float64)
    k = np.concatenate([pooled_k[idx], raw_k[rows]], axis=0)
    if pooled_v is None:
        v = None
    else:
        v = np.concatenate([pooled_v[idx], raw_v[rows]], axis=0)
    return pos, k, v


def attend_decode(q, pooled_k, pooled_v, raw_k, raw_v, t, m, W, mode, scale,
                  raw_pos_base=None, sel_idx=None, sink=None, rmsnorm_eps=None,
                  rope_dims=0, rope_base=10000.0):
    """Decode attention for one query per sequence ([mSeek] "How LBCA works",
    step 4; [HCA]/[CSA] "What is implemented").

    q [B, Hq, d]; pooled_k/pooled_v [B, Hkv, N, d]; raw_k/raw_v [B, Hkv, R, d];
    t [B] query positions; raw_pos_base [B] (default 0); sel_idx [B, k] selected
    pooled entries (-1 empty) or None for all visible; sink [Hq] or None.
    ``pooled_v``/``raw_v`` None means one shared series used as K and V (MQA).
    With ``rmsnorm_eps`` / ``rope_dims`` set (shared series only), q and every
    visible row are normalised and rotated at their positions, V is the treated
    row, and the output's rotated dims are turned back by -t.
    Returns o [B, Hq, d] and lse [B, Hq].
    """
    q = _f64(q)
    pk, pv, rk, rv = _f64(pooled_k), _f64(pooled_v), _f64(raw_k), _f64(raw_v)
    shared = pv is None
    if (rv is None) != shared:
        raise ValueError("pooled_v and raw_v must both be given or both be None")
    treat = rmsnorm_eps is not None or rope_dims
    if treat and not shared:
        raise NotImplementedError("entry treatment is defined for a shared K=V series")
    B, Hq, d = q.shape
    Hkv = pk.shape[1]
    G = Hq // Hkv
    o = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    for b in range(B):
        tb = int(t[b])
        base = 0 if raw_pos_base is None else int(raw_pos_base[b])
        sel = None if sel_idx is None else sel_idx[b]
        for kh in range(Hkv):
            pos, krows, vrows = _rows_for_query(
                tb, m, W, mode, pk[b, kh], None if shared else pv[b, kh],
                rk[b, kh], None if shared else rv[b, kh], base, sel)
            if rmsnorm_eps is not None:
                krows = rmsnorm(krows, rmsnorm_eps)
            if rope_dims:
                krows = rope(krows, pos, rope_dims, rope_base)
            if shared:
                vrows = krows
            for g in range(G):
                h = kh * G + g
                qv = q[b, h]
                if rmsnorm_eps is not None:
                    qv = rmsnorm(qv, rmsnorm_eps)
                if rope_dims:
                    qv = rope(qv, tb, rope_dims, rope_base)
                ov, lv = attend_rows(qv, krows, vrows, scale,
                                     None if sink is None else _f64(sink)[h])
                if rope_dims:
                    ov = rope(ov, -tb, rope_dims, rope_base)
                o[b, h] = ov
                lse[b, h] = lv
    return o, lse


def attend_prefill(q, q_pos0, pooled_k, pooled_v, raw_k, raw_v, raw_pos_base, m, W,
                   mode, scale, sink=None):
    """Prefill: every query position t = q_pos0 + i runs the decode rule with its
    own visibility ([mSeek] "How LBCA works", steps 4-5: a query never sees a
    summary that holds a later token, nor one still inside its window).

    q [B, Tq, Hq, d]; pooled_k/pooled_v [B, Hkv, N, d]; raw_k/raw_v
    [B, Hkv, R, d] with row r = position raw_pos_base + r.  Returns
    o [B, Tq, Hq, d], lse [B, Tq, Hq].
    """
    q = _f64(q)
    pk, pv, rk, rv = _f64(pooled_k), _f64(pooled_v), _f64(raw_k), _f64(raw_v)
    B, Tq, Hq, d = q.shape
    Hkv = pk.shape[1]
    G = Hq // Hkv
    sk = None if sink is None else _f64(sink)
    o = np.zeros((B, Tq, Hq, d))
    lse = np.zeros((B, Tq, Hq))
    for i in range(Tq):
        t = q_pos0 + i
        for b in range(B):
            for kh in range(Hkv):
                _, krows, vrows = _rows_for_query(
                    t, m, W, mode, pk[b, kh], None if pv is None else pv[b, kh],
                    rk[b, kh], None if rv is None else rv[b, kh], raw_pos_base, None)
                if vrows is None:
                    vrows = krows
                for g in range(G):
                    h = kh * G + g
                    o[b, i, h], lse[b, i, h] = attend_rows(
                        q[b, i, h], krows, vrows, scale, None if sk is None else sk[h])
    return o, lse


def prefill_chunked(q, keys, values, logits, bias, m, W, chunk, scale, sink=None):
    """Chunked LBCA prefill over a whole context, as a chunked pipeline runs it.

    For each chunk of queries [c0, c1): first pool every block that the chunk's
    last query may see (blocks complete and older than its window), then let
    the chunk's queries attend, each with its own visibility.  keys/values/
    logits are [B, Hkv, T, d], q [B, T, Hq, d], bias [Hkv, m, d].
    Returns o [B, T, Hq, d] and lse [B, T, Hq].
    """
    keys, values = _f64(keys), _f64(values)
    T = keys.shape[-2]
    B, Hkv, _, d = keys.shape
    cap = T // m
    pk = np.zeros((B, Hkv, cap, d))
    pv = np.zeros((B, Hkv, cap, d))
    done = 0
    outs, lses = [], []
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        need, _ = visible_range(c1 - 1, m, W, EXCLUSIVE)
        if need > done:
            a, b_ = pool_single(keys, logits, bias, m, done, need, values=values)
            pk[:, :, done:need] = a
            pv[:, :, done:need] = b_
            done = need
        o, l = attend_prefill(q[:, c0:c1], c0, pk, pv, keys, values, 0, m, W,
                              EXCLUSIVE, scale, sink)
        outs.append(o)
        lses.append(l)
    return np.concatenate(outs, axis=1), np.concatenate(lses, axis=1)


# ----------------------------------------------------------------------------
# a8-a9. CSA lightning indexer and top-k
# ----------------------------------------------------------------------------
def index_scores(qi, w, ki, n_visible):
    """I_j = sum_h w_h * relu(q_h . k_j) for the first ``n_visible`` keys
    ([CSA] "What is implemented", second item: per-head ReLU scores against the
    compressed indexer keys, mixed by learned head weights).

    qi [HI, dI], w [HI], ki [N, dI].  Returns fp64 scores [n_visible].
    """
    qi, w, ki = _f64(qi), _f64(w), _f64(ki)
    s = ki[:n_visible] @ qi.T                    # [n, HI]
    return np.maximum(s, 0.0) @ w


def topk_select(scores, k):
    """Indices of the k largest scores; ties go to the lower index; fewer than
    k candidates -> all of them, padded with -1; returned in ascending index order
    ([CSA] "What is implemented", second item: top-k over visible entries)."""
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[0]
    order = np.lexsort((np.arange(n), -scores))   # primary: -score, secondary: index
    chosen = np.sort(order[:k])
    out = np.full(k, -1, dtype=np.int64)
    out[:chosen.size] = chosen
    return out


def topk_margin(scores, k):
    """Gap between the k-th and (k+1)-th largest score (inf if <= k candidates)."""
    s = np.sort(np.asarray(scores, dtype=np.float64))[::-1]
    if s.size <= k:
        return np.inf
    return s[k - 1] - s[k]


def csa_index_topk(qi, w, ki, t, m, k):
    """Per sequence: visible = floor((t+1)/m) compressed keys (OVERLAP rule);
    score, then select.  qi [B, HI, dI], w [B, HI], ki [B, N, dI], t [B].
    Returns idx [B, k] int64 and the fp64 scores of the selected entries
    (NaN where padded)."""
    B = len(t)
    idx = np.full((B, k), -1, dtype=np.int64)
    sc = np.full((B, k), np.nan)
    for b in range(B):
        n_vis = min((int(t[b]) + 1) // m, ki.shape[1])
        s = index_scores(qi[b], w[b], ki[b], n_vis)
        sel = topk_select(s, k)
        idx[b] = sel
        ok = sel >= 0
        sc[b, ok] = s[sel[ok]]
    return idx, sc


def csa_sparse_prefill(qi, w, ki, q, entries, raw, raw_pos_base, q_pos0, m, W, k, scale,
                       sink=None, rmsnorm_eps=None, rope_dims=0, rope_base=10000.0):
    """CSA prefill of a chunk of consecutive queries ([CSA] "What is implemented",
    second and third items, taken for every query of a chunk): query i sits at
    t = q_pos0 + i, scores the indexer keys visible at t (OVERLAP rule), keeps
    its own top-k, and attends to those entries plus its W-token raw window
    under one softmax (MQA, shared K = V series), exactly the decode rule at t.

    qi [B, Tq, HI, dI], w [B, Tq, HI], ki [B, N, dI]; q [B, Tq, Hq, d];
    entries [B, N, d] (pooled, before the treatment); raw [B, R, d] with row r
    at position raw_pos_base + r.  Returns idx [B, Tq, k] (ascending, -1
    padded), o [B, Tq, Hq, d], lse [B, Tq, Hq].
    """
    B, Tq = q.shape[0], q.shape[1]
    idx = np.full((B, Tq, k), -1, dtype=np.int64)
    o = np.zeros(q.shape)
    lse = np.zeros(q.shape[:3])
    for b in range(B):
        for i in range(Tq):
            t = q_pos0 + i
            sel, _ = csa_index_topk(qi[b, i][None], w[b, i][None], ki[b][None], [t], m, k)
            idx[b, i] = sel[0]
            ob, lb = attend_decode(q[b, i][None], entries[b][None, None], None, raw[b][None, None], None,
                                   [t], m, W, OVERLAP, scale, raw_pos_base=[raw_pos_base], sel_idx=sel,
                                   sink=sink, rmsnorm_eps=rmsnorm_eps, rope_dims=rope_dims,
                                   rope_base=rope_base)
            o[b, i], lse[b, i] = ob[0], lb[0]
    return idx, o, lse


# ----------------------------------------------------------------------------
# Projections around the path ([CSA] "What is implemented", second item: low-rank
# indexer queries; third item and [HCA] "What is implemented": grouped output
# projection).  The pages name both without formulas; the readings:
#   * low-rank indexer queries: q^I_t = W^IUQ c^Q_t, where c^Q_t is the query's
#     low-rank latent (d_c dims) and W^IUQ maps it to all indexer heads at once
#     ([heads * head_dim, d_c]); the result is split into heads;
#   * pooling logits: the content-dependent pooling weights of a series
#     ([CSA] "What is implemented", first item: Z^a, Z^b beside C^a, C^b; [HCA]
#     the same for its single series) are a linear map of the token's hidden
#     state, z_t = W^Z h_t, one row of logits per pooled channel;
#   * grouped output projection: the attention output of a token (all query
#     heads concatenated) is cut into g groups of consecutive heads; group i is
#     projected by its own matrix W_i to an intermediate width, the g results are
#     concatenated and projected by W_O to the model width.
# Weights are stored [out_features, in_features] (each output feature is a
# dot product with one weight row).
# ----------------------------------------------------------------------------
def grouped_projection(x, w):
    """Block-diagonal projection.  x [..., g * K]; w [g, N, K].  The input's last
    axis is cut into g consecutive slices of K; slice i is multiplied by w[i]^T.
    Returns [..., g * N] (group i in columns i*N .. (i+1)*N - 1)."""
    x, w = _f64(x), _f64(w)
    g, N, K = w.shape
    if x.shape[-1] != g * K:
        raise ValueError("input width must be groups x in_features")
    xs = x.reshape(x.shape[:-1] + (g, K))
    out = np.empty(x.shape[:-1] + (g, N))
    for i in range(g):
        out[..., i, :] = xs[..., i, :] @ w[i].T
    return out.reshape(x.shape[:-1] + (g * N,))


def indexer_queries(c_q, w_uq, heads):
    """Low-rank indexer queries: c_q [..., d_c], w_uq [heads * d_I, d_c] ->
    [..., heads, d_I]."""
    q = _f64(c_q) @ _f64(w_uq).T
    return q.reshape(q.shape[:-1] + (heads, q.shape[-1] // heads))


def pooling_logits(h, w_z, dim):
    """Pooling logits of hidden states h [..., d_model]: w_z [series * dim,
    d_model] (series stacked, e.g. Z^a then Z^b) -> [..., series, dim]."""
    z = _f64(h) @ _f64(w_z).T
    return z.reshape(z.shape[:-1] + (z.shape[-1] // dim, dim))


def output_projection(o, w_groups, w_out):
    """Grouped output projection of attention outputs o [..., H, c] (heads
    consecutive): w_groups [g, d_g, (H/g) * c], w_out [d_model, g * d_g]."""
    o = _f64(o)
    flat = o.reshape(o.shape[:-2] + (o.shape[-2] * o.shape[-1],))
    mid = grouped_projection(flat, w_groups)
    return mid @ _f64(w_out).T


# ----------------------------------------------------------------------------
# Attention backward (training the compressed layer: [mSeek] "Experiment at a
# glance", continued pretraining; the gradients of the attention over pooled
# entries plus the window, per query with its own visibility).  Forward per
# query t and query head h: logits l_j = scale * q . k_j over the visible rows
# (pooled entries j < n_p(t), then the raw span), p = softmax(l) with exp(sigma_h)
# added to the denominator when a sink is given, o = sum_j p_j v_j.  For an
# upstream gradient g = dL/do:
#   D = g . o,  dp_j = g . v_j,  ds_j = p_j (dp_j - D)
#   dq = scale * sum_j ds_j k_j,  dk_j += scale * ds_j q,  dv_j += p_j g
#   dsigma_h = -sum over queries of p_sink * D,  p_sink = exp(sigma_h - lse).
# ----------------------------------------------------------------------------
def attend_prefill_backward(q, q_pos0, pooled_k, pooled_v, raw_k, raw_v, raw_pos_base, m, W, mode, scale,
                            grad_out, sink=None):
    """Gradients of attend_prefill (separate K and V series).  Shapes as
    attend_prefill; grad_out [B, Tq, Hq, d].  Returns dq [B, Tq, Hq, d],
    dpooled_k, dpooled_v [B, Hkv, N, d], draw_k, draw_v [B, Hkv, R, d] and dsink
    [Hq] (None without a sink)."""
    q, gout = _f64(q), _f64(grad_out)
    pk, pv, rk, rv = _f64(pooled_k), _f64(pooled_v), _f64(raw_k), _f64(raw_v)
    B, Tq, Hq, d = q.shape
    Hkv = pk.shape[1]
    G = Hq // Hkv
    sk = None if sink is None else _f64(sink)
    dq = np.zeros_like(q)
    dpk, dpv, drk, drv = np.zeros_like(pk), np.zeros_like(pv), np.zeros_like(rk), np.zeros_like(rv)
    dsink = None if sk is None else np.zeros(Hq)
    for i in range(Tq):
        t = q_pos0 + i
        n_p, rb = visible_range(t, m, W, mode)
        rows = np.arange(rb, t + 1) - raw_pos_base
        for b in range(B):
            for kh in range(Hkv):
                keys = np.concatenate([pk[b, kh, :n_p], rk[b, kh, rows]], axis=0)
                vals = np.concatenate([pv[b, kh, :n_p], rv[b, kh, rows]], axis=0)
                for g in range(G):
                    h = kh * G + g
                    lg = scale * (keys @ q[b, i, h])
                    mx = lg.max()
                    if sk is not None:
                        mx = max(mx, sk[h])
                    e = np.exp(lg - mx)
                    den = e.sum() + (0.0 if sk is None else np.exp(sk[h] - mx))
                    p = e / den
                    o = p @ vals
                    go = gout[b, i, h]
                    D = go @ o
                    ds = p * (vals @ go - D)
                    dq[b, i, h] = scale * (ds @ keys)
                    dk = scale * np.outer(ds, q[b, i, h])
                    dv = np.outer(p, go)
                    dpk[b, kh, :n_p] += dk[:n_p]
                    dpv[b, kh, :n_p] += dv[:n_p]
                    drk[b, kh, rows] += dk[n_p:]
                    drv[b, kh, rows] += dv[n_p:]
                    if sk is not None:
                        dsink[h] -= np.exp(sk[h] - mx) / den * D
    return dq, dpk, dpv, drk, drv, dsink
