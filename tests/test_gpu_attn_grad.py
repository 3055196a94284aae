"""GPU parity of the attention backward (lbca_attend_prefill_backward) against the
fp64 oracle (oracle.lbca_oracle.attend_prefill_backward), through the C ABI.

The forward's output and lse come from lbca_attend_prefill on the GPU (they are
inputs of the backward only; the oracle recomputes everything from q, K, V and
the upstream gradient).  Sizes span several 128-key workgroups, query runs
split across workgroups (more than 1024 flattened rows), ragged tails, both
visibility rules, GQA groups of 2 and 3, a shared K=V series with a sink, a raw
buffer that starts past position 0, chunked backward with accumulation, and an
empty chunk.  Tolerance: the bf16 bar of tests/parity_util.py on every gradient.
"""
import math

import numpy as np
import pytest
import torch

from block_compressed_kv_amd import synth
from oracle import lbca_oracle as O

from parity_util import check_bf16, host, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(tag, B, Tq, Hq, Hkv, d, N, R, shared, sink):
    g = lambda n, shape: synth.normal(shape, synth.seed_of("attn-grad", tag, n), dtype="bf16", device=DEV)
    x = dict(q=g("q", (B, Tq, Hq, d)), pk=g("pk", (B, Hkv, N, d)), rk=g("rk", (B, Hkv, R, d)),
             do=g("do", (B, Tq, Hq, d)))
    x["pv"] = None if shared else g("pv", (B, Hkv, N, d))
    x["rv"] = None if shared else g("rv", (B, Hkv, R, d))
    x["sink"] = synth.normal((Hq,), synth.seed_of("attn-grad", tag, "sink"), device=DEV) if sink else None
    return x


def _oracle(x, q0, rpb, m, W, mode, scale, sl=slice(None)):
    """Oracle gradients for queries sl of x; a shared series is passed as both K and V
    and its gradient is the sum of both roles."""
    pk, rk = host(x["pk"]), host(x["rk"])
    pv = pk if x["pv"] is None else host(x["pv"])
    rv = rk if x["rv"] is None else host(x["rv"])
    sink = None if x["sink"] is None else host(x["sink"])
    q, do = host(x["q"][:, sl]), host(x["do"][:, sl])
    start = sl.start or 0
    dq, dpk, dpv, drk, drv, ds = O.attend_prefill_backward(q, q0 + start, pk, pv, rk, rv, rpb, m, W, mode, scale,
                                                          do, sink=sink)
    if x["pv"] is None:
        return dq, dpk + dpv, None, drk + drv, None, ds
    return dq, dpk, dpv, drk, drv, ds


def _check_all(got, ref, what):
    names = ("dq", "d pooled k", "d pooled v", "d raw k", "d raw v", "d sink")
    for n, g, r in zip(names, got, ref):
        if r is None:
            assert g is None, (what, n)
            continue
        check_bf16(host(g), r, f"{what}: {n}")


@pytest.mark.parametrize("case", [
    # tag, B, Tq, q0, Hq, Hkv, d, m, W, mode, raw base, shared, sink, out dtype
    ("excl-d64-split", 1, 700, 0, 4, 2, 64, 2, 6, O.EXCLUSIVE, 0, False, False, torch.float32),
    ("ovl-d128-shared-sink", 2, 300, 200, 6, 2, 128, 8, 32, O.OVERLAP, 150, True, True, torch.bfloat16),
    ("excl-d128-gqa3", 1, 1200, 0, 6, 2, 128, 16, 128, O.EXCLUSIVE, 0, False, False, torch.float32),
    ("ovl-d64-mqa-sink", 2, 260, 77, 8, 1, 64, 4, 16, O.OVERLAP, 0, False, True, torch.float32),
])
def test_attention_backward(lib, case):
    tag, B, Tq, q0, Hq, Hkv, d, m, W, mode, rpb, shared, sink, odt = case
    last = q0 + Tq - 1
    N = O.visible_range(last, m, W, mode)[0] + 3       # 3 entries no query sees: zero gradient
    R = last + 1 - rpb
    say(f"attention backward {tag}: B={B} Tq={Tq} q0={q0} Hq={Hq} Hkv={Hkv} d={d} m={m} W={W} N={N} R={R}")
    x = _inputs(tag, B, Tq, Hq, Hkv, d, N, R, shared, sink)
    scale = 1 / math.sqrt(d)
    o, lse = lib.attend_prefill(x["q"], q0, x["pk"], x["rk"], rpb, m, W, mode, pooled_v=x["pv"], raw_v=x["rv"],
                                sink=x["sink"], out_dtype=odt)
    got = lib.attend_prefill_backward(x["q"], q0, x["pk"], x["rk"], rpb, m, W, mode, o, lse, x["do"],
                                      pooled_v=x["pv"], raw_v=x["rv"], sink=x["sink"])
    torch.cuda.synchronize()
    _check_all(got, _oracle(x, q0, rpb, m, W, mode, scale), tag)
    assert (got[1][:, :, N - 3:] == 0).all()


def test_chunked_backward_accumulates(lib):
    # two query chunks, the second adding into the first's key/value/sink gradients,
    # equal the one-shot oracle gradients
    B, Tq, Hq, Hkv, d, m, W, mode = 1, 640, 6, 2, 128, 4, 24, O.EXCLUSIVE
    N = O.visible_range(Tq - 1, m, W, mode)[0]
    x = _inputs("chunked", B, Tq, Hq, Hkv, d, N, Tq, False, True)
    o, lse = lib.attend_prefill(x["q"], 0, x["pk"], x["rk"], 0, m, W, mode, pooled_v=x["pv"], raw_v=x["rv"],
                                sink=x["sink"], out_dtype=torch.float32)
    dq = torch.empty((B, Tq, Hq, d), dtype=torch.float32, device=DEV)
    bufs = None
    for c0, c1 in ((0, 250), (250, Tq)):
        sub = lambda t: t[:, c0:c1] if t.dim() == 4 else t[:, c0:c1].contiguous()  # lse stays dense
        kw = {} if bufs is None else dict(zip(("grad_pooled_k", "grad_pooled_v", "grad_raw_k", "grad_raw_v",
                                               "grad_sink"), bufs))
        g = lib.attend_prefill_backward(sub(x["q"]), c0, x["pk"], x["rk"], 0, m, W, mode, sub(o), sub(lse),
                                        sub(x["do"]), pooled_v=x["pv"], raw_v=x["rv"], sink=x["sink"],
                                        accumulate=bufs is not None, **kw)
        dq[:, c0:c1] = g[0]
        bufs = g[1:]
    torch.cuda.synchronize()
    _check_all((dq,) + tuple(bufs), _oracle(x, 0, 0, m, W, mode, 1 / math.sqrt(d)), "chunked")


def test_empty_chunk_zeroes_key_gradients(lib):
    B, Hq, Hkv, d, N, R = 1, 4, 2, 64, 10, 50
    x = _inputs("empty", B, 1, Hq, Hkv, d, N, R, False, True)
    q = x["q"][:, :0]
    o = torch.empty((B, 0, Hq, d), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, 0, Hq), dtype=torch.float32, device=DEV)
    bufs = [torch.full(s, 5.0, device=DEV) for s in ((B, Hkv, N, d), (B, Hkv, N, d), (B, Hkv, R, d),
                                                     (B, Hkv, R, d), (Hq,))]
    g = lib.attend_prefill_backward(q, 20, x["pk"], x["rk"], 0, 4, 8, O.EXCLUSIVE, o, lse, q, pooled_v=x["pv"],
                                    raw_v=x["rv"], sink=x["sink"], grad_pooled_k=bufs[0], grad_pooled_v=bufs[1],
                                    grad_raw_k=bufs[2], grad_raw_v=bufs[3], grad_sink=bufs[4])
    torch.cuda.synchronize()
    for t in g[1:]:
        assert (t == 0).all()
