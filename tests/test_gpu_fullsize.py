"""GPU parity at the workloads' full sizes, in the launch shapes bench.py times.

The GPU runs every call at full size; the fp64 oracle recomputes sampled
outputs (whole units, query positions or sequences) one by one, from the same
seeded inputs copied exactly to the host.  Tolerances: tests/parity_util.py.

  * Llama-3.2-3B decode at 32K, batch 16: all 510 blocks pooled, one decode
    launch; three (sequence, KV head) units checked (pooled entries and the
    three query heads of each).
  * Chunked prefill at 16K in 2048-token chunks: every chunk pools its new
    blocks then attends; all pooled entries and 16 query positions (chunk
    edges, window edges, random) checked for all 24 heads.
  * Attention backward at 16K, one call over all 16384 queries (the
    Llama-shaped layer, 1016 pooled entries, random bf16 inputs and upstream
    gradient): 12 query positions' dq, 6 raw positions' and 4 pooled entries'
    dK/dV recomputed from exactly the queries that see them (the entries seen
    by more than 1024 rows span two query runs).
  * HCA at 1M context, batch 4: 8192 treated entries pooled, decode with
    RMSNorm, partial RoPE and a sink; one sequence recomputed by the oracle,
    which streams its 2^20 tokens block range by block range.
  * CSA at 128K, batch 2: dual pooling of 32768 treated entries, indexer
    top-512 over 32768 keys (sets compared exactly), decode over the selection
    plus the window.
"""
import math

import numpy as np
import pytest
import torch

from block_compressed_kv_amd import synth
from oracle import lbca_oracle as O

from parity_util import check_bf16, host, index_score_bound, index_ws_scores, say, topk_matches

pytestmark = pytest.mark.gpu
DEV = "cuda"
EPS, RD, BASE = 1e-6, 64, 10000.0


def _cpu(t):
    return t.detach().to("cpu")


def test_llama_decode_32k_batch16(lib):
    B, Hq, Hkv, d, m, W, T, N = 16, 24, 8, 128, 64, 128, 32768, 510
    say(f"full-size LBCA decode B={B} T={T}: generating")
    L = synth.lbca_layer(("full-llama-32k",), B, Hq, Hkv, T, d, m, "bf16", "f32", device=DEV)
    pk = torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, device=DEV)
    pv = torch.empty_like(pk)
    say("pool 510 blocks, decode at t=32767")
    lib.pool_blocks(L["k"], L["z"], L["bias"], m, 0, N, pk, v=L["v"], out_v=pv)
    q = L["q"][:, 0]
    pos = torch.full((B,), T - 1, dtype=torch.int64, device=DEV)
    o, lse = lib.attend_decode(q, pk, L["k"], pos, m, W, O.EXCLUSIVE, pooled_v=pv, raw_v=L["v"])
    torch.cuda.synchronize()
    bias = _cpu(L["bias"])
    for b in range(B):  # every (sequence, KV head) unit, one sequence at a time (about 1 s of oracle each)
        say(f"oracle sequence {b}: pooling of 8 KV heads, decode of 24 query heads")
        ks, vs, zs = _cpu(L["k"][b:b + 1]), _cpu(L["v"][b:b + 1]), _cpu(L["z"][b:b + 1])
        rk, rv = O.pool_single(ks, zs, bias, m, 0, N, values=vs)
        check_bf16(host(pk[b]), rk[0], f"pooled K b={b}")
        check_bf16(host(pv[b]), rv[0], f"pooled V b={b}")
        ro, rl = O.attend_decode(_cpu(q[b:b + 1]), rk, rv, ks, vs, [T - 1], m, W, O.EXCLUSIVE, 1 / math.sqrt(d))
        check_bf16(host(o[b]), ro[0], f"decode out b={b}")
        check_bf16(host(lse[b]), rl[0], f"decode lse b={b}")


def test_llama_chunked_prefill_16k(lib):
    B, Hq, Hkv, d, m, W, T, chunk = 1, 24, 8, 128, 16, 128, 16384, 2048
    say(f"full-size chunked prefill T={T} chunk={chunk}: generating")
    L = synth.lbca_layer(("full-prefill-16k",), B, Hq, Hkv, T, d, m, "bf16", "f32", device=DEV, q_len=T)
    N = T // m
    pk = torch.zeros((B, Hkv, N, d), dtype=torch.bfloat16, device=DEV)
    pv = torch.zeros_like(pk)
    out = torch.empty((B, T, Hq, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, T, Hq), dtype=torch.float32, device=DEV)
    done = 0
    for c0 in range(0, T, chunk):
        need, _ = O.visible_range(c0 + chunk - 1, m, W, O.EXCLUSIVE)
        lib.pool_blocks(L["k"], L["z"], L["bias"], m, done, need, pk, v=L["v"], out_v=pv)
        done = need
        qc = L["q"][:, c0:c0 + chunk]
        lib.attend_prefill(qc, c0, pk, L["k"], 0, m, W, O.EXCLUSIVE, out=out[:, c0:c0 + chunk],
                            lse=lse[:, c0:c0 + chunk], pooled_v=pv, raw_v=L["v"])
    torch.cuda.synchronize()
    say("oracle pooling of every block")
    ks, vs, zs, bias = _cpu(L["k"]), _cpu(L["v"]), _cpu(L["z"]), _cpu(L["bias"])
    rk, rv = O.pool_single(ks, zs, bias, m, 0, done, values=vs)
    check_bf16(host(pk[:, :, :done]), rk, "pooled K")
    check_bf16(host(pv[:, :, :done]), rv, "pooled V")
    rng = np.random.default_rng(16384)
    # the chunk and window edges plus 500 random positions (every query head of each)
    ts = sorted({0, 1, 127, 128, 2047, 2048, 4095, 8191, 8192 + 77, 14335, 14336, 16383,
                 *rng.integers(0, T, 500).tolist()})
    say(f"oracle prefill at {len(ts)} query positions")
    q = _cpu(L["q"])
    oh, lh = host(out), host(lse)
    for t in ts:
        ro, rl = O.attend_prefill(q[:, t:t + 1], t, rk, rv, ks, vs, 0, m, W, O.EXCLUSIVE,
                                  1 / math.sqrt(d))
        check_bf16(oh[:, t:t + 1], ro, f"prefill out t={t}")
        check_bf16(lh[:, t:t + 1], rl, f"prefill lse t={t}")


def test_llama_attention_backward_16k(lib):
    B, Hq, Hkv, d, m, W, T = 1, 24, 8, 128, 16, 128, 16384
    EX = O.EXCLUSIVE
    N = O.visible_range(T - 1, m, W, EX)[0]
    say(f"full-size attention backward T={T} N={N}: generating")
    g = lambda n, shape: synth.normal(shape, synth.seed_of("full-attn-grad-16k", n), dtype="bf16", device=DEV)
    q, do = g("q", (B, T, Hq, d)), g("do", (B, T, Hq, d))
    pk, pv, rk, rv = g("pk", (B, Hkv, N, d)), g("pv", (B, Hkv, N, d)), g("rk", (B, Hkv, T, d)), g("rv", (B, Hkv, T, d))
    o, lse = lib.attend_prefill(q, 0, pk, rk, 0, m, W, EX, pooled_v=pv, raw_v=rv, out_dtype=torch.bfloat16)
    dq, dpk, dpv, drk, drv, _ = lib.attend_prefill_backward(q, 0, pk, rk, 0, m, W, EX, o, lse, do,
                                                           pooled_v=pv, raw_v=rv)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(d)
    qh, doh = _cpu(q), _cpu(do)
    keys = tuple(_cpu(t) for t in (pk, pv, rk, rv))

    def oracle(t0, t1):
        return O.attend_prefill_backward(qh[:, t0:t1], t0, *keys, 0, m, W, EX, scale, doh[:, t0:t1])

    rng = np.random.default_rng(1601)
    for t in sorted({0, 1, 127, 128, 143, 144, 8191, 16383, *rng.integers(0, T, 4).tolist()}):
        check_bf16(host(dq[:, t:t + 1]), oracle(t, t + 1)[0], f"dq t={t}")
    for p in (0, 100, 129, 8000, 16300, 16383):
        t_last = min(T - 1, (p // m + 1) * m + W - 2)    # last query whose window holds p
        r = oracle(p, t_last + 1)
        check_bf16(host(drk[:, :, p]), r[3][:, :, p], f"raw dK p={p}")
        check_bf16(host(drv[:, :, p]), r[4][:, :, p], f"raw dV p={p}")
    for j in (990, 1000, 1014, 1015):
        t_first = (j + 1) * m + W - 1                    # first query that sees entry j
        say(f"pooled entry {j}: queries from {t_first}")
        r = oracle(t_first, T)
        check_bf16(host(dpk[:, :, j]), r[1][:, :, j], f"pooled dK j={j}")
        check_bf16(host(dpv[:, :, j]), r[2][:, :, j], f"pooled dV j={j}")


def test_hca_decode_1m_batch4(lib):
    B, Hq, d, m, W, T = 4, 64, 512, 128, 128, 1 << 20
    N = T // m
    say(f"full-size HCA decode B={B} T={T}: generating")
    H = synth.hca_layer(("full-hca-1m",), B, Hq, T, d, m, device=DEV)
    ent = torch.empty((B, 1, N, d), dtype=torch.bfloat16, device=DEV)
    say("pool 8192 treated entries, decode at t=2^20-1")
    lib.pool_blocks(H["c"], H["z"], H["bias"], m, 0, N, ent, rmsnorm_eps=EPS, rope_dims=RD, rope_base=BASE)
    pos = torch.full((B,), T - 1, dtype=torch.int64, device=DEV)
    o, lse = lib.attend_decode(H["q"], ent, H["c"], pos, m, W, O.OVERLAP, sink=H["sink"],
                                rmsnorm_eps=EPS, rope_dims=RD, rope_base=BASE)
    torch.cuda.synchronize()
    bias = _cpu(H["bias"])
    for b in range(B):  # every sequence, its history streamed through the oracle 1024 blocks at a time
        say(f"oracle: stream sequence {b} ({N} blocks)")
        parts = []
        step = 1024
        for j0 in range(0, N, step):
            cs = _cpu(H["c"][b:b + 1, :, j0 * m:(j0 + step) * m])
            zs = _cpu(H["z"][b:b + 1, :, j0 * m:(j0 + step) * m])
            parts.append(O.pool_single(cs, zs, bias, m, 0, step))
        pooled = np.concatenate(parts, axis=2)                       # [1, 1, N, d]
        treated = O.rope(O.rmsnorm(pooled, EPS), np.arange(N) * m, RD, BASE)
        check_bf16(host(ent[b:b + 1]), treated, f"treated HCA entries b={b}")
        raw = _cpu(H["c"][b:b + 1, :, T - W:])
        ro, rl = O.attend_decode(_cpu(H["q"][b:b + 1]), pooled, None, raw, None, [T - 1], m, W, O.OVERLAP,
                                 1 / math.sqrt(d), raw_pos_base=[T - W], sink=_cpu(H["sink"]),
                                 rmsnorm_eps=EPS, rope_dims=RD, rope_base=BASE)
        check_bf16(host(o[b:b + 1]), ro, f"HCA decode out b={b}")
        check_bf16(host(lse[b:b + 1]), rl, f"HCA decode lse b={b}")


def test_csa_decode_128k_batch2(lib):
    B, Hq, d, m, W, T, HI, dI, k = 2, 64, 512, 4, 128, 1 << 17, 8, 64, 512
    N = T // m
    say(f"full-size CSA decode B={B} T={T}: generating")
    C = synth.csa_layer(("full-csa-128k",), B, Hq, T, d, m, HI, dI, device=DEV)
    # the indexer consumes compressed keys; both sides read these bf16 keys
    keys = synth.normal((B, N, dI), synth.seed_of("full-csa-128k", "index-keys"), dtype="bf16", device=DEV)
    ent = torch.empty((B, 1, N, d), dtype=torch.bfloat16, device=DEV)
    treat = dict(rmsnorm_eps=EPS, rope_dims=RD, rope_base=BASE)
    say("dual pooling of 32768 treated entries, indexer top-512, decode")
    lib.pool_blocks(C["ca"], C["za"], C["bias_a"], m, 0, N, ent, xb=C["cb"], zb=C["zb"],
                     bias_b=C["bias_b"], **treat)
    pos = torch.full((B,), T - 1, dtype=torch.int64, device=DEV)
    ws = torch.empty(lib.index_workspace_bytes(C["qi"], C["w"], keys, pos, m, k), dtype=torch.uint8, device=DEV)
    idx, _ = lib.csa_index_topk(C["qi"], C["w"], keys, pos, m, k, workspace=ws)
    o, lse = lib.attend_decode(C["q"], ent, C["ca"], pos, m, W, O.OVERLAP, sel_idx=idx, sink=C["sink"],
                                **treat)
    torch.cuda.synchronize()
    gidx = _cpu(idx).numpy()
    gs = index_ws_scores(ws, B, N)
    qi, w, kh = _cpu(C["qi"]), _cpu(C["w"]), _cpu(keys)
    sel = np.zeros((B, k), dtype=np.int64)
    for b in range(B):
        say(f"oracle indexer sequence {b}")
        s = O.index_scores(qi[b], w[b], kh[b], N)
        margin, band = topk_matches(gidx[b], s, k, f"CSA top-k b={b}", index_score_bound(qi[b], w[b], kh[b], N),
                                    gpu_scores=gs[b])
        say(f"top-512 of sequence {b}: margin {margin:.3e}" +
            (" (in the fp32 tie band: exact against the kernel's own fp32 scores, which are within their bounds)"
             if band else " (set exact)"))
        sel[b] = gidx[b] if band else O.topk_select(s, k)
    # oracle entries for the selected ids only (entry i: a-block i and b-block i-1)
    pooled = np.zeros((B, 1, N, d))
    ba, bb = _cpu(C["bias_a"][0]), _cpu(C["bias_b"][0])
    for b in range(B):
        say(f"oracle dual pooling of the selected entries, sequence {b}")
        for i in sel[b]:
            lo = max(0, i - 1) * m
            sl = slice(lo, (i + 1) * m)
            e = O.pool_dual(_cpu(C["ca"][b:b + 1, :, sl]), _cpu(C["za"][b:b + 1, :, sl]), ba,
                            _cpu(C["cb"][b:b + 1, :, sl]), _cpu(C["zb"][b:b + 1, :, sl]), bb, m,
                            i - lo // m, i - lo // m + 1)
            pooled[b, 0, i] = e[0, 0, 0]
        treated = O.rope(O.rmsnorm(pooled[b, 0, sel[b]], EPS), sel[b] * m, RD, BASE)
        check_bf16(host(ent[b, 0, torch.as_tensor(sel[b], device=DEV)]), treated, f"treated CSA entries b={b}")
    raw = _cpu(C["ca"][:, :, T - W:])
    ro, rl = O.attend_decode(_cpu(C["q"]), pooled, None, raw, None, [T - 1] * B, m, W, O.OVERLAP,
                             1 / math.sqrt(d), raw_pos_base=[T - W] * B, sel_idx=sel,
                             sink=_cpu(C["sink"]), **treat)
    check_bf16(host(o), ro, "CSA decode out")
    check_bf16(host(lse), rl, "CSA decode lse")


def test_csa_sparse_prefill_128k_chunk_batch2(lib):
    # the bench's sparse prefill: the last 2048 queries of each 128K sequence, sampled queries
    B, Hq, d, m, W, T, HI, dI, k, CH = 2, 64, 512, 4, 128, 1 << 17, 8, 64, 512, 2048
    N, t0 = T // m, T - CH
    say(f"full-size CSA sparse prefill B={B} T={T} chunk={CH}: generating")
    C = synth.csa_layer(("full-csa-128k-chunk",), B, Hq, T, d, m, HI, dI, device=DEV, q_len=CH)
    keys = synth.normal((B, N, dI), synth.seed_of("full-csa-128k-chunk", "index-keys"), dtype="bf16", device=DEV)
    ent = torch.empty((B, 1, N, d), dtype=torch.bfloat16, device=DEV)
    treat = dict(rmsnorm_eps=EPS, rope_dims=RD, rope_base=BASE)
    lib.pool_blocks(C["ca"], C["za"], C["bias_a"], m, 0, N, ent, xb=C["cb"], zb=C["zb"],
                    bias_b=C["bias_b"], **treat)
    rbase = t0 - W + 1
    raw = C["ca"][:, 0, rbase:]
    say("sparse prefill of the chunk")
    o, lse, idx = lib.csa_sparse_prefill(C["qi"], C["w"], keys, C["q"], ent[:, 0], raw, t0, rbase, m, W, k,
                                         sink=C["sink"], **treat)
    torch.cuda.synchronize()
    gidx = _cpu(idx).numpy()
    kh, rawh = _cpu(keys), _cpu(raw)
    ba, bb = _cpu(C["bias_a"][0]), _cpu(C["bias_b"][0])
    for b in range(B):
        for i in (0, 1, 1023, CH - 2, CH - 1):
            t = t0 + i
            n_vis = (t + 1) // m
            say(f"oracle: sequence {b} query {i} (t = {t})")
            s = O.index_scores(_cpu(C["qi"][b, i]), _cpu(C["w"][b, i]), kh[b], n_vis)
            _, band = topk_matches(gidx[b, i], s, k, f"sparse prefill top-k b={b} i={i}",
                                   index_score_bound(_cpu(C["qi"][b, i]), _cpu(C["w"][b, i]), kh[b], n_vis),
                                   allow_band=True)
            if band:
                say(f"sequence {b} query {i}: selection in the fp32 tie band (validity checked)")
            sel = gidx[b, i]
            pooled = np.zeros((1, 1, N, d))
            for j in sel[sel >= 0]:
                lo = max(0, j - 1) * m
                sl = slice(lo, (j + 1) * m)
                e = O.pool_dual(_cpu(C["ca"][b:b + 1, :, sl]), _cpu(C["za"][b:b + 1, :, sl]), ba,
                                _cpu(C["cb"][b:b + 1, :, sl]), _cpu(C["zb"][b:b + 1, :, sl]), bb, m,
                                j - lo // m, j - lo // m + 1)
                pooled[0, 0, j] = e[0, 0, 0]
            ro, rl = O.attend_decode(_cpu(C["q"][b, i])[None], pooled, None, rawh[b][None, None], None, [t], m, W,
                                     O.OVERLAP, 1 / math.sqrt(d), raw_pos_base=[rbase], sel_idx=sel[None],
                                     sink=_cpu(C["sink"]), **treat)
            check_bf16(host(o[b, i]), ro[0], f"sparse prefill out b={b} i={i}")
            check_bf16(host(lse[b, i]), rl[0], f"sparse prefill lse b={b} i={i}")
