"""GPU parity: every entry point of liblbca against the fp64 oracle, through the C ABI.

Sizes span several tiles plus a ragged tail and finish in seconds on the oracle;
the full workload sizes are in test_gpu_fullsize.py.  Inputs come from the
seeded generators (block_compressed_kv_amd.synth) and are copied exactly to the
oracle.  Tolerances: see tests/parity_util.py.
"""
import math

import numpy as np
import pytest
import torch

from block_compressed_kv_amd import synth
from oracle import lbca_oracle as O

from parity_util import check, check_bf16, check_f32_rows, host, index_score_bound, index_ws_scores, say, topk_matches

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _dev(d):
    return {k: v.to(DEV) for k, v in d.items()}


# ---------------------------------------------------------------------------
# pooling
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kv,zt,B,H,T,d,m,b0,b1", [
    ("f32", "f32", 1, 1, 1025, 64, 16, 0, 64),       # tiny fp32 layer (all complete blocks)
    ("bf16", "f32", 2, 8, 4096, 128, 64, 3, 61),     # Llama-shaped GQA layer, ragged range
    ("bf16", "bf16", 1, 2, 640, 256, 16, 0, 40),
    ("f32", "bf16", 2, 3, 300, 32, 7, 1, 42),        # odd block size (m % 4 != 0)
])
def test_pool_single(lib, kv, zt, B, H, T, d, m, b0, b1):
    say(f"pool {kv}/{zt} B={B} H={H} T={T} d={d} m={m} blocks [{b0},{b1})")
    L = _dev(synth.lbca_layer(f"pool-{kv}-{d}-{m}", B, H, H, T, d, m, kv, zt))
    N = T // m
    ok = torch.full((B, H, N, d), 7.0, dtype=L["k"].dtype, device=DEV)
    ov = torch.full_like(ok, 7.0)
    lib.pool_blocks(L["k"], L["z"], L["bias"], m, b0, b1, ok, v=L["v"], out_v=ov)
    torch.cuda.synchronize()
    rk, rv = O.pool_single(host(L["k"]), host(L["z"]), host(L["bias"]), m, b0, b1, values=host(L["v"]))
    check(kv, host(ok[:, :, b0:b1]), rk, "pooled K")
    check(kv, host(ov[:, :, b0:b1]), rv, "pooled V")
    # rows outside the range are untouched
    assert (ok[:, :, :b0] == 7.0).all() and (ok[:, :, b1:] == 7.0).all()


def test_pool_pos_base_window(lib):
    # token buffer that starts at position 640: pool blocks 10..19 (m=64) from it
    B, H, T, d, m = 1, 2, 2048, 128, 64
    L = _dev(synth.lbca_layer("pool-base", B, H, H, T, d, m, "bf16", "f32"))
    base = 640
    sub = {k: L[k][:, :, base:] for k in ("k", "v", "z")}
    ok = torch.zeros((B, H, 32, d), dtype=torch.bfloat16, device=DEV)
    ov = torch.zeros_like(ok)
    lib.pool_blocks(sub["k"], sub["z"], L["bias"], m, 10, 20, ok, v=sub["v"], out_v=ov, pos_base=base)
    rk, rv = O.pool_single(host(L["k"]), host(L["z"]), host(L["bias"]), m, 10, 20, values=host(L["v"]))
    check_bf16(host(ok[:, :, 10:20]), rk, "pooled K (pos_base)")
    check_bf16(host(ov[:, :, 10:20]), rv, "pooled V (pos_base)")


@pytest.mark.parametrize("treat", [False, True])
def test_pool_shared_hca(lib, treat):
    B, T, d, m = 2, 128 * 9 + 50, 512, 128
    H = _dev(synth.hca_layer(f"pool-hca-{treat}", B, 4, T, d, m))
    N = T // m
    out = torch.zeros((B, 1, N, d), dtype=torch.bfloat16, device=DEV)
    kw = dict(rmsnorm_eps=1e-6, rope_dims=64, rope_base=10000.0) if treat else {}
    lib.pool_blocks(H["c"], H["z"], H["bias"], m, 0, N, out, **kw)
    ref = O.pool_single(host(H["c"]), host(H["z"]), host(H["bias"]), m, 0, N)
    if treat:
        ref = O.rope(O.rmsnorm(ref, 1e-6), (np.arange(N) * m)[None, None], 64, 10000.0)
    check_bf16(host(out), ref, f"HCA entries treat={treat}")


@pytest.mark.parametrize("d,treat", [(512, False), (512, True), (64, False)])
def test_pool_dual_csa(lib, d, treat):
    B, m, T = 2, 4, 4 * 301
    C = _dev(synth.csa_layer(f"pool-dual-{d}", B, 4, T, d, m, 8, 64))
    N = T // m
    out = torch.zeros((B, 1, N, d), dtype=torch.bfloat16, device=DEV)
    kw = dict(rmsnorm_eps=1e-6, rope_dims=64, rope_base=10000.0) if treat else {}
    lib.pool_blocks(C["ca"], C["za"], C["bias_a"], m, 0, N, out, xb=C["cb"], zb=C["zb"],
                    bias_b=C["bias_b"], **kw)
    ref = O.pool_dual(host(C["ca"]), host(C["za"]), host(C["bias_a"][0]), host(C["cb"]), host(C["zb"]),
                      host(C["bias_b"][0]), m, 0, N)
    if treat:
        ref = O.rope(O.rmsnorm(ref, 1e-6), (np.arange(N) * m)[None, None], 64, 10000.0)
    check_bf16(host(out), ref, f"CSA dual entries d={d} treat={treat}")
    # a sub-range starting mid-sequence reads block i-1 of the b-series
    out2 = torch.zeros_like(out)
    lib.pool_blocks(C["ca"], C["za"], C["bias_a"], m, 17, 90, out2, xb=C["cb"], zb=C["zb"],
                    bias_b=C["bias_b"], **kw)
    assert torch.equal(out2[:, :, 17:90], out[:, :, 17:90])


@pytest.mark.parametrize("xdt,zdt,B,H,T,d,m,b0,b1,pb,with_v", [
    ("bf16", "f32", 2, 3, 300, 128, 16, 2, 17, 0, True),     # LBCA-shaped, ragged block range
    ("f32", "f32", 1, 2, 700, 64, 64, 3, 10, 64, False),     # raw rows start at position 64
    ("bf16", "bf16", 2, 1, 520, 512, 16, 0, 32, 0, True),    # 512 dims (m * d = 8192)
    ("bf16", "f32", 3, 2, 130, 128, 64, 0, 2, 0, True),      # four tokens per lane, few blocks
    ("bf16", "f32", 1, 2, 64, 128, 1, 5, 60, 0, True),       # m = 1: most lane phases empty
])
def test_pool_backward(lib, xdt, zdt, B, H, T, d, m, b0, b1, pb, with_v):
    say(f"pool backward {xdt}/{zdt} B={B} H={H} d={d} m={m} blocks [{b0},{b1}) pos_base={pb}")
    L = _dev(synth.lbca_layer(f"pool-grad-{xdt}-{d}-{m}", B, H, H, T, d, m, xdt, zdt))
    N = T // m
    g = lambda n: synth.normal((B, H, N, d), synth.seed_of("pool-grad", xdt, d, m, n), dtype=xdt, device=DEV)
    gx, gv = g("gx"), (g("gv") if with_v else None)
    sub = lambda t: t[:, :, pb:]
    x, z = sub(L["k"]), sub(L["z"])
    v = sub(L["v"]) if with_v else None
    dx, dz = torch.full_like(x, 7.0), torch.full_like(z, 7.0)
    dv = torch.full_like(v, 7.0) if with_v else None
    lib.pool_blocks_backward(x, z, L["bias"], m, b0, b1, gx, v=v, grad_v=gv, dx=dx, dv=dv, dz=dz, pos_base=pb)
    _, _, _, dbias = lib.pool_blocks_backward(x, z, L["bias"], m, b0, b1, gx, v=v, grad_v=gv, pos_base=pb)
    rx, rv, rz, rb = O.pool_single_backward(host(L["k"]), host(L["z"]), host(L["bias"]), m, b0, b1,
                                            host(gx)[:, :, b0:b1], values=host(L["v"]) if with_v else None,
                                            grad_values=host(gv)[:, :, b0:b1] if with_v else None)
    lo, hi = b0 * m, b1 * m
    check(xdt, host(dx[:, :, lo - pb:hi - pb]), rx[:, :, lo:hi], "d series")
    check(zdt, host(dz[:, :, lo - pb:hi - pb]), rz[:, :, lo:hi], "d logits")
    if with_v:
        check(xdt, host(dv[:, :, lo - pb:hi - pb]), rv[:, :, lo:hi], "d values")
    check("f32", host(dbias), rb, "d bias")
    # rows outside the pooled blocks are untouched
    assert (dx[:, :, :lo - pb] == 7.0).all() and (dx[:, :, hi - pb:] == 7.0).all()
    assert (dz[:, :, :lo - pb] == 7.0).all() and (dz[:, :, hi - pb:] == 7.0).all()
    # bitwise reproducible
    dx2, dv2, dz2, db2 = lib.pool_blocks_backward(x, z, L["bias"], m, b0, b1, gx, v=v, grad_v=gv, pos_base=pb)
    assert torch.equal(dx2[:, :, lo - pb:hi - pb], dx[:, :, lo - pb:hi - pb]) and torch.equal(db2, dbias)
    assert torch.equal(dz2[:, :, lo - pb:hi - pb], dz[:, :, lo - pb:hi - pb])
    # an empty range writes a zero bias gradient and nothing else
    _, _, dz3, db3 = lib.pool_blocks_backward(x, z, L["bias"], m, b1, b1, gx, v=v, grad_v=gv, pos_base=pb)
    assert (db3 == 0).all() and (dz3 == 0).all()


@pytest.mark.parametrize("form,d,m,b0,b1", [
    ("hca", 512, 16, 2, 30),      # shared series, RMSNorm + RoPE on the stored entries
    ("csa", 512, 4, 3, 40),       # dual series (block j with b-block j-1), treated
    ("csa-plain", 64, 4, 0, 45),  # dual series without treatment, entry 0 without a b-part
])
def test_pool_backward_treated_and_dual(lib, form, d, m, b0, b1):
    say(f"pool backward {form} d={d} m={m} blocks [{b0},{b1})")
    B, T = 2, 4 * 128
    N = T // m
    treat = {} if form == "csa-plain" else dict(rmsnorm_eps=1e-6, rope_dims=64, rope_base=10000.0)
    g = synth.normal((B, 1, N, d), synth.seed_of("pool-grad-treat", form), dtype="bf16", device=DEV)
    gi = host(g)[:, :, b0:b1]
    pos = (np.arange(b0, b1) * m)[None, None, :]          # each entry's block start
    if form == "hca":
        H = _dev(synth.hca_layer(f"pool-grad-{form}", B, 4, T, d, m))
        x, z, bias = H["c"], H["z"], H["bias"]
        dx, _, dz, dbias = lib.pool_blocks_backward(x, z, bias, m, b0, b1, g, **treat)
        pooled = O.pool_single(host(x), host(z), host(bias), m, b0, b1)
        ge = O.treat_backward(pooled, gi, 1e-6, 64, 10000.0, pos)
        rx, _, rz, rb = O.pool_single_backward(host(x), host(z), host(bias), m, b0, b1, ge)
    else:
        C = _dev(synth.csa_layer(f"pool-grad-{form}", B, 4, T, d, m, 8, 64))
        x, z, bias = C["ca"], C["za"], C["bias_a"]
        dx, _, dz, dbias, dxb, dzb, dbias_b = lib.pool_blocks_backward(
            x, z, bias, m, b0, b1, g, xb=C["cb"], zb=C["zb"], bias_b=C["bias_b"], **treat)
        pooled = O.pool_dual(host(x), host(z), host(bias[0]), host(C["cb"]), host(C["zb"]), host(C["bias_b"][0]),
                             m, b0, b1)
        ge = O.treat_backward(pooled, gi, 1e-6, 64, 10000.0, pos) if treat else gi
        rx, rz, rb, rxb, rzb, rbb = O.pool_dual_backward(host(x), host(z), host(bias[0]), host(C["cb"]),
                                                         host(C["zb"]), host(C["bias_b"][0]), m, b0, b1, ge)
        lo_b, hi_b = (max(b0, 1) - 1) * m, (b1 - 1) * m
        check_bf16(host(dxb[:, :, lo_b:hi_b]), rxb[:, :, lo_b:hi_b], "d b-series")
        check_bf16(host(dzb[:, :, lo_b:hi_b]), rzb[:, :, lo_b:hi_b], "d b-logits")
        check("f32", host(dbias_b[0]), rbb, "d bias_b")
        assert (dxb[:, :, :lo_b] == 0).all() and (dxb[:, :, hi_b:] == 0).all()
    lo, hi = b0 * m, b1 * m
    check_bf16(host(dx[:, :, lo:hi]), rx[:, :, lo:hi], "d series")
    check_bf16(host(dz[:, :, lo:hi]), rz[:, :, lo:hi], "d logits")
    check("f32", host(dbias if form == "hca" else dbias[0]), rb, "d bias")
    assert (dx[:, :, :lo] == 0).all() and (dx[:, :, hi:] == 0).all()


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
def test_decode_tiny_fp32_layer(lib):
    # seq_len 1024 fp32 layer, decode at position 1024 (its own K/V cached): 56 pooled + 129 raw
    T, t, m, W = 1025, 1024, 16, 128
    L = _dev(synth.lbca_layer("c1", 1, 2, 1, T, 64, m, "f32", "f32", q_len=1))
    n_p, _ = O.visible_range(t, m, W, O.EXCLUSIVE)
    assert n_p == 56
    pk = torch.zeros((1, 1, 64, 64), device=DEV)
    pv = torch.zeros_like(pk)
    lib.pool_blocks(L["k"], L["z"], L["bias"], m, 0, n_p, pk, v=L["v"], out_v=pv)
    q = L["q"][:, 0]
    pos = torch.tensor([t], device=DEV)
    for sink in (None, torch.tensor([0.3, -1.1], device=DEV)):
        o, lse = lib.attend_decode(q, pk, L["k"], pos, m, W, O.EXCLUSIVE, pooled_v=pv, raw_v=L["v"],
                                   sink=sink)
        rpk, rpv = O.pool_single(host(L["k"]), host(L["z"]), host(L["bias"]), m, 0, n_p, values=host(L["v"]))
        ro, rl = O.attend_decode(host(q), rpk, rpv, host(L["k"]), host(L["v"]), [t], m, W, O.EXCLUSIVE,
                                 1 / 8, sink=None if sink is None else host(sink))
        check_f32_rows(host(o), ro, f"tiny decode sink={sink is not None}")
        check_f32_rows(host(lse)[..., None], rl[..., None], "tiny decode lse")


@pytest.mark.parametrize("t_list", [[4095, 1000, 130, 0], [127, 128, 191, 192]])
def test_decode_gqa_bf16(lib, t_list):
    # Llama-shaped GQA decode (24 q heads over 8 KV heads, d=128), ragged positions
    B, Hq, Hkv, d, m, W, T = len(t_list), 24, 8, 128, 64, 128, 4096
    g = lambda n, shape: synth.normal(shape, synth.seed_of("dec-gqa", n, tuple(t_list)), dtype="bf16",
                                      device=DEV)
    q = g("q", (B, Hq, d))
    pk, pv = g("pk", (B, Hkv, 64, d)), g("pv", (B, Hkv, 64, d))
    rk, rv = g("rk", (B, Hkv, T, d)), g("rv", (B, Hkv, T, d))
    pos = torch.tensor(t_list, device=DEV)
    sink = synth.normal((Hq,), 5, device=DEV)
    o, lse = lib.attend_decode(q, pk, rk, pos, m, W, O.EXCLUSIVE, pooled_v=pv, raw_v=rv, sink=sink)
    ro, rl = O.attend_decode(host(q), host(pk), host(pv), host(rk), host(rv), t_list, m, W, O.EXCLUSIVE,
                             1 / math.sqrt(d), sink=host(sink))
    check_bf16(host(o), ro, "GQA decode out")
    check_bf16(host(lse), rl, "GQA decode lse")
    # bitwise reproducible
    o2, lse2 = lib.attend_decode(q, pk, rk, pos, m, W, O.EXCLUSIVE, pooled_v=pv, raw_v=rv, sink=sink)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_decode_workspace_reuse_and_graph_replay(lib):
    # split path: one workspace reused by many calls, eager and replayed from a graph,
    # with other work in between, always reproduces the first result bit for bit
    B, Hq, Hkv, d, m, W = 2, 24, 8, 128, 64, 128
    g = lambda n, shape: synth.normal(shape, synth.seed_of("dec-reuse", n), dtype="bf16", device=DEV)
    q, q2 = g("q", (B, Hq, d)), g("q2", (B, Hq, d))
    pk, pv = g("pk", (B, Hkv, 2048, d)), g("pv", (B, Hkv, 2048, d))
    rk, rv = g("rk", (B, Hkv, 256, d)), g("rv", (B, Hkv, 256, d))
    t_list = [2048 * 64 + 127, 1300 * 64 + 77]                        # 2048 and 1299 pooled entries
    base = [O.visible_range(t, m, W, O.EXCLUSIVE)[1] for t in t_list]
    pos, rpb = torch.tensor(t_list, device=DEV), torch.tensor(base, device=DEV)
    kw = dict(pooled_v=pv, raw_v=rv, raw_pos_base=rpb)
    need = lib.decode_workspace_bytes(q, pk, rk, pos, m, W, O.EXCLUSIVE, **kw)
    assert need > 0, "this shape should split the rows across workgroups"
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    ref_o, ref_l = lib.attend_decode(q, pk, rk, pos, m, W, O.EXCLUSIVE, **kw)
    ro, _ = O.attend_decode(host(q), host(pk), host(pv), host(rk), host(rv), t_list, m, W,
                            O.EXCLUSIVE, 1 / math.sqrt(d), raw_pos_base=base)
    check_bf16(host(ref_o), ro, "reference call")
    for _ in range(5):
        lib.attend_decode(q, pk, rk, pos, m, W, O.EXCLUSIVE, out=out, lse=lse, workspace=ws, **kw)
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
    torch.cuda.synchronize()
    # graph of the same call on the same workspace
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        lib.attend_decode(q, pk, rk, pos, m, W, O.EXCLUSIVE, out=out, lse=lse, workspace=ws, **kw)
    torch.cuda.synchronize()
    other = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for i in range(4):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {i}"
        # eager work in between, on another workspace and other queries
        lib.attend_decode(q2, pk, rk, pos, m, W, O.EXCLUSIVE, workspace=other, **kw)
        torch.cuda.synchronize()


@pytest.mark.parametrize("d,Hq,Hkv,shared", [(128, 24, 8, False), (128, 16, 8, True), (64, 8, 8, False)])
def test_decode_one_split_rows_past_the_list(lib, d, Hq, Hkv, shared):
    # 16 sequences x 8 KV heads: one workgroup (group) per unit, the path that
    # requests the first pooled rows before reading the position.  Every row
    # outside a sequence's visible list (pooled capacity past n_pooled, raw rows
    # past t) holds NaN and must not reach the output.
    m, W, cap = 64, 128, 520
    t_list = [33000, 32767, 32768 + 63, 200, 0, 127, 128, 191, 192, 5000, 20000, 33407, 1000,
              64 * 300 + 5, 64 * 17, 64 * 23 + 127]
    B = len(t_list)
    g = lambda n, shape: synth.normal(shape, synth.seed_of("dec-1split", n, d, shared), dtype="bf16",
                                      device=DEV)
    q = g("q", (B, Hq, d))
    pk, rk = g("pk", (B, Hkv, cap, d)), g("rk", (B, Hkv, 256, d))
    pv, rv = (None, None) if shared else (g("pv", (B, Hkv, cap, d)), g("rv", (B, Hkv, 256, d)))
    base = []
    for b, t in enumerate(t_list):
        n_p, rb = O.visible_range(t, m, W, O.EXCLUSIVE)
        base.append(rb)
        for x in (pk, pv):
            if x is not None:
                x[b, :, n_p:] = float("nan")
        for x in (rk, rv):
            if x is not None:
                x[b, :, t - rb + 1:] = float("nan")
    pos, rpb = torch.tensor(t_list, device=DEV), torch.tensor(base, device=DEV)
    kw = dict(pooled_v=pv, raw_v=rv, raw_pos_base=rpb)
    assert lib.decode_workspace_bytes(q, pk, rk, pos, m, W, O.EXCLUSIVE, **kw) == 0, "expected one split"
    o, lse = lib.attend_decode(q, pk, rk, pos, m, W, O.EXCLUSIVE, **kw)
    hv = lambda x: None if x is None else host(x)
    ro, rl = O.attend_decode(host(q), host(pk), hv(pv), host(rk), hv(rv), t_list, m, W, O.EXCLUSIVE,
                             1 / math.sqrt(d), raw_pos_base=base)
    say(f"one-split decode d={d} Hq={Hq} Hkv={Hkv} shared={shared}")
    check_bf16(host(o), ro, "one-split decode out")
    check_bf16(host(lse), rl, "one-split decode lse")


def test_decode_raw_pos_base_and_overlap(lib):
    B, Hq, Hkv, d, m, W = 3, 8, 2, 64, 16, 40
    t_list, base = [700, 333, 45], [600, 290, 0]
    g = lambda n, shape: synth.normal(shape, synth.seed_of("dec-base", n), dtype="bf16", device=DEV)
    q = g("q", (B, Hq, d))
    pk, pv = g("pk", (B, Hkv, 50, d)), g("pv", (B, Hkv, 50, d))
    rk, rv = g("rk", (B, Hkv, 128, d)), g("rv", (B, Hkv, 128, d))
    pos = torch.tensor(t_list, device=DEV)
    rpb = torch.tensor(base, device=DEV)
    o, lse = lib.attend_decode(q, pk, rk, pos, m, W, O.OVERLAP, pooled_v=pv, raw_v=rv, raw_pos_base=rpb)
    ro, rl = O.attend_decode(host(q), host(pk), host(pv), host(rk), host(rv), t_list, m, W, O.OVERLAP,
                             1 / 8, raw_pos_base=base)
    check_bf16(host(o), ro, "decode OVERLAP + raw_pos_base")
    check_bf16(host(lse), rl, "lse")


def test_decode_invalid_sequence_gets_nan(lib):
    B, Hq, Hkv, d, m, W = 3, 4, 1, 64, 16, 32
    q = synth.normal((B, Hq, d), 1, dtype="bf16", device=DEV)
    pk = synth.normal((B, Hkv, 8, d), 2, dtype="bf16", device=DEV)
    rk = synth.normal((B, Hkv, 256, d), 3, dtype="bf16", device=DEV)
    # seq 0 fine; seq 1 needs 13 pooled entries (> 8); seq 2 position beyond the raw buffer
    pos = torch.tensor([100, 240, 300], device=DEV)
    o, lse = lib.attend_decode(q, pk, rk, pos, m, W, O.OVERLAP)
    assert torch.isfinite(o[0]).all() and torch.isfinite(lse[0]).all()
    assert torch.isnan(o[1]).all() and torch.isnan(lse[1]).all()
    assert torch.isnan(o[2]).all() and torch.isnan(lse[2]).all()


@pytest.mark.parametrize("rd,nb", [(0, 12), (64, 12), (64, 300)])
def test_decode_hca_treated(lib, rd, nb):
    # HCA-style MQA: shared series, 64 heads, d=512, m'=128, RMSNorm, partial RoPE, sink;
    # 300 blocks split each sequence's rows over several workgroups
    B, Hq, d, m, W = 2, 64, 512, 128, 128
    T = 128 * nb + 77
    H = _dev(synth.hca_layer(f"dec-hca-{rd}-{nb}", B, Hq, T, d, m))
    t_list = [T - 1, 128 * 5 + 3]
    N = T // m
    entries = torch.zeros((B, 1, N, d), dtype=torch.bfloat16, device=DEV)
    lib.pool_blocks(H["c"], H["z"], H["bias"], m, 0, N, entries, rmsnorm_eps=1e-6, rope_dims=rd)
    pos = torch.tensor(t_list, device=DEV)
    o, lse = lib.attend_decode(H["q"], entries, H["c"], pos, m, W, O.OVERLAP, sink=H["sink"],
                               rmsnorm_eps=1e-6, rope_dims=rd)
    pooled = O.pool_single(host(H["c"]), host(H["z"]), host(H["bias"]), m, 0, N)
    ro, rl = O.attend_decode(host(H["q"]), pooled, None, host(H["c"]), None, t_list, m, W, O.OVERLAP,
                             1 / math.sqrt(d), sink=host(H["sink"]), rmsnorm_eps=1e-6, rope_dims=rd)
    check_bf16(host(o), ro, f"HCA decode rope={rd}")
    check_bf16(host(lse), rl, "HCA lse")


@pytest.mark.parametrize("Hq,B,nb", [(16, 3, 40), (32, 2, 40), (48, 1, 7), (32, 1, 300)])
def test_decode_mqa_512_head_counts(lib, Hq, B, nb):
    # 512-dim shared-series MQA with 16 or 48 query heads (16-head groups) and
    # 32 (one 32-head block of the wide kernel), treated, with a sink
    d, m, W = 512, 128, 128
    T = 128 * nb + 33
    H = _dev(synth.hca_layer(f"dec-mqa512-{Hq}-{B}-{nb}", B, Hq, T, d, m))
    t_list = [T - 1, 128 * 3 + 5, 900][:B]
    N = T // m
    entries = torch.zeros((B, 1, N, d), dtype=torch.bfloat16, device=DEV)
    treat = dict(rmsnorm_eps=1e-6, rope_dims=64)
    lib.pool_blocks(H["c"], H["z"], H["bias"], m, 0, N, entries, **treat)
    pos = torch.tensor(t_list, device=DEV)
    o, lse = lib.attend_decode(H["q"], entries, H["c"], pos, m, W, O.OVERLAP, sink=H["sink"], **treat)
    pooled = O.pool_single(host(H["c"]), host(H["z"]), host(H["bias"]), m, 0, N)
    ro, rl = O.attend_decode(host(H["q"]), pooled, None, host(H["c"]), None, t_list, m, W, O.OVERLAP,
                             1 / math.sqrt(d), sink=host(H["sink"]), **treat)
    check_bf16(host(o), ro, f"MQA-512 decode Hq={Hq}")
    check_bf16(host(lse), rl, "lse")


def test_decode_mqa_512_first_positions(lib):
    # the wide path at the smallest positions: t = 0 (one raw row, no pooled entry),
    # t = 1, t = 127 (one complete block, window 0..127) and t = 128
    B, Hq, d, m, W = 4, 64, 512, 128, 128
    T = 512
    H = _dev(synth.hca_layer("dec-mqa512-first", B, Hq, T, d, m))
    t_list = [0, 1, 127, 128]
    N = T // m
    entries = torch.zeros((B, 1, N, d), dtype=torch.bfloat16, device=DEV)
    treat = dict(rmsnorm_eps=1e-6, rope_dims=64)
    lib.pool_blocks(H["c"], H["z"], H["bias"], m, 0, N, entries, **treat)
    pos = torch.tensor(t_list, device=DEV)
    o, lse = lib.attend_decode(H["q"], entries, H["c"], pos, m, W, O.OVERLAP, sink=H["sink"], **treat)
    pooled = O.pool_single(host(H["c"]), host(H["z"]), host(H["bias"]), m, 0, N)
    ro, rl = O.attend_decode(host(H["q"]), pooled, None, host(H["c"]), None, t_list, m, W, O.OVERLAP,
                             1 / math.sqrt(d), sink=host(H["sink"]), **treat)
    check_bf16(host(o), ro, "MQA-512 first positions")
    check_bf16(host(lse), rl, "lse")


@pytest.mark.parametrize("path", ["gqa128", "mqa512"])
def test_decode_merge_64_splits(lib, path):
    # one sequence whose rows are cut into the most splits (64), so the merge
    # combines 64 partials per head: split maxima and sums reduced over the
    # splits of 16 waves.  gqa128: unnormalised fp32 partials of the GQA path;
    # mqa512: normalised bf16 partials of the wide path (entries pooled and
    # treated from a raw series with 4-token blocks, sink).
    say(f"64-split decode {path}")
    if path == "gqa128":
        Hq, Hkv, d, m, W, N = 24, 8, 128, 64, 128, 65000
        t = N * m + 127
        n_p, rb = O.visible_range(t, m, W, O.EXCLUSIVE)
        assert n_p == N
        g = lambda n, shape: synth.normal(shape, synth.seed_of("dec-64splits", n), dtype="bf16", device=DEV)
        q = g("q", (1, Hq, d))
        pk, pv = g("pk", (1, Hkv, N, d)), g("pv", (1, Hkv, N, d))
        rk, rv = g("rk", (1, Hkv, 256, d)), g("rv", (1, Hkv, 256, d))
        pos, rpb = torch.tensor([t], device=DEV), torch.tensor([rb], device=DEV)
        kw = dict(pooled_v=pv, raw_v=rv, raw_pos_base=rpb)
        need = lib.decode_workspace_bytes(q, pk, rk, pos, m, W, O.EXCLUSIVE, **kw)
        assert need == Hkv * 64 * 16 * (2 * 4 + d * 4), need      # 64 fp32 partials per unit
        o, lse = lib.attend_decode(q, pk, rk, pos, m, W, O.EXCLUSIVE, **kw)
        ro, rl = O.attend_decode(host(q), host(pk), host(pv), host(rk), host(rv), [t], m, W, O.EXCLUSIVE,
                                 1 / math.sqrt(d), raw_pos_base=[rb])
    else:
        Hq, d, m, W = 64, 512, 4, 128
        T = 4 * 5888 + 3  # 184 + 4 tiles of 32 rows, raw tiles counting twice: 64 ranges of cost 3
        N = T // m
        H = _dev(synth.hca_layer("dec-64splits-mqa", 1, Hq, T, d, m))
        entries = torch.zeros((1, 1, N, d), dtype=torch.bfloat16, device=DEV)
        treat = dict(rmsnorm_eps=1e-6, rope_dims=64)
        lib.pool_blocks(H["c"], H["z"], H["bias"], m, 0, N, entries, **treat)
        t = T - 1
        pos = torch.tensor([t], device=DEV)
        kw = dict(sink=H["sink"], **treat)
        need = lib.decode_workspace_bytes(H["q"], entries, H["c"], pos, m, W, O.OVERLAP, **kw)
        assert need == (Hq // 16) * 64 * 16 * (2 * 4 + d * 2), need  # 64 bf16 partials per unit
        o, lse = lib.attend_decode(H["q"], entries, H["c"], pos, m, W, O.OVERLAP, **kw)
        pooled = O.pool_single(host(H["c"]), host(H["z"]), host(H["bias"]), m, 0, N)
        ro, rl = O.attend_decode(host(H["q"]), pooled, None, host(H["c"]), None, [t], m, W, O.OVERLAP,
                                 1 / math.sqrt(d), sink=host(H["sink"]), **treat)
    check_bf16(host(o), ro, f"64-split decode {path}")
    check_bf16(host(lse), rl, "lse")


def test_decode_selected_entries(lib):
    # CSA-style: dual-pooled treated entries, a selection with -1 padding and invisible
    # ids, plus the 128-token window; MQA 64 heads, d=512
    B, Hq, d, m, W, k = 2, 64, 512, 4, 128, 40
    T = 4 * 300
    C = _dev(synth.csa_layer("dec-sel", B, Hq, T, d, m, 8, 64))
    N = T // m
    entries = torch.zeros((B, 1, N, d), dtype=torch.bfloat16, device=DEV)
    treat = dict(rmsnorm_eps=1e-6, rope_dims=64, rope_base=10000.0)
    lib.pool_blocks(C["ca"], C["za"], C["bias_a"], m, 0, N, entries, xb=C["cb"], zb=C["zb"],
                    bias_b=C["bias_b"], **treat)
    t_list = [T - 1, 4 * 100 + 2]
    rng = np.random.default_rng(3)
    sel = np.stack([np.sort(rng.choice(300, k, replace=False)), np.sort(rng.choice(150, k, replace=False))])
    sel[0, -3:] = -1                 # empty slots
    sel_t = torch.tensor(sel, dtype=torch.int32, device=DEV)   # seq 1 also lists ids >= 100 (invisible)
    pos = torch.tensor(t_list, device=DEV)
    o, lse = lib.attend_decode(C["q"], entries, C["ca"], pos, m, W, O.OVERLAP, sel_idx=sel_t,
                               sink=C["sink"], **treat)
    pooled = O.pool_dual(host(C["ca"]), host(C["za"]), host(C["bias_a"][0]), host(C["cb"]),
                         host(C["zb"]), host(C["bias_b"][0]), m, 0, N)
    ro, rl = O.attend_decode(host(C["q"]), pooled, None, host(C["ca"]), None, t_list, m, W, O.OVERLAP,
                             1 / math.sqrt(d), sel_idx=sel, sink=host(C["sink"]), **treat)
    check_bf16(host(o), ro, "selected decode")
    check_bf16(host(lse), rl, "selected lse")


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------
def test_prefill_tiny_fp32_layer(lib):
    T, m, W = 1024, 16, 128
    L = _dev(synth.lbca_layer("c1", 1, 2, 1, T + 1, 64, m, "f32", "f32", q_len=T))
    n_p, _ = O.visible_range(T - 1, m, W, O.EXCLUSIVE)
    pk = torch.zeros((1, 1, 64, 64), device=DEV)
    pv = torch.zeros_like(pk)
    lib.pool_blocks(L["k"], L["z"], L["bias"], m, 0, n_p, pk, v=L["v"], out_v=pv)
    o, lse = lib.attend_prefill(L["q"], 0, pk, L["k"], 0, m, W, O.EXCLUSIVE, pooled_v=pv, raw_v=L["v"])
    k, v, z, bias = (host(L[n]) for n in ("k", "v", "z", "bias"))
    ro, rl = O.prefill_chunked(host(L["q"]), k[:, :, :T], v[:, :, :T], z[:, :, :T], bias, m, W, T, 1 / 8)
    check_f32_rows(host(o), ro, "tiny prefill")
    check_f32_rows(host(lse)[..., None], rl[..., None], "tiny prefill lse")


@pytest.mark.parametrize("chunk", [256, 300])
def test_prefill_chunked_bf16(lib, chunk):
    # Llama-shaped GQA layer, m=16, W=128, chunked: pool the chunk's newly visible blocks, attend
    B, Hq, Hkv, d, m, W, T = 1, 24, 8, 128, 16, 128, 1200
    L = _dev(synth.lbca_layer("prefill-bf16", B, Hq, Hkv, T, d, m, "bf16", "f32", q_len=T))
    pk = torch.zeros((B, Hkv, T // m, d), dtype=torch.bfloat16, device=DEV)
    pv = torch.zeros_like(pk)
    out = torch.empty((B, T, Hq, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, T, Hq), dtype=torch.float32, device=DEV)
    done = 0
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        need, _ = O.visible_range(c1 - 1, m, W, O.EXCLUSIVE)
        if need > done:
            lib.pool_blocks(L["k"], L["z"], L["bias"], m, done, need, pk, v=L["v"], out_v=pv)
            done = need
        lib.attend_prefill(L["q"][:, c0:c1], c0, pk, L["k"], 0, m, W, O.EXCLUSIVE,
                           out=out[:, c0:c1], lse=lse[:, c0:c1], pooled_v=pv, raw_v=L["v"])
    ro, rl = O.prefill_chunked(host(L["q"]), host(L["k"]), host(L["v"]), host(L["z"]), host(L["bias"]),
                               m, W, 400, 1 / math.sqrt(d))
    check_bf16(host(out), ro, f"chunked prefill chunk={chunk}")
    check_bf16(host(lse), rl, "prefill lse")


@pytest.mark.parametrize("q0,q_len", [(0, 1), (777, 1), (500, 3)])
def test_prefill_tiny_chunks(lib, q0, q_len):
    # chunks of one to three queries (one 16-row group, mostly padding), GQA bf16, EXCLUSIVE
    B, Hq, Hkv, d, m, W = 2, 24, 8, 128, 16, 128
    T = 800
    L = _dev(synth.lbca_layer("prefill-tiny", B, Hq, Hkv, T, d, m, "bf16", "f32", q_len=T))
    need, _ = O.visible_range(q0 + q_len - 1, m, W, O.EXCLUSIVE)
    pk = torch.zeros((B, Hkv, T // m, d), dtype=torch.bfloat16, device=DEV)
    pv = torch.zeros_like(pk)
    if need > 0:
        lib.pool_blocks(L["k"], L["z"], L["bias"], m, 0, need, pk, v=L["v"], out_v=pv)
    q = L["q"][:, q0:q0 + q_len]
    o, lse = lib.attend_prefill(q, q0, pk, L["k"], 0, m, W, O.EXCLUSIVE, pooled_v=pv, raw_v=L["v"],
                                out_dtype=torch.float32)
    rpk, rpv = O.pool_single(host(L["k"]), host(L["z"]), host(L["bias"]), m, 0, T // m, values=host(L["v"]))
    ro, rl = O.attend_prefill(host(q), q0, rpk, rpv, host(L["k"]), host(L["v"]), 0, m, W, O.EXCLUSIVE,
                              1 / math.sqrt(d))
    check_bf16(host(o), ro, f"prefill q0={q0} len={q_len}")
    check_bf16(host(lse), rl, "lse")


def test_prefill_overlap_shared_sink(lib):
    # OVERLAP visibility, shared K=V series, sink, fp32 output, MQA-like 8 heads over 1 KV head, d=64
    B, Hq, d, m, W, T = 2, 8, 64, 8, 24, 333
    g = lambda n, shape: synth.normal(shape, synth.seed_of("prefill-ov", n), dtype="bf16", device=DEV)
    q = g("q", (B, 100, Hq, d))
    pooled, raw = g("p", (B, 1, T // m, d)), g("r", (B, 1, T, d))
    sink = synth.normal((Hq,), 9, device=DEV)
    o, lse = lib.attend_prefill(q, T - 100, pooled, raw, 0, m, W, O.OVERLAP, sink=sink,
                                out_dtype=torch.float32)
    ro, rl = O.attend_prefill(host(q), T - 100, host(pooled), None, host(raw), None, 0, m, W, O.OVERLAP,
                              1 / 8, sink=host(sink))
    check_bf16(host(o), ro, "prefill overlap shared")
    check_bf16(host(lse), rl, "lse")


# ---------------------------------------------------------------------------
# indexer + top-k
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N,k,t_list", [
    (2000, 64, [7999, 3001]), (700, 512, [2799, 100]), (5000, 2048, [19999, 19999]),
    # two-stage selection (slices of 4096): 5 slices with a ragged last one, 3 visible
    # slices, one slice holding more than k, fewer visible than k
    (20000, 300, [79999, 35999, 2399, 999]),
    # k at a quarter of a slice; the 4th slice empty or holding a single entry
    (12289, 1024, [49155, 49159]),
])
def test_index_topk(lib, N, k, t_list):
    B, HI, dI, m = len(t_list), 8, 64, 4
    g = lambda n, shape: synth.normal(shape, synth.seed_of("idx", N, n), dtype="bf16", device=DEV)
    qi, keys = g("qi", (B, HI, dI)), g("k", (B, N, dI))
    w = synth.uniform((B, HI), synth.seed_of("idx", N, "w"), device=DEV)
    pos = torch.tensor(t_list, device=DEV)
    ws = torch.empty(lib.index_workspace_bytes(qi, w, keys, pos, m, k), dtype=torch.uint8, device=DEV)
    idx, score = lib.csa_index_topk(qi, w, keys, pos, m, k, workspace=ws)
    idx, score = idx.cpu().numpy(), score.cpu().numpy()
    gs = index_ws_scores(ws, B, N)
    for b, t in enumerate(t_list):
        n_vis = min((t + 1) // m, N)
        s = O.index_scores(host(qi[b]), host(w[b]), host(keys[b]), n_vis)
        margin, band = topk_matches(idx[b], s, k, f"top-k seq {b}",
                                    index_score_bound(host(qi[b]), host(w[b]), host(keys[b]), n_vis),
                                    gpu_scores=gs[b, :n_vis] if n_vis > k else None)
        say(f"top-k seq {b}: n_vis={n_vis} k={k} margin={margin:.3e}" + (" in the fp32 tie band" if band else ""))
        sel = idx[b][idx[b] >= 0]
        np.testing.assert_allclose(score[b][:sel.size], s[sel], rtol=1e-5, atol=1e-5)
        assert np.isnan(score[b][sel.size:]).all()


@pytest.mark.parametrize("N,k,t_list", [(600, 50, [-1, -7]), (20000, 300, [1199, -1])])
def test_index_topk_no_or_exactly_k_visible(lib, N, k, t_list):
    # t < 0 sees nothing (an all -1 row); t = 1199 with m = 4 sees exactly k = 300 entries
    B, HI, dI, m = len(t_list), 8, 64, 4
    g = lambda n, shape: synth.normal(shape, synth.seed_of("idx-edge", N, n), dtype="bf16", device=DEV)
    qi, keys = g("qi", (B, HI, dI)), g("k", (B, N, dI))
    w = synth.uniform((B, HI), synth.seed_of("idx-edge", N, "w"), device=DEV)
    idx, score = lib.csa_index_topk(qi, w, keys, torch.tensor(t_list, device=DEV), m, k)
    idx, score = idx.cpu().numpy(), score.cpu().numpy()
    for b, t in enumerate(t_list):
        n_vis = 0 if t < 0 else min((t + 1) // m, N)
        s = O.index_scores(host(qi[b]), host(w[b]), host(keys[b]), n_vis)
        assert list(idx[b]) == list(O.topk_select(s, k)), f"seq {b} t={t}"
        np.testing.assert_allclose(score[b][:n_vis], s, rtol=1e-5, atol=1e-5)
        assert np.isnan(score[b][n_vis:]).all()


def test_topk_two_stage_ties_across_slices(lib):
    # exact small-integer scores: 300 nines spread over every slice, eights every 20th
    # entry from 3000 on (55 of them in slice 0), ones elsewhere; the top 500 are the
    # nines plus the 200 lowest-index eights, which straddle the slice 0 / 1 boundary
    B, HI, dI, N, m, k = 1, 1, 32, 16384, 1, 500
    vals = np.ones(N)
    vals[3000::20] = 8
    rng = np.random.default_rng(synth.seed_of("ties-two-stage") % (1 << 32))
    vals[rng.choice(N, 300, replace=False)] = 9
    qi = torch.zeros((B, HI, dI), dtype=torch.bfloat16, device=DEV)
    qi[0, 0, 0] = 1.0
    keys = torch.zeros((B, N, dI), dtype=torch.bfloat16, device=DEV)
    keys[0, :, 0] = torch.tensor(vals, dtype=torch.bfloat16)
    w = torch.ones((B, HI), device=DEV)
    idx, score = lib.csa_index_topk(qi, w, keys, torch.tensor([N - 1], device=DEV), m, k)
    ref = O.topk_select(vals.astype(np.float64), k)
    got = idx[0].cpu().numpy()
    assert list(got) == list(ref)
    assert (np.sort(vals)[::-1][:k] == np.sort(vals[got])[::-1]).all()
    np.testing.assert_array_equal(score[0].cpu().numpy(), vals[got].astype(np.float32))


def test_topk_ties_and_zero_scores(lib):
    # planted exact ties: small-integer data makes every score exact in fp32 and fp64
    B, HI, dI, N, m, k = 1, 2, 32, 96, 1, 10
    qi = torch.zeros((B, HI, dI), dtype=torch.bfloat16, device=DEV)
    qi[0, 0, 0] = 1.0
    keys = torch.zeros((B, N, dI), dtype=torch.bfloat16, device=DEV)
    vals = [3, 5, 5, 1, 5, 2, 2, 7, -4, 2] * 9 + [0] * 6
    keys[0, :, 0] = torch.tensor(vals, dtype=torch.bfloat16)
    w = torch.tensor([[1.0, 0.5]], device=DEV)
    idx, score = lib.csa_index_topk(qi, w, keys, torch.tensor([N - 1], device=DEV), m, k)
    s = np.maximum(np.array(vals, dtype=np.float64), 0)
    ref = O.topk_select(s, k)
    assert list(idx[0].cpu().numpy()) == list(ref)


# ---------------------------------------------------------------------------
# CSA sparse prefill (a query chunk: indexer, per-query top-k, selected attention)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,Tq,p0,HI,dI,k,treated", [
    (2, 70, 2330, 8, 64, 64, True),     # two query groups (64 + ragged 6), k well below the visible count
    (1, 40, 0, 16, 128, 16, True),      # 16 indexer heads, early queries see fewer than k (or no) entries
    (1, 33, 1000, 5, 32, 100, False),   # padded indexer heads, odd query tail, untreated
    (1, 520, 2000, 8, 64, 64, True),    # 520 rows: one 8-wave attention workgroup per query
])
def test_csa_sparse_prefill(lib, B, Tq, p0, HI, dI, k, treated):
    Hq, d, m, W = 64, 512, 4, 128
    T = p0 + Tq
    N = T // m
    C = _dev(synth.csa_layer(f"csa-pf-{p0}", B, Hq, T, d, m, HI, dI, q_len=Tq))
    treat = dict(rmsnorm_eps=1e-6, rope_dims=64, rope_base=10000.0) if treated else {}
    entries = torch.zeros((B, 1, N, d), dtype=torch.bfloat16, device=DEV)
    lib.pool_blocks(C["ca"], C["za"], C["bias_a"], m, 0, N, entries, xb=C["cb"], zb=C["zb"],
                    bias_b=C["bias_b"], **treat)
    ikeys = torch.zeros((B, 1, N, dI), dtype=torch.bfloat16, device=DEV)
    lib.pool_blocks(C["ica"], C["iza"], C["ibias_a"], m, 0, N, ikeys, xb=C["icb"], zb=C["izb"],
                    bias_b=C["ibias_b"])
    say(f"csa sparse prefill B={B} Tq={Tq} p0={p0} HI={HI} dI={dI} k={k}")
    o, lse, idx = lib.csa_sparse_prefill(C["qi"], C["w"], ikeys[:, 0], C["q"], entries[:, 0], C["ca"][:, 0],
                                         p0, 0, m, W, k, sink=C["sink"], **treat)
    o, lse, idx = host(o), host(lse), idx.cpu().numpy()
    pooled = O.pool_dual(host(C["ca"]), host(C["za"]), host(C["bias_a"][0]), host(C["cb"]),
                         host(C["zb"]), host(C["bias_b"][0]), m, 0, N)
    qi, w, ki, q, raw = host(C["qi"]), host(C["w"]), host(ikeys[:, 0]), host(C["q"]), host(C["ca"])
    sink = host(C["sink"])
    band_rows = 0
    for b in range(B):
        ro = np.zeros((Tq, Hq, d))
        rl = np.zeros((Tq, Hq))
        for i in range(Tq):
            t = p0 + i
            n_vis = min((t + 1) // m, N)
            band_rows += topk_matches(idx[b, i], O.index_scores(qi[b, i], w[b, i], ki[b], n_vis), k,
                                      f"seq {b} query {i}", index_score_bound(qi[b, i], w[b, i], ki[b], n_vis),
                                      allow_band=True)[1]
            # the attention over the GPU's (valid) selection
            oo, ll = O.attend_decode(q[b, i][None], pooled[b][None], None, raw[b][None], None, [t], m, W,
                                     O.OVERLAP, 1 / math.sqrt(d), raw_pos_base=[0], sel_idx=idx[b, i][None],
                                     sink=sink, **treat)
            ro[i], rl[i] = oo[0], ll[0]
        check_bf16(o[b], ro, f"sparse prefill out seq {b}")
        check_bf16(lse[b], rl, f"sparse prefill lse seq {b}")
    say(f"sparse prefill: {band_rows} of {B * Tq} selections in the fp32 tie band (validity checked)")


@pytest.mark.parametrize("Tq,N", [
    (20, 12500),    # 20 rows: the per-query selection runs in two stages (4 slices of 4096)
    (300, 20000),   # 300 rows: one selection workgroup per row over up to 20000 entries
])
def test_csa_sparse_prefill_two_stage_selection(lib, Tq, N):
    B, Hq, d, m, W, HI, dI, k = 1, 32, 512, 4, 128, 8, 64, 512
    p0 = N * m - Tq
    g = lambda n, shape: synth.normal(shape, synth.seed_of("csa-pf-2s", N, n), dtype="bf16", device=DEV)
    qi, ki, q, ent, raw = g("qi", (B, Tq, HI, dI)), g("ki", (B, N, dI)), g("q", (B, Tq, Hq, d)), \
        g("e", (B, N, d)), g("raw", (B, Tq + W, d))
    w = synth.uniform((B, Tq, HI), synth.seed_of("csa-pf-2s", N, "w"), device=DEV)
    base = p0 - W + 1
    o, lse, idx = lib.csa_sparse_prefill(qi, w, ki, q, ent, raw, p0, base, m, W, k)
    o, lse, idx = host(o), host(lse), idx.cpu().numpy()
    qh, wh, kh, eh, rh = host(qi), host(w), host(ki), host(ent), host(raw)
    ro, rl = np.zeros((Tq, Hq, d)), np.zeros((Tq, Hq))
    for i in range(Tq):
        t = p0 + i
        n_vis = min((t + 1) // m, N)
        topk_matches(idx[0, i], O.index_scores(qh[0, i], wh[0, i], kh[0], n_vis), k, f"query {i}",
                     index_score_bound(qh[0, i], wh[0, i], kh[0], n_vis), allow_band=True)
        oo, ll = O.attend_decode(host(q)[0, i][None], eh[0][None, None], None, rh[0][None, None], None, [t], m, W,
                                 O.OVERLAP, 1 / math.sqrt(d), raw_pos_base=[base], sel_idx=idx[0, i][None])
        ro[i], rl[i] = oo[0], ll[0]
    check_bf16(o[0], ro, "two-stage sparse prefill out")
    check_bf16(lse[0], rl, "two-stage sparse prefill lse")
