"""Strided tensors at the C ABI: every call, given non-contiguous views (rows
padded inside a wider buffer, slices of longer caches, head-interleaved
[batch, rows, heads, dim] buffers seen as [batch, heads, rows, dim], queries
taken from a fused projection output), returns bitwise what it returns for
the same values in dense tensors, and writes strided outputs in place without
touching the rest of their buffers.  The unused elements of every input buffer
hold NaN, so a read outside a view poisons the outputs.  Decode and prefill
over strided inputs are also checked against the fp64 oracle directly.

Bitwise equality holds because strides change only addresses: the kernel
instance, the split plan and the order of every sum are the same.  The
attention backward adds dq and the sink gradient with floating-point atomics,
so those two are compared at 1e-5 relative instead.
"""
import math

import numpy as np
import pytest
import torch

from block_compressed_kv_amd import synth
from oracle import lbca_oracle as O

from parity_util import check_bf16, check_f32_rows, host, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
SENT = 1152.0  # fill of output buffers outside the views (exact in bf16)


def _g(tag, shape, dtype="bf16", std=1.0):
    return synth.normal(shape, synth.seed_of("strided", tag), std=std, dtype=dtype, device=DEV)


def view(t, layout, fill=float("nan")):
    """A non-contiguous view holding t's values; the rest of its buffer holds fill."""
    shp = list(t.shape)
    if layout == "pad":        # rows of d inside rows of d + 16
        buf = torch.full(shp[:-1] + [shp[-1] + 16], fill, dtype=t.dtype, device=t.device)
        v = buf[..., : shp[-1]]
    elif layout == "swap":     # dims 1 and 2 stored the other way round (head-interleaved)
        s2 = list(shp)
        s2[1], s2[2] = s2[2], s2[1]
        buf = torch.full(s2, fill, dtype=t.dtype, device=t.device)
        v = buf.transpose(1, 2)
    elif layout == "slice1":   # dim 1 a slice of a longer buffer, not at its start
        buf = torch.full(shp[:1] + [shp[1] + 3] + shp[2:], fill, dtype=t.dtype, device=t.device)
        v = buf[:, 2: 2 + shp[1]]
    elif layout == "slice2":   # dim 2 (rows) a slice of a longer buffer
        buf = torch.full(shp[:2] + [shp[2] + 5] + shp[3:], fill, dtype=t.dtype, device=t.device)
        v = buf[:, :, 1: 1 + shp[2]]
    else:
        raise ValueError(layout)
    assert not v.is_contiguous() and v.stride(-1) == 1
    v.copy_(t)
    return v, buf


def out_view(shape, dtype, layout, zero=False):
    """An output view inside a buffer of sentinels (its own elements zero or unset)."""
    v, buf = view(torch.zeros(shape, dtype=dtype, device=DEV), layout, fill=SENT)
    if not zero:
        v.fill_(-7.0)
    return v, buf


def untouched(v, buf, what):
    """Everything of buf outside the view still holds the sentinel."""
    assert int((buf == SENT).sum()) == buf.numel() - v.numel(), f"{what}: writes outside the view"


def same(a, b, what):
    assert a.shape == b.shape, what
    assert torch.equal(a, b), f"{what}: strided result differs from dense (max {float((a.float() - b.float()).abs().max())})"


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("case", [
    # tag, B, Hq, Hkv, d, entries, raw rows, t0, m, W, shared
    ("gqa128-split", 2, 6, 2, 128, 6100, 96, 24000, 4, 32, False),
    ("gqa64-shared", 3, 8, 2, 64, 330, 80, 5000, 16, 48, True),
])
def test_decode_strided(lib, case):
    tag, B, Hq, Hkv, d, N, R, t0, m, W, shared = case
    say(f"strided decode {tag}")
    fused = _g(f"{tag}-qkv", (B, Hq + 2 * Hkv, d))
    q = fused[:, :Hq]                                               # query part of a fused projection
    pk = _g(f"{tag}-pk", (B, Hkv, N, d))
    rk = _g(f"{tag}-rk", (B, Hkv, R, d))
    pv = None if shared else _g(f"{tag}-pv", (B, Hkv, N, d))
    rv = None if shared else _g(f"{tag}-rv", (B, Hkv, R, d))
    pos = torch.tensor([t0 + 37 * b for b in range(B)], dtype=torch.int64, device=DEV)
    rpb = torch.tensor([O.visible_range(t0 + 37 * b, m, W, O.EXCLUSIVE)[1] - 3 for b in range(B)],
                       dtype=torch.int64, device=DEV)
    sink = _g(f"{tag}-sink", (Hq,), "f32")
    dense = lib.attend_decode(q.contiguous(), pk, rk, pos, m, W, O.EXCLUSIVE, pooled_v=pv, raw_v=rv,
                              raw_pos_base=rpb, sink=sink)
    spk, _ = view(pk, "slice2")
    srk, _ = view(rk, "swap")
    spv = None if shared else view(pv, "pad")[0]
    srv = None if shared else view(rv, "slice1")[0]
    out, obuf = out_view((B, Hq, d), torch.float32, "pad")
    got = lib.attend_decode(q, spk, srk, pos, m, W, O.EXCLUSIVE, out=out, pooled_v=spv, raw_v=srv,
                            raw_pos_base=rpb, sink=sink)
    torch.cuda.synchronize()
    same(got[0], dense[0], f"{tag} out")
    same(got[1], dense[1], f"{tag} lse")
    untouched(out, obuf, f"{tag} out")
    # and against the oracle (one sequence)
    hv = lambda t: host(t)
    ro, rl = O.attend_decode(hv(q)[:1], hv(pk)[:1], hv(pk if shared else pv)[:1], hv(rk)[:1],
                             hv(rk if shared else rv)[:1], [t0], m, W, O.EXCLUSIVE, 1 / math.sqrt(d),
                             raw_pos_base=[int(rpb[0])], sink=hv(sink))
    check_bf16(host(got[0])[:1], ro, f"{tag} vs oracle")


def test_decode_strided_f32_and_noalloc(lib):
    B, Hq, Hkv, d, N, R, t, m, W = 2, 4, 2, 64, 40, 48, 300, 8, 16
    q = _g("f32-q", (B, Hq, d), "f32")
    pk, pv = _g("f32-pk", (B, Hkv, N, d), "f32"), _g("f32-pv", (B, Hkv, N, d), "f32")
    rk, rv = _g("f32-rk", (B, Hkv, R, d), "f32"), _g("f32-rv", (B, Hkv, R, d), "f32")
    pos = torch.tensor([t, t - 5], dtype=torch.int64, device=DEV)
    rpb = torch.tensor([260, 250], dtype=torch.int64, device=DEV)
    dense = lib.attend_decode(q, pk, rk, pos, m, W, O.EXCLUSIVE, pooled_v=pv, raw_v=rv, raw_pos_base=rpb)
    args = [view(q, "slice1")[0], view(pk, "swap")[0], view(rk, "pad")[0], pos, m, W, O.EXCLUSIVE]
    out, obuf = out_view((B, Hq, d), torch.float32, "slice1")
    got = lib.attend_decode(*args, out=out, pooled_v=view(pv, "slice2")[0], raw_v=view(rv, "swap")[0],
                            raw_pos_base=rpb)
    torch.cuda.synchronize()
    same(got[0], dense[0], "f32 out")
    same(got[1], dense[1], "f32 lse")
    untouched(out, obuf, "f32 out")
    ref_o, _ = O.attend_decode(host(q), host(pk), host(pv), host(rk), host(rv), [t, t - 5], m, W, O.EXCLUSIVE,
                               1 / math.sqrt(d), raw_pos_base=[260, 250])
    check_f32_rows(host(got[0]), ref_o, "f32 strided vs oracle")
    # the allocation-free entry point takes the same views (bf16 copy of the case)
    bq, bpk, brk = (x.to(torch.bfloat16) for x in (q, pk, rk))
    bpv, brv = pv.to(torch.bfloat16), rv.to(torch.bfloat16)
    o1 = torch.empty((B, Hq, d), dtype=torch.float32, device=DEV)
    l1 = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    lib.attend_decode_noalloc(bq, bpk, brk, pos, m, W, O.EXCLUSIVE, o1, l1, pooled_v=bpv, raw_v=brv,
                              raw_pos_base=rpb)
    o2, ob2 = out_view((B, Hq, d), torch.float32, "pad")
    l2 = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    lib.attend_decode_noalloc(view(bq, "slice1")[0], view(bpk, "swap")[0], view(brk, "slice2")[0], pos, m, W,
                              O.EXCLUSIVE, o2, l2, pooled_v=view(bpv, "pad")[0], raw_v=view(brv, "pad")[0],
                              raw_pos_base=rpb)
    torch.cuda.synchronize()
    same(o2, o1, "noalloc out")
    same(l2, l1, "noalloc lse")
    untouched(o2, ob2, "noalloc out")


def test_decode_strided_wide_selected(lib):
    # 512-dim MQA with the HCA/CSA treatment and a selection (wide path, split and merged)
    B, Hq, d, N, R, t, m, W, k = 2, 64, 512, 3100, 160, 12100, 4, 128, 512
    q = _g("wide-q", (B, Hq, d))
    ent = _g("wide-e", (B, 1, N, d))
    raw = _g("wide-r", (B, 1, R, d))
    pos = torch.tensor([t, t - 9], dtype=torch.int64, device=DEV)
    rpb = torch.tensor([t - 150, t - 159], dtype=torch.int64, device=DEV)
    sel = torch.stack([torch.randperm(3000, generator=torch.Generator().manual_seed(5 + b))[:k].sort().values
                       for b in range(B)]).to(torch.int32).to(DEV)
    kw = dict(raw_pos_base=rpb, sel_idx=sel, rmsnorm_eps=1e-6, rope_dims=64)
    dense = lib.attend_decode(q, ent, raw, pos, m, W, O.OVERLAP, **kw)
    out, obuf = out_view((B, Hq, d), torch.float32, "pad")
    got = lib.attend_decode(view(q, "slice1")[0], view(ent, "slice2")[0], view(raw, "pad")[0], pos, m, W,
                            O.OVERLAP, out=out, **kw)
    torch.cuda.synchronize()
    same(got[0], dense[0], "wide out")
    same(got[1], dense[1], "wide lse")
    untouched(out, obuf, "wide out")


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("case", [
    # tag, B, Tq, q0, Hq, Hkv, d, m, W, mode, shared, dtype, out dtype
    ("p128", 2, 300, 900, 6, 2, 128, 8, 64, O.EXCLUSIVE, False, "bf16", torch.float32),
    ("p64-shared", 1, 400, 150, 8, 2, 64, 4, 40, O.OVERLAP, True, "bf16", torch.bfloat16),
    ("pf32", 1, 70, 200, 4, 2, 64, 4, 16, O.EXCLUSIVE, False, "f32", torch.float32),
])
def test_prefill_strided(lib, case):
    tag, B, Tq, q0, Hq, Hkv, d, m, W, mode, shared, dt, odt = case
    say(f"strided prefill {tag}")
    last = q0 + Tq - 1
    N = O.visible_range(last, m, W, mode)[0] + 2
    rpb = max(0, O.visible_range(q0, m, W, mode)[1] - 5)
    R = last + 1 - rpb + 4
    fused = _g(f"{tag}-qkv", (B, Tq, Hq + 2 * Hkv, d), dt)
    q = fused[:, :, Hkv: Hkv + Hq]                                   # not at the start of the row either
    pk, rk = _g(f"{tag}-pk", (B, Hkv, N, d), dt), _g(f"{tag}-rk", (B, Hkv, R, d), dt)
    pv = None if shared else _g(f"{tag}-pv", (B, Hkv, N, d), dt)
    rv = None if shared else _g(f"{tag}-rv", (B, Hkv, R, d), dt)
    sink = _g(f"{tag}-sink", (Hq,), "f32")
    dense = lib.attend_prefill(q.contiguous(), q0, pk, rk, rpb, m, W, mode, pooled_v=pv, raw_v=rv, sink=sink,
                               out_dtype=odt)
    out, obuf = out_view((B, Tq, Hq, d), odt, "pad")
    got = lib.attend_prefill(q, q0, view(pk, "pad")[0], view(rk, "swap")[0], rpb, m, W, mode, out=out,
                             pooled_v=None if shared else view(pv, "swap")[0],
                             raw_v=None if shared else view(rv, "slice2")[0], sink=sink)
    torch.cuda.synchronize()
    same(got[0], dense[0], f"{tag} out")
    same(got[1], dense[1], f"{tag} lse")
    untouched(out, obuf, f"{tag} out")
    sl = slice(0, min(Tq, 48))
    ro, rl = O.attend_prefill(host(q)[:, sl], q0, host(pk), host(pk if shared else pv), host(rk),
                              host(rk if shared else rv), rpb, m, W, mode, 1 / math.sqrt(d), sink=host(sink))
    (check_f32_rows if dt == "f32" else check_bf16)(host(got[0])[:, sl], ro, f"{tag} vs oracle")


def test_attention_backward_strided(lib):
    B, Tq, q0, Hq, Hkv, d, m, W, mode = 1, 520, 0, 6, 2, 128, 8, 64, O.EXCLUSIVE
    last = q0 + Tq - 1
    N = O.visible_range(last, m, W, mode)[0] + 1
    R = Tq
    fused = _g("bw-qkv", (B, Tq, Hq + 2 * Hkv, d))
    q = fused[:, :, :Hq]
    pk, pv = _g("bw-pk", (B, Hkv, N, d)), _g("bw-pv", (B, Hkv, N, d))
    rk, rv = _g("bw-rk", (B, Hkv, R, d)), _g("bw-rv", (B, Hkv, R, d))
    do = _g("bw-do", (B, Tq, Hq, d))
    sink = _g("bw-sink", (Hq,), "f32")
    o, lse = lib.attend_prefill(q.contiguous(), q0, pk, rk, 0, m, W, mode, pooled_v=pv, raw_v=rv, sink=sink,
                                out_dtype=torch.float32)
    dense = lib.attend_prefill_backward(q.contiguous(), q0, pk, rk, 0, m, W, mode, o, lse, do, pooled_v=pv,
                                        raw_v=rv, sink=sink)
    outs = [out_view(s, torch.float32, lay) for s, lay in (((B, Tq, Hq, d), "pad"), ((B, Hkv, N, d), "slice2"),
                                                            ((B, Hkv, N, d), "swap"), ((B, Hkv, R, d), "pad"),
                                                            ((B, Hkv, R, d), "swap"))]
    got = lib.attend_prefill_backward(q, q0, view(pk, "swap")[0], view(rk, "slice2")[0], 0, m, W, mode,
                                      view(o, "pad")[0], lse, view(do, "pad")[0], pooled_v=view(pv, "pad")[0],
                                      raw_v=view(rv, "swap")[0], sink=sink, grad_q=outs[0][0],
                                      grad_pooled_k=outs[1][0], grad_pooled_v=outs[2][0], grad_raw_k=outs[3][0],
                                      grad_raw_v=outs[4][0])
    torch.cuda.synchronize()
    names = ("dq", "d pooled k", "d pooled v", "d raw k", "d raw v", "d sink")
    for i, n in enumerate(names):
        if n in ("dq", "d sink"):   # summed with atomics: order of the adds varies
            err = (got[i] - dense[i]).abs().max() / dense[i].abs().max()
            assert float(err) <= 1e-5, f"{n}: {float(err)}"
        else:
            same(got[i], dense[i], n)
    for i, (v, buf) in enumerate(outs):
        untouched(v, buf, names[i])


# ---------------------------------------------------------------------------
def test_pool_strided(lib):
    B, H, T, d, m = 2, 3, 96, 64, 16
    N = T // m
    x, v = _g("pool-x", (B, H, T, d)), _g("pool-v", (B, H, T, d))
    z = _g("pool-z", (B, H, T, d), "f32")
    bias = _g("pool-b", (H, m, d), "f32", std=0.1)
    ox = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=DEV)
    ov = torch.empty_like(ox)
    lib.pool_blocks(x, z, bias, m, 0, N, ox, v=v, out_v=ov)
    sx, bx = out_view((B, H, N, d), torch.bfloat16, "swap")
    sv, bv = out_view((B, H, N, d), torch.bfloat16, "pad")
    lib.pool_blocks(view(x, "swap")[0], view(z, "slice2")[0], bias, m, 0, N, sx, v=view(v, "pad")[0], out_v=sv)
    # shared series with the treatment, dual CSA mode
    hx = _g("pool-hx", (B, 1, T, 128))
    hz = _g("pool-hz", (B, 1, T, 128), "f32")
    hb = _g("pool-hb", (1, m, 128), "f32", std=0.1)
    hxb, hzb = _g("pool-hxb", (B, 1, T, 128)), _g("pool-hzb", (B, 1, T, 128), "f32")
    hbb = _g("pool-hbb", (1, m, 128), "f32", std=0.1)
    tr = dict(rmsnorm_eps=1e-6, rope_dims=64)
    od = torch.empty((B, 1, N, 128), dtype=torch.bfloat16, device=DEV)
    lib.pool_blocks(hx, hz, hb, m, 0, N, od, xb=hxb, zb=hzb, bias_b=hbb, **tr)
    sd, bd = out_view((B, 1, N, 128), torch.bfloat16, "slice2")
    lib.pool_blocks(view(hx, "pad")[0], view(hz, "slice2")[0], hb, m, 0, N, sd, xb=view(hxb, "slice2")[0],
                    zb=view(hzb, "pad")[0], bias_b=hbb, **tr)
    torch.cuda.synchronize()
    same(sx, ox, "pooled K")
    same(sv, ov, "pooled V")
    same(sd, od, "dual treated entries")
    for t, b_, n in ((sx, bx, "K"), (sv, bv, "V"), (sd, bd, "dual")):
        untouched(t, b_, n)


def test_pool_backward_strided(lib):
    B, H, T, d, m = 2, 2, 64, 64, 16
    N = T // m
    x, v = _g("pg-x", (B, H, T, d)), _g("pg-v", (B, H, T, d))
    z = _g("pg-z", (B, H, T, d), "f32")
    bias = _g("pg-b", (H, m, d), "f32", std=0.1)
    gx, gv = _g("pg-gx", (B, H, N, d)), _g("pg-gv", (B, H, N, d))
    dense = lib.pool_blocks_backward(x, z, bias, m, 0, N, gx, v=v, grad_v=gv)
    dx, bdx = out_view((B, H, T, d), torch.bfloat16, "swap", zero=True)
    dv, bdv = out_view((B, H, T, d), torch.bfloat16, "pad", zero=True)
    dz, bdz = out_view((B, H, T, d), torch.float32, "slice2", zero=True)
    got = lib.pool_blocks_backward(view(x, "pad")[0], view(z, "swap")[0], bias, m, 0, N, view(gx, "slice2")[0],
                                   v=view(v, "slice1")[0], grad_v=view(gv, "swap")[0], dx=dx, dv=dv, dz=dz)
    torch.cuda.synchronize()
    for i, n in enumerate(("dx", "dv", "dz", "dbias")):
        same(got[i], dense[i], n)
    for t, b_, n in ((dx, bdx, "dx"), (dv, bdv, "dv"), (dz, bdz, "dz")):
        untouched(t, b_, n)


# ---------------------------------------------------------------------------
def test_cache_and_fused_step_strided(lib):
    # the same token stream through dense and strided rings / pooled caches /
    # token rows: lbca_cache_append + lbca_attend_decode and lbca_decode_step
    B, Hq, H, d, m, W, ring, T = 2, 4, 2, 64, 16, 32, 56, 150
    L = synth.lbca_layer("strided-step", B, Hq, H, T, d, m, "bf16", "f32", device=DEV)
    k, v, z, bias = L["k"], L["v"], L["z"], L["bias"]
    N = T // m + 1

    def state(strided):
        # rings start as NaN (every row is written before it is read), entries as 7
        def f(shp, dt, lay, val=float("nan")):
            t = torch.full(shp, val, dtype=dt, device=DEV)
            return view(t, lay)[0] if strided else t
        return dict(rk=f((B, H, 2 * ring, d), torch.bfloat16, "swap"), rv=f((B, H, 2 * ring, d), torch.bfloat16, "pad"),
                    rz=f((B, H, 2 * ring, d), torch.float32, "slice2"),
                    pk=f((B, H, N, d), torch.bfloat16, "slice2", 7.0), pv=f((B, H, N, d), torch.bfloat16, "swap", 7.0),
                    rpb=torch.zeros((B,), dtype=torch.int64, device=DEV))

    sd, ss, fd, fs = state(False), state(True), state(False), state(True)
    qs = _g("step-q", (8, B, Hq + 2 * H, d))
    for t in range(T):
        pos = torch.full((B,), t, dtype=torch.int64, device=DEV)
        tok = [x[:, :, t] for x in (k, v, z)]                        # [B, H, d] views of the history
        q = qs[t % 8][:, :Hq]
        for st, toks in ((sd, [x.contiguous() for x in tok]), (ss, tok)):
            lib.cache_append(toks[0], toks[2], st["rk"], st["rz"], bias, pos, st["rpb"], m, W, O.EXCLUSIVE, st["pk"],
                             v_new=toks[1], raw_v=st["rv"], out_v=st["pv"])
        od = lib.attend_decode(q.contiguous(), sd["pk"], sd["rk"], pos, m, W, O.EXCLUSIVE, pooled_v=sd["pv"],
                               raw_v=sd["rv"], raw_pos_base=sd["rpb"])
        os_ = lib.attend_decode(q, ss["pk"], ss["rk"], pos, m, W, O.EXCLUSIVE, pooled_v=ss["pv"], raw_v=ss["rv"],
                                raw_pos_base=ss["rpb"])
        fo_d = lib.decode_step(q.contiguous(), *[x.contiguous() for x in tok], fd["rk"], fd["rv"], fd["rz"], bias,
                               fd["pk"], fd["pv"], pos, fd["rpb"], m, W)
        out, obuf = out_view((B, Hq, d), torch.float32, "pad")
        fo_s = lib.decode_step(q, *tok, fs["rk"], fs["rv"], fs["rz"], bias, fs["pk"], fs["pv"], pos, fs["rpb"], m, W,
                               out=out)
        same(os_[0], od[0], f"cache step {t}: out")
        same(fo_s[0], fo_d[0], f"fused step {t}: out")
        same(fo_s[1], fo_d[1], f"fused step {t}: lse")
        untouched(out, obuf, f"fused step {t}: out")
    torch.cuda.synchronize()
    for n in ("rk", "rv", "rz", "pk", "pv"):
        same(ss[n], sd[n], f"cache state {n}")
        same(fs[n], fd[n], f"fused state {n}")


# ---------------------------------------------------------------------------
def test_index_and_sparse_prefill_strided(lib):
    B, Tq, HI, dI, Hq, d, m, W, k = 2, 70, 8, 64, 64, 512, 4, 128, 64
    q0 = 2600
    N = (q0 + Tq) // m + 2
    R = Tq + W + 3
    rpb = q0 - W - 1
    qi_f = _g("sp-qi", (B, Tq, HI + 2, dI))
    q_idx = qi_f[:, :, 1: 1 + HI]
    head_w = _g("sp-w", (B, Tq, HI), "f32")
    keys = _g("sp-k", (B, N, dI))
    q = _g("sp-q", (B, Tq, Hq, d))
    ent = _g("sp-e", (B, N, d))
    raw = _g("sp-r", (B, R, d))
    tr = dict(rmsnorm_eps=1e-6, rope_dims=64)
    dense = lib.csa_sparse_prefill(q_idx.contiguous(), head_w, keys, q, ent, raw, q0, rpb, m, W, k, **tr)
    out, obuf = out_view((B, Tq, Hq, d), torch.float32, "pad")
    got = lib.csa_sparse_prefill(q_idx, head_w, view(keys, "pad")[0], view(q, "slice1")[0],
                                 view(ent.unsqueeze(1), "slice2")[0][:, 0], view(raw, "pad")[0], q0, rpb, m, W, k,
                                 out=out, **tr)
    torch.cuda.synchronize()
    same(got[2], dense[2], "selections")
    same(got[0], dense[0], "sparse prefill out")
    same(got[1], dense[1], "sparse prefill lse")
    untouched(out, obuf, "sparse prefill out")
    # decode-time indexer on strided queries and keys
    pos = torch.tensor([q0, q0 + 33], dtype=torch.int64, device=DEV)
    qd = qi_f[:, 5, 1: 1 + HI]
    wd = head_w[:, 5].contiguous()
    di, ds = lib.csa_index_topk(qd.contiguous(), wd, keys, pos, m, k)
    si, ss = lib.csa_index_topk(qd, wd, view(keys, "pad")[0], pos, m, k)
    torch.cuda.synchronize()
    same(si, di, "index ids")
    same(ss, ds, "index scores")
    for b in range(B):
        nv = (int(pos[b]) + 1) // m
        ref_scores = O.index_scores(host(qd)[b], host(wd)[b], host(keys)[b], nv)
        ids = host(si)[b].astype(np.int64)
        ids = ids[ids >= 0]
        assert len(ids) == min(k, nv)
        np.testing.assert_allclose(host(ss)[b][: len(ids)], ref_scores[ids], rtol=1e-5, atol=1e-5)
