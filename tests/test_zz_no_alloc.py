"""lbca_attend_decode_noalloc (split partials in the library's static scratch)
against lbca_attend_decode (the same kernels with a caller workspace), through
the C ABI: bitwise equal on two calls in a row, the second with a smaller
input, on both decode kernels' split paths; within the parity bar of the
oracle; a size beyond the scratch is rejected before any device work."""
import math

import numpy as np
import pytest
import torch

from block_compressed_kv_amd import synth
from oracle import lbca_oracle as O

from parity_util import check_bf16, host, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _hca(tag, B, N, T, treat):
    g = lambda n, shape: synth.normal(shape, synth.seed_of("noalloc", tag, n), dtype="bf16", device=DEV)
    q, ent, raw = g("q", (B, 64, 512)), g("e", (B, 1, N, 512)), g("r", (B, 1, 256, 512))
    pos = torch.tensor([T - 1 - 3 * b for b in range(B)], device=DEV)
    rpb = torch.full((B,), T - 256, dtype=torch.int64, device=DEV)
    sink = synth.normal((64,), synth.seed_of("noalloc", tag, "sink"), device=DEV)
    kw = dict(raw_pos_base=rpb, sink=sink)
    if treat:  # q and raw rows treated in the kernel (entries count as stored, treated)
        kw.update(rmsnorm_eps=1e-6, rope_dims=64)
    return q, ent, raw, pos, kw


def _lbca(tag, B, N):
    g = lambda n, shape: synth.normal(shape, synth.seed_of("noalloc", tag, n), dtype="bf16", device=DEV)
    q = g("q", (B, 24, 128))
    pk, pv = g("pk", (B, 8, N, 128)), g("pv", (B, 8, N, 128))
    rk, rv = g("rk", (B, 8, 256, 128)), g("rv", (B, 8, 256, 128))
    t_list = [N * 64 + 127 - 700 * b for b in range(B)]
    base = [O.visible_range(t, 64, 128, O.EXCLUSIVE)[1] for t in t_list]
    pos = torch.tensor(t_list, device=DEV)
    return q, pk, rk, pos, dict(pooled_v=pv, raw_v=rv, raw_pos_base=torch.tensor(base, device=DEV))


def _both(lib, q, pk, rk, pos, m, W, mode, kw):
    need = lib.decode_workspace_bytes(q, pk, rk, pos, m, W, mode, **kw)
    assert 0 < need <= lib.NOALLOC_SCRATCH_BYTES, need
    ref_o, ref_l = lib.attend_decode(q, pk, rk, pos, m, W, mode, **kw)
    out = torch.full_like(ref_o, float("nan"))
    lse = torch.full_like(ref_l, float("nan"))
    lib.attend_decode_noalloc(q, pk, rk, pos, m, W, mode, out, lse, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), "no-allocation decode differs"
    return out, lse, need


def test_noalloc_wide_path_two_calls(lib):
    # HCA-shaped (512 dims, 64 heads, treated): the wide kernel's bf16 partials
    T = 1 << 20
    for B, N in ((4, 8192), (2, 3000)):
        q, ent, raw, pos, kw = _hca(f"wide{B}", B, N, T, treat=B == 4)
        if N < 8192:
            pos = torch.tensor([N * 128 + 50, N * 128 - 700], device=DEV)
            kw["raw_pos_base"] = pos - 200
        o, lse, need = _both(lib, q, ent, raw, pos, 128, 128, O.OVERLAP, kw)
        say(f"no-alloc wide path B={B} N={N}: {need} bytes of scratch")
        if B == 2:  # also within the parity bar of the oracle
            ro, rl = O.attend_decode(host(q), host(ent), None, host(raw), None, host(pos).astype(int), 128, 128,
                                     O.OVERLAP, 1 / math.sqrt(512), raw_pos_base=host(kw["raw_pos_base"]).astype(int),
                                     sink=host(kw["sink"]))
            check_bf16(host(o), ro, "no-alloc wide out")
            check_bf16(host(lse), rl, "no-alloc wide lse")


def test_noalloc_narrow_path_two_calls(lib):
    # Llama-shaped GQA with long lists: the narrow kernel's fp32 partials and the merge
    for B, N in ((3, 2048), (1, 1300)):
        q, pk, rk, pos, kw = _lbca(f"narrow{B}", B, N)
        o, lse, need = _both(lib, q, pk, rk, pos, 64, 128, O.EXCLUSIVE, kw)
        say(f"no-alloc narrow path B={B} N={N}: {need} bytes of scratch")
    ro, rl = O.attend_decode(host(q), host(pk), host(kw["pooled_v"]), host(rk), host(kw["raw_v"]),
                             host(pos).astype(int), 64, 128, O.EXCLUSIVE, 1 / math.sqrt(128),
                             raw_pos_base=host(kw["raw_pos_base"]).astype(int))
    check_bf16(host(o), ro, "no-alloc narrow out")
    check_bf16(host(lse), rl, "no-alloc narrow lse")


def test_noalloc_rejects_beyond_scratch(lib):
    # GQA decode of 32 sequences over 8192 entries at m = 4: about 19 MB of fp32
    # partials, beyond the 16 MiB scratch (validation fails before any launch, so
    # the inputs need no values)
    B, N = 32, 8192
    e = lambda *shape: torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    q, pk, pv, rk, rv = e(B, 24, 128), e(B, 8, N, 128), e(B, 8, N, 128), e(B, 8, 256, 128), e(B, 8, 256, 128)
    pos = torch.full((B,), N * 4 + 127, dtype=torch.int64, device=DEV)
    kw = dict(pooled_v=pv, raw_v=rv, raw_pos_base=pos - 200)
    assert lib.decode_workspace_bytes(q, pk, rk, pos, 4, 128, O.EXCLUSIVE, **kw) > lib.NOALLOC_SCRATCH_BYTES
    out = torch.full((B, 24, 128), 7.0, device=DEV)
    lse = torch.full((B, 24), 7.0, device=DEV)
    with pytest.raises(lib.LbcaError) as err:
        lib.attend_decode_noalloc(q, pk, rk, pos, 4, 128, O.EXCLUSIVE, out, lse, **kw)
    assert err.value.status == lib.ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert (out == 7.0).all() and (lse == 7.0).all(), "outputs untouched"


def test_noalloc_without_split_uses_no_scratch(lib):
    # one workgroup per unit (the headline batch-16 shape): no partials at all
    B, N = 16, 510
    g = lambda n, shape: synth.normal(shape, synth.seed_of("noalloc-1split", n), dtype="bf16", device=DEV)
    q, pk, pv, rk, rv = g("q", (B, 24, 128)), g("pk", (B, 8, N, 128)), g("pv", (B, 8, N, 128)), \
        g("rk", (B, 8, 128, 128)), g("rv", (B, 8, 128, 128))
    pos = torch.full((B,), 32767, dtype=torch.int64, device=DEV)
    kw = dict(pooled_v=pv, raw_v=rv, raw_pos_base=torch.full((B,), 32640, dtype=torch.int64, device=DEV))
    assert lib.decode_workspace_bytes(q, pk, rk, pos, 64, 128, O.EXCLUSIVE, **kw) == 0
    ref_o, ref_l = lib.attend_decode(q, pk, rk, pos, 64, 128, O.EXCLUSIVE, **kw)
    out, lse = torch.empty_like(ref_o), torch.empty_like(ref_l)
    lib.attend_decode_noalloc(q, pk, rk, pos, 64, 128, O.EXCLUSIVE, out, lse, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
