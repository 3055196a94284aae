"""Exact indexing probes of every MFMA attention path, through the C ABI.

The bf16 parity bound (2e-2 + 1e-2 |ref|) is as large as a typical attention
output, so it cannot see a dropped tile, a window that starts one row late or a
wrong selected id.  These probes choose inputs whose results are exact in the
kernels' own arithmetic, so any such mistake shows:

* Uniform probe: q = 0 makes every logit exactly 0 on both sides, every softmax
  weight exactly 1 (0 after the max is subtracted), so the output is the plain
  mean of the visible value rows and lse = ln(number of visible rows) ("mSeek:
  learned KV-cache compression in a 3B model", "How LBCA works", steps 4-5: one
  softmax over every visible summary plus the exact window).  Value rows name
  themselves (``codes``): small integers, exact in bf16 and in fp32 sums, with
  the base-8 digits of the row's entry id or position, a raw/pooled flag, the KV
  head and the sequence.  A missing, extra or substituted row moves lse by at
  least ln(n/(n-1)) or one channel of the mean by at least 1/n, both far above
  the fp32 rounding of a division (checked by ``_power``).
* Spike probe: q = (64, 0, ...) and one chosen row with 64 in channel 0 (every
  other row 0 there): that row's logit is 4096 * scale and every other row's
  weight underflows to exactly 0, so the output is exactly the chosen row when
  it is visible and the mean of the visible rows (channel 0 = 0) when it is not.
  Spikes sit on the boundaries: the last visible and the first invisible pooled
  entry, the first raw row and the one before it, the query's own row and the
  one after it, tile edges, selected and unselected ids.

Expected values come from ``probe_util.expect`` (the oracle's visibility rule
and exact fp64 sums; pinned against the oracle's attention in
tests/test_probe_util.py), or the oracle itself for the selections.  Paths whose split partials are stored in bf16 (the 512-dim wide decode
with row ranges split over workgroups) keep lse exact and the spike probes
exact; their uniform-probe means carry the bf16 rounding of each partial, so
their identity checks rest on the spikes.
"""
import math

import numpy as np
import pytest
import torch

from oracle import lbca_oracle as O

from parity_util import host, say
from probe_util import SPIKE, codes, expect

pytestmark = pytest.mark.gpu
DEV = "cuda"
OUT_REL, OUT_ABS = 1e-6, 1e-7         # fp32 rounding of one division, with margin
LSE_ABS, LSE_REL = 4e-6, 2e-7         # fp32 log / logit rounding, with margin
BF16_PARTIAL_ABS = 2.0 ** -8 * 16     # a bf16 split partial of codes up to 15


def bf(x):
    t = torch.as_tensor(np.asarray(x), dtype=torch.float32).to(torch.bfloat16)
    assert torch.equal(t.float().double(), torch.as_tensor(np.asarray(x), dtype=torch.float64)), "not exact in bf16"
    return t.to(DEV)


def check_out(got, ref, what, abs_tol=OUT_ABS):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    bound = abs_tol + OUT_REL * np.abs(ref)
    bad = np.argwhere(~(err <= bound))
    assert bad.size == 0, f"{what}: {len(bad)} elements off, first at {tuple(bad[0])}: " \
                          f"got {got[tuple(bad[0])]} want {ref[tuple(bad[0])]}"


def check_lse(got, ref, what):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    bound = LSE_ABS + LSE_REL * np.abs(ref)
    bad = np.argwhere(~(err <= bound))
    assert bad.size == 0, f"{what}: lse off at {tuple(bad[0])}: got {got[tuple(bad[0])]} want {ref[tuple(bad[0])]}"


def _power(n_max):
    # one row more or less moves lse by ln(1 + 1/n) > 1/(n+1); the bound must be well below it
    assert 1.0 / (n_max + 1) > 2 * (LSE_ABS + LSE_REL * math.log(n_max + 1)), n_max


def _visible_count(t, m, W, mode, sel=None):
    n_p, rb = O.visible_range(t, m, W, mode)
    if sel is not None:
        s = np.asarray(sel)
        n_p = int(((s >= 0) & (s < n_p)).sum())
    return n_p + t - rb + 1


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
def decode_probe(lib, *, B, Hq, Hkv, d, N, R, m, W, mode, t_list, rpb, shared, spikes=None, sel=None,
                 sink=False, bf16_partials=False, what=""):
    """One probe launch.  spikes: None (uniform probe) or per sequence ("pool", j) /
    ("raw", position) / None."""
    b_, h_ = np.arange(B)[:, None, None], np.arange(Hkv)[None, :, None]
    P = codes(np.arange(N)[None, None, :], 0, h_, b_, d)
    Rw = codes(np.asarray(rpb)[:, None, None] + np.arange(R)[None, None, :], 1, h_, b_, d)
    Kp, Kr = (P, Rw) if shared else (np.zeros_like(P), np.zeros_like(Rw))
    q = np.zeros((B, Hq, d))
    if spikes is None:
        _power(max(_visible_count(t, m, W, mode, None if sel is None else sel[b]) for b, t in enumerate(t_list)))
    else:
        q[..., 0] = SPIKE
        for b, sp in enumerate(spikes):
            if sp is not None:
                where, idx = sp
                if where == "pool":
                    Kp[b, :, idx, 0] = SPIKE
                else:
                    Kr[b, :, idx - rpb[b], 0] = SPIKE
    pos = torch.tensor(t_list, dtype=torch.int64, device=DEV)
    rpbd = torch.tensor(rpb, dtype=torch.int64, device=DEV)
    sk = torch.zeros(Hq, device=DEV) if sink else None
    seld = None if sel is None else torch.as_tensor(np.asarray(sel), dtype=torch.int32).to(DEV)
    kw = dict(raw_pos_base=rpbd, sel_idx=seld, sink=sk)
    if not shared:
        kw.update(pooled_v=bf(P), raw_v=bf(Rw))
    tag = f"{what} ({'uniform' if spikes is None else 'spike'})"
    say(f"probe decode {tag}: B={B} Hq={Hq} Hkv={Hkv} d={d} N={N} m={m} W={W} mode={mode}")
    o, lse = lib.attend_decode(bf(q), bf(Kp), bf(Kr), pos, m, W, mode, **kw)
    torch.cuda.synchronize()
    G = Hq // Hkv
    ro, rl = np.zeros((B, Hq, d)), np.zeros((B, Hq))
    for b, t in enumerate(t_list):
        sp = None if spikes is None else spikes[b]
        for kh in range(Hkv):
            row = None
            if sp is not None:
                row = (Kp if shared else P)[b, kh, sp[1]] if sp[0] == "pool" else \
                    (Kr if shared else Rw)[b, kh, sp[1] - rpb[b]]
            oo, ll = expect(P[b, kh] if not shared else Kp[b, kh], Rw[b, kh] if not shared else Kr[b, kh], rpb[b],
                            [t], m, W, mode, 1 / math.sqrt(d), sel=None if sel is None else sel[b],
                            sink=0.0 if sink else None, spike=sp, spike_row=row)
            ro[b, kh * G:(kh + 1) * G] = oo[0]
            rl[b, kh * G:(kh + 1) * G] = ll[0]
    # with bf16 split partials only a visible spike (one row, exact in bf16) is exact
    spike_seen = rl[:, 0] > 0.5 * SPIKE * SPIKE / math.sqrt(d)
    for b in range(B):
        loose = bf16_partials and not spike_seen[b]
        check_out(host(o[b]), ro[b], f"{tag} seq {b}", abs_tol=BF16_PARTIAL_ABS if loose else OUT_ABS)
    check_lse(host(lse), rl, tag)
    if spikes is not None:
        say(f"  spikes seen by sequence: {spike_seen.astype(int).tolist()}")


def _llama_positions():
    # 32K decode, batch 16: the query at t = 32767 and its neighbours across the
    # block and window boundaries (m = 64, W = 128); all raw spans inside rows
    # [32512, 32768) and at most 510 pooled entries
    return [32767, 32766, 32765, 32703, 32702, 32704, 32705, 32735, 32736, 32639, 32640, 32641, 32670,
            32671, 32767, 32700]


@pytest.mark.parametrize("sink", [False, True])
def test_probe_decode_llama_32k_batch16(lib, sink):
    # headline decode launch shape: 24 query heads over 8 KV heads, d = 128, 510 entries
    t_list = _llama_positions()
    B, lo = len(t_list), 32512
    kw = dict(B=B, Hq=24, Hkv=8, d=128, N=510, R=256, m=64, W=128, mode=O.EXCLUSIVE, t_list=t_list,
              rpb=[lo] * B, shared=False, what="32K batch 16")
    decode_probe(lib, sink=sink, **kw)
    if sink:
        return
    spikes = []
    for b, t in enumerate(t_list):
        n_p, rb = O.visible_range(t, 64, 128, O.EXCLUSIVE)
        spikes.append([("pool", n_p - 1), ("pool", n_p) if n_p < 510 else ("pool", 0), ("raw", rb),
                       ("raw", rb - 1) if rb > lo else ("raw", t), ("raw", t), ("raw", min(t + 1, 32767)),
                       ("pool", 31), ("pool", 32), ("raw", rb + 31), ("raw", rb + 32), ("pool", 0),
                       ("pool", 479), ("pool", 480), ("raw", t - 127), ("raw", lo), ("pool", n_p // 2)][b])
    decode_probe(lib, spikes=spikes, **kw)
    # the same boundary rows shifted by one sequence, so each position meets other spikes
    decode_probe(lib, spikes=spikes[1:] + spikes[:1], **kw)


@pytest.mark.parametrize("mode", [O.EXCLUSIVE, O.OVERLAP])
def test_probe_decode_early_positions(lib, mode):
    # the first positions: no pooled entry yet, the first block, the window edge
    t_list = [0, 1, 2, 63, 64, 126, 127, 128, 129, 190, 191, 192, 193, 255, 256, 300]
    B = len(t_list)
    kw = dict(B=B, Hq=24, Hkv=8, d=128, N=8, R=320, m=64, W=128, mode=mode, t_list=t_list, rpb=[0] * B,
              shared=False, what=f"early positions mode {mode}")
    decode_probe(lib, **kw)
    spikes = []
    for b, t in enumerate(t_list):
        n_p, rb = O.visible_range(t, 64, 128, mode)
        spikes.append(("raw", rb) if b % 3 == 0 else ("raw", max(rb - 1, 0)) if b % 3 == 1 else
                      ("pool", max(n_p - 1, 0)))
    decode_probe(lib, spikes=spikes, **kw)


@pytest.mark.parametrize("d,Hq,Hkv,B", [
    (64, 8, 8, 16),      # 64 dims: one workgroup per unit, no dim split
    (128, 40, 2, 3),     # 20 heads per KV head: two 16-head groups, dim-split twins
    (256, 8, 2, 4),      # 256 dims
])
def test_probe_decode_shapes(lib, d, Hq, Hkv, B):
    m, W = 16, 40
    t_list = [700 + 37 * b for b in range(B)]
    rpb = [O.visible_range(t, m, W, O.EXCLUSIVE)[1] - 5 for t in t_list]
    kw = dict(B=B, Hq=Hq, Hkv=Hkv, d=d, N=100, R=80, m=m, W=W, mode=O.EXCLUSIVE, t_list=t_list, rpb=rpb,
              shared=False, what=f"d={d} Hq={Hq} Hkv={Hkv}")
    decode_probe(lib, **kw)
    spikes = [("raw", O.visible_range(t, m, W, O.EXCLUSIVE)[1] - (b % 2)) for b, t in enumerate(t_list)]
    decode_probe(lib, spikes=spikes, **kw)


def test_probe_decode_split_rows(lib):
    # long lists (about 8000 entries at m = 4): rows split over workgroups with
    # fp32 partials and the fixed-order merge
    m, W = 4, 128
    t_list = [32767, 30001, 9999]
    B = len(t_list)
    rpb = [32000, 29500, 9700]
    kw = dict(B=B, Hq=24, Hkv=8, d=128, N=8192, R=768, m=m, W=W, mode=O.EXCLUSIVE, t_list=t_list, rpb=rpb,
              shared=False, what="split rows")
    q0 = torch.zeros((B, 24, 128), dtype=torch.bfloat16, device=DEV)
    need = lib.decode_workspace_bytes(q0, torch.zeros((B, 8, 8192, 128), dtype=torch.bfloat16, device=DEV),
                                      torch.zeros((B, 8, 768, 128), dtype=torch.bfloat16, device=DEV),
                                      torch.tensor(t_list, device=DEV), m, W, O.EXCLUSIVE,
                                      pooled_v=torch.zeros((B, 8, 8192, 128), dtype=torch.bfloat16, device=DEV),
                                      raw_v=torch.zeros((B, 8, 768, 128), dtype=torch.bfloat16, device=DEV))
    assert need > 0, "this shape splits the rows"
    decode_probe(lib, **kw)
    decode_probe(lib, spikes=[("pool", O.visible_range(t, m, W, O.EXCLUSIVE)[0] - 1) for t in t_list], **kw)
    decode_probe(lib, spikes=[("pool", 4000), ("raw", 30001), ("raw", O.visible_range(9999, m, W, 0)[1] - 1)], **kw)


def test_probe_decode_shared_512_narrow(lib):
    # 512-dim shared series with 16 query heads (not a multiple of 32: the
    # narrow kernel with 16-row tiles), selected entries with padding and ids
    # that are not visible
    B, Hq, d, m, W, N = 2, 16, 512, 4, 128, 3000
    t_list = [11999, 6000]
    rng = np.random.default_rng(11)
    sel = np.full((B, 300), -1, dtype=np.int64)
    for b, t in enumerate(t_list):
        n_p = O.visible_range(t, m, W, O.OVERLAP)[0]
        sel[b, :250] = np.sort(rng.choice(n_p, 250, replace=False))
        sel[b, 250:260] = n_p + np.arange(10)          # not visible (past the buffer for b = 0): skipped
    rpb = [t - 200 for t in t_list]
    kw = dict(B=B, Hq=Hq, Hkv=1, d=d, N=N, R=256, m=m, W=W, mode=O.OVERLAP, t_list=t_list, rpb=rpb,
              shared=True, sel=sel, what="512 narrow + selection")
    decode_probe(lib, **kw)
    unselected = [int(np.setdiff1d(np.arange(100), sel[b])[0]) for b in range(B)]
    decode_probe(lib, spikes=[("pool", int(sel[0, 17])), ("pool", unselected[1])], **kw)
    decode_probe(lib, spikes=[("raw", t_list[0] - W), ("pool", int(sel[1, 250]))], **kw)


def test_probe_decode_hca_1m_batch4(lib):
    # HCA decode launch shape: 64 query heads, one shared 512-dim series, 8192
    # entries (m' = 128), window 128, positions near 2^20
    T = 1 << 20
    t_list = [T - 1, T - 2, T - 128, T - 129]
    B, m, W, R = 4, 128, 128, 300
    rpb = [T - R] * B
    kw = dict(B=B, Hq=64, Hkv=1, d=512, N=8192, R=R, m=m, W=W, mode=O.OVERLAP, t_list=t_list, rpb=rpb,
              shared=True, bf16_partials=True, what="HCA 1M batch 4")
    need = lib.decode_workspace_bytes(torch.zeros((B, 64, 512), dtype=torch.bfloat16, device=DEV),
                                      torch.zeros((B, 1, 8192, 512), dtype=torch.bfloat16, device=DEV),
                                      torch.zeros((B, 1, R, 512), dtype=torch.bfloat16, device=DEV),
                                      torch.tensor(t_list, device=DEV), m, W, O.OVERLAP)
    assert need > 0, "the HCA launch splits its rows (bf16 partials)"
    decode_probe(lib, **kw)
    spikes = []
    for b, t in enumerate(t_list):
        n_p, rb = O.visible_range(t, m, W, O.OVERLAP)
        spikes.append([("pool", n_p - 1), ("pool", n_p), ("raw", rb), ("raw", rb - 1)][b])
    decode_probe(lib, spikes=spikes, **kw)
    decode_probe(lib, spikes=[("raw", T - 1), ("pool", 0), ("pool", 4095), ("pool", 4096)], **kw)
    decode_probe(lib, spikes=[("pool", 8191), ("raw", T - 1), ("raw", T - 128), ("pool", 8190)], **kw)


def test_probe_decode_csa_128k_selection(lib):
    # CSA core attention launch shape: top-512 selected of 32768 entries plus the
    # window, 64 heads x 512, batch 2; selections include -1 padding, an id past
    # the visible count and an unsorted order
    T, m, W, N, k = 1 << 17, 4, 128, 32768, 512
    t_list = [T - 1, T - 3]
    B = 2
    rng = np.random.default_rng(5)
    sel = np.full((B, k), -1, dtype=np.int64)
    for b, t in enumerate(t_list):
        n_p = O.visible_range(t, m, W, O.OVERLAP)[0]
        pick = rng.choice(n_p, 500, replace=False)
        sel[b, :500] = pick if b else np.sort(pick)
    sel[1, 500] = 32767                                  # not visible at t = 2^17 - 3
    rpb = [T - 256] * B
    kw = dict(B=B, Hq=64, Hkv=1, d=512, N=N, R=256, m=m, W=W, mode=O.OVERLAP, t_list=t_list, rpb=rpb,
              shared=True, sel=sel, bf16_partials=True, what="CSA 128K selection")
    decode_probe(lib, **kw)
    unsel = [int(np.setdiff1d(np.arange(2000), sel[b])[0]) for b in range(B)]
    decode_probe(lib, spikes=[("pool", int(sel[0, 0])), ("pool", unsel[1])], **kw)
    decode_probe(lib, spikes=[("pool", unsel[0]), ("pool", 32767)], **kw)
    decode_probe(lib, spikes=[("raw", t_list[0] - W), ("raw", t_list[1] - W + 1)], **kw)


def test_probe_decode_selection_at_split_limit(lib):
    # the largest selection plus raw span the wide path plans: 2048 ids and a
    # 63488-row window = 2048 tiles of 32 rows over 64 ranges of 1024 staged ids
    B, Hq, d, m, k, W = 1, 64, 512, 4, 2048, 63488
    t = 80000
    n_p = O.visible_range(t, m, W, O.OVERLAP)[0]
    N = n_p
    sel = np.sort(np.random.default_rng(3).choice(n_p, k, replace=False))[None]
    rpb = [t - W + 1]
    kw = dict(B=B, Hq=Hq, Hkv=1, d=d, N=N, R=W, m=m, W=W, mode=O.OVERLAP, t_list=[t], rpb=rpb, shared=True,
              sel=sel, bf16_partials=True, what="64 ranges")
    decode_probe(lib, **kw)
    decode_probe(lib, spikes=[("pool", int(sel[0, -1]))], **kw)
    decode_probe(lib, spikes=[("raw", t - W + 1)], **kw)


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------
def prefill_probe(lib, *, B, Tq, q_pos0, Hq, Hkv, d, N, R, rpb, m, W, mode, shared, spikes=None, what=""):
    """spikes: None (uniform probe) or one ("pool", j) / ("raw", position) per sequence."""
    b_, h_ = np.arange(B)[:, None, None], np.arange(Hkv)[None, :, None]
    P = codes(np.arange(N)[None, None, :], 0, h_, b_, d)
    Rw = codes(rpb + np.arange(R)[None, None, :], 1, h_, b_, d)
    Kp, Kr = (P, Rw) if shared else (np.zeros_like(P), np.zeros_like(Rw))
    q = np.zeros((B, Tq, Hq, d))
    if spikes is None:
        _power(_visible_count(q_pos0 + Tq - 1, m, W, mode))
    else:
        q[..., 0] = SPIKE
        for b, (where, idx) in enumerate(spikes):
            if where == "pool":
                Kp[b, :, idx, 0] = SPIKE
            else:
                Kr[b, :, idx - rpb, 0] = SPIKE
    kw = {} if shared else dict(pooled_v=bf(P), raw_v=bf(Rw))
    tag = f"{what} ({'uniform' if spikes is None else 'spike'})"
    say(f"probe prefill {tag}: B={B} Tq={Tq} q_pos0={q_pos0} Hq={Hq} Hkv={Hkv} d={d} m={m} W={W} mode={mode}")
    o, lse = lib.attend_prefill(bf(q), q_pos0, bf(Kp), bf(Kr), rpb, m, W, mode, out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    G = Hq // Hkv
    ts = q_pos0 + np.arange(Tq)
    ro, rl = np.zeros((B, Tq, Hq, d)), np.zeros((B, Tq, Hq))
    for b in range(B):
        sp = None if spikes is None else spikes[b]
        for kh in range(Hkv):
            Pv, Rv = (Kp[b, kh], Kr[b, kh]) if shared else (P[b, kh], Rw[b, kh])
            row = None if sp is None else (Pv[sp[1]] if sp[0] == "pool" else Rv[sp[1] - rpb])
            oo, ll = expect(Pv, Rv, rpb, ts, m, W, mode, 1 / math.sqrt(d), spike=sp, spike_row=row)
            ro[b, :, kh * G:(kh + 1) * G] = oo[:, None]
            rl[b, :, kh * G:(kh + 1) * G] = ll[:, None]
    check_out(host(o), ro, tag)
    check_lse(host(lse), rl, tag)


@pytest.mark.parametrize("q_pos0,Tq", [(14336, 2048), (0, 2048), (2048, 2048), (1000, 333)])
def test_probe_prefill_llama_chunks(lib, q_pos0, Tq):
    # 16K chunked prefill shape: 24 query heads over 8 KV heads, d = 128, m = 16,
    # W = 128; the raw buffer starts exactly at the first query's raw span.  The
    # spikes (one per sequence of a batch of 4) sit on an entry that becomes
    # visible inside the chunk, the chunk's middle position (causal edge, then
    # the window edge), the first query's first raw row and the last query's row.
    m, W = 16, 128
    n_last, _ = O.visible_range(q_pos0 + Tq - 1, m, W, O.EXCLUSIVE)
    n0, rb0 = O.visible_range(q_pos0, m, W, O.EXCLUSIVE)
    kw = dict(Tq=Tq, q_pos0=q_pos0, Hq=24, Hkv=8, d=128, N=max(n_last, 1), R=q_pos0 + Tq - rb0, rpb=rb0,
              m=m, W=W, mode=O.EXCLUSIVE, shared=False, what=f"chunk at {q_pos0}")
    prefill_probe(lib, B=1, **kw)
    spikes = [("pool", min(n0 + 3, n_last - 1)) if n_last > 0 else ("raw", rb0), ("raw", q_pos0 + Tq // 2),
              ("raw", rb0), ("raw", q_pos0 + Tq - 1)]
    prefill_probe(lib, B=4, spikes=spikes, **kw)


@pytest.mark.parametrize("mode,shared,d", [(O.OVERLAP, True, 64), (O.EXCLUSIVE, True, 128),
                                           (O.OVERLAP, False, 64)])
def test_probe_prefill_modes(lib, mode, shared, d):
    B, Tq, q_pos0, Hq, Hkv, m, W = 2, 300, 700, 8, 2, 16, 100
    n_last, _ = O.visible_range(q_pos0 + Tq - 1, m, W, mode)
    _, rb0 = O.visible_range(q_pos0, m, W, mode)
    rpb = rb0 - 3
    kw = dict(B=B, Tq=Tq, q_pos0=q_pos0, Hq=Hq, Hkv=Hkv, d=d, N=n_last + 2, R=q_pos0 + Tq - rpb + 5, rpb=rpb, m=m,
              W=W, mode=mode, shared=shared, what=f"mode {mode} shared {shared} d {d}")
    prefill_probe(lib, **kw)
    prefill_probe(lib, **dict(kw, spikes=[("raw", q_pos0 + 150), ("pool", n_last - 1)]))
    prefill_probe(lib, **dict(kw, spikes=[("raw", rb0), ("raw", rb0 + W)]))


# ---------------------------------------------------------------------------
# CSA: exact-arithmetic indexer data, sparse prefill
# ---------------------------------------------------------------------------
def dyadic(shape, seed, lim=2.0):
    """Values k/8 with |k| <= 8*lim: every indexer product and every sum of them is
    exact in fp32, so the GPU's fp32 scores equal the oracle's fp64 scores and the
    selection (ties included, lower index first) must match exactly."""
    rng = np.random.default_rng(seed)
    return np.clip(np.round(rng.standard_normal(shape) * 4) / 8, -lim, lim)


def weights16(shape, seed):
    return np.random.default_rng(seed).integers(0, 17, size=shape) / 16.0


def _exact_scores_bound(HI, dI, lim=2.0):
    # |q.k| <= dI * lim^2 in units of 1/64; times w (units 1/16), summed over HI
    # heads: the largest score in units of 1/1024 stays below 2^24
    assert HI * dI * lim * lim * 1024 < 2 ** 24


@pytest.mark.parametrize("t_list", [[(1 << 17) - 1, (1 << 17) - 2], [2047, 40000]])
def test_probe_index_topk_exact_128k(lib, t_list):
    # CSA indexer launch shape (8 heads x 64, top-512 of 32768, batch 2) on exact data:
    # the selected sets, with their many exact ties, must equal the oracle's
    B, HI, dI, N, m, k = 2, 8, 64, 32768, 4, 512
    _exact_scores_bound(HI, dI)
    qi, keys, w = dyadic((B, HI, dI), 1), dyadic((B, N, dI), 2), weights16((B, HI), 3)
    idx, score = lib.csa_index_topk(bf(qi), torch.tensor(w, dtype=torch.float32, device=DEV), bf(keys),
                                    torch.tensor(t_list, device=DEV), m, k)
    idx, score = idx.cpu().numpy(), score.cpu().numpy()
    for b, t in enumerate(t_list):
        n_vis = min((t + 1) // m, N)
        s = O.index_scores(qi[b], w[b], keys[b], n_vis)
        ref = O.topk_select(s, k)
        ties = int((s == np.sort(s)[::-1][min(k, n_vis) - 1]).sum())
        say(f"exact top-k seq {b}: n_vis={n_vis}, {ties} entries share the k-th score")
        assert list(idx[b]) == list(ref), f"seq {b}: selection differs"
        sel = ref[ref >= 0]
        assert np.array_equal(score[b][:sel.size].astype(np.float64), s[sel]), "scores are exact"


@pytest.mark.parametrize("B,Tq,p0,k", [
    (2, 520, 2600, 64),     # 1040 query rows: one 8-wave attention workgroup per query, no split
    (1, 40, 0, 16),         # the first 40 positions: fewer than k (or no) entries visible
])
def test_probe_csa_sparse_prefill_exact(lib, B, Tq, p0, k):
    Hq, d, m, W, HI, dI = 64, 512, 4, 128, 8, 64
    T = p0 + Tq
    N = T // m + 3
    _exact_scores_bound(HI, dI)
    qi, ki, w = dyadic((B, Tq, HI, dI), 7), dyadic((B, N, dI), 8), weights16((B, Tq, HI), 9)
    b_ = np.arange(B)[:, None]
    ent = codes(np.arange(N)[None, :], 0, 0, b_, d)
    raw = codes(np.arange(T)[None, :], 1, 0, b_, d)
    _power(k + W)
    wd = torch.tensor(w, dtype=torch.float32, device=DEV)
    say(f"probe csa sparse prefill B={B} Tq={Tq} p0={p0} k={k}")
    o, lse, idx = lib.csa_sparse_prefill(bf(qi), wd, bf(ki), bf(np.zeros((B, Tq, Hq, d))), bf(ent), bf(raw), p0, 0,
                                         m, W, k)
    torch.cuda.synchronize()
    o, lse, idx = host(o), host(lse), idx.cpu().numpy()
    for b in range(B):
        ro, rl = np.zeros((Tq, Hq, d)), np.zeros((Tq, Hq))
        for i in range(Tq):
            t = p0 + i
            n_vis = min((t + 1) // m, N)
            ref = O.topk_select(O.index_scores(qi[b, i], w[b, i], ki[b], n_vis), k)
            assert list(idx[b, i]) == list(ref), f"seq {b} query {i}: selection differs"
            oo, ll = expect(ent[b], raw[b], 0, [t], m, W, O.OVERLAP, 1 / math.sqrt(d), sel=ref)
            ro[i], rl[i] = oo[0], ll[0]
        twins = B * Tq < 512          # fewer than 512 rows: twin workgroups with split bf16 partials
        check_out(o[b], ro, f"sparse prefill seq {b}", abs_tol=BF16_PARTIAL_ABS if twins else OUT_ABS)
        check_lse(lse[b], rl, f"sparse prefill lse seq {b}")


# ---------------------------------------------------------------------------
# decode through the cache ring
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", [O.EXCLUSIVE, O.OVERLAP])
def test_probe_decode_through_ring(lib, mode):
    # Token-by-token loop: each token's K/V rows name their position; logits z
    # and the bias are 0, so each pooled entry is the exact mean of its block
    # (block-aligned base-8 digits average to k + 0.5 or stay constant).  At the
    # checked steps decode reads the ring with q = 0 and must give the exact mean
    # of the visible rows and lse = ln(count).
    from test_gpu_cache import _loop

    B, H, Hq, d, m, W, T = 3, 2, 6, 64, 16, 32, 300
    ring = W + m + 8 if mode == O.EXCLUSIVE else W + 8
    offsets = [0, 21, 77]
    xs = codes(np.arange(T)[None, None, :], 1, np.arange(H)[None, :, None], np.arange(B)[:, None, None], d)
    x, v = bf(xs), bf(xs)
    z = torch.zeros((B, H, T, d), dtype=torch.float32, device=DEV)
    bias = torch.zeros((H, m, d), dtype=torch.float32, device=DEV)
    q = torch.zeros((B, Hq, d), dtype=torch.bfloat16, device=DEV)
    G = Hq // H
    n_blocks = T // m
    pooled = xs[:, :, :n_blocks * m].reshape(B, H, n_blocks, m, d).mean(axis=3)   # uniform weights: block means
    steps = T - 1
    checked = []

    def on_check(step, t_list, raw_x, raw_v, raw_z, rpb, out_x, out_v):
        pos = torch.tensor(t_list, dtype=torch.int64, device=DEV)
        o, lse = lib.attend_decode(q, out_x, raw_x, pos, m, W, mode, pooled_v=out_v, raw_v=raw_v, raw_pos_base=rpb)
        o, lse = host(o), host(lse)
        for b, t in enumerate(t_list):
            if t < 0:
                continue
            for kh in range(H):
                oo, ll = expect(pooled[b, kh], xs[b, kh], 0, [t], m, W, mode, 1 / math.sqrt(d))
                check_out(o[b, kh * G:(kh + 1) * G], np.repeat(oo, G, 0), f"ring decode step {step} seq {b}")
                check_lse(lse[b, kh * G:(kh + 1) * G], np.repeat(ll, G), f"ring decode step {step} seq {b}")
        checked.append(step)

    check_at = set(range(0, steps, 7)) | {steps - 1, 47, 48, 49, 63, 64, 159, 160}
    _loop(lib, x, z, bias, m, W, mode, ring, n_blocks + 1, offsets, steps, check_at, v=v, on_check=on_check)
    say(f"probe ring decode mode {mode}: {len(checked)} steps checked")
    assert len(checked) == len(check_at)
