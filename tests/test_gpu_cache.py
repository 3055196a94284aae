"""GPU parity of the decode-time cache step (lbca_cache_append) and of the
fused decode step (lbca_decode_step) through the C ABI.

Each case replays a decode loop token by token over a seeded history, with
sequences that start at different steps (position < 0 = not started yet), on
a mirrored raw ring whose size is not a multiple of the block, so blocks
straddle the mirror.  Checked against what the method fixes for the state after
tokens 0..t ("mSeek: learned KV-cache compression in a 3B model", "How LBCA
works" steps 1-5):
- the ring rows of every position of the raw span of t hold that token, bit
  for bit, at row (position - raw_pos_base), and raw_pos_base follows the
  header's rule;
- every entry that became visible equals, bit for bit, what lbca_pool_blocks
  writes from the linear history (same pooling code), and the oracle's pooled
  entry within the bf16 / fp32 tolerance;
- decode through the ring equals the oracle's attention over the linear
  history.
"""
import math

import numpy as np
import pytest
import torch

from block_compressed_kv_amd import synth
from oracle import lbca_oracle as O

from parity_util import check, check_bf16, host, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _dev(d):
    return {k: v.to(DEV) for k, v in d.items()}


def _loop(lib, series, z, bias, m, W, mode, ring, entries, offsets, steps, check_at, v=None, treat=None,
          on_check=None, dual=None):
    """Append tokens 0.. of each sequence (sequence b starts at step offsets[b]); call
    on_check(step, t_list, raw_x, raw_v, raw_z, rpb, out_x, out_v) at the listed steps."""
    treat = treat or {}
    B, H, T, d = series.shape
    raw_x = torch.full((B, H, 2 * ring, d), float("nan"), dtype=series.dtype, device=DEV)
    raw_z = torch.full((B, H, 2 * ring, d), float("nan"), dtype=z.dtype, device=DEV)
    raw_v = None if v is None else torch.full_like(raw_x, float("nan"))
    out_x = torch.full((B, H, entries, d), 7.0, dtype=series.dtype, device=DEV)
    out_v = None if v is None else torch.full_like(out_x, 7.0)
    rpb = torch.full((B,), -123, dtype=torch.int64, device=DEV)
    bidx = torch.arange(B, device=DEV)
    if dual is not None:  # (xb, zb, bias_b): the b-series of dual (CSA) pooling
        xb, zb, bias_b = dual
        raw_xb, raw_zb = torch.full_like(raw_x, float("nan")), torch.full_like(raw_z, float("nan"))
        dual_kw = lambda ti: dict(xb_new=xb[bidx, :, ti], zb_new=zb[bidx, :, ti],
                                  raw_xb=raw_xb, raw_zb=raw_zb, bias_b=bias_b)
    for step in range(steps):
        t_list = [step - o for o in offsets]
        assert max(t_list) < T, "the history covers every appended position"
        pos = torch.tensor(t_list, dtype=torch.int64, device=DEV)
        ti = pos.clamp(min=0)
        x_new = series[bidx, :, ti]
        z_new = z[bidx, :, ti]
        v_new = None if v is None else v[bidx, :, ti]
        lib.cache_append(x_new, z_new, raw_x, raw_z, bias, pos, rpb, m, W, mode, out_x, v_new=v_new,
                         raw_v=raw_v, out_v=out_v, **treat, **(dual_kw(ti) if dual is not None else {}))
        if step in check_at:
            torch.cuda.synchronize()
            on_check(step, t_list, raw_x, raw_v, raw_z, rpb, out_x, out_v)
    if dual is not None:
        torch.cuda.synchronize()
        _check_ring([steps - 1 - o for o in offsets], m, W, mode, ring, raw_xb, raw_zb, rpb, xb, zb)
    return raw_x, raw_v, raw_z, rpb, out_x, out_v


def _check_ring(t_list, m, W, mode, ring, raw_x, raw_z, rpb, series, z, raw_v=None, v=None):
    base = host(rpb).astype(np.int64)
    for b, t in enumerate(t_list):
        if t < 0:
            assert base[b] == -123, "a sequence that has not started keeps its raw base"
            continue
        _, rb = O.visible_range(t, m, W, mode)
        assert base[b] == rb - rb % ring, (b, t, base[b], rb)
        rows = torch.arange(rb, t + 1, device=DEV) - int(base[b])
        assert int(rows.min()) >= 0 and int(rows.max()) < 2 * ring
        assert torch.equal(raw_x[b][:, rows], series[b][:, rb:t + 1]), f"ring x, sequence {b}"
        assert torch.equal(raw_z[b][:, rows], z[b][:, rb:t + 1]), f"ring z, sequence {b}"
        if v is not None:
            assert torch.equal(raw_v[b][:, rows], v[b][:, rb:t + 1]), f"ring v, sequence {b}"
        # the mirror: both rows of each of the last `ring` positions hold the token
        lo = max(0, t - ring + 1)
        slots = torch.arange(lo, t + 1, device=DEV) % ring
        assert torch.equal(raw_x[b][:, slots], raw_x[b][:, slots + ring])


@pytest.mark.parametrize("xdt,zdt,d", [("bf16", "f32", 128), ("f32", "f32", 64)])
def test_cache_exclusive_gqa(lib, xdt, zdt, d):
    # LBCA rule, separate K and V, 2 KV heads x 3 query heads each, ragged starts
    H, Hq, m, W, ring, T = 2, 6, 16, 32, 56, 420
    offsets = [0, 37, 101]
    B = len(offsets)
    L = _dev(synth.lbca_layer(f"cache-excl-{xdt}-{d}", B, Hq, H, T, d, m, xdt, zdt))
    k, v, z, bias = L["k"], L["v"], L["z"], L["bias"]
    entries = T // m + 2
    steps = 400                       # sequence 0 ends at t = 399, within its history
    q = synth.normal((B, Hq, d), synth.seed_of("cache-excl-q", xdt, d), dtype=xdt, device=DEV)
    checked = []

    def on_check(step, t_list, raw_x, raw_v, raw_z, rpb, out_x, out_v):
        _check_ring(t_list, m, W, O.EXCLUSIVE, ring, raw_x, raw_z, rpb, k, z, raw_v, v)
        pos = torch.tensor(t_list, dtype=torch.int64, device=DEV)
        o, lse = lib.attend_decode(q, out_x, raw_x, pos, m, W, O.EXCLUSIVE, pooled_v=out_v, raw_v=raw_v,
                                   raw_pos_base=rpb)
        live = [b for b, t in enumerate(t_list) if t >= 0]
        n_max = max(O.visible_range(t_list[b], m, W, O.EXCLUSIVE)[0] for b in live)
        rk, rv = O.pool_single(host(k), host(z), host(bias), m, 0, max(n_max, 1), values=host(v))
        ro, rl = O.attend_decode(host(q)[live], rk[live], rv[live], host(k)[live], host(v)[live],
                                 [t_list[b] for b in live], m, W, O.EXCLUSIVE, 1 / math.sqrt(d))
        check(xdt, host(o)[live], ro, f"decode through the ring at step {step}")
        check(xdt, host(lse)[live][..., None], rl[..., None], "lse")
        checked.append(step)

    check_at = {0, 1, 47, 48, 63, 64, 65, 130, 200, 311, 312, steps - 1}
    say(f"cache EXCLUSIVE {xdt}/{zdt} d={d}: {steps} steps")
    raw_x, raw_v, raw_z, rpb, out_x, out_v = _loop(lib, k, z, bias, m, W, O.EXCLUSIVE, ring, entries, offsets,
                                                   steps, check_at, v=v, on_check=on_check)
    assert len(checked) == len(check_at)
    # every entry that became visible: bitwise the linear-history pooling, and the oracle's
    t_end = [steps - 1 - o for o in offsets]
    ref_x = torch.full_like(out_x, 7.0)
    ref_v = torch.full_like(out_v, 7.0)
    lib.pool_blocks(k, z, bias, m, 0, T // m, ref_x, v=v, out_v=ref_v)
    rk, rv = O.pool_single(host(k), host(z), host(bias), m, 0, T // m, values=host(v))
    for b, t in enumerate(t_end):
        n_p, _ = O.visible_range(t, m, W, O.EXCLUSIVE)
        assert torch.equal(out_x[b, :, :n_p], ref_x[b, :, :n_p]) and torch.equal(out_v[b, :, :n_p], ref_v[b, :, :n_p])
        assert (out_x[b, :, n_p:] == 7.0).all(), "entries not yet visible are untouched"
        check(xdt, host(out_x[b, :, :n_p]), rk[b, :, :n_p], f"entries of sequence {b}")
        check(xdt, host(out_v[b, :, :n_p]), rv[b, :, :n_p], f"value entries of sequence {b}")


@pytest.mark.parametrize("Hq", [16, 32])
def test_cache_overlap_hca_treated(lib, Hq):
    # HCA rule: shared 512-dim series, RMSNorm + RoPE on entries, sink; the due block ends
    # with the token appended in the same call; 32 heads take the wide decode path
    B, d, m, W, ring, T = 2, 512, 8, 16, 20, 170
    offsets = [0, 13]
    H = _dev(synth.hca_layer(f"cache-hca-{Hq}", B, Hq, T, d, m))
    c, z, bias, q, sink = H["c"], H["z"], H["bias"], H["q"], H["sink"]
    treat = dict(rmsnorm_eps=1e-6, rope_dims=64)
    entries = T // m + 1
    steps = 160
    checked = []

    def on_check(step, t_list, raw_x, raw_v, raw_z, rpb, out_x, out_v):
        _check_ring(t_list, m, W, O.OVERLAP, ring, raw_x, raw_z, rpb, c, z)
        pos = torch.tensor(t_list, dtype=torch.int64, device=DEV)
        o, lse = lib.attend_decode(q, out_x, raw_x, pos, m, W, O.OVERLAP, raw_pos_base=rpb, sink=sink, **treat)
        live = [b for b, t in enumerate(t_list) if t >= 0]
        n_max = max(O.visible_range(t_list[b], m, W, O.OVERLAP)[0] for b in live)
        pooled = O.pool_single(host(c), host(z), host(bias), m, 0, max(n_max, 1))
        ro, rl = O.attend_decode(host(q)[live], pooled[live], None, host(c)[live], None,
                                 [t_list[b] for b in live], m, W, O.OVERLAP, 1 / math.sqrt(d),
                                 sink=host(sink), **treat)
        check_bf16(host(o)[live], ro, f"treated decode through the ring at step {step}")
        check_bf16(host(lse)[live], rl, "lse")
        checked.append(step)

    check_at = {0, 7, 8, 19, 20, 21, 40, 99, steps - 1}
    say(f"cache OVERLAP HCA Hq={Hq}: {steps} steps")
    raw_x, _, raw_z, rpb, out_x, _ = _loop(lib, c, z, bias, m, W, O.OVERLAP, ring, entries, offsets, steps,
                                           check_at, treat=treat, on_check=on_check)
    assert len(checked) == len(check_at)
    ref = torch.full_like(out_x, 7.0)
    lib.pool_blocks(c, z, bias, m, 0, T // m, ref, **treat)
    pooled = O.pool_single(host(c), host(z), host(bias), m, 0, T // m)
    treated = O.rope(O.rmsnorm(pooled, 1e-6), (np.arange(T // m) * m)[None, None], 64, 10000.0)
    for b, o in enumerate(offsets):
        n_p, _ = O.visible_range(steps - 1 - o, m, W, O.OVERLAP)
        assert torch.equal(out_x[b, :, :n_p], ref[b, :, :n_p]), f"entries of sequence {b}"
        check_bf16(host(out_x[b, :, :n_p]), treated[b, :, :n_p], f"treated entries of sequence {b}")


def test_cache_due_entry_past_capacity(lib):
    # entries beyond the pooled buffer are not written (pooling skipped) while the ring
    # and the raw base still advance; decode then reports such a sequence as not fitting
    H, d, m, W, ring, T = 1, 64, 8, 16, 24, 120
    offsets = [0, 60]
    B = len(offsets)
    L = _dev(synth.lbca_layer("cache-cap", B, 2, H, T, d, m, "bf16", "f32"))
    k, v, z, bias = L["k"], L["v"], L["z"], L["bias"]
    entries = 6                       # blocks 0..5 fit; sequence 0 makes blocks up to 11 visible
    steps = 119
    raw_x, raw_v, raw_z, rpb, out_x, out_v = _loop(lib, k, z, bias, m, W, O.EXCLUSIVE, ring, entries, offsets,
                                                   steps, set(), v=v)
    torch.cuda.synchronize()
    t_end = [steps - 1 - o for o in offsets]
    _check_ring(t_end, m, W, O.EXCLUSIVE, ring, raw_x, raw_z, rpb, k, z, raw_v, v)
    ref_x = torch.full_like(out_x, 7.0)
    ref_v = torch.full_like(out_v, 7.0)
    lib.pool_blocks(k, z, bias, m, 0, entries, ref_x, v=v, out_v=ref_v)
    for b, t in enumerate(t_end):
        n = min(O.visible_range(t, m, W, O.EXCLUSIVE)[0], entries)
        assert torch.equal(out_x[b, :, :n], ref_x[b, :, :n]) and torch.equal(out_v[b, :, :n], ref_v[b, :, :n])
        assert (out_x[b, :, n:] == 7.0).all()
    q = synth.normal((B, 2, d), 5, dtype="bf16", device=DEV)
    pos = torch.tensor(t_end, dtype=torch.int64, device=DEV)
    o, lse = lib.attend_decode(q, out_x, raw_x, pos, m, W, O.EXCLUSIVE, pooled_v=out_v, raw_v=raw_v,
                               raw_pos_base=rpb)
    n_p = [O.visible_range(t, m, W, O.EXCLUSIVE)[0] for t in t_end]
    assert n_p[0] > entries and n_p[1] <= entries
    assert torch.isnan(o[0]).all() and torch.isfinite(o[1]).all()


def test_cache_overlap_csa_dual(lib):
    # CSA: dual overlapped pooling (block j of the a-series with block j-1 of the b-series
    # under one softmax), treated 512-dim entries, 4-token blocks, ring of 2m..W slots;
    # 64 heads take the wide decode path
    B, Hq, d, m, W, ring, T = 2, 64, 512, 4, 16, 20, 120
    offsets = [0, 9]
    C = _dev(synth.csa_layer("cache-csa", B, Hq, T, d, m, 8, 64))
    treat = dict(rmsnorm_eps=1e-6, rope_dims=64)
    entries = T // m
    steps = 110
    say(f"cache OVERLAP CSA dual: {steps} steps")
    raw_x, _, raw_z, rpb, out_x, _ = _loop(lib, C["ca"], C["za"], C["bias_a"], m, W, O.OVERLAP, ring, entries,
                                           offsets, steps, set(), treat=treat,
                                           dual=(C["cb"], C["zb"], C["bias_b"]))
    t_end = [steps - 1 - o for o in offsets]
    _check_ring(t_end, m, W, O.OVERLAP, ring, raw_x, raw_z, rpb, C["ca"], C["za"])
    ref = torch.full_like(out_x, 7.0)
    lib.pool_blocks(C["ca"], C["za"], C["bias_a"], m, 0, entries, ref, xb=C["cb"], zb=C["zb"], bias_b=C["bias_b"],
                    **treat)
    pooled = O.pool_dual(host(C["ca"]), host(C["za"]), host(C["bias_a"][0]), host(C["cb"]), host(C["zb"]),
                         host(C["bias_b"][0]), m, 0, entries)
    treated = O.rope(O.rmsnorm(pooled, 1e-6), (np.arange(entries) * m)[None, None], 64, 10000.0)
    for b, t in enumerate(t_end):
        n_p, _ = O.visible_range(t, m, W, O.OVERLAP)
        assert torch.equal(out_x[b, :, :n_p], ref[b, :, :n_p]), f"entries of sequence {b}"
        assert (out_x[b, :, n_p:] == 7.0).all()
        check_bf16(host(out_x[b, :, :n_p]), treated[b, :, :n_p], f"treated dual entries of sequence {b}")
    pos = torch.tensor(t_end, dtype=torch.int64, device=DEV)
    o, lse = lib.attend_decode(C["q"], out_x, raw_x, pos, m, W, O.OVERLAP, raw_pos_base=rpb, sink=C["sink"], **treat)
    ro, rl = O.attend_decode(host(C["q"]), pooled, None, host(C["ca"]), None, t_end, m, W, O.OVERLAP,
                             1 / math.sqrt(d), sink=host(C["sink"]), **treat)
    check_bf16(host(o), ro, "decode over dual entries through the ring")
    check_bf16(host(lse), rl, "lse")


# ---------------------------------------------------------------------------
# the fused step: append, pool on completion and decode in one launch
# ---------------------------------------------------------------------------
def _step_state(B, H, ring, entries, d, xdt, zdt):
    nanx = lambda: torch.full((B, H, 2 * ring, d), float("nan"), dtype=xdt, device=DEV)
    st = dict(rk=nanx(), rv=nanx(), rz=torch.full((B, H, 2 * ring, d), float("nan"), dtype=zdt, device=DEV),
              pk=torch.full((B, H, entries, d), 7.0, dtype=xdt, device=DEV),
              rpb=torch.full((B,), -123, dtype=torch.int64, device=DEV))
    st["pv"] = torch.full_like(st["pk"], 7.0)
    return st


def _run_steps(lib, L, qs, offsets, m, W, first_step, steps, fused, plain, check_at=(), on_check=None):
    """Advance both states over the given steps: fused by lbca_decode_step, plain by
    lbca_cache_append + lbca_attend_decode; the live sequences' outputs must be bitwise equal."""
    k, v, z, bias = L["k"], L["v"], L["z"], L["bias"]
    B = k.shape[0]
    bidx = torch.arange(B, device=DEV)
    for step in range(first_step, first_step + steps):
        t_list = [step - o for o in offsets]
        pos = torch.tensor(t_list, dtype=torch.int64, device=DEV)
        ti = pos.clamp(min=0)
        k_new, v_new, z_new = (x[bidx, :, ti] for x in (k, v, z))
        q = qs[step % qs.shape[0]]
        of, lf = lib.decode_step(q, k_new, v_new, z_new, fused["rk"], fused["rv"], fused["rz"], bias, fused["pk"],
                                 fused["pv"], pos, fused["rpb"], m, W)
        lib.cache_append(k_new, z_new, plain["rk"], plain["rz"], bias, pos, plain["rpb"], m, W, O.EXCLUSIVE,
                         plain["pk"], v_new=v_new, raw_v=plain["rv"], out_v=plain["pv"])
        ou, lu = lib.attend_decode(q, plain["pk"], plain["rk"], pos, m, W, O.EXCLUSIVE, pooled_v=plain["pv"],
                                   raw_v=plain["rv"], raw_pos_base=plain["rpb"])
        live = [b for b, t in enumerate(t_list) if t >= 0]
        assert torch.equal(of[live], ou[live]) and torch.equal(lf[live], lu[live]), f"fused step {step} differs"
        assert torch.equal(fused["rpb"][live], plain["rpb"][live]), "raw base"
        if step in check_at:
            torch.cuda.synchronize()
            on_check(step, t_list, q, of, lf)
    return [first_step + steps - 1 - o for o in offsets]


def _decode_vs_oracle(L, m, W, d, xdt):
    k, v, z, bias = (host(L[n]) for n in ("k", "v", "z", "bias"))

    def on_check(step, t_list, q, o, lse):
        live = [b for b, t in enumerate(t_list) if t >= 0]
        n_max = max(O.visible_range(t_list[b], m, W, O.EXCLUSIVE)[0] for b in live)
        rk, rv = O.pool_single(k, z, bias, m, 0, max(n_max, 1), values=v)
        ro, rl = O.attend_decode(host(q)[live], rk[live], rv[live], k[live], v[live], [t_list[b] for b in live], m,
                                 W, O.EXCLUSIVE, 1 / math.sqrt(d))
        check(xdt, host(o)[live], ro, f"fused decode step {step}")
        check(xdt, host(lse)[live][..., None], rl[..., None], "lse")
    return on_check


@pytest.mark.parametrize("zdt,d,Hq", [("f32", 128, 6), ("bf16", 64, 4)])
def test_decode_step_fused(lib, zdt, d, Hq):
    # lbca_decode_step token by token from the start, ragged starts, ring not a
    # multiple of the block: every step bitwise equal to the separate cache step +
    # decode, decode against the oracle at the listed steps, the ring rows as the
    # rule places them, and every block completed so far pooled bitwise as
    # lbca_pool_blocks writes it from the linear history (later entries untouched)
    H, m, W, ring, T = 2, 16, 32, 56, 420
    offsets = [0, 37, 101]
    B = len(offsets)
    L = _dev(synth.lbca_layer(f"step-{zdt}-{d}", B, Hq, H, T, d, m, "bf16", zdt))
    entries = T // m + 2
    steps = 400
    qs = synth.normal((steps, B, Hq, d), synth.seed_of("step-q", zdt, d), dtype="bf16", device=DEV)
    xdt, zt = torch.bfloat16, L["z"].dtype
    fused, plain = _step_state(B, H, ring, entries, d, xdt, zt), _step_state(B, H, ring, entries, d, xdt, zt)
    check_at = {0, 1, 15, 16, 47, 48, 63, 64, 65, 130, 311, 312, steps - 1}
    say(f"fused decode step bf16/{zdt} d={d}: {steps} steps")
    t_end = _run_steps(lib, L, qs, offsets, m, W, 0, steps, fused, plain, check_at, _decode_vs_oracle(L, m, W, d, "bf16"))
    torch.cuda.synchronize()
    _check_ring(t_end, m, W, O.EXCLUSIVE, ring, fused["rk"], fused["rz"], fused["rpb"], L["k"], L["z"], fused["rv"],
                L["v"])
    ref_k = torch.full_like(fused["pk"], 7.0)
    ref_v = torch.full_like(fused["pv"], 7.0)
    lib.pool_blocks(L["k"], L["z"], L["bias"], m, 0, T // m, ref_k, v=L["v"], out_v=ref_v)
    for b, t in enumerate(t_end):
        done = (t + 1) // m                    # blocks completed by t
        assert torch.equal(fused["pk"][b, :, :done], ref_k[b, :, :done])
        assert torch.equal(fused["pv"][b, :, :done], ref_v[b, :, :done])
        assert (fused["pk"][b, :, done:] == 7.0).all(), "blocks not completed yet are untouched"


def test_decode_step_split_rows(lib):
    # decode at t ~ 20000 (1250 pooled blocks): the rows are split across
    # workgroups, so the step is the fused launch plus the merge; state set up as
    # a prefill would leave it (every completed block pooled, the ring filled)
    B, Hq, H, d, m, W, ring, t0, steps = 1, 6, 2, 128, 16, 128, 160, 20000, 40
    T = t0 + steps
    L = _dev(synth.lbca_layer("step-split", B, Hq, H, T, d, m, "bf16", "f32"))
    entries = T // m + 1
    qs = synth.normal((4, B, Hq, d), synth.seed_of("step-split-q"), dtype="bf16", device=DEV)
    xdt, zt = torch.bfloat16, torch.float32
    states = []
    for _ in range(2):
        st = _step_state(B, H, ring, entries, d, xdt, zt)
        lib.pool_blocks(L["k"], L["z"], L["bias"], m, 0, t0 // m, st["pk"], v=L["v"], out_v=st["pv"])
        s = torch.arange(t0 - ring + 1, t0, device=DEV)
        for key, src in (("rk", "k"), ("rv", "v"), ("rz", "z")):
            st[key][:, :, s % ring] = L[src][:, :, s]
            st[key][:, :, s % ring + ring] = L[src][:, :, s]
        states.append(st)
    say(f"fused decode step with split rows: t from {t0}, {steps} steps")
    _run_steps(lib, L, qs, [0], m, W, t0, steps, states[0], states[1], {t0, t0 + 1, t0 + 15, t0 + steps - 1},
               _decode_vs_oracle(L, m, W, d, "bf16"))
