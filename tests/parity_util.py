"""Shared helpers of the GPU parity tests (tolerances, conversions, progress)."""
import sys

import numpy as np
import torch

# Tolerances (the stated parity bar):
#   fp32 inputs: per output row, max |gpu - oracle| <= 1e-5 * max |oracle row|
#   bf16 inputs with fp32 accumulation: |gpu - oracle| <= 2e-2 + 1e-2 * |oracle|
#   integer / index work: exact
F32_ROW_REL = 1e-5
BF16_ATOL, BF16_RTOL = 2e-2, 1e-2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def host(t):
    """Exact fp64 copy of a device tensor."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def check_f32_rows(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    g = got.reshape(-1, got.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    err = np.abs(g - r).max(axis=1)
    bound = F32_ROW_REL * np.maximum(np.abs(r).max(axis=1), 1e-30)
    worst = int(np.argmax(err / bound))
    assert (err <= bound).all(), f"{what}: row {worst} err {err[worst]:.3e} > {bound[worst]:.3e}"
    return float((err / bound).max())


def check_bf16(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = BF16_ATOL + BF16_RTOL * np.abs(ref)
    worst = np.unravel_index(int(np.argmax(err - bound)), err.shape)
    assert (err <= bound).all(), (f"{what}: at {worst} got {got[worst]:.6f} ref {ref[worst]:.6f} "
                                  f"(max abs err {err.max():.3e})")
    return float(err.max())


def check_scalar_f32(got, ref, what, rel=F32_ROW_REL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    assert (err <= rel * np.maximum(np.abs(ref), 1.0)).all(), f"{what}: max err {err.max():.3e}"


def check(dtype, got, ref, what):
    return check_f32_rows(got, ref, what) if dtype == "f32" else check_bf16(got, ref, what)


def topk_matches(gpu_idx, oracle_scores, k, what, margin_rel=1e-5):
    """Selection parity: the oracle's fp64 scores decide.  Where the gap between
    the k-th and (k+1)-th oracle score exceeds an fp32 error bound the sets must
    be identical; inside the band the GPU set must still be a valid top-k
    (everything it picked is >= every score it left out, up to the bound)."""
    s = np.asarray(oracle_scores, dtype=np.float64)
    n = s.shape[0]
    idx = np.asarray(gpu_idx)
    want = min(k, n)
    assert (idx[want:] == -1).all(), f"{what}: padding"
    chosen = idx[:want]
    assert (np.diff(chosen) > 0).all() and chosen.min(initial=0) >= 0 and chosen.max(initial=-1) < n, \
        f"{what}: ids not ascending / in range"
    if want == n:
        assert (chosen == np.arange(n)).all()
        return np.inf
    order = np.lexsort((np.arange(n), -s))
    ref = np.sort(order[:k])
    srt = np.sort(s)[::-1]
    bound = margin_rel * max(np.abs(s).max(), 1e-30)
    margin = srt[k - 1] - srt[k]
    if margin > bound:
        assert (chosen == ref).all(), f"{what}: set differs (margin {margin:.3e} > {bound:.3e})"
    else:
        rest = np.setdiff1d(np.arange(n), chosen)
        assert s[chosen].min() >= s[rest].max() - bound, f"{what}: invalid selection in tie band"
    return margin
