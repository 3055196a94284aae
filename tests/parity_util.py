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


def index_score_bound(qi, w, ki, n_visible):
    """A rigorous bound on |fp32 score - exact score| for each visible key, for any
    summation order: the dot product of dI terms, the ReLU (exact), the weight
    multiply and the sum over HI heads accumulate at most (dI + HI + 2) unit
    roundings of the absolute terms, so |error_j| <= gamma * sum_h w_h sum_i
    |q_hi k_ji| with gamma = n u / (1 - n u), n = dI + HI + 2, u = 2^-24; doubled
    for margin (MFMA accumulation order and internal width are unspecified)."""
    qi, w, ki = (x.double().numpy() if isinstance(x, torch.Tensor) else np.asarray(x, dtype=np.float64)
                 for x in (qi, w, ki))
    n = qi.shape[-1] + qi.shape[0] + 2
    u = 2.0 ** -24
    gamma = n * u / (1 - n * u)
    return 2 * gamma * ((np.abs(ki[:n_visible]) @ np.abs(qi).T) @ np.abs(w))


def index_ws_scores(ws, batch, entries):
    """The fp32 indexer scores csa_index_topk leaves at the head of its workspace:
    ``batch`` rows of ``entries`` scores, each row padded to a multiple of 4
    (16-byte rows).  Read after the call, on the host."""
    stride = (entries + 3) & ~3
    return ws[:batch * stride * 4].view(torch.float32).view(batch, stride)[:, :entries].cpu().numpy()


def topk_matches(gpu_idx, oracle_scores, k, what, err, allow_band=False, gpu_scores=None):
    """Selection parity against the oracle's fp64 scores.  err[j] bounds the fp32
    error of score j (``index_score_bound``).  Where the k-th and (k+1)-th oracle
    scores differ by more than their two bounds the GPU set must be the oracle's
    set exactly.  Otherwise the row lies in the fp32 tie band, where the exact
    set is not decidable from fp32 scores.  With ``gpu_scores`` (the kernel's own
    fp32 scores of the visible entries) the selection is pinned exactly anyway:
    every GPU score lies within its bound of the oracle's, and the GPU set is
    exactly the top-k of those fp32 scores (ties to the lower index), band or
    not.  Without them a band row fails unless ``allow_band`` (tests over
    thousands of query rows, where some rows land there), which reports it
    (returned band flag) and still requires a top-k of some scores within the
    bounds: every chosen entry's upper bound reaches every other entry's lower
    bound.  Returns (margin, in_band)."""
    s = np.asarray(oracle_scores, dtype=np.float64)
    e = np.asarray(err, dtype=np.float64)
    n = s.shape[0]
    idx = np.asarray(gpu_idx)
    want = min(k, n)
    assert (idx[want:] == -1).all(), f"{what}: padding"
    chosen = idx[:want]
    assert (np.diff(chosen) > 0).all() and chosen.min(initial=0) >= 0 and chosen.max(initial=-1) < n, \
        f"{what}: ids not ascending / in range"
    if want == n:
        assert (chosen == np.arange(n)).all(), f"{what}: every visible entry must be selected"
        return np.inf, False
    order = np.lexsort((np.arange(n), -s))
    ref = np.sort(order[:k])
    a, b = order[k - 1], order[k]
    margin = s[a] - s[b]
    if gpu_scores is not None:
        g = np.asarray(gpu_scores, dtype=np.float32).astype(np.float64)
        assert g.shape == (n,), f"{what}: {g.shape} GPU scores for {n} visible entries"
        bad = np.abs(g - s) > e
        assert not bad.any(), f"{what}: {bad.sum()} GPU scores outside their fp32 bound of the oracle's"
        own = np.sort(np.lexsort((np.arange(n), -g))[:k])
        assert (chosen == own).all(), f"{what}: set is not the top-k of the kernel's own fp32 scores"
        return margin, bool(margin <= e[a] + e[b])
    if margin > e[a] + e[b]:
        assert (chosen == ref).all(), f"{what}: set differs outside the fp32 band (margin {margin:.3e})"
        return margin, False
    assert allow_band, (f"{what}: the seeded case lands in the fp32 tie band (margin {margin:.3e} within "
                        f"the bounds {e[a] + e[b]:.3e}); choose another seed")
    # some fp32 rounding within the bounds ranks every chosen entry at or above every other
    rest = np.setdiff1d(np.arange(n), chosen)
    assert (s[chosen] + e[chosen]).min() >= (s[rest] - e[rest]).max(), \
        f"{what}: not a top-k of any scores within the fp32 bounds"
    return margin, True
