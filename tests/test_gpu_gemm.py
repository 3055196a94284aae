"""GPU parity of the grouped projection GEMM (lbca_grouped_gemm) and the two
projections built on it, against the oracle (oracle.lbca_oracle:
grouped_projection, indexer_queries, output_projection), through the C ABI.

Reading: an fp32 input A is rounded to bf16 (nearest even) before the
contraction, so the oracle gets the rounded values; what remains is fp32
accumulation against fp64, bounded per output by 2e-5 * sum_l |a_l w_l| (plus
half a bf16 unit of the result when C is stored in bf16)."""
import numpy as np
import pytest
import torch

from block_compressed_kv_amd import synth
from oracle import lbca_oracle as O

from parity_util import host, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _check(got, a_used, w, ref, c_bf16, what):
    mag = O.grouped_projection(np.abs(a_used), np.abs(w))
    bound = 2e-5 * mag + 1e-30 + (2.0 ** -8 * np.abs(ref) if c_bf16 else 0.0)
    err = np.abs(got - ref)
    bad = np.argwhere(~(err <= bound))
    assert bad.size == 0, f"{what}: {len(bad)} off, first {tuple(bad[0])} got {got[tuple(bad[0])]} ref {ref[tuple(bad[0])]}"
    return float((err / np.maximum(bound, 1e-30)).max())


@pytest.mark.parametrize("G,M,N,K,a_dt,c_dt", [
    (1, 300, 200, 512, "bf16", "f32"),      # ragged row and column tiles
    (3, 129, 130, 200, "f32", "bf16"),      # K tail (200 = 3 x 64 + 8), fp32 A rounded on load
    (2, 1, 257, 64, "bf16", "bf16"),        # one row
    (4, 513, 96, 1024, "f32", "f32"),
    (2, 70, 140, 136, "bf16", "f32"),       # bf16 K tail (136 = 2 x 64 + 8)
    (1, 65, 64, 40, "bf16", "bf16"),        # K below one step: the only step is the tail
])
def test_grouped_gemm(lib, G, M, N, K, a_dt, c_dt):
    say(f"grouped gemm G={G} M={M} N={N} K={K} a={a_dt} c={c_dt}")
    a = synth.normal((M, G * K), synth.seed_of("gemm", G, M, N, K, "a"), dtype=a_dt, device=DEV)
    w = synth.normal((G, N, K), synth.seed_of("gemm", G, M, N, K, "w"), dtype="bf16", device=DEV)
    out = lib.grouped_gemm(a, w, groups=G, out_dtype=torch.float32 if c_dt == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    a_used = host(a.to(torch.bfloat16))
    ref = O.grouped_projection(a_used, host(w))
    r = _check(host(out), a_used, host(w), ref, c_dt == "bf16", "grouped gemm")
    say(f"  worst error / bound {r:.3f}")
    # bitwise reproducible
    out2 = lib.grouped_gemm(a, w, groups=G, out_dtype=out.dtype)
    assert torch.equal(out, out2)


def test_grouped_gemm_strided_views(lib):
    # A read through a column slice of a wider buffer (lda > K per group), C written into a
    # wider buffer: through the raw C ABI with explicit strides
    import ctypes
    M, N, K, G = 200, 160, 128, 2
    big = synth.normal((M, 3 * G * K), synth.seed_of("gemm-strided", "a"), dtype="bf16", device=DEV)
    w = synth.normal((G, N, K), synth.seed_of("gemm-strided", "w"), dtype="bf16", device=DEV)
    cbuf = torch.full((M, 2 * G * N + 4), 7.0, device=DEV)
    off = G * K  # A starts at column G*K of each row
    args = lib.GemmArgs(big.data_ptr() + off * 2, w.data_ptr(), cbuf.data_ptr() + 4 * 4, G, M, N, K, 3 * G * K, K,
                        2 * G * N + 4, K, N * K, N, lib.BF16, lib.F32)
    assert lib.lib().lbca_grouped_gemm(ctypes.byref(args), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    torch.cuda.synchronize()
    a_used = host(big[:, off:off + G * K])
    ref = O.grouped_projection(a_used, host(w))
    _check(host(cbuf[:, 4:4 + G * N]), a_used, host(w), ref, False, "strided gemm")
    assert (cbuf[:, :4] == 7.0).all() and (cbuf[:, 4 + G * N:] == 7.0).all(), "outside C untouched"


def test_projections_csa_shapes(lib):
    # the paper dims: 64 query heads x 512 dims, query latent d_c = 1024, 8 x 64 indexer heads;
    # grouped output projection in 8 groups of 8 heads to 1024 each, then to a 4096-wide model
    T, H, c, dc, HI, dI, g, dg, dm = 512, 64, 512, 1024, 8, 64, 8, 1024, 4096
    seed = lambda n: synth.seed_of("proj-csa", n)
    cq = synth.normal((T, dc), seed("cq"), dtype="bf16", device=DEV)
    wuq = synth.normal((HI * dI, dc), seed("wuq"), std=dc ** -0.5, dtype="bf16", device=DEV)
    o = synth.normal((T, H, c), seed("o"), device=DEV)                   # attention output, fp32
    wg = synth.normal((g, dg, H // g * c), seed("wg"), std=(H // g * c) ** -0.5, dtype="bf16", device=DEV)
    wo = synth.normal((dm, g * dg), seed("wo"), std=(g * dg) ** -0.5, dtype="bf16", device=DEV)
    qi = lib.indexer_queries(cq, wuq, HI)
    y = lib.output_projection(o, wg, wo)
    torch.cuda.synchronize()
    assert qi.shape == (T, HI, dI) and y.shape == (T, dm)
    rq = O.indexer_queries(host(cq), host(wuq), HI)
    _check(host(qi).reshape(T, -1), host(cq), host(wuq)[None], rq.reshape(T, -1), True, "indexer queries")
    # output projection on sampled tokens: stage 1 then stage 2 as the kernel rounds them
    rows = [0, 1, 255, 511]
    o_used = host(o.to(torch.bfloat16))[rows].reshape(len(rows), -1)
    mid = O.grouped_projection(o_used, host(wg))
    mid_bf = host(torch.as_tensor(mid, dtype=torch.float32).to(torch.bfloat16))   # stage 1 stores bf16
    ref = O.grouped_projection(mid_bf, host(wo)[None])
    _check(host(y)[rows], mid_bf, host(wo)[None], ref, False, "output projection")
    # stage 1 itself within its bound
    mid_gpu = lib.grouped_gemm(o.reshape(T, -1), wg, groups=g)
    _check(host(mid_gpu)[rows], o_used, host(wg), mid, True, "output projection stage 1")
    # pooling logits of CSA's two series (Z^a, Z^b: 512 channels each) from the hidden state
    h = synth.normal((T, dm), seed("h"), dtype="bf16", device=DEV)
    wz = synth.normal((2 * c, dm), seed("wz"), std=dm ** -0.5, dtype="bf16", device=DEV)
    z = lib.pooling_logits(h, wz, c)
    torch.cuda.synchronize()
    assert z.shape == (T, 2, c) and z.dtype == torch.float32
    rz = O.pooling_logits(host(h), host(wz), c)
    _check(host(z).reshape(T, -1), host(h), host(wz)[None], rz.reshape(T, -1), False, "pooling logits")
