"""Benchmark: LBCA decode at 32K context on one MI355X (plus pooling and prefill lines).

Headline workload: Llama-3.2-3B-shaped LBCA layers (24 query heads over 8 KV
heads, head dim 128, bf16 K/V/Q, fp32 pooling logits, 64-token blocks, 128-token
raw window), 14 layers with independent seeded inputs, batch 16, one decode
step at position t = 32767: per layer, decode attention over 510 pooled
entries + 128 raw tokens per KV head.  ``value`` = decode layer-steps per
second (one lbca_attend_decode launch per layer-step).

Inputs are resident in HBM before timing.  Each layer keeps what a decode step
touches (pooled cache, the last 192 raw tokens, the due block's logits); the
14 layers together (590 MB at batch 16) exceed the 256 MB Infinity Cache, so
every step streams from HBM.  The 14 launches are captured once as a HIP graph
and replayed; HIP events on the launch stream bracket the timed region.

Also reported: the decode launch's HBM roofline fraction (and its HBM traffic
from stored counter passes), the oracle on the host cores (cpu_baseline), batch
1 and 4, the step with the due block pooled first (a block leaves the window
every 64 steps), an incremental decode loop (64 steps of lbca_cache_append into a
mirrored raw ring, the due block pooled on its step, then decode from the ring),
the pooling gradients of one layer's history (GB/s),
pooling GB/s for the whole history, chunked prefill (16K
context in 2048-token chunks) TFLOP/s, HCA decode at 1M context (batch 4, 64
query heads x 512, pooling GB/s of the whole history) and CSA at 128K (batch 2:
indexer scores + top-512, decode over the selection, dual pooling GB/s, its
treated dual pooling gradients, and the sparse prefill of a 2048-query chunk per
sequence: chunk indexer, per-query top-512 and selected attention); the
measured ceilings of the part (streaming read, one launch reading the decode's
bytes, a bf16 MFMA loop, the empty-kernel launch floor) with each kernel's
fraction of them; and the oracle timed beside prefill, HCA and CSA on bounded
samples.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
    python bench.py --counters    # only what the FETCH_SIZE / WRITE_SIZE passes profile
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time
import types

import torch

from block_compressed_kv_amd import lbca, synth

METRIC = "LBCA decode layer-steps/s + achieved HBM GB/s at 32K ctx; prefill TFLOP/s"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
EXCL, OVER = lbca.EXCLUSIVE, lbca.OVERLAP


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def ev():
    return torch.cuda.Event(enable_timing=True)


# ---------------------------------------------------------------------------
# 32K decode layers
# ---------------------------------------------------------------------------
CTX, HQ, HKV, D, M, W, LAYERS = 32768, 24, 8, 128, 64, 128, 14
T_POS = CTX - 1                        # query position
N_POOLED = 510                         # visible pooled entries at T_POS
RAW0 = 509 * M                         # first token kept raw: block 509 (due) + window
RAW_ROWS = CTX - RAW0                  # 192


# HBM traffic of the batch-16 decode launch, from two rocprofv3 --pmc passes over
# `python bench.py --counters` (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch, median over the
# decode dispatches).  Each counter is scaled by what it reads for the 256 MiB device-to-device
# copy in the same run (FETCH_SIZE reports half the bytes a copy reads, WRITE_SIZE all it
# writes).  The figure holds only for the decode source it was taken on: when the hash of
# decode.hip + decode_common.h differs, bench reports traffic as null.
COUNTERS = {"fetch_kib": 20576.09375, "write_kib": 197.0,
            "copy_fetch_kib": 131083.5, "copy_write_kib": 262144.0, "copy_bytes": 256 << 20,
            "source_sha256": "9e873176720507b068ec0b39428f13e1d11f61f658d4a7ff5be3bbcc8e9cc51b"}
COUNTER_SOURCES = ("decode.hip", "decode_common.h")


def decode_source_sha256():
    import hashlib
    h = hashlib.sha256()
    base = os.path.join(os.path.dirname(os.path.abspath(__file__)), "block_compressed_kv_amd", "csrc")
    for f in COUNTER_SOURCES:
        with open(os.path.join(base, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic_bytes():
    """HBM bytes per decode launch from the stored counter passes, or None if the source moved."""
    c = COUNTERS
    if c["source_sha256"] != decode_source_sha256():
        return None
    fetch = c["fetch_kib"] * c["copy_bytes"] / (c["copy_fetch_kib"] * 1024.0)
    write = c["write_kib"] * c["copy_bytes"] / (c["copy_write_kib"] * 1024.0)
    return (fetch + write) * 1024.0


def counter_pass():
    """What the --pmc passes profile: a 256 MiB copy (the counters' scale) and 3 decode steps."""
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    B = 16
    pos = torch.full((B,), T_POS, dtype=torch.int64, device="cuda")
    rpb = torch.full((B,), RAW0, dtype=torch.int64, device="cuda")
    layers = [DecodeLayer(l, B, pos, rpb) for l in range(LAYERS)]
    torch.cuda.synchronize()
    for _ in range(3):
        for L in layers:
            L.decode()
    torch.cuda.synchronize()
    log(f"[bench] counter pass: 3 copies of {n} B, {3 * LAYERS} decode launches at batch {B}")


def decode_bytes_per_seq_layer():
    # K and V of every visible row (pooled + raw window) in bf16, q in bf16, out in fp32
    n_rows = N_POOLED + (T_POS - (N_POOLED * M) + 1)
    return n_rows * HKV * D * 2 * 2 + HQ * D * 2 + HQ * D * 4


class DecodeLayer:
    def __init__(self, layer, B, pos, rpb, pool_timer=None):
        tag = ("bench-32k", layer, B)
        dev = "cuda"
        full = synth.lbca_layer(tag, B, HQ, HKV, CTX, D, M, "bf16", "f32", device=dev)
        self.bias = full["bias"]
        self.pk = torch.empty((B, HKV, N_POOLED, D), dtype=torch.bfloat16, device=dev)
        self.pv = torch.empty_like(self.pk)
        # prefill-time pooling of blocks 0..508 from the whole history (timed as pooling GB/s)
        e0, e1 = ev(), ev()
        e0.record()
        lbca.pool_blocks(full["k"], full["z"], self.bias, M, 0, N_POOLED - 1, self.pk, v=full["v"],
                         out_v=self.pv)
        e1.record()
        if pool_timer is not None:
            pool_timer.append((e0, e1, B * HKV * (N_POOLED - 1) * M * D * (2 + 2 + 4)))
        # the raw window in buffers of its own, as a serving cache holds it (the
        # ring of lbca_cache_append): views into the 32K history would scatter
        # each (sequence, head)'s rows 8 MB apart
        self.rk = full["k"][:, :, RAW0:].contiguous()
        self.rv = full["v"][:, :, RAW0:].contiguous()
        self.z = full["z"][:, :, RAW0:].contiguous()
        del full
        self.q = synth.normal((B, HQ, D), synth.seed_of(*tag, "q1"), dtype="bf16", device=dev)
        self.pos, self.rpb = pos, rpb  # one positions tensor for every layer, as in a model
        self.out = torch.empty((B, HQ, D), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, HQ), dtype=torch.float32, device=dev)
        nbytes = lbca.decode_workspace_bytes(self.q, self.pk, self.rk, self.pos, M, W, EXCL,
                                             pooled_v=self.pv, raw_v=self.rv, raw_pos_base=self.rpb)
        self.ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=dev)

    def pool_due(self):
        lbca.pool_blocks(self.rk, self.z, self.bias, M, N_POOLED - 1, N_POOLED, self.pk, v=self.rv,
                         out_v=self.pv, pos_base=RAW0)

    def decode(self):
        lbca.attend_decode(self.q, self.pk, self.rk, self.pos, M, W, EXCL, out=self.out, lse=self.lse,
                           pooled_v=self.pv, raw_v=self.rv, raw_pos_base=self.rpb, workspace=self.ws)


def capture(fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm the allocator / module loading outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph(g, reps):
    e0, e1 = ev(), ev()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps  # ms


def run_decode(B, steps, warmup, pool_timer=None):
    pos = torch.full((B,), T_POS, dtype=torch.int64, device="cuda")
    rpb = torch.full((B,), RAW0, dtype=torch.int64, device="cuda")
    layers = [DecodeLayer(l, B, pos, rpb, pool_timer) for l in range(LAYERS)]
    torch.cuda.synchronize()

    def step_with_pool():
        for L in layers:
            L.pool_due()
            L.decode()

    def step():
        for L in layers:
            L.decode()

    # eager reference, then check graph replays reproduce it bitwise
    step_with_pool()
    torch.cuda.synchronize()
    ref = [L.out.clone() for L in layers]
    g_pool = capture(step_with_pool)
    g_step = capture(step)
    for _ in range(max(1, warmup)):
        g_step.replay()
    torch.cuda.synchronize()
    for L, r in zip(layers, ref):
        if not torch.equal(L.out, r):
            raise RuntimeError("graph replay differs from the eager step")
    ms_step = time_graph(g_step, steps)          # 14 decode launches
    ms_pool_step = time_graph(g_pool, steps)     # 14 x (pool due block + decode)
    return layers, ms_step, ms_pool_step


# ---------------------------------------------------------------------------
# incremental decode loop: the cache step (token into the raw ring, due block
# pooled on its step) followed by decode, as a decode loop runs it
# ---------------------------------------------------------------------------
RING = W + M          # ring slots (the raw buffers hold 2 * RING mirrored rows)
INC_STEPS = M         # one block period: each layer pools exactly one due block


def run_incremental(B, reps):
    """Decode steps at positions T_POS-63 .. T_POS of 14 layers at batch 16 (the last
    step makes block 509 visible).  Per layer and step, lbca_cache_append writes the
    token to the mirrored raw ring (pooling the due block on its step), then
    lbca_attend_decode reads the pooled entries and the ring.  A second graph runs the
    same decodes alone (raw bases precomputed), so the cache step's share is the
    difference."""
    dev = "cuda"
    t0 = T_POS - INC_STEPS + 1
    poss = [torch.full((B,), t0 + s, dtype=torch.int64, device=dev) for s in range(INC_STEPS)]
    bases = []
    for pos in poss:
        _, rb = lbca.visible_range(int(pos[0]), M, W, EXCL)
        bases.append(torch.full((B,), rb - rb % RING, dtype=torch.int64, device=dev))
    layers = []
    for l in range(LAYERS):
        g = lambda n, shape, dt="bf16": synth.normal(shape, synth.seed_of("bench-inc", l, B, n), dtype=dt,
                                                     device=dev)
        L = types.SimpleNamespace()
        L.pk, L.pv = g("pk", (B, HKV, N_POOLED + 2, D)), g("pv", (B, HKV, N_POOLED + 2, D))
        L.rk, L.rv, L.rz = g("rk", (B, HKV, 2 * RING, D)), g("rv", (B, HKV, 2 * RING, D)), \
            g("rz", (B, HKV, 2 * RING, D), "f32")
        L.xk, L.xv, L.xz = g("xk", (B, HKV, D)), g("xv", (B, HKV, D)), g("xz", (B, HKV, D), "f32")
        L.bias = synth.normal((HKV, M, D), synth.seed_of("bench-inc", l, "bias"), std=0.1, device=dev)
        L.q = g("q", (B, HQ, D))
        L.rpb = torch.zeros((B,), dtype=torch.int64, device=dev)
        L.out = torch.empty((B, HQ, D), dtype=torch.float32, device=dev)
        L.lse = torch.empty((B, HQ), dtype=torch.float32, device=dev)
        nb = lbca.decode_workspace_bytes(L.q, L.pk, L.rk, poss[0], M, W, EXCL, pooled_v=L.pv, raw_v=L.rv,
                                         raw_pos_base=L.rpb)
        L.ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device=dev)
        layers.append(L)

    def decode(L, pos, rpb):
        lbca.attend_decode(L.q, L.pk, L.rk, pos, M, W, EXCL, out=L.out, lse=L.lse, pooled_v=L.pv, raw_v=L.rv,
                           raw_pos_base=rpb, workspace=L.ws)

    def loop():
        for pos in poss:
            for L in layers:
                lbca.cache_append(L.xk, L.xz, L.rk, L.rz, L.bias, pos, L.rpb, M, W, EXCL, L.pk, v_new=L.xv,
                                  raw_v=L.rv, out_v=L.pv)
                decode(L, pos, L.rpb)

    def decode_only():
        for pos, rpb in zip(poss, bases):
            for L in layers:
                decode(L, pos, rpb)

    def fused():  # lbca_decode_step: append, pool on completion and decode in one launch
        for pos in poss:
            for L in layers:
                lbca.decode_step(L.q, L.xk, L.xv, L.xz, L.rk, L.rv, L.rz, L.bias, L.pk, L.pv, pos, L.rpb, M, W,
                                 out=L.out, lse=L.lse, workspace=L.ws)

    loop()  # eager pass; the graphs then revisit the same 64 positions with the same tokens
    torch.cuda.synchronize()
    ref = [L.out.clone() for L in layers]
    if not all(torch.equal(L.rpb, bases[-1]) for L in layers):
        raise RuntimeError("cache step left an unexpected raw base")
    fused()  # the same positions through the fused step (entries the loop pooled are read back)
    torch.cuda.synchronize()
    if not all(torch.equal(L.out, r) for L, r in zip(layers, ref)):
        raise RuntimeError("the fused decode step differs from cache step + decode")
    g_loop, g_dec, g_fused = capture(loop), capture(decode_only), capture(fused)
    g_loop.replay()
    torch.cuda.synchronize()
    if not all(torch.equal(L.out, r) for L, r in zip(layers, ref)):
        raise RuntimeError("graph replay of the decode loop differs from the eager pass")
    ms_loop, ms_dec, ms_fused = time_graph(g_loop, reps), time_graph(g_dec, reps), time_graph(g_fused, reps)
    n = INC_STEPS * LAYERS
    return {"layer_steps_per_s": n / (ms_loop * 1e-3), "layer_step_us": ms_loop * 1e3 / n,
            "decode_us": ms_dec * 1e3 / n, "cache_append_us": (ms_loop - ms_dec) * 1e3 / n,
            "fused_layer_step_us": ms_fused * 1e3 / n, "fused_layer_steps_per_s": n / (ms_fused * 1e-3),
            "fused_over_decode_us": (ms_fused - ms_dec) * 1e3 / n,
            "workload": f"batch {B}, 14 layers, positions {t0}..{T_POS} (one due block per layer), "
                        f"mirrored raw ring of {RING} slots; fused: lbca_decode_step, one launch per layer-step"}


def run_pool_backward(B, reps):
    """Gradients of the pooling of one layer's 509-block history at batch 16 (K, V bf16,
    logits fp32): reads x, v, z and writes dx, dv, dz once per token channel (16 B) plus
    the upstream rows; the bias gradient is reduced in a second small launch."""
    dev = "cuda"
    tag = ("bench-pool-grad", B)
    L = synth.lbca_layer(tag, B, HQ, HKV, RAW0, D, M, "bf16", "f32", device=dev)
    n = N_POOLED - 1
    gx = synth.normal((B, HKV, n, D), synth.seed_of(*tag, "gx"), dtype="bf16", device=dev)
    gv = synth.normal((B, HKV, n, D), synth.seed_of(*tag, "gv"), dtype="bf16", device=dev)
    dx, dv, dz = torch.empty_like(L["k"]), torch.empty_like(L["v"]), torch.empty_like(L["z"])
    dbias = torch.empty_like(L["bias"])
    nb = lbca.pool_blocks_backward_workspace_bytes(L["k"], L["z"], L["bias"], M, 0, n, gx, v=L["v"], grad_v=gv)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
    call = lambda: lbca.pool_blocks_backward(L["k"], L["z"], L["bias"], M, 0, n, gx, v=L["v"], grad_v=gv,
                                             dx=dx, dv=dv, dz=dz, dbias=dbias, workspace=ws)
    call()
    torch.cuda.synchronize()
    ref = dbias.clone()
    g = capture(call)
    g.replay()
    torch.cuda.synchronize()
    if not torch.equal(dbias, ref):
        raise RuntimeError("graph replay of the pooling backward differs from the eager call")
    ms = time_graph(g, reps)
    tok = B * HKV * n * M * D
    nbytes = tok * (2 + 2 + 4) * 2 + 2 * B * HKV * n * D * 2 + HKV * M * D * 4
    del L, dx, dv, dz
    return {"ms": ms, "GBps": nbytes / (ms * 1e-3) / 1e9, "bytes": nbytes, "workspace_bytes": nb,
            "workload": f"batch {B}, 8 KV heads, {n} blocks of {M} tokens, d={D}: gradients of K, V "
                        f"(bf16), logits (fp32) and bias"}


# ---------------------------------------------------------------------------
# chunked prefill, 16K context
# ---------------------------------------------------------------------------
P_CTX, P_M, P_CHUNK = 16384, 16, 2048


def prefill_flops():
    tot = 0
    for t in range(P_CTX):
        n_p, rb = lbca.visible_range(t, P_M, W, EXCL)
        tot += 4 * HQ * D * (n_p + t - rb + 1)
    return tot


def prefill_executed_flops():
    """FLOPs the kernels execute for the 16K chunked prefill: each workgroup (256
    rows of the flattened (position, GQA head) space of one KV head) multiplies
    its rows by every 32-key tile of the union of its rows' visible spans (the
    pooled prefix of its last position, then the raw band from its first
    position's window start to its last position), masked or not."""
    G = HQ // HKV
    tot = 0
    for c0 in range(0, P_CTX, P_CHUNK):
        rows = P_CHUNK * G
        for r0 in range(0, rows, 256):
            r1 = min(rows, r0 + 256) - 1
            p_first, p_last = c0 + r0 // G, c0 + r1 // G
            n_p, _ = lbca.visible_range(p_last, P_M, W, EXCL)
            _, rb = lbca.visible_range(p_first, P_M, W, EXCL)
            tiles = -(-n_p // 32) + -(-(p_last - rb + 1) // 32)
            tot += HKV * 256 * tiles * 32 * D * 4
    return tot


def run_prefill(reps):
    dev = "cuda"
    L = synth.lbca_layer(("bench-prefill-16k",), 1, HQ, HKV, P_CTX, D, P_M, "bf16", "f32", device=dev,
                         q_len=P_CTX)
    pk = torch.zeros((1, HKV, P_CTX // P_M, D), dtype=torch.bfloat16, device=dev)
    pv = torch.zeros_like(pk)
    out = torch.empty((1, P_CTX, HQ, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((1, P_CTX, HQ), dtype=torch.float32, device=dev)
    qs = [L["q"][:, c:c + P_CHUNK] for c in range(0, P_CTX, P_CHUNK)]
    plan = []
    done = 0
    for i, c0 in enumerate(range(0, P_CTX, P_CHUNK)):
        need, _ = lbca.visible_range(c0 + P_CHUNK - 1, P_M, W, EXCL)
        plan.append((i, c0, done, need))
        done = need

    def attend(i, c0):
        lbca.attend_prefill(qs[i], c0, pk, L["k"], 0, P_M, W, EXCL, out=out[:, c0:c0 + P_CHUNK],
                            lse=lse[:, c0:c0 + P_CHUNK], pooled_v=pv, raw_v=L["v"])

    def full():
        for i, c0, b0, b1 in plan:
            lbca.pool_blocks(L["k"], L["z"], L["bias"], P_M, b0, b1, pk, v=L["v"], out_v=pv)
            attend(i, c0)

    def attn_only():
        for i, c0, _, _ in plan:
            attend(i, c0)

    g_full = capture(full)
    g_attn = capture(attn_only)
    g_full.replay()
    ms_full = time_graph(g_full, reps)
    ms_attn = time_graph(g_attn, reps)
    return ms_full, ms_attn


# ---------------------------------------------------------------------------
# attention backward over one 16K sequence (same layer shape, one call)
# ---------------------------------------------------------------------------
def run_attention_backward(reps):
    """Gradients of attention over all 16384 queries of one sequence (pooled
    entries 0..1015 plus the window; random bf16 inputs and upstream gradient):
    the D / dq-zeroing pass and the key-major gradient kernel, timed as one graph."""
    dev = "cuda"
    N = lbca.visible_range(P_CTX - 1, P_M, W, EXCL)[0]
    g = lambda n, shape: synth.normal(shape, synth.seed_of("bench-attn-grad-16k", n), dtype="bf16", device=dev)
    q, do = g("q", (1, P_CTX, HQ, D)), g("do", (1, P_CTX, HQ, D))
    pk, pv = g("pk", (1, HKV, N, D)), g("pv", (1, HKV, N, D))
    rk, rv = g("rk", (1, HKV, P_CTX, D)), g("rv", (1, HKV, P_CTX, D))
    o, lse = lbca.attend_prefill(q, 0, pk, rk, 0, P_M, W, EXCL, pooled_v=pv, raw_v=rv, out_dtype=torch.bfloat16)
    f32 = dict(dtype=torch.float32, device=dev)
    bufs = dict(grad_q=torch.empty((1, P_CTX, HQ, D), **f32), grad_pooled_k=torch.empty((1, HKV, N, D), **f32),
                grad_pooled_v=torch.empty((1, HKV, N, D), **f32), grad_raw_k=torch.empty((1, HKV, P_CTX, D), **f32),
                grad_raw_v=torch.empty((1, HKV, P_CTX, D), **f32))
    ws = torch.empty(lbca.attend_prefill_backward_workspace_bytes(tuple(q.shape), 0, HKV, N, P_CTX, 0, P_M, W, EXCL),
                     dtype=torch.uint8, device=dev)

    def step():
        lbca.attend_prefill_backward(q, 0, pk, rk, 0, P_M, W, EXCL, o, lse, do, pooled_v=pv, raw_v=rv,
                                     workspace=ws, **bufs)

    gr = capture(step)
    ms = time_graph(gr, reps)
    fl = 5 * prefill_flops() // 2    # S, dP, dV, dK, dQ: 10 d flops per visible (row, key) pair
    del q, do, pk, pv, rk, rv, o, lse, bufs, ws
    return {"ms": ms, "tflops": fl / (ms * 1e-3) / 1e12, "algorithmic_flops": fl,
            "frac_of_bf16_peak": fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "workload": f"one sequence of {P_CTX} queries, 24 query / 8 KV heads, d=128, m={P_M}, W={W}, "
                        f"{N} pooled entries; gradients of q, pooled and raw K and V (fp32)"}


# ---------------------------------------------------------------------------
# HCA decode at 1M context and CSA decode at 128K (MQA, 64 query heads, dim 512)
# ---------------------------------------------------------------------------
X_HQ, X_D, X_RD, X_EPS, X_BASE = 64, 512, 64, 1e-6, 10000.0
HCA_T, HCA_M, HCA_B = 1 << 20, 128, 4
CSA_T, CSA_M, CSA_B, CSA_HI, CSA_DI, CSA_K = 1 << 17, 4, 2, 8, 64, 512
CSA_CHUNK = 2048  # sparse prefill: queries per sequence in the timed chunk
ROTATE_BYTES = 600 << 20   # distinct bytes a timing loop cycles through (> 2 x Infinity Cache)


def mqa_step_bytes(B, rows):
    """Algorithmic bytes of one MQA decode call: every visible (or selected) row
    read once in bf16 (K = V), the queries in bf16, out and LSE in fp32."""
    return B * (rows * X_D * 2 + X_HQ * X_D * 2 + X_HQ * X_D * 4 + X_HQ * 4)


def run_hca(reps):
    """Pool the whole 1M history once (timed, GB/s), then time decode at t = 2^20 - 1
    over instances that rotate through more than the Infinity Cache holds."""
    dev = "cuda"
    B, T, m = HCA_B, HCA_T, HCA_M
    N = T // m
    treat = dict(rmsnorm_eps=X_EPS, rope_dims=X_RD, rope_base=X_BASE)
    H = synth.hca_layer(("bench-hca-1m",), B, X_HQ, T, X_D, m, device=dev)
    ent = torch.empty((B, 1, N, X_D), dtype=torch.bfloat16, device=dev)
    pool = lambda: lbca.pool_blocks(H["c"], H["z"], H["bias"], m, 0, N, ent, **treat)
    pool()
    g_pool = capture(pool)
    ms_pool = time_graph(g_pool, 3)
    pool_bytes = B * T * X_D * 2 * 2 + B * N * X_D * 2
    raw = H["c"][:, :, T - W:].contiguous()  # the window in its own buffer, as a serving cache holds it
    pos = torch.full((B,), T - 1, dtype=torch.int64, device=dev)
    rpb = torch.full((B,), T - W, dtype=torch.int64, device=dev)
    sink = H["sink"]
    del H, g_pool
    torch.cuda.empty_cache()
    per_inst = ent.numel() * 2 + raw.numel() * 2
    n_inst = max(2, -(-ROTATE_BYTES // per_inst))
    inst = []
    for i in range(n_inst):
        inst.append(dict(ent=ent.clone(), raw=raw.clone(),
                         q=synth.normal((B, X_HQ, X_D), synth.seed_of("bench-hca-1m", "q", i), dtype="bf16",
                                        device=dev),
                         out=torch.empty((B, X_HQ, X_D), device=dev), lse=torch.empty((B, X_HQ), device=dev)))
    kw = dict(raw_pos_base=rpb, sink=sink, **treat)
    x = inst[0]
    nws = lbca.decode_workspace_bytes(x["q"], x["ent"], x["raw"], pos, m, W, OVER, **kw)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)

    def step():
        for x in inst:
            lbca.attend_decode(x["q"], x["ent"], x["raw"], pos, m, W, OVER, out=x["out"], lse=x["lse"],
                               workspace=ws, **kw)

    g = capture(step)
    g.replay()
    us = time_graph(g, reps) * 1e3 / n_inst
    rows = N + W
    by = mqa_step_bytes(B, rows)
    fl = B * X_HQ * rows * X_D * 4
    return {"decode_us": us, "decode_GBps": by / (us * 1e-6) / 1e9,
            "decode_frac_of_hbm_peak": by / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "decode_tflops": fl / (us * 1e-6) / 1e12, "decode_algorithmic_bytes": by,
            "decode_workspace_bytes": nws, "instances": n_inst,
            "pool_ms": ms_pool, "pool_GBps": pool_bytes / (ms_pool * 1e-3) / 1e9, "pool_bytes": pool_bytes,
            "workload": f"HCA batch {B}, t = 2^20 - 1: {N} treated entries + {W} raw, 64 query heads x 512"}


def run_csa(reps):
    """Dual-pool the 128K history once (timed), then time indexer top-512 and decode over
    the selection at t = 2^17 - 1, rotating through instances with their own keys."""
    dev = "cuda"
    B, T, m, k = CSA_B, CSA_T, CSA_M, CSA_K
    N = T // m
    treat = dict(rmsnorm_eps=X_EPS, rope_dims=X_RD, rope_base=X_BASE)
    C = synth.csa_layer(("bench-csa-128k",), B, X_HQ, T, X_D, m, CSA_HI, CSA_DI, device=dev)
    ent = torch.empty((B, 1, N, X_D), dtype=torch.bfloat16, device=dev)
    pool = lambda: lbca.pool_blocks(C["ca"], C["za"], C["bias_a"], m, 0, N, ent, xb=C["cb"], zb=C["zb"],
                                    bias_b=C["bias_b"], **treat)
    pool()
    g_pool = capture(pool)
    ms_pool = time_graph(g_pool, 3)
    pool_bytes = B * T * X_D * 2 * 4 + B * N * X_D * 2
    # gradients of that pooling (dual series, treated entries) for one upstream gradient per entry
    gd = synth.normal((B, 1, N, X_D), synth.seed_of("bench-csa-128k", "grad"), dtype="bf16", device=dev)
    outs = dict(dx=torch.empty_like(C["ca"]), dz=torch.empty_like(C["za"]), dbias=torch.empty_like(C["bias_a"]),
                dxb=torch.empty_like(C["cb"]), dzb=torch.empty_like(C["zb"]), dbias_b=torch.empty_like(C["bias_b"]))
    dual = dict(xb=C["cb"], zb=C["zb"], bias_b=C["bias_b"])
    nbw = lbca.pool_blocks_backward_workspace_bytes(C["ca"], C["za"], C["bias_a"], m, 0, N, gd, **dual, **treat)
    wsb = torch.empty(max(nbw, 16), dtype=torch.uint8, device=dev)
    back = lambda: lbca.pool_blocks_backward(C["ca"], C["za"], C["bias_a"], m, 0, N, gd, workspace=wsb, **dual,
                                             **treat, **outs)
    back()
    g_back = capture(back)
    ms_back = time_graph(g_back, 3)
    back_bytes = B * T * X_D * 2 * 4 * 2 + B * N * X_D * 2  # a- and b-series rows and logits read and written
    del gd, outs, dual, wsb, g_back
    # sparse prefill of the context's last chunk of CSA_CHUNK queries per sequence: chunk indexer,
    # per-query top-k and the selected-entry attention (treated entries as above)
    CH, tg = CSA_CHUNK, "bench-csa-128k-chunk"
    t0 = T - CH
    pf = dict(qi=synth.normal((B, CH, CSA_HI, CSA_DI), synth.seed_of(tg, "qi"), dtype="bf16", device=dev),
              w=synth.uniform((B, CH, CSA_HI), synth.seed_of(tg, "w"), device=dev),
              keys=synth.normal((B, N, CSA_DI), synth.seed_of(tg, "keys"), dtype="bf16", device=dev),
              q=synth.normal((B, CH, X_HQ, X_D), synth.seed_of(tg, "q"), dtype="bf16", device=dev))
    rbase = t0 - W + 1
    rawc = C["ca"][:, 0, rbase:].contiguous()  # the chunk's raw rows in their own buffer
    pf_out = torch.empty((B, CH, X_HQ, X_D), device=dev)
    pf_lse = torch.empty((B, CH, X_HQ), device=dev)
    pf_idx = torch.empty((B, CH, k), dtype=torch.int32, device=dev)
    pf_args = (pf["qi"], pf["w"], pf["keys"], pf["q"], ent[:, 0], rawc, t0, rbase, m, W, k)
    pf_kw = dict(sink=C["sink"], out=pf_out, lse=pf_lse, out_idx=pf_idx, **treat)
    ws_pf = torch.empty(max(lbca.csa_sparse_prefill_workspace_bytes(*pf_args, **pf_kw), 16), dtype=torch.uint8,
                        device=dev)
    sparse = lambda: lbca.csa_sparse_prefill(*pf_args, workspace=ws_pf, **pf_kw)
    sparse()
    g_sp = capture(sparse)
    ms_sp = time_graph(g_sp, 3)
    n_vis_sum = sum((t + 1) // m for t in range(t0, T))
    sp_index_flop = B * n_vis_sum * CSA_HI * CSA_DI * 2
    sp_attn_flop = B * CH * X_HQ * (k + W) * X_D * 4
    del pf, rawc, pf_out, pf_lse, pf_idx, ws_pf, g_sp, pf_args, pf_kw
    raw = C["ca"][:, :, T - W:].contiguous()  # the window in its own buffer, as a serving cache holds it
    sink = C["sink"]
    del C, g_pool
    torch.cuda.empty_cache()
    pos = torch.full((B,), T - 1, dtype=torch.int64, device=dev)
    rpb = torch.full((B,), T - W, dtype=torch.int64, device=dev)
    tag = "bench-csa-128k"
    # distinct bytes per instance that one step touches: keys + the gathered rows + window
    per_inst = B * (N * CSA_DI * 2 + (k + W) * X_D * 2)
    n_inst = max(2, -(-ROTATE_BYTES // per_inst))
    inst = []
    for i in range(n_inst):
        inst.append(dict(
            ent=ent.clone(), raw=raw.clone(),
            keys=synth.normal((B, N, CSA_DI), synth.seed_of(tag, "keys", i), dtype="bf16", device=dev),
            qi=synth.normal((B, CSA_HI, CSA_DI), synth.seed_of(tag, "qi", i), dtype="bf16", device=dev),
            w=synth.uniform((B, CSA_HI), synth.seed_of(tag, "w", i), device=dev),
            q=synth.normal((B, X_HQ, X_D), synth.seed_of(tag, "q", i), dtype="bf16", device=dev),
            idx=torch.empty((B, k), dtype=torch.int32, device=dev),
            sc=torch.empty((B, k), dtype=torch.float32, device=dev),
            out=torch.empty((B, X_HQ, X_D), device=dev), lse=torch.empty((B, X_HQ), device=dev)))
    kw = dict(raw_pos_base=rpb, sink=sink, **treat)
    x = inst[0]
    ws_i = torch.empty(lbca.index_workspace_bytes(x["qi"], x["w"], x["keys"], pos, m, k), dtype=torch.uint8,
                       device=dev)
    nws = lbca.decode_workspace_bytes(x["q"], x["ent"], x["raw"], pos, m, W, OVER, sel_idx=x["idx"], **kw)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)

    def index(x):
        lbca.csa_index_topk(x["qi"], x["w"], x["keys"], pos, m, k, out_idx=x["idx"], out_score=x["sc"],
                            workspace=ws_i)

    def decode(x):
        lbca.attend_decode(x["q"], x["ent"], x["raw"], pos, m, W, OVER, out=x["out"], lse=x["lse"],
                           sel_idx=x["idx"], workspace=ws, **kw)

    g_both = capture(lambda: [(index(x), decode(x)) for x in inst])
    g_idx = capture(lambda: [index(x) for x in inst])
    g_dec = capture(lambda: [decode(x) for x in inst])
    g_both.replay()
    us_both = time_graph(g_both, reps) * 1e3 / n_inst
    us_idx = time_graph(g_idx, reps) * 1e3 / n_inst
    us_dec = time_graph(g_dec, reps) * 1e3 / n_inst
    by_idx = B * (N * CSA_DI * 2 + CSA_HI * CSA_DI * 2 + CSA_HI * 4 + k * 8)
    by_dec = mqa_step_bytes(B, k + W)
    by = by_idx + by_dec
    return {"sparse_prefill_chunk": {"workload": f"batch {B}, last {CSA_CHUNK} queries of a {T}-token context, "
                                              f"top-{k} of {N} entries plus the {W}-token window, {X_HQ} heads x {X_D}",
                                  "ms": ms_sp, "queries_per_s": B * CSA_CHUNK / (ms_sp * 1e-3),
                                  "index_GFLOP": sp_index_flop / 1e9, "attention_GFLOP": sp_attn_flop / 1e9,
                                  "TFLOPs": (sp_index_flop + sp_attn_flop) / (ms_sp * 1e-3) / 1e12},
            "step_us": us_both, "step_GBps": by / (us_both * 1e-6) / 1e9, "step_algorithmic_bytes": by,
            "index_topk_us": us_idx, "index_GBps": by_idx / (us_idx * 1e-6) / 1e9,
            "decode_us": us_dec, "decode_GBps": by_dec / (us_dec * 1e-6) / 1e9,
            "decode_workspace_bytes": nws, "instances": n_inst,
            "pool_ms": ms_pool, "pool_GBps": pool_bytes / (ms_pool * 1e-3) / 1e9, "pool_bytes": pool_bytes,
            "pool_backward_ms": ms_back, "pool_backward_GBps": back_bytes / (ms_back * 1e-3) / 1e9,
            "workload": f"CSA batch {B}, t = 2^17 - 1: top-{k} of {N} entries (8 x 64 indexer) + {W} raw, "
                        f"64 query heads x 512"}


# ---------------------------------------------------------------------------
# projections around the path, at the CSA sparse prefill chunk (batch 2 x 2048 tokens)
# ---------------------------------------------------------------------------
PJ_T, PJ_H, PJ_C, PJ_DC, PJ_HI, PJ_DI, PJ_G, PJ_DG, PJ_DM = 4096, 64, 512, 1024, 8, 64, 8, 1024, 4096


def run_projections(reps):
    """Low-rank indexer queries (d_c = 1024 -> 8 x 64), the grouped output
    projection (64 heads x 512 in 8 groups to 1024 each, then to 4096) and the
    pooling logits of CSA's two series (4096 -> 2 x 512, fp32) of 4096 tokens,
    each lbca_grouped_gemm launch captured in a graph of its own."""
    dev = "cuda"
    sd = lambda n: synth.seed_of("bench-proj", n)
    cq = synth.normal((PJ_T, PJ_DC), sd("cq"), dtype="bf16", device=dev)
    wuq = synth.normal((PJ_HI * PJ_DI, PJ_DC), sd("wuq"), std=PJ_DC ** -0.5, dtype="bf16", device=dev)
    o = synth.normal((PJ_T, PJ_H, PJ_C), sd("o"), device=dev)
    wg = synth.normal((PJ_G, PJ_DG, PJ_H // PJ_G * PJ_C), sd("wg"), std=(PJ_H // PJ_G * PJ_C) ** -0.5,
                      dtype="bf16", device=dev)
    wo = synth.normal((PJ_DM, PJ_G * PJ_DG), sd("wo"), std=(PJ_G * PJ_DG) ** -0.5, dtype="bf16", device=dev)
    qi = torch.empty((PJ_T, PJ_HI * PJ_DI), dtype=torch.bfloat16, device=dev)
    mid = torch.empty((PJ_T, PJ_G * PJ_DG), dtype=torch.bfloat16, device=dev)
    y = torch.empty((PJ_T, PJ_DM), dtype=torch.float32, device=dev)
    flat = o.reshape(PJ_T, -1)
    parts = {
        "indexer_queries": (lambda: lbca.grouped_gemm(cq, wuq, out=qi), 2 * PJ_T * PJ_DC * PJ_HI * PJ_DI),
        "output_groups": (lambda: lbca.grouped_gemm(flat, wg, out=mid, groups=PJ_G),
                          2 * PJ_T * PJ_H * PJ_C * PJ_DG),
        "output_model": (lambda: lbca.grouped_gemm(mid, wo, out=y), 2 * PJ_T * PJ_G * PJ_DG * PJ_DM),
    }
    h = synth.normal((PJ_T, PJ_DM), sd("h"), dtype="bf16", device=dev)
    wz = synth.normal((2 * PJ_C, PJ_DM), sd("wz"), std=PJ_DM ** -0.5, dtype="bf16", device=dev)
    z = torch.empty((PJ_T, 2 * PJ_C), dtype=torch.float32, device=dev)
    parts["pooling_logits"] = (lambda: lbca.grouped_gemm(h, wz, out=z), 2 * PJ_T * PJ_DM * 2 * PJ_C)
    res = {"workload": f"{PJ_T} tokens: indexer queries {PJ_DC} -> {PJ_HI} x {PJ_DI}; output projection "
                       f"{PJ_H} heads x {PJ_C} in {PJ_G} groups -> {PJ_G} x {PJ_DG} -> {PJ_DM} "
                       f"(fp32 attention output rounded to bf16 on load); pooling logits of two series "
                       f"{PJ_DM} -> 2 x {PJ_C} (fp32)"}
    tot_ms, tot_fl = 0.0, 0
    for name, (fn, fl) in parts.items():
        g = capture(fn)
        ms = time_graph(g, reps)
        res[name] = {"ms": ms, "tflops": fl / (ms * 1e-3) / 1e12, "flops": fl}
        tot_ms += ms
        tot_fl += fl
    res["total_ms"] = tot_ms
    res["tflops"] = tot_fl / (tot_ms * 1e-3) / 1e12
    res["frac_of_bf16_peak"] = res["tflops"] / BF16_PEAK_TFLOPS
    return res


# ---------------------------------------------------------------------------
# measured ceilings of this part (probe kernels in libceilings.so)
# ---------------------------------------------------------------------------
def run_ceilings():
    """Streaming HBM read (1 GiB), one launch reading the batch-16 decode's bytes
    (14 distinct buffers in a graph, like the decode step), a bf16 MFMA loop and
    the empty-kernel launch floor."""
    import ctypes

    from block_compressed_kv_amd import build as B
    if not os.path.exists(B.CEIL_LIB):
        raise RuntimeError(f"{B.CEIL_LIB} is missing: build it with `python -m block_compressed_kv_amd.build`")
    L = ctypes.CDLL(B.CEIL_LIB)
    L.ceil_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.ceil_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    L.ceil_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.ceil_lds.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.ceil_empty.argtypes = [ctypes.c_void_p]
    stream = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def ok(r):
        if r != 0:
            raise RuntimeError(f"ceiling probe failed (hip error {r})")

    res = {}
    grid = 2048
    out = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
    big = torch.zeros(1 << 30, dtype=torch.uint8, device="cuda")
    g = capture(lambda: ok(L.ceil_read(big.data_ptr(), big.numel(), out.data_ptr(), grid, stream())))
    res["hbm_read_GBps"] = big.numel() / (time_graph(g, 20) * 1e-3) / 1e9
    dst = torch.empty_like(big)
    g = capture(lambda: ok(L.ceil_copy(big.data_ptr(), dst.data_ptr(), big.numel(), grid, stream())))
    res["hbm_copy_GBps"] = 2 * big.numel() / (time_graph(g, 20) * 1e-3) / 1e9  # bytes read + written
    del big, dst, g
    nb = decode_bytes_per_seq_layer() * 16
    bufs = [torch.zeros(nb, dtype=torch.uint8, device="cuda") for _ in range(LAYERS)]
    for grid_dec in (256, 1024):
        g = capture(lambda: [ok(L.ceil_read(b.data_ptr(), nb, out.data_ptr(), grid_dec, stream())) for b in bufs])
        res[f"read_decode_bytes_one_launch_us_grid{grid_dec}"] = time_graph(g, 50) * 1e3 / LAYERS
    del bufs, g
    lg, lit = 1024, 2048
    lsrc = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    lo_ = torch.empty(lg * 256, dtype=torch.int32, device="cuda")
    g = capture(lambda: ok(L.ceil_lds(lsrc.data_ptr(), lo_.data_ptr(), lg, lit, stream())))
    lds_s = time_graph(g, 10) * 1e-3
    res["lds_read_TBps"] = lg * 256 * 8 * lit * 16 / lds_s / 1e12
    res["lds_read_bytes_per_clock_per_cu_at_2p4GHz"] = res["lds_read_TBps"] * 1e12 / 256 / 2.4e9
    mg, iters = 1024, 4096
    mo = torch.empty(mg * 256, dtype=torch.float32, device="cuda")
    g = capture(lambda: ok(L.ceil_mfma(mo.data_ptr(), mg, iters, stream())))
    res["mfma_bf16_TFLOPs"] = mg * 4 * iters * 4 * 32768 / (time_graph(g, 5) * 1e-3) / 1e12
    L.ceil_mfma16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    mg16 = 2048
    mo16 = torch.empty(mg16 * 256, dtype=torch.float32, device="cuda")
    g = capture(lambda: ok(L.ceil_mfma16(mo16.data_ptr(), mg16, iters, stream())))
    res["mfma16_bf16_TFLOPs"] = mg16 * 4 * iters * 8 * 16384 / (time_graph(g, 5) * 1e-3) / 1e12
    g = capture(lambda: [ok(L.ceil_empty(stream())) for _ in range(LAYERS)])
    res["empty_launch_us"] = time_graph(g, 200) * 1e3 / LAYERS
    res["note"] = ("hbm_read: 2048 workgroups streaming 1 GiB; hbm_copy: the same workgroups copying 1 GiB "
                   "(bytes read + written); lds_read: 1024 workgroups x 256 threads each reading 16 B per step "
                   "from LDS, eight reads in flight; read_decode_bytes_one_launch: one launch reading "
                   f"{nb} B (the batch-16 decode's algorithmic bytes), 14 distinct buffers per graph replay; "
                   "mfma: 1024 workgroups x 4 waves x 4 chains of v_mfma_f32_32x32x16_bf16; "
                   "mfma16: 2048 workgroups x 4 waves x 8 chains of v_mfma_f32_16x16x32_bf16; "
                   "empty_launch: 14 empty kernels per graph replay")
    return res


# ---------------------------------------------------------------------------
# oracle on the host
# ---------------------------------------------------------------------------
def cpu_baseline(layer, budget_s=12.0):
    """The oracle's decode attention per layer-step (batch 16, fp64 NumPy), bounded sample."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import lbca_oracle as O

    host = lambda t: t.detach().cpu().to(torch.float64).numpy()
    B = layer.q.shape[0]
    q, pk, pv = host(layer.q), host(layer.pk), host(layer.pv)
    rk, rv = host(layer.rk), host(layer.rv)
    n = 0
    t0 = time.perf_counter()
    while True:
        O.attend_decode(q, pk, pv, rk, rv, [T_POS] * B, M, W, O.EXCLUSIVE, 1 / math.sqrt(D),
                        raw_pos_base=[RAW0] * B)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": n / el, "unit": "layer-steps/s", "cores": blas, "kind": "oracle",
            "sample": f"{n} oracle decode layer-steps (batch {B}, 32K context, 510 pooled + 128 raw "
                      f"per KV head, fp64 NumPy) in {el:.1f} s; BLAS threads {blas}, "
                      f"{len(os.sched_getaffinity(0))} cores available"}


def _timed(fn, budget_s):
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            return el / n, n


def oracle_samples(budget_s=3.0):
    """The oracle beside the other timed ops, each on a bounded sample of its
    workload (fp64 NumPy on the host cores; seeded synthetic inputs of the
    workload's shapes): batch-1 32K decode per layer-step, queries of the last
    16K prefill chunk (time per chunk extrapolated from the sample), one HCA
    sequence's decode at 1M and one CSA sequence's indexer + top-512 + decode
    at 128K (per step = per sequence x batch)."""
    import numpy as np

    from oracle import lbca_oracle as O

    f64 = lambda t: t.to(torch.float64).numpy()
    res = {}
    # 32K decode at batch 1
    tag = ("bench-oracle-32k",)
    q = f64(synth.normal((1, HQ, D), synth.seed_of(*tag, "q"), dtype="bf16"))
    pk, pv = (f64(synth.normal((1, HKV, N_POOLED, D), synth.seed_of(*tag, n), dtype="bf16")) for n in ("pk", "pv"))
    rk, rv = (f64(synth.normal((1, HKV, RAW_ROWS, D), synth.seed_of(*tag, n), dtype="bf16")) for n in ("rk", "rv"))
    sec, n = _timed(lambda: O.attend_decode(q, pk, pv, rk, rv, [T_POS], M, W, O.EXCLUSIVE, 1 / math.sqrt(D),
                                            raw_pos_base=[RAW0]), budget_s)
    res["decode_32k_b1"] = {"oracle_s": sec, "sample": f"{n} layer-steps"}
    # prefill: the last 16 query positions of chunk 7 (positions 16368..16383)
    tag = ("bench-oracle-prefill",)
    nq, n_pool = 16, P_CTX // P_M
    qp = f64(synth.normal((1, nq, HQ, D), synth.seed_of(*tag, "q"), dtype="bf16"))
    ppk, ppv = (f64(synth.normal((1, HKV, n_pool, D), synth.seed_of(*tag, n), dtype="bf16")) for n in ("pk", "pv"))
    prk, prv = (f64(synth.normal((1, HKV, P_CTX, D), synth.seed_of(*tag, n), dtype="bf16")) for n in ("rk", "rv"))
    sec, n = _timed(lambda: O.attend_prefill(qp, P_CTX - nq, ppk, ppv, prk, prv, 0, P_M, W, O.EXCLUSIVE,
                                             1 / math.sqrt(D)), budget_s)
    res["prefill_16k_chunk7"] = {"oracle_s_per_chunk_est": sec * P_CHUNK / nq,
                                 "sample": f"{n} runs of the last {nq} queries of chunk 7, scaled to {P_CHUNK}"}
    # HCA decode, one sequence at t = 2^20 - 1
    tag = ("bench-oracle-hca",)
    treat = dict(rmsnorm_eps=X_EPS, rope_dims=X_RD, rope_base=X_BASE)
    N = HCA_T // HCA_M
    qh = f64(synth.normal((1, X_HQ, X_D), synth.seed_of(*tag, "q"), dtype="bf16"))
    eh = f64(synth.normal((1, 1, N, X_D), synth.seed_of(*tag, "ent"), dtype="bf16"))
    rh = f64(synth.normal((1, 1, W, X_D), synth.seed_of(*tag, "raw"), dtype="bf16"))
    sk = f64(synth.normal((X_HQ,), synth.seed_of(*tag, "sink")))
    sec, n = _timed(lambda: O.attend_decode(qh, eh, None, rh, None, [HCA_T - 1], HCA_M, W, O.OVERLAP,
                                            1 / math.sqrt(X_D), raw_pos_base=[HCA_T - W], sink=sk, **treat),
                    budget_s)
    res["hca_1m_step"] = {"oracle_s": sec * HCA_B, "sample": f"{n} decodes of one sequence, x {HCA_B} sequences"}
    # CSA: indexer scores + top-512 + decode over the selection, one sequence at t = 2^17 - 1
    tag = ("bench-oracle-csa",)
    N = CSA_T // CSA_M
    qi = f64(synth.normal((CSA_HI, CSA_DI), synth.seed_of(*tag, "qi"), dtype="bf16"))
    wi = f64(synth.uniform((CSA_HI,), synth.seed_of(*tag, "w")))
    ki = f64(synth.normal((N, CSA_DI), synth.seed_of(*tag, "keys"), dtype="bf16"))
    qc = f64(synth.normal((1, X_HQ, X_D), synth.seed_of(*tag, "q"), dtype="bf16"))
    ec = f64(synth.normal((1, 1, N, X_D), synth.seed_of(*tag, "ent"), dtype="bf16"))
    rc = f64(synth.normal((1, 1, W, X_D), synth.seed_of(*tag, "raw"), dtype="bf16"))

    def csa_step():
        sel = O.topk_select(O.index_scores(qi, wi, ki, N), CSA_K)
        return O.attend_decode(qc, ec, None, rc, None, [CSA_T - 1], CSA_M, W, O.OVERLAP, 1 / math.sqrt(X_D),
                               raw_pos_base=[CSA_T - W], sel_idx=sel[None], sink=sk, **treat)

    sec, n = _timed(csa_step, budget_s)
    res["csa_128k_step"] = {"oracle_s": sec * CSA_B, "sample": f"{n} steps of one sequence, x {CSA_B} sequences"}
    del np
    return res


# ---------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--batch", type=int, default=16)
    ap.add_argument("--no-cpu", action="store_true", help="skip the host oracle timing")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-incremental", action="store_true", help="skip the cache-step decode loop")
    ap.add_argument("--no-backward", action="store_true", help="skip the pooling-gradient line")
    ap.add_argument("--no-small-batch", action="store_true")
    ap.add_argument("--no-mqa", action="store_true", help="skip the HCA 1M and CSA 128K lines")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured-ceiling probes")
    ap.add_argument("--no-proj", action="store_true", help="skip the projection GEMM line")
    ap.add_argument("--no-attn-grad", action="store_true", help="skip the attention-backward line")
    ap.add_argument("--counters", action="store_true",
                    help="only run what the FETCH_SIZE / WRITE_SIZE counter passes profile")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the decode/prefill hot path here has no multi-GPU "
              f"path (requested --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    lbca.lib()  # fail loudly if the library is missing
    if args.counters:
        counter_pass()
        return

    B = args.batch
    log(f"[bench] decode 32K: building {LAYERS} layers at batch {B}")
    pool_timer = []
    layers, ms_step, ms_pool_step = run_decode(B, args.steps, args.warmup, pool_timer)
    torch.cuda.synchronize()
    pool_ms = sum(a.elapsed_time(b) for a, b, _ in pool_timer)
    pool_bytes = sum(n for _, _, n in pool_timer)
    us_launch = ms_step * 1e3 / LAYERS
    log(f"[bench] step {ms_step * 1e3:.1f} us ({LAYERS} decode launches, {us_launch:.2f} us each); "
        f"with the due block pooled first {ms_pool_step * 1e3:.1f} us")

    per_launch_bytes = decode_bytes_per_seq_layer() * B
    achieved = per_launch_bytes / (us_launch * 1e-6) / 1e9
    traffic = measured_traffic_bytes()
    value = LAYERS / (ms_step * 1e-3)
    us_pool = (ms_pool_step - ms_step) * 1e3 / LAYERS
    extra = {
        "decode_launch_us": us_launch,
        "decode_algorithmic_bytes_per_launch": per_launch_bytes,
        "due_block_pool_us": us_pool,
        "step_with_due_pool_layer_steps_per_s": LAYERS / (ms_pool_step * 1e-3),
        "amortised_layer_steps_per_s": 1e6 / (us_launch + us_pool / M),
        "history_pool_GBps": pool_bytes / (pool_ms * 1e-3) / 1e9,
        "history_pool_bytes": pool_bytes,
        "decode_traffic_over_algorithmic": None if traffic is None else traffic / per_launch_bytes,
    }

    cpu = None
    if not args.no_cpu:
        log("[bench] oracle on host cores (bounded sample)")
        cpu = cpu_baseline(layers[0])
    del layers
    torch.cuda.empty_cache()

    if not args.no_small_batch:
        for b in (1, 4):
            log(f"[bench] decode 32K batch {b}")
            ls, st, _ = run_decode(b, args.steps, args.warmup)
            by = decode_bytes_per_seq_layer() * b
            us = st * 1e3 / LAYERS
            extra[f"b{b}"] = {"layer_steps_per_s": LAYERS / (st * 1e-3), "decode_launch_us": us,
                              "decode_GBps": by / (us * 1e-6) / 1e9,
                              "note": "14 layers fit in the 256 MB Infinity Cache at this batch"}
            del ls
            torch.cuda.empty_cache()

    if not args.no_backward:
        log("[bench] pooling gradients of a 32K history (batch 16)")
        extra["pool_backward_32k"] = run_pool_backward(B, max(3, args.steps // 40))
        torch.cuda.empty_cache()

    if not args.no_incremental:
        log("[bench] incremental decode loop 32K (cache step + decode, 64 steps)")
        extra["incremental_32k"] = run_incremental(B, max(5, args.steps // 10))
        torch.cuda.empty_cache()

    if not args.no_prefill:
        log("[bench] chunked prefill 16K (8 x 2048)")
        ms_full, ms_attn = run_prefill(max(5, args.steps // 10))
        fl = prefill_flops()
        fx = prefill_executed_flops()
        extra["prefill"] = {"tflops": fl / (ms_attn * 1e-3) / 1e12, "attention_ms": ms_attn,
                            "with_pooling_ms": ms_full, "algorithmic_flops": fl,
                            "frac_of_bf16_peak": fl / (ms_attn * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                            "executed_tile_flops": fx, "executed_tflops": fx / (ms_attn * 1e-3) / 1e12}

    if not args.no_attn_grad:
        log("[bench] attention backward 16K (one call)")
        extra["attention_backward_16k"] = run_attention_backward(max(3, args.steps // 20))
        torch.cuda.empty_cache()

    if not args.no_proj:
        log("[bench] projections around the path (grouped GEMM, 4096 tokens)")
        extra["projections"] = run_projections(max(5, args.steps // 20))
        torch.cuda.empty_cache()

    if not args.no_mqa:
        log("[bench] HCA decode 1M (batch 4)")
        extra["hca_1m"] = run_hca(max(5, args.steps // 4))
        torch.cuda.empty_cache()
        log("[bench] CSA index top-512 + decode 128K (batch 2)")
        extra["csa_128k"] = run_csa(max(5, args.steps // 4))
        torch.cuda.empty_cache()

    if not args.no_ceilings:
        log("[bench] measured ceilings (streaming read, MFMA loop, launch floor)")
        ce = run_ceilings()
        ce["decode_launch_vs_one_launch_read"] = min(ce["read_decode_bytes_one_launch_us_grid256"],
                                                     ce["read_decode_bytes_one_launch_us_grid1024"]) / us_launch
        ce["decode_GBps_vs_stream_read"] = achieved / ce["hbm_read_GBps"]
        if "prefill" in extra:
            ce["prefill_vs_mfma_loop"] = extra["prefill"]["tflops"] / ce["mfma_bf16_TFLOPs"]
        if "attention_backward_16k" in extra:
            ce["attention_backward_vs_mfma_loop"] = (extra["attention_backward_16k"]["tflops"]
                                                     / ce["mfma_bf16_TFLOPs"])
        if "projections" in extra:
            ce["projections_vs_mfma_loop"] = extra["projections"]["tflops"] / ce["mfma_bf16_TFLOPs"]
        if "pool_backward_32k" in extra:
            ce["pool_backward_vs_copy"] = extra["pool_backward_32k"]["GBps"] / ce["hbm_copy_GBps"]
        extra["ceilings"] = ce
        torch.cuda.empty_cache()

    if not args.no_cpu:
        log("[bench] oracle samples beside the other timed ops")
        osm = oracle_samples()
        osm["decode_32k_b1"]["gpu_s"] = extra["b1"]["decode_launch_us"] * 1e-6 if "b1" in extra else None
        if "prefill" in extra:
            osm["prefill_16k_chunk7"]["gpu_s_mean_chunk"] = extra["prefill"]["attention_ms"] * 1e-3 / 8
        if "hca_1m" in extra:
            osm["hca_1m_step"]["gpu_s"] = extra["hca_1m"]["decode_us"] * 1e-6
        if "csa_128k" in extra:
            osm["csa_128k_step"]["gpu_s"] = extra["csa_128k"]["step_us"] * 1e-6
        for v in osm.values():
            o = v.get("oracle_s", v.get("oracle_s_per_chunk_est"))
            gs = v.get("gpu_s", v.get("gpu_s_mean_chunk"))
            v["speedup"] = o / gs if o and gs else None
        extra["oracle_vs_gpu"] = osm

    line = {
        "metric": METRIC, "value": value, "unit": "layer-steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"lbca-decode-32k-b{B}-14layers", "batch": B, "context": CTX,
                   "q_heads": HQ, "kv_heads": HKV, "head_dim": D, "block": M, "window": W,
                   "layers": LAYERS, "step": "one lbca_attend_decode launch per layer"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "decode_kernel (lbca_attend_decode, one workgroup per unit at batch 16)"},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
