"""Seeded synthetic inputs shaped like the pages' workloads.

This module holds no arithmetic of the method: it only draws seeded random
numbers (torch's Philox-based generator on the GPU, its Mersenne-Twister one on
the CPU) and rounds them to the storage dtype (round-to-nearest-even for bf16).
Both the HIP path and the oracle consume exactly these tensors.

Workload shapes (the pages' settings): Llama-3.2-3B GQA layers (24 query heads
over 8 KV heads, head dim 128) with 16- or 64-token blocks and a 128-token raw
window; DeepSeek-V4 paper dims for HCA/CSA (MQA over 64 query heads, head dim
512, 128-token pooling for HCA, 4-token dual pooling and an 8x64 indexer with
top-512 for CSA).  Every tensor is N(0,1) unless noted: positional biases are
N(0, 0.1); indexer head weights are U(0, 1).
"""
from __future__ import annotations

import hashlib

import torch

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def seed_of(*keys) -> int:
    """Stable 63-bit seed from a tuple of labels (config, layer, tensor, ...)."""
    h = hashlib.sha256(repr(keys).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def normal(shape, seed, std=1.0, dtype="f32", device="cpu"):
    """fp32 N(0, std^2) draws, then rounded to ``dtype``."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(_DT.get(dtype, dtype))


def uniform(shape, seed, lo=0.0, hi=1.0, dtype="f32", device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.rand(tuple(shape), generator=g, device=device, dtype=torch.float32)
    x = x * (hi - lo) + lo
    return x.to(_DT.get(dtype, dtype))


# ---------------------------------------------------------------------------
# Workload recipes.  Each returns a dict of named tensors.
# ---------------------------------------------------------------------------
def lbca_layer(tag, B, Hq, Hkv, T, d, m, kv_dtype, z_dtype, device="cpu",
               q_len=1, bias_std=0.1):
    """One LBCA (GQA) layer: K, V [B,Hkv,T,d], pooling logits z [B,Hkv,T,d],
    bias [Hkv,m,d] fp32, queries q [B,q_len,Hq,d] (all positions' queries when
    q_len = T)."""
    return {
        "k": normal((B, Hkv, T, d), seed_of(tag, "k"), dtype=kv_dtype, device=device),
        "v": normal((B, Hkv, T, d), seed_of(tag, "v"), dtype=kv_dtype, device=device),
        "z": normal((B, Hkv, T, d), seed_of(tag, "z"), dtype=z_dtype, device=device),
        "bias": normal((Hkv, m, d), seed_of(tag, "bias"), std=bias_std, device=device),
        "q": normal((B, q_len, Hq, d), seed_of(tag, "q"), dtype=kv_dtype, device=device),
    }


def hca_layer(tag, B, Hq, T, d, m, dtype="bf16", device="cpu", bias_std=0.1):
    """HCA: one shared series c [B,1,T,d], logits z [B,1,T,d], bias [1,m,d],
    decode queries q [B,Hq,d], sink logits [Hq] ~ N(0,1)."""
    return {
        "c": normal((B, 1, T, d), seed_of(tag, "c"), dtype=dtype, device=device),
        "z": normal((B, 1, T, d), seed_of(tag, "z"), dtype=dtype, device=device),
        "bias": normal((1, m, d), seed_of(tag, "bias"), std=bias_std, device=device),
        "q": normal((B, Hq, d), seed_of(tag, "q"), dtype=dtype, device=device),
        "sink": normal((Hq,), seed_of(tag, "sink"), device=device),
    }


def csa_layer(tag, B, Hq, T, d, m, HI, dI, dtype="bf16", device="cpu", bias_std=0.1, q_len=None):
    """CSA: a- and b-series with logits and biases for the core entries (dim d)
    and for the indexer keys (dim dI), decode queries, indexer queries and head
    weights U(0,1), sink logits.  With q_len, a chunk of q_len queries per
    sequence: q [B, q_len, Hq, d], qi [B, q_len, HI, dI], w [B, q_len, HI]."""
    lead = (B,) if q_len is None else (B, q_len)
    out = {}
    for s in ("a", "b"):
        out["c" + s] = normal((B, 1, T, d), seed_of(tag, "c" + s), dtype=dtype, device=device)
        out["z" + s] = normal((B, 1, T, d), seed_of(tag, "z" + s), dtype=dtype, device=device)
        out["bias_" + s] = normal((1, m, d), seed_of(tag, "bias_" + s), std=bias_std, device=device)
        out["ic" + s] = normal((B, 1, T, dI), seed_of(tag, "ic" + s), dtype=dtype, device=device)
        out["iz" + s] = normal((B, 1, T, dI), seed_of(tag, "iz" + s), dtype=dtype, device=device)
        out["ibias_" + s] = normal((1, m, dI), seed_of(tag, "ibias_" + s), std=bias_std, device=device)
    out["q"] = normal(lead + (Hq, d), seed_of(tag, "q"), dtype=dtype, device=device)
    out["qi"] = normal(lead + (HI, dI), seed_of(tag, "qi"), dtype=dtype, device=device)
    out["w"] = uniform(lead + (HI,), seed_of(tag, "w"), device=device)
    out["sink"] = normal((Hq,), seed_of(tag, "sink"), device=device)
    return out
