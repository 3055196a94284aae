"""Thin ctypes binding over liblbca.so (the C ABI in include/lbca.h).

Argument marshalling only: every step of the method runs in the HIP kernels.
PyTorch supplies device memory and the current HIP stream.  Tensors must
already be contiguous and on the GPU; nothing is copied or converted here.
Missing outputs and workspaces are allocated with ``torch.empty`` (plumbing).
If ``liblbca.so`` has not been built, the first call raises ``RuntimeError``.
"""
from __future__ import annotations

import ctypes
import math
import os
import re

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblbca.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "lbca.h")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4
F32, BF16 = 0, 1
EXCLUSIVE, OVERLAP = 0, 1

_i64, _i32, _f32, _vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p


class PoolArgs(ctypes.Structure):
    _fields_ = [("x", _vp), ("v", _vp), ("z", _vp), ("bias", _vp), ("xb", _vp), ("zb", _vp),
                ("bias_b", _vp), ("out_x", _vp), ("out_v", _vp),
                ("batch", _i64), ("heads", _i64), ("tokens", _i64), ("dim", _i64), ("block", _i64),
                ("entries", _i64), ("block_begin", _i64), ("block_end", _i64), ("pos_base", _i64),
                ("x_dtype", _i32), ("z_dtype", _i32), ("rmsnorm_eps", _f32), ("rope_dims", _i32),
                ("rope_base", _f32)]


class PoolGradArgs(ctypes.Structure):
    _fields_ = [("x", _vp), ("v", _vp), ("z", _vp), ("bias", _vp), ("grad_x", _vp), ("grad_v", _vp),
                ("dx", _vp), ("dv", _vp), ("dz", _vp), ("dbias", _vp),
                ("batch", _i64), ("heads", _i64), ("tokens", _i64), ("dim", _i64), ("block", _i64),
                ("entries", _i64), ("block_begin", _i64), ("block_end", _i64), ("pos_base", _i64),
                ("x_dtype", _i32), ("z_dtype", _i32), ("rmsnorm_eps", _f32), ("rope_dims", _i32),
                ("rope_base", _f32), ("xb", _vp), ("zb", _vp), ("bias_b", _vp), ("dxb", _vp), ("dzb", _vp),
                ("dbias_b", _vp)]


class CacheArgs(ctypes.Structure):
    _fields_ = [("x_new", _vp), ("v_new", _vp), ("z_new", _vp), ("raw_x", _vp), ("raw_v", _vp),
                ("raw_z", _vp), ("bias", _vp), ("out_x", _vp), ("out_v", _vp), ("pos", _vp),
                ("raw_pos_base", _vp),
                ("batch", _i64), ("heads", _i64), ("dim", _i64), ("block", _i64), ("window", _i64),
                ("ring", _i64), ("entries", _i64), ("mode", _i32), ("x_dtype", _i32), ("z_dtype", _i32),
                ("rmsnorm_eps", _f32), ("rope_dims", _i32), ("rope_base", _f32),
                ("xb_new", _vp), ("zb_new", _vp), ("raw_xb", _vp), ("raw_zb", _vp), ("bias_b", _vp)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("q", _vp), ("pooled_k", _vp), ("pooled_v", _vp), ("raw_k", _vp), ("raw_v", _vp),
                ("pos", _vp), ("raw_pos_base", _vp), ("sel_idx", _vp), ("sink", _vp), ("out", _vp),
                ("lse", _vp),
                ("batch", _i64), ("q_heads", _i64), ("kv_heads", _i64), ("dim", _i64), ("entries", _i64),
                ("raw_rows", _i64), ("k_sel", _i64), ("block", _i64), ("window", _i64),
                ("mode", _i32), ("dtype", _i32), ("scale", _f32), ("rmsnorm_eps", _f32),
                ("rope_dims", _i32), ("rope_base", _f32)]


class PrefillArgs(ctypes.Structure):
    _fields_ = [("q", _vp), ("pooled_k", _vp), ("pooled_v", _vp), ("raw_k", _vp), ("raw_v", _vp),
                ("sink", _vp), ("out", _vp), ("lse", _vp),
                ("batch", _i64), ("q_len", _i64), ("q_heads", _i64), ("kv_heads", _i64), ("dim", _i64),
                ("entries", _i64), ("raw_rows", _i64), ("q_pos0", _i64), ("raw_pos_base", _i64),
                ("block", _i64), ("window", _i64), ("mode", _i32), ("dtype", _i32), ("out_dtype", _i32),
                ("scale", _f32)]


class IndexArgs(ctypes.Structure):
    _fields_ = [("q_idx", _vp), ("head_w", _vp), ("keys", _vp), ("pos", _vp), ("out_idx", _vp),
                ("out_score", _vp),
                ("batch", _i64), ("heads", _i64), ("dim", _i64), ("entries", _i64), ("k", _i64),
                ("block", _i64), ("dtype", _i32)]


class CsaPrefillArgs(ctypes.Structure):
    _fields_ = [("q_idx", _vp), ("head_w", _vp), ("idx_keys", _vp), ("q", _vp), ("entries", _vp),
                ("raw", _vp), ("sink", _vp), ("out", _vp), ("lse", _vp), ("out_idx", _vp),
                ("batch", _i64), ("q_len", _i64), ("idx_heads", _i64), ("idx_dim", _i64),
                ("q_heads", _i64), ("dim", _i64), ("n_entries", _i64), ("raw_rows", _i64), ("k", _i64),
                ("q_pos0", _i64), ("raw_pos_base", _i64), ("block", _i64), ("window", _i64),
                ("dtype", _i32), ("scale", ctypes.c_float), ("rmsnorm_eps", ctypes.c_float),
                ("rope_dims", _i32), ("rope_base", ctypes.c_float)]


class LbcaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = lib().lbca_status_string(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")


_lib = None


def lib():
    """Open liblbca.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_compressed_kv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.lbca_abi_version.restype = ctypes.c_int
        L.lbca_status_string.restype = ctypes.c_char_p
        L.lbca_status_string.argtypes = [ctypes.c_int]
        L.lbca_visible_range.argtypes = [_i64, _i64, _i64, _i32, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]
        L.lbca_pool_blocks.argtypes = [ctypes.POINTER(PoolArgs), _vp]
        L.lbca_cache_append.argtypes = [ctypes.POINTER(CacheArgs), _vp]
        L.lbca_pool_blocks_backward_workspace.argtypes = [ctypes.POINTER(PoolGradArgs),
                                                          ctypes.POINTER(ctypes.c_size_t)]
        L.lbca_pool_blocks_backward.argtypes = [ctypes.POINTER(PoolGradArgs), _vp, ctypes.c_size_t, _vp]
        L.lbca_attend_decode_workspace.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.POINTER(ctypes.c_size_t)]
        L.lbca_attend_decode.argtypes = [ctypes.POINTER(DecodeArgs), _vp, ctypes.c_size_t, _vp]
        L.lbca_attend_prefill.argtypes = [ctypes.POINTER(PrefillArgs), _vp]
        L.csa_index_topk_workspace.argtypes = [ctypes.POINTER(IndexArgs), ctypes.POINTER(ctypes.c_size_t)]
        L.csa_index_topk.argtypes = [ctypes.POINTER(IndexArgs), _vp, ctypes.c_size_t, _vp]
        L.csa_sparse_prefill_workspace.argtypes = [ctypes.POINTER(CsaPrefillArgs), ctypes.POINTER(ctypes.c_size_t)]
        L.csa_sparse_prefill.argtypes = [ctypes.POINTER(CsaPrefillArgs), _vp, ctypes.c_size_t, _vp]
        for name in exported_names():
            getattr(L, name).restype = ctypes.c_int if name != "lbca_status_string" else ctypes.c_char_p
        if L.lbca_abi_version() != 1:
            raise RuntimeError("liblbca ABI version mismatch")
        _lib = L
    return _lib


def exported_names():
    """Every entry point declared in include/lbca.h."""
    text = open(HEADER).read()
    return re.findall(r"LBCA_API\s+(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", text)


def _check(status, where):
    if status != OK:
        raise LbcaError(status, where)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dt(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t, name, ndim=None):
    if t is None:
        return
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def visible_range(t, m, W, mode):
    """Host-only visibility rule from the library: (n_pooled, raw_begin)."""
    n, rb = _i64(), _i64()
    _check(lib().lbca_visible_range(t, m, W, mode, ctypes.byref(n), ctypes.byref(rb)),
           "lbca_visible_range")
    return n.value, rb.value


# ---------------------------------------------------------------------------
def pool_blocks(x, z, bias, block, block_begin, block_end, out_x, v=None, out_v=None, xb=None,
                zb=None, bias_b=None, pos_base=0, rmsnorm_eps=None, rope_dims=0,
                rope_base=10000.0, stream=None):
    """lbca_pool_blocks: x, v, z, xb, zb [B,H,T,d]; bias [H,m,d]; out [B,H,N,d]."""
    for t, n in ((x, "x"), (v, "v"), (z, "z"), (xb, "xb"), (zb, "zb"), (out_x, "out_x"), (out_v, "out_v")):
        _need(t, n, 4)
    _need(bias, "bias", 3)
    _need(bias_b, "bias_b", 3)
    B, H, T, d = x.shape
    a = PoolArgs(_p(x), _p(v), _p(z), _p(bias), _p(xb), _p(zb), _p(bias_b), _p(out_x), _p(out_v),
                 B, H, T, d, block, out_x.shape[2], block_begin, block_end, pos_base,
                 _dt(x), _dt(z), -1.0 if rmsnorm_eps is None else float(rmsnorm_eps), int(rope_dims),
                 float(rope_base))
    _check(lib().lbca_pool_blocks(ctypes.byref(a), _stream(stream)), "lbca_pool_blocks")
    return out_x if out_v is None else (out_x, out_v)


def _pool_grad_args(x, z, bias, block, block_begin, block_end, grad_x, dx, dz, dbias, v, grad_v, dv,
                    pos_base, rmsnorm_eps=None, rope_dims=0, rope_base=10000.0, xb=None, zb=None, bias_b=None,
                    dxb=None, dzb=None, dbias_b=None):
    for t, n in ((x, "x"), (v, "v"), (z, "z"), (grad_x, "grad_x"), (grad_v, "grad_v"), (dx, "dx"),
                 (dv, "dv"), (dz, "dz"), (xb, "xb"), (zb, "zb"), (dxb, "dxb"), (dzb, "dzb")):
        _need(t, n, 4)
    for t, n in ((bias, "bias"), (dbias, "dbias"), (bias_b, "bias_b"), (dbias_b, "dbias_b")):
        _need(t, n, 3)
    B, H, T, d = x.shape
    return PoolGradArgs(_p(x), _p(v), _p(z), _p(bias), _p(grad_x), _p(grad_v), _p(dx), _p(dv), _p(dz),
                        _p(dbias), B, H, T, d, block, grad_x.shape[2], block_begin, block_end, pos_base,
                        _dt(x), _dt(z), -1.0 if rmsnorm_eps is None else float(rmsnorm_eps), int(rope_dims),
                        float(rope_base), _p(xb), _p(zb), _p(bias_b), _p(dxb), _p(dzb), _p(dbias_b))


def pool_blocks_backward(x, z, bias, block, block_begin, block_end, grad_x, v=None, grad_v=None, dx=None,
                         dv=None, dz=None, dbias=None, pos_base=0, workspace=None, rmsnorm_eps=None, rope_dims=0,
                         rope_base=10000.0, xb=None, zb=None, bias_b=None, dxb=None, dzb=None, dbias_b=None,
                         stream=None):
    """lbca_pool_blocks_backward: gradients of pool_blocks (single series with optional values,
    the shared series with its entry treatment, or dual mode with xb, zb, bias_b).
    Returns (dx, dv or None, dz, dbias), plus (dxb, dzb, dbias_b) in dual mode; missing outputs
    are allocated (rows outside the pooled blocks of new outputs are zeros)."""
    dx = torch.zeros_like(x) if dx is None else dx
    dz = torch.zeros_like(z) if dz is None else dz
    if v is not None and dv is None:
        dv = torch.zeros_like(v)
    if dbias is None:
        dbias = torch.empty_like(bias)
    dual = xb is not None
    if dual:
        dxb = torch.zeros_like(xb) if dxb is None else dxb
        dzb = torch.zeros_like(zb) if dzb is None else dzb
        dbias_b = torch.empty_like(bias_b) if dbias_b is None else dbias_b
    a = _pool_grad_args(x, z, bias, block, block_begin, block_end, grad_x, dx, dz, dbias, v, grad_v, dv,
                        pos_base, rmsnorm_eps, rope_dims, rope_base, xb, zb, bias_b, dxb, dzb, dbias_b)
    if workspace is None:
        n = ctypes.c_size_t()
        _check(lib().lbca_pool_blocks_backward_workspace(ctypes.byref(a), ctypes.byref(n)),
               "lbca_pool_blocks_backward_workspace")
        workspace = torch.empty(max(n.value, 16), dtype=torch.uint8, device=x.device)
    _check(lib().lbca_pool_blocks_backward(ctypes.byref(a), _p(workspace), workspace.numel(), _stream(stream)),
           "lbca_pool_blocks_backward")
    return (dx, dv, dz, dbias, dxb, dzb, dbias_b) if dual else (dx, dv, dz, dbias)


def pool_blocks_backward_workspace_bytes(x, z, bias, block, block_begin, block_end, grad_x, v=None,
                                         grad_v=None, pos_base=0, xb=None, zb=None, bias_b=None, **treat):
    a = _pool_grad_args(x, z, bias, block, block_begin, block_end, grad_x, x, z, bias, v, grad_v, v, pos_base,
                        treat.get("rmsnorm_eps"), treat.get("rope_dims", 0), treat.get("rope_base", 10000.0),
                        xb, zb, bias_b, xb, zb, bias_b)
    n = ctypes.c_size_t()
    _check(lib().lbca_pool_blocks_backward_workspace(ctypes.byref(a), ctypes.byref(n)),
           "lbca_pool_blocks_backward_workspace")
    return n.value


def cache_append(x_new, z_new, raw_x, raw_z, bias, pos, raw_pos_base, block, window, mode, out_x,
                 v_new=None, raw_v=None, out_v=None, rmsnorm_eps=None, rope_dims=0, rope_base=10000.0,
                 xb_new=None, zb_new=None, raw_xb=None, raw_zb=None, bias_b=None, stream=None):
    """lbca_cache_append: x_new, v_new, z_new [B,H,d]; raw_* [B,H,2*ring,d] (mirrored ring);
    bias [H,m,d]; out [B,H,N,d]; pos, raw_pos_base [B] int64 (raw_pos_base is written).
    Dual (CSA) mode: xb_new, zb_new, raw_xb, raw_zb, bias_b for the b-series."""
    for t, n, nd in ((x_new, "x_new", 3), (v_new, "v_new", 3), (z_new, "z_new", 3), (raw_x, "raw_x", 4),
                     (raw_v, "raw_v", 4), (raw_z, "raw_z", 4), (bias, "bias", 3), (out_x, "out_x", 4),
                     (out_v, "out_v", 4), (pos, "pos", 1), (raw_pos_base, "raw_pos_base", 1),
                     (xb_new, "xb_new", 3), (zb_new, "zb_new", 3), (raw_xb, "raw_xb", 4), (raw_zb, "raw_zb", 4),
                     (bias_b, "bias_b", 3)):
        _need(t, n, nd)
    B, H, d = x_new.shape
    if raw_x.shape[2] % 2:
        raise ValueError("raw buffers hold 2 * ring rows")
    a = CacheArgs(_p(x_new), _p(v_new), _p(z_new), _p(raw_x), _p(raw_v), _p(raw_z), _p(bias), _p(out_x),
                  _p(out_v), _p(pos), _p(raw_pos_base), B, H, d, block, window, raw_x.shape[2] // 2,
                  out_x.shape[2], mode, _dt(x_new), _dt(z_new),
                  -1.0 if rmsnorm_eps is None else float(rmsnorm_eps), int(rope_dims), float(rope_base),
                  _p(xb_new), _p(zb_new), _p(raw_xb), _p(raw_zb), _p(bias_b))
    _check(lib().lbca_cache_append(ctypes.byref(a), _stream(stream)), "lbca_cache_append")


def _decode_args(q, pooled_k, raw_k, pos, block, window, mode, out, lse, pooled_v, raw_v,
                 raw_pos_base, sel_idx, sink, scale, rmsnorm_eps, rope_dims, rope_base):
    for t, n, nd in ((q, "q", 3), (pooled_k, "pooled_k", 4), (pooled_v, "pooled_v", 4),
                     (raw_k, "raw_k", 4), (raw_v, "raw_v", 4), (sel_idx, "sel_idx", 2),
                     (out, "out", 3)):
        _need(t, n, nd)
    B, Hq, d = q.shape
    Hkv, N = pooled_k.shape[1], pooled_k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return DecodeArgs(_p(q), _p(pooled_k), _p(pooled_v), _p(raw_k), _p(raw_v), _p(pos),
                      _p(raw_pos_base), _p(sel_idx), _p(sink), _p(out), _p(lse),
                      B, Hq, Hkv, d, N, raw_k.shape[2], 0 if sel_idx is None else sel_idx.shape[1],
                      block, window, mode, _dt(q), float(scale),
                      -1.0 if rmsnorm_eps is None else float(rmsnorm_eps), int(rope_dims),
                      float(rope_base))


def decode_workspace_bytes(q, pooled_k, raw_k, pos, block, window, mode, **kw):
    out = kw.pop("out", None)
    a = _decode_args(q, pooled_k, raw_k, pos, block, window, mode, out if out is not None else q,
                     kw.get("lse"), kw.get("pooled_v"), kw.get("raw_v"), kw.get("raw_pos_base"),
                     kw.get("sel_idx"), kw.get("sink"), kw.get("scale"), kw.get("rmsnorm_eps"),
                     kw.get("rope_dims", 0), kw.get("rope_base", 10000.0))
    n = ctypes.c_size_t()
    _check(lib().lbca_attend_decode_workspace(ctypes.byref(a), ctypes.byref(n)),
           "lbca_attend_decode_workspace")
    return n.value


def attend_decode(q, pooled_k, raw_k, pos, block, window, mode, out=None, lse=None, pooled_v=None,
                  raw_v=None, raw_pos_base=None, sel_idx=None, sink=None, scale=None,
                  rmsnorm_eps=None, rope_dims=0, rope_base=10000.0, workspace=None, stream=None):
    """lbca_attend_decode; returns (out [B,Hq,d] fp32, lse [B,Hq] fp32)."""
    B, Hq, d = q.shape
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    a = _decode_args(q, pooled_k, raw_k, pos, block, window, mode, out, lse, pooled_v, raw_v,
                     raw_pos_base, sel_idx, sink, scale, rmsnorm_eps, rope_dims, rope_base)
    need = ctypes.c_size_t()
    _check(lib().lbca_attend_decode_workspace(ctypes.byref(a), ctypes.byref(need)),
           "lbca_attend_decode_workspace")
    if workspace is None and need.value > 0:  # split partials; contents on entry do not matter
        workspace = torch.empty(need.value, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().lbca_attend_decode(ctypes.byref(a), _p(workspace), ws_bytes, _stream(stream)),
           "lbca_attend_decode")
    return out, lse


def attend_prefill(q, q_pos0, pooled_k, raw_k, raw_pos_base, block, window, mode, out=None,
                   lse=None, pooled_v=None, raw_v=None, sink=None, scale=None, out_dtype=None,
                   stream=None):
    """lbca_attend_prefill: q [B,Tq,Hq,d]; returns (out [B,Tq,Hq,d], lse [B,Tq,Hq])."""
    for t, n, nd in ((q, "q", 4), (pooled_k, "pooled_k", 4), (pooled_v, "pooled_v", 4),
                     (raw_k, "raw_k", 4), (raw_v, "raw_v", 4)):
        _need(t, n, nd)
    B, Tq, Hq, d = q.shape
    if out is None:
        out = torch.empty((B, Tq, Hq, d), dtype=out_dtype or q.dtype, device=q.device)
    _need(out, "out", 4)
    if lse is None:
        lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    a = PrefillArgs(_p(q), _p(pooled_k), _p(pooled_v), _p(raw_k), _p(raw_v), _p(sink), _p(out), _p(lse),
                    B, Tq, Hq, pooled_k.shape[1], d, pooled_k.shape[2], raw_k.shape[2], q_pos0,
                    raw_pos_base, block, window, mode, _dt(q), _dt(out), float(scale))
    _check(lib().lbca_attend_prefill(ctypes.byref(a), _stream(stream)), "lbca_attend_prefill")
    return out, lse


def index_workspace_bytes(q_idx, head_w, keys, pos, block, k):
    """csa_index_topk_workspace: bytes of workspace csa_index_topk needs for these shapes
    (the query's buffer stands in for the output, which the size does not depend on)."""
    B, HI, dI = q_idx.shape
    a = IndexArgs(_p(q_idx), _p(head_w), _p(keys), _p(pos), _p(q_idx), None,
                  B, HI, dI, keys.shape[1], k, block, _dt(q_idx))
    need = ctypes.c_size_t()
    _check(lib().csa_index_topk_workspace(ctypes.byref(a), ctypes.byref(need)), "csa_index_topk_workspace")
    return need.value


def csa_index_topk(q_idx, head_w, keys, pos, block, k, out_idx=None, out_score=None,
                   workspace=None, stream=None):
    """csa_index_topk: q_idx [B,HI,dI], head_w [B,HI], keys [B,N,dI]; returns (idx, score)."""
    for t, n, nd in ((q_idx, "q_idx", 3), (head_w, "head_w", 2), (keys, "keys", 3)):
        _need(t, n, nd)
    B, HI, dI = q_idx.shape
    if out_idx is None:
        out_idx = torch.empty((B, k), dtype=torch.int32, device=q_idx.device)
    if out_score is None:
        out_score = torch.empty((B, k), dtype=torch.float32, device=q_idx.device)
    a = IndexArgs(_p(q_idx), _p(head_w), _p(keys), _p(pos), _p(out_idx), _p(out_score),
                  B, HI, dI, keys.shape[1], k, block, _dt(q_idx))
    need = ctypes.c_size_t()
    _check(lib().csa_index_topk_workspace(ctypes.byref(a), ctypes.byref(need)), "csa_index_topk_workspace")
    if workspace is None and need.value > 0:
        workspace = torch.empty(need.value, dtype=torch.uint8, device=q_idx.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().csa_index_topk(ctypes.byref(a), _p(workspace), ws_bytes, _stream(stream)),
           "csa_index_topk")
    return out_idx, out_score


def _csa_prefill_args(q_idx, head_w, idx_keys, q, entries, raw, q_pos0, raw_pos_base, block, window, k,
                      out, lse, out_idx, sink, scale, rmsnorm_eps, rope_dims, rope_base):
    for t, n, nd in ((q_idx, "q_idx", 4), (head_w, "head_w", 3), (idx_keys, "idx_keys", 3), (q, "q", 4),
                     (entries, "entries", 3), (raw, "raw", 3), (out, "out", 4), (out_idx, "out_idx", 3)):
        _need(t, n, nd)
    B, Tq, Hq, d = q.shape
    HI, dI = q_idx.shape[2], q_idx.shape[3]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return CsaPrefillArgs(_p(q_idx), _p(head_w), _p(idx_keys), _p(q), _p(entries), _p(raw), _p(sink), _p(out),
                          _p(lse), _p(out_idx), B, Tq, HI, dI, Hq, d, entries.shape[1], raw.shape[1], k,
                          q_pos0, raw_pos_base, block, window, _dt(q), float(scale),
                          -1.0 if rmsnorm_eps is None else float(rmsnorm_eps), int(rope_dims), float(rope_base))


def csa_sparse_prefill_workspace_bytes(q_idx, head_w, idx_keys, q, entries, raw, q_pos0, raw_pos_base, block,
                                      window, k, out=None, lse=None, out_idx=None, sink=None, scale=None,
                                      rmsnorm_eps=None, rope_dims=0, rope_base=10000.0):
    """csa_sparse_prefill_workspace: bytes of workspace csa_sparse_prefill needs for these shapes
    (the query's buffer stands in for an absent output, which the size does not depend on)."""
    a = _csa_prefill_args(q_idx, head_w, idx_keys, q, entries, raw, q_pos0, raw_pos_base, block, window, k,
                          q if out is None else out, lse, out_idx, sink, scale, rmsnorm_eps, rope_dims, rope_base)
    need = ctypes.c_size_t()
    _check(lib().csa_sparse_prefill_workspace(ctypes.byref(a), ctypes.byref(need)), "csa_sparse_prefill_workspace")
    return need.value


def csa_sparse_prefill(q_idx, head_w, idx_keys, q, entries, raw, q_pos0, raw_pos_base, block, window, k,
                       out=None, lse=None, out_idx=None, sink=None, scale=None, rmsnorm_eps=None, rope_dims=0,
                       rope_base=10000.0, workspace=None, stream=None):
    """csa_sparse_prefill: q_idx [B,Tq,HI,dI], head_w [B,Tq,HI], idx_keys [B,N,dI], q [B,Tq,Hq,d],
    entries [B,N,d], raw [B,R,d]; returns (out [B,Tq,Hq,d] fp32, lse [B,Tq,Hq], idx [B,Tq,k] int32)."""
    B, Tq, Hq, d = q.shape
    if out is None:
        out = torch.empty((B, Tq, Hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=q.device)
    if out_idx is None:
        out_idx = torch.empty((B, Tq, k), dtype=torch.int32, device=q.device)
    a = _csa_prefill_args(q_idx, head_w, idx_keys, q, entries, raw, q_pos0, raw_pos_base, block, window, k,
                          out, lse, out_idx, sink, scale, rmsnorm_eps, rope_dims, rope_base)
    need = ctypes.c_size_t()
    _check(lib().csa_sparse_prefill_workspace(ctypes.byref(a), ctypes.byref(need)), "csa_sparse_prefill_workspace")
    if workspace is None:  # positions, selections, scores; contents on entry do not matter
        workspace = torch.empty(max(need.value, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().csa_sparse_prefill(ctypes.byref(a), _p(workspace), ws_bytes, _stream(stream)),
           "csa_sparse_prefill")
    return out, lse, out_idx
