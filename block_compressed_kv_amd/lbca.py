"""Thin ctypes binding over liblbca.so (the C ABI in include/lbca.h).

Argument marshalling only: every step of the method runs in the HIP kernels.
PyTorch supplies device memory and the current HIP stream.  Tensors must be
on the GPU.  Queries, keys, values, logits, outputs and their gradients may be
strided views (their last dimension contiguous): their strides go to the
library as they are.  Per-head and per-sequence vectors, positions, index
lists and biases must be contiguous.  Nothing is copied or converted here.
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

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_TOO_LARGE = 0, -1, -2, -3, -4, -5
NOALLOC_SCRATCH_BYTES = 16 << 20
F32, BF16 = 0, 1
EXCLUSIVE, OVERLAP = 0, 1

_i64, _i32, _f32, _vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p


class Strides(ctypes.Structure):
    """lbca_strides: element strides of every dimension but the last, outermost first."""
    _fields_ = [("s", _i64 * 3)]


def _stf(*names):
    return [(n, Strides) for n in names]


class PoolArgs(ctypes.Structure):
    _fields_ = [("x", _vp), ("v", _vp), ("z", _vp), ("bias", _vp), ("xb", _vp), ("zb", _vp),
                ("bias_b", _vp), ("out_x", _vp), ("out_v", _vp),
                ("batch", _i64), ("heads", _i64), ("tokens", _i64), ("dim", _i64), ("block", _i64),
                ("entries", _i64), ("block_begin", _i64), ("block_end", _i64), ("pos_base", _i64),
                ("x_dtype", _i32), ("z_dtype", _i32), ("rmsnorm_eps", _f32), ("rope_dims", _i32),
                ("rope_base", _f32)] + _stf("x_st", "v_st", "z_st", "xb_st", "zb_st", "out_x_st", "out_v_st")


class PoolGradArgs(ctypes.Structure):
    _fields_ = [("x", _vp), ("v", _vp), ("z", _vp), ("bias", _vp), ("grad_x", _vp), ("grad_v", _vp),
                ("dx", _vp), ("dv", _vp), ("dz", _vp), ("dbias", _vp),
                ("batch", _i64), ("heads", _i64), ("tokens", _i64), ("dim", _i64), ("block", _i64),
                ("entries", _i64), ("block_begin", _i64), ("block_end", _i64), ("pos_base", _i64),
                ("x_dtype", _i32), ("z_dtype", _i32), ("rmsnorm_eps", _f32), ("rope_dims", _i32),
                ("rope_base", _f32), ("xb", _vp), ("zb", _vp), ("bias_b", _vp), ("dxb", _vp), ("dzb", _vp),
                ("dbias_b", _vp)] + _stf("x_st", "v_st", "z_st", "grad_x_st", "grad_v_st", "dx_st", "dv_st",
                                          "dz_st", "xb_st", "zb_st", "dxb_st", "dzb_st")


class CacheArgs(ctypes.Structure):
    _fields_ = [("x_new", _vp), ("v_new", _vp), ("z_new", _vp), ("raw_x", _vp), ("raw_v", _vp),
                ("raw_z", _vp), ("bias", _vp), ("out_x", _vp), ("out_v", _vp), ("pos", _vp),
                ("raw_pos_base", _vp),
                ("batch", _i64), ("heads", _i64), ("dim", _i64), ("block", _i64), ("window", _i64),
                ("ring", _i64), ("entries", _i64), ("mode", _i32), ("x_dtype", _i32), ("z_dtype", _i32),
                ("rmsnorm_eps", _f32), ("rope_dims", _i32), ("rope_base", _f32),
                ("xb_new", _vp), ("zb_new", _vp), ("raw_xb", _vp), ("raw_zb", _vp), ("bias_b", _vp)] + _stf(
                    "x_new_st", "v_new_st", "z_new_st", "raw_x_st", "raw_v_st", "raw_z_st", "out_x_st", "out_v_st",
                    "xb_new_st", "zb_new_st", "raw_xb_st", "raw_zb_st")


class DecodeArgs(ctypes.Structure):
    _fields_ = [("q", _vp), ("pooled_k", _vp), ("pooled_v", _vp), ("raw_k", _vp), ("raw_v", _vp),
                ("pos", _vp), ("raw_pos_base", _vp), ("sel_idx", _vp), ("sink", _vp), ("out", _vp),
                ("lse", _vp),
                ("batch", _i64), ("q_heads", _i64), ("kv_heads", _i64), ("dim", _i64), ("entries", _i64),
                ("raw_rows", _i64), ("k_sel", _i64), ("block", _i64), ("window", _i64),
                ("mode", _i32), ("dtype", _i32), ("scale", _f32), ("rmsnorm_eps", _f32),
                ("rope_dims", _i32), ("rope_base", _f32)] + _stf("q_st", "pooled_k_st", "pooled_v_st", "raw_k_st",
                                                                  "raw_v_st", "out_st")


class PrefillArgs(ctypes.Structure):
    _fields_ = [("q", _vp), ("pooled_k", _vp), ("pooled_v", _vp), ("raw_k", _vp), ("raw_v", _vp),
                ("sink", _vp), ("out", _vp), ("lse", _vp),
                ("batch", _i64), ("q_len", _i64), ("q_heads", _i64), ("kv_heads", _i64), ("dim", _i64),
                ("entries", _i64), ("raw_rows", _i64), ("q_pos0", _i64), ("raw_pos_base", _i64),
                ("block", _i64), ("window", _i64), ("mode", _i32), ("dtype", _i32), ("out_dtype", _i32),
                ("scale", _f32)] + _stf("q_st", "pooled_k_st", "pooled_v_st", "raw_k_st", "raw_v_st", "out_st")


class PrefillGradArgs(ctypes.Structure):
    _fields_ = [("q", _vp), ("pooled_k", _vp), ("pooled_v", _vp), ("raw_k", _vp), ("raw_v", _vp),
                ("sink", _vp), ("out", _vp), ("lse", _vp), ("grad_out", _vp), ("grad_q", _vp),
                ("grad_pooled_k", _vp), ("grad_pooled_v", _vp), ("grad_raw_k", _vp), ("grad_raw_v", _vp),
                ("grad_sink", _vp),
                ("batch", _i64), ("q_len", _i64), ("q_heads", _i64), ("kv_heads", _i64), ("dim", _i64),
                ("entries", _i64), ("raw_rows", _i64), ("q_pos0", _i64), ("raw_pos_base", _i64),
                ("block", _i64), ("window", _i64), ("mode", _i32), ("dtype", _i32), ("out_dtype", _i32),
                ("accumulate", _i32), ("scale", _f32)] + _stf(
                    "q_st", "pooled_k_st", "pooled_v_st", "raw_k_st", "raw_v_st", "out_st", "grad_out_st",
                    "grad_q_st", "grad_pooled_k_st", "grad_pooled_v_st", "grad_raw_k_st", "grad_raw_v_st")


class StepArgs(ctypes.Structure):
    _fields_ = [("q", _vp), ("k_new", _vp), ("v_new", _vp), ("z_new", _vp), ("raw_k", _vp), ("raw_v", _vp),
                ("raw_z", _vp), ("bias", _vp), ("pooled_k", _vp), ("pooled_v", _vp), ("pos", _vp),
                ("raw_pos_base", _vp), ("sink", _vp), ("out", _vp), ("lse", _vp),
                ("batch", _i64), ("q_heads", _i64), ("kv_heads", _i64), ("dim", _i64), ("block", _i64),
                ("window", _i64), ("ring", _i64), ("entries", _i64), ("dtype", _i32), ("z_dtype", _i32),
                ("scale", _f32)] + _stf("q_st", "k_new_st", "v_new_st", "z_new_st", "raw_k_st", "raw_v_st",
                                        "raw_z_st", "pooled_k_st", "pooled_v_st", "out_st")


class IndexArgs(ctypes.Structure):
    _fields_ = [("q_idx", _vp), ("head_w", _vp), ("keys", _vp), ("pos", _vp), ("out_idx", _vp),
                ("out_score", _vp),
                ("batch", _i64), ("heads", _i64), ("dim", _i64), ("entries", _i64), ("k", _i64),
                ("block", _i64), ("dtype", _i32)] + _stf("q_idx_st", "keys_st")


class CsaPrefillArgs(ctypes.Structure):
    _fields_ = [("q_idx", _vp), ("head_w", _vp), ("idx_keys", _vp), ("q", _vp), ("entries", _vp),
                ("raw", _vp), ("sink", _vp), ("out", _vp), ("lse", _vp), ("out_idx", _vp),
                ("batch", _i64), ("q_len", _i64), ("idx_heads", _i64), ("idx_dim", _i64),
                ("q_heads", _i64), ("dim", _i64), ("n_entries", _i64), ("raw_rows", _i64), ("k", _i64),
                ("q_pos0", _i64), ("raw_pos_base", _i64), ("block", _i64), ("window", _i64),
                ("dtype", _i32), ("scale", ctypes.c_float), ("rmsnorm_eps", ctypes.c_float),
                ("rope_dims", _i32), ("rope_base", ctypes.c_float)] + _stf(
                    "q_idx_st", "idx_keys_st", "q_st", "entries_st", "raw_st", "out_st")


class GemmArgs(ctypes.Structure):
    _fields_ = [("a", _vp), ("w", _vp), ("c", _vp), ("groups", _i64), ("m", _i64), ("n", _i64), ("k", _i64),
                ("lda", _i64), ("ldw", _i64), ("ldc", _i64), ("a_group_stride", _i64), ("w_group_stride", _i64),
                ("c_group_stride", _i64), ("a_dtype", _i32), ("c_dtype", _i32)]


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
        L.lbca_attend_decode_noalloc.argtypes = [ctypes.POINTER(DecodeArgs), _vp]
        L.lbca_attend_prefill.argtypes = [ctypes.POINTER(PrefillArgs), _vp]
        L.lbca_decode_step_workspace.argtypes = [ctypes.POINTER(StepArgs), ctypes.POINTER(ctypes.c_size_t)]
        L.lbca_decode_step.argtypes = [ctypes.POINTER(StepArgs), _vp, ctypes.c_size_t, _vp]
        L.lbca_attend_prefill_backward_workspace.argtypes = [ctypes.POINTER(PrefillGradArgs),
                                                             ctypes.POINTER(ctypes.c_size_t)]
        L.lbca_attend_prefill_backward.argtypes = [ctypes.POINTER(PrefillGradArgs), _vp, ctypes.c_size_t, _vp]
        L.csa_index_topk_workspace.argtypes = [ctypes.POINTER(IndexArgs), ctypes.POINTER(ctypes.c_size_t)]
        L.csa_index_topk.argtypes = [ctypes.POINTER(IndexArgs), _vp, ctypes.c_size_t, _vp]
        L.csa_sparse_prefill_workspace.argtypes = [ctypes.POINTER(CsaPrefillArgs), ctypes.POINTER(ctypes.c_size_t)]
        L.csa_sparse_prefill.argtypes = [ctypes.POINTER(CsaPrefillArgs), _vp, ctypes.c_size_t, _vp]
        L.lbca_grouped_gemm.argtypes = [ctypes.POINTER(GemmArgs), _vp]
        for name in exported_names():
            getattr(L, name).restype = ctypes.c_int if name != "lbca_status_string" else ctypes.c_char_p
        if L.lbca_abi_version() != 2:
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


_EMPTY = 256  # non-null, aligned address passed for a buffer with no elements (never dereferenced)


def _p(t):
    """Device pointer of t for the C ABI; None stays NULL (an absent optional buffer).
    A tensor with no elements may have a null data pointer, which the ABI would read
    as an absent buffer, so it is passed as a placeholder address: the library never
    reads or writes a buffer of size 0."""
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr() if t.numel() > 0 else _EMPTY)


def _dt(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t, name, ndim=None):
    if t is None:
        return
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


_FLOAT = (torch.float32, torch.bfloat16)


def _expect(t, name, shape, dtypes=_FLOAT, device=None, strided=False):
    """The library sees raw pointers only, so every buffer's full shape, dtype and
    device are checked here: a short buffer would otherwise be read or written
    past its end.  strided: a view whose last dimension is contiguous (its
    strides are passed with it), else a contiguous tensor."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be one of {dtypes}, got {t.dtype}")
    if strided:
        if t.dim() > 0 and t.shape[-1] > 1 and t.stride(-1) != 1:
            raise ValueError(f"{name} must have a contiguous last dimension")
        if t.numel() > 1 and all(st == 0 for st, n in zip(t.stride()[:-1], t.shape[:-1]) if n > 1) and \
                any(n > 1 for n in t.shape[:-1]):
            raise ValueError(f"{name}: a view that repeats one row everywhere is not accepted")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _st(t):
    """lbca_strides of t: its element strides but the last (0 for dimensions of extent 1)."""
    st = Strides()
    if t is not None:
        for i, (n, s) in enumerate(zip(t.shape[:-1], t.stride()[:-1])):
            st.s[i] = s if n > 1 else 0
    return st


def _set_st(a, **tensors):
    """Fills the named stride fields of the argument struct a from the tensors."""
    for name, t in tensors.items():
        setattr(a, name + "_st", _st(t))
    return a


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
    _need(x, "x", 4)
    _need(out_x, "out_x", 4)
    B, H, T, d = x.shape
    N, dev, xt = out_x.shape[2], x.device, (x.dtype,)
    _expect(x, "x", (B, H, T, d), strided=True)
    _expect(z, "z", (B, H, T, d), device=dev, strided=True)
    for t, n in ((v, "v"), (xb, "xb")):
        _expect(t, n, (B, H, T, d), xt, dev, strided=True)
    _expect(zb, "zb", (B, H, T, d), (z.dtype,), dev, strided=True)
    for t, n in ((out_x, "out_x"), (out_v, "out_v")):
        _expect(t, n, (B, H, N, d), xt, dev, strided=True)
    for t, n in ((bias, "bias"), (bias_b, "bias_b")):
        _expect(t, n, (H, block, d), (torch.float32,), dev)
    a = PoolArgs(_p(x), _p(v), _p(z), _p(bias), _p(xb), _p(zb), _p(bias_b), _p(out_x), _p(out_v),
                 B, H, T, d, block, out_x.shape[2], block_begin, block_end, pos_base,
                 _dt(x), _dt(z), -1.0 if rmsnorm_eps is None else float(rmsnorm_eps), int(rope_dims),
                 float(rope_base))
    _set_st(a, x=x, v=v, z=z, xb=xb, zb=zb, out_x=out_x, out_v=out_v)
    _check(lib().lbca_pool_blocks(ctypes.byref(a), _stream(stream)), "lbca_pool_blocks")
    return out_x if out_v is None else (out_x, out_v)


def _pool_grad_args(x, z, bias, block, block_begin, block_end, grad_x, dx, dz, dbias, v, grad_v, dv,
                    pos_base, rmsnorm_eps=None, rope_dims=0, rope_base=10000.0, xb=None, zb=None, bias_b=None,
                    dxb=None, dzb=None, dbias_b=None):
    _need(x, "x", 4)
    _need(grad_x, "grad_x", 4)
    B, H, T, d = x.shape
    N, dev, xt, zt = grad_x.shape[2], x.device, (x.dtype,), (z.dtype,)
    _expect(x, "x", (B, H, T, d), strided=True)
    _expect(z, "z", (B, H, T, d), device=dev, strided=True)
    for t, n in ((v, "v"), (dx, "dx"), (dv, "dv"), (xb, "xb"), (dxb, "dxb")):
        _expect(t, n, (B, H, T, d), xt, dev, strided=True)
    for t, n in ((dz, "dz"), (zb, "zb"), (dzb, "dzb")):
        _expect(t, n, (B, H, T, d), zt, dev, strided=True)
    for t, n in ((grad_x, "grad_x"), (grad_v, "grad_v")):
        _expect(t, n, (B, H, N, d), xt, dev, strided=True)
    for t, n in ((bias, "bias"), (dbias, "dbias"), (bias_b, "bias_b"), (dbias_b, "dbias_b")):
        _expect(t, n, (H, block, d), (torch.float32,), dev)
    a = PoolGradArgs(_p(x), _p(v), _p(z), _p(bias), _p(grad_x), _p(grad_v), _p(dx), _p(dv), _p(dz),
                     _p(dbias), B, H, T, d, block, grad_x.shape[2], block_begin, block_end, pos_base,
                     _dt(x), _dt(z), -1.0 if rmsnorm_eps is None else float(rmsnorm_eps), int(rope_dims),
                     float(rope_base), _p(xb), _p(zb), _p(bias_b), _p(dxb), _p(dzb), _p(dbias_b))
    return _set_st(a, x=x, v=v, z=z, grad_x=grad_x, grad_v=grad_v, dx=dx, dv=dv, dz=dz, xb=xb, zb=zb, dxb=dxb,
                   dzb=dzb)


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
    for t, n, nd in ((x_new, "x_new", 3), (raw_x, "raw_x", 4), (out_x, "out_x", 4)):
        _need(t, n, nd)
    B, H, d = x_new.shape
    if raw_x.shape[2] % 2:
        raise ValueError("raw buffers hold 2 * ring rows")
    R2, N, dev, xt, zt = raw_x.shape[2], out_x.shape[2], x_new.device, (x_new.dtype,), (z_new.dtype,)
    _expect(x_new, "x_new", (B, H, d), strided=True)
    for t, n in ((v_new, "v_new"), (xb_new, "xb_new")):
        _expect(t, n, (B, H, d), xt, dev, strided=True)
    for t, n in ((z_new, "z_new"), (zb_new, "zb_new")):
        _expect(t, n, (B, H, d), zt, dev, strided=True)
    for t, n in ((raw_x, "raw_x"), (raw_v, "raw_v"), (raw_xb, "raw_xb")):
        _expect(t, n, (B, H, R2, d), xt, dev, strided=True)
    for t, n in ((raw_z, "raw_z"), (raw_zb, "raw_zb")):
        _expect(t, n, (B, H, R2, d), zt, dev, strided=True)
    for t, n in ((out_x, "out_x"), (out_v, "out_v")):
        _expect(t, n, (B, H, N, d), xt, dev, strided=True)
    for t, n in ((bias, "bias"), (bias_b, "bias_b")):
        _expect(t, n, (H, block, d), (torch.float32,), dev)
    for t, n in ((pos, "pos"), (raw_pos_base, "raw_pos_base")):
        _expect(t, n, (B,), (torch.int64,), dev)
    a = CacheArgs(_p(x_new), _p(v_new), _p(z_new), _p(raw_x), _p(raw_v), _p(raw_z), _p(bias), _p(out_x),
                  _p(out_v), _p(pos), _p(raw_pos_base), B, H, d, block, window, raw_x.shape[2] // 2,
                  out_x.shape[2], mode, _dt(x_new), _dt(z_new),
                  -1.0 if rmsnorm_eps is None else float(rmsnorm_eps), int(rope_dims), float(rope_base),
                  _p(xb_new), _p(zb_new), _p(raw_xb), _p(raw_zb), _p(bias_b))
    _set_st(a, x_new=x_new, v_new=v_new, z_new=z_new, raw_x=raw_x, raw_v=raw_v, raw_z=raw_z, out_x=out_x,
            out_v=out_v, xb_new=xb_new, zb_new=zb_new, raw_xb=raw_xb, raw_zb=raw_zb)
    _check(lib().lbca_cache_append(ctypes.byref(a), _stream(stream)), "lbca_cache_append")


def decode_step(q, k_new, v_new, z_new, raw_k, raw_v, raw_z, bias, pooled_k, pooled_v, pos, raw_pos_base,
                block, window, out=None, lse=None, sink=None, scale=None, workspace=None, stream=None):
    """lbca_decode_step (EXCLUSIVE rule): append k/v/z_new [B,Hkv,d] to the mirrored ring
    raw_* [B,Hkv,2*ring,d], pool the block the token completes into pooled_* [B,Hkv,N,d],
    write raw_pos_base [B], and decode q [B,Hq,d] at pos [B]; returns (out, lse)."""
    for t, n, nd in ((q, "q", 3), (k_new, "k_new", 3), (raw_k, "raw_k", 4), (pooled_k, "pooled_k", 4)):
        _need(t, n, nd)
    B, Hq, d = q.shape
    Hkv, R2, N, dev, qt, zt = k_new.shape[1], raw_k.shape[2], pooled_k.shape[2], q.device, (q.dtype,), (z_new.dtype,)
    if R2 % 2:
        raise ValueError("raw buffers hold 2 * ring rows")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    _expect(q, "q", (B, Hq, d), strided=True)
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _expect(t, n, (B, Hkv, d), qt, dev, strided=True)
    _expect(z_new, "z_new", (B, Hkv, d), device=dev, strided=True)
    for t, n in ((raw_k, "raw_k"), (raw_v, "raw_v")):
        _expect(t, n, (B, Hkv, R2, d), qt, dev, strided=True)
    _expect(raw_z, "raw_z", (B, Hkv, R2, d), zt, dev, strided=True)
    _expect(bias, "bias", (Hkv, block, d), (torch.float32,), dev)
    for t, n in ((pooled_k, "pooled_k"), (pooled_v, "pooled_v")):
        _expect(t, n, (B, Hkv, N, d), qt, dev, strided=True)
    for t, n in ((pos, "pos"), (raw_pos_base, "raw_pos_base")):
        _expect(t, n, (B,), (torch.int64,), dev)
    _expect(sink, "sink", (Hq,), (torch.float32,), dev)
    _expect(out, "out", (B, Hq, d), (torch.float32,), dev, strided=True)
    _expect(lse, "lse", (B, Hq), (torch.float32,), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    a = StepArgs(_p(q), _p(k_new), _p(v_new), _p(z_new), _p(raw_k), _p(raw_v), _p(raw_z), _p(bias), _p(pooled_k),
                 _p(pooled_v), _p(pos), _p(raw_pos_base), _p(sink), _p(out), _p(lse), B, Hq, Hkv, d, block,
                 window, R2 // 2, N, _dt(q), _dt(z_new), float(scale))
    _set_st(a, q=q, k_new=k_new, v_new=v_new, z_new=z_new, raw_k=raw_k, raw_v=raw_v, raw_z=raw_z,
            pooled_k=pooled_k, pooled_v=pooled_v, out=out)
    need = ctypes.c_size_t()
    _check(lib().lbca_decode_step_workspace(ctypes.byref(a), ctypes.byref(need)), "lbca_decode_step_workspace")
    if workspace is None and need.value > 0:
        workspace = torch.empty(need.value, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().lbca_decode_step(ctypes.byref(a), _p(workspace), ws_bytes, _stream(stream)), "lbca_decode_step")
    return out, lse


def _decode_args(q, pooled_k, raw_k, pos, block, window, mode, out, lse, pooled_v, raw_v,
                 raw_pos_base, sel_idx, sink, scale, rmsnorm_eps, rope_dims, rope_base, check_out=True):
    for t, n, nd in ((q, "q", 3), (pooled_k, "pooled_k", 4), (raw_k, "raw_k", 4), (sel_idx, "sel_idx", 2)):
        _need(t, n, nd)
    B, Hq, d = q.shape
    Hkv, N, R, dev, qt = pooled_k.shape[1], pooled_k.shape[2], raw_k.shape[2], q.device, (q.dtype,)
    _expect(q, "q", (B, Hq, d), strided=True)
    for t, n in ((pooled_k, "pooled_k"), (pooled_v, "pooled_v")):
        _expect(t, n, (B, Hkv, N, d), qt, dev, strided=True)
    for t, n in ((raw_k, "raw_k"), (raw_v, "raw_v")):
        _expect(t, n, (B, Hkv, R, d), qt, dev, strided=True)
    for t, n in ((pos, "pos"), (raw_pos_base, "raw_pos_base")):
        _expect(t, n, (B,), (torch.int64,), dev)
    if sel_idx is not None:
        _expect(sel_idx, "sel_idx", (B, sel_idx.shape[1]), (torch.int32,), dev)
    _expect(sink, "sink", (Hq,), (torch.float32,), dev)
    if check_out:
        _expect(out, "out", (B, Hq, d), (torch.float32,), dev, strided=True)
        _expect(lse, "lse", (B, Hq), (torch.float32,), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    a = DecodeArgs(_p(q), _p(pooled_k), _p(pooled_v), _p(raw_k), _p(raw_v), _p(pos),
                   _p(raw_pos_base), _p(sel_idx), _p(sink), _p(out), _p(lse),
                   B, Hq, Hkv, d, N, raw_k.shape[2], 0 if sel_idx is None else sel_idx.shape[1],
                   block, window, mode, _dt(q), float(scale),
                   -1.0 if rmsnorm_eps is None else float(rmsnorm_eps), int(rope_dims),
                   float(rope_base))
    return _set_st(a, q=q, pooled_k=pooled_k, pooled_v=pooled_v, raw_k=raw_k, raw_v=raw_v,
                   out=out if check_out else None)


def decode_workspace_bytes(q, pooled_k, raw_k, pos, block, window, mode, **kw):
    out = kw.pop("out", None)
    a = _decode_args(q, pooled_k, raw_k, pos, block, window, mode, out if out is not None else q,
                     kw.get("lse"), kw.get("pooled_v"), kw.get("raw_v"), kw.get("raw_pos_base"),
                     kw.get("sel_idx"), kw.get("sink"), kw.get("scale"), kw.get("rmsnorm_eps"),
                     kw.get("rope_dims", 0), kw.get("rope_base", 10000.0), check_out=out is not None)
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


def attend_decode_noalloc(q, pooled_k, raw_k, pos, block, window, mode, out, lse, pooled_v=None, raw_v=None,
                          raw_pos_base=None, sel_idx=None, sink=None, scale=None, rmsnorm_eps=None, rope_dims=0,
                          rope_base=10000.0, stream=None):
    """lbca_attend_decode_noalloc: lbca_attend_decode with the split partials in the
    library's static scratch; the caller passes the outputs (nothing is allocated)."""
    a = _decode_args(q, pooled_k, raw_k, pos, block, window, mode, out, lse, pooled_v, raw_v,
                     raw_pos_base, sel_idx, sink, scale, rmsnorm_eps, rope_dims, rope_base)
    _check(lib().lbca_attend_decode_noalloc(ctypes.byref(a), _stream(stream)), "lbca_attend_decode_noalloc")
    return out, lse


def attend_prefill(q, q_pos0, pooled_k, raw_k, raw_pos_base, block, window, mode, out=None,
                   lse=None, pooled_v=None, raw_v=None, sink=None, scale=None, out_dtype=None,
                   stream=None):
    """lbca_attend_prefill: q [B,Tq,Hq,d]; returns (out [B,Tq,Hq,d], lse [B,Tq,Hq])."""
    for t, n, nd in ((q, "q", 4), (pooled_k, "pooled_k", 4), (raw_k, "raw_k", 4)):
        _need(t, n, nd)
    B, Tq, Hq, d = q.shape
    Hkv, N, R, dev, qt = pooled_k.shape[1], pooled_k.shape[2], raw_k.shape[2], q.device, (q.dtype,)
    if out is None:
        out = torch.empty((B, Tq, Hq, d), dtype=out_dtype or q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=q.device)
    _expect(q, "q", (B, Tq, Hq, d), strided=True)
    for t, n in ((pooled_k, "pooled_k"), (pooled_v, "pooled_v")):
        _expect(t, n, (B, Hkv, N, d), qt, dev, strided=True)
    for t, n in ((raw_k, "raw_k"), (raw_v, "raw_v")):
        _expect(t, n, (B, Hkv, R, d), qt, dev, strided=True)
    _expect(sink, "sink", (Hq,), (torch.float32,), dev)
    _expect(out, "out", (B, Tq, Hq, d), device=dev, strided=True)
    _expect(lse, "lse", (B, Tq, Hq), (torch.float32,), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    a = PrefillArgs(_p(q), _p(pooled_k), _p(pooled_v), _p(raw_k), _p(raw_v), _p(sink), _p(out), _p(lse),
                    B, Tq, Hq, pooled_k.shape[1], d, pooled_k.shape[2], raw_k.shape[2], q_pos0,
                    raw_pos_base, block, window, mode, _dt(q), _dt(out), float(scale))
    _set_st(a, q=q, pooled_k=pooled_k, pooled_v=pooled_v, raw_k=raw_k, raw_v=raw_v, out=out)
    _check(lib().lbca_attend_prefill(ctypes.byref(a), _stream(stream)), "lbca_attend_prefill")
    return out, lse


def attend_prefill_backward(q, q_pos0, pooled_k, raw_k, raw_pos_base, block, window, mode, out, lse,
                            grad_out, pooled_v=None, raw_v=None, sink=None, scale=None, grad_q=None,
                            grad_pooled_k=None, grad_pooled_v=None, grad_raw_k=None, grad_raw_v=None,
                            grad_sink=None, accumulate=False, workspace=None, stream=None):
    """lbca_attend_prefill_backward: gradients of attend_prefill given its out and lse and
    the upstream gradient grad_out [B,Tq,Hq,d].  Returns (grad_q, grad_pooled_k,
    grad_pooled_v, grad_raw_k, grad_raw_v, grad_sink), all float32; with pooled_v/raw_v
    None (one series as K and V) the value gradients are None and the key gradients
    hold both roles; grad_sink is None without a sink.  accumulate=True adds the key,
    value and sink gradients into the given buffers (chunked backward)."""
    for t, n, nd in ((q, "q", 4), (pooled_k, "pooled_k", 4), (raw_k, "raw_k", 4)):
        _need(t, n, nd)
    B, Tq, Hq, d = q.shape
    Hkv, N, R, dev, qt = pooled_k.shape[1], pooled_k.shape[2], raw_k.shape[2], q.device, (q.dtype,)
    shared = pooled_v is None
    f32 = torch.float32

    def new(shape):
        return torch.empty(shape, dtype=f32, device=dev)

    if accumulate and (grad_pooled_k is None or grad_raw_k is None or (not shared and (
            grad_pooled_v is None or grad_raw_v is None)) or (sink is not None and grad_sink is None)):
        raise ValueError("accumulate=True needs the gradient buffers to add into")
    grad_q = new((B, Tq, Hq, d)) if grad_q is None else grad_q
    grad_pooled_k = new((B, Hkv, N, d)) if grad_pooled_k is None else grad_pooled_k
    grad_raw_k = new((B, Hkv, R, d)) if grad_raw_k is None else grad_raw_k
    if not shared:
        grad_pooled_v = new((B, Hkv, N, d)) if grad_pooled_v is None else grad_pooled_v
        grad_raw_v = new((B, Hkv, R, d)) if grad_raw_v is None else grad_raw_v
    elif grad_pooled_v is not None or grad_raw_v is not None:
        raise ValueError("one shared K/V series has no separate value gradients")
    if sink is not None and grad_sink is None:
        grad_sink = new((Hq,))
    _expect(q, "q", (B, Tq, Hq, d), strided=True)
    _expect(grad_out, "grad_out", (B, Tq, Hq, d), qt, dev, strided=True)
    for t, n in ((pooled_k, "pooled_k"), (pooled_v, "pooled_v")):
        _expect(t, n, (B, Hkv, N, d), qt, dev, strided=True)
    for t, n in ((raw_k, "raw_k"), (raw_v, "raw_v")):
        _expect(t, n, (B, Hkv, R, d), qt, dev, strided=True)
    _expect(sink, "sink", (Hq,), (f32,), dev)
    _expect(out, "out", (B, Tq, Hq, d), device=dev, strided=True)
    _expect(lse, "lse", (B, Tq, Hq), (f32,), dev)
    _expect(grad_q, "grad_q", (B, Tq, Hq, d), (f32,), dev, strided=True)
    for t, n in ((grad_pooled_k, "grad_pooled_k"), (grad_pooled_v, "grad_pooled_v")):
        _expect(t, n, (B, Hkv, N, d), (f32,), dev, strided=True)
    for t, n in ((grad_raw_k, "grad_raw_k"), (grad_raw_v, "grad_raw_v")):
        _expect(t, n, (B, Hkv, R, d), (f32,), dev, strided=True)
    _expect(grad_sink, "grad_sink", (Hq,), (f32,), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    a = PrefillGradArgs(_p(q), _p(pooled_k), _p(pooled_v), _p(raw_k), _p(raw_v), _p(sink), _p(out), _p(lse),
                        _p(grad_out), _p(grad_q), _p(grad_pooled_k), _p(grad_pooled_v), _p(grad_raw_k),
                        _p(grad_raw_v), _p(grad_sink), B, Tq, Hq, Hkv, d, N, R, q_pos0, raw_pos_base, block,
                        window, mode, _dt(q), _dt(out), int(bool(accumulate)), float(scale))
    _set_st(a, q=q, pooled_k=pooled_k, pooled_v=pooled_v, raw_k=raw_k, raw_v=raw_v, out=out, grad_out=grad_out,
            grad_q=grad_q, grad_pooled_k=grad_pooled_k, grad_pooled_v=grad_pooled_v, grad_raw_k=grad_raw_k,
            grad_raw_v=grad_raw_v)
    need = ctypes.c_size_t()
    _check(lib().lbca_attend_prefill_backward_workspace(ctypes.byref(a), ctypes.byref(need)),
           "lbca_attend_prefill_backward_workspace")
    if workspace is not None and workspace.numel() * workspace.element_size() < need.value:
        raise ValueError(f"workspace needs {need.value} bytes")
    if workspace is None and need.value > 0:
        workspace = torch.empty(need.value, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().lbca_attend_prefill_backward(ctypes.byref(a), _p(workspace), ws_bytes, _stream(stream)),
           "lbca_attend_prefill_backward")
    return grad_q, grad_pooled_k, grad_pooled_v, grad_raw_k, grad_raw_v, grad_sink


def attend_prefill_backward_workspace_bytes(q_shape, q_pos0, kv_heads, entries, raw_rows, raw_pos_base, block,
                                            window, mode, shared=False, dtype=torch.bfloat16):
    """lbca_attend_prefill_backward_workspace for these sizes (B, Tq, Hq, d = q_shape); no
    buffer is touched, so placeholder addresses stand in for them."""
    B, Tq, Hq, d = q_shape
    ph = ctypes.c_void_p(_EMPTY)
    a = PrefillGradArgs(ph, ph, None if shared else ph, ph, None if shared else ph, None, ph, ph, ph, ph, ph,
                        None if shared else ph, ph, None if shared else ph, None, B, Tq, Hq, kv_heads, d, entries,
                        raw_rows, q_pos0, raw_pos_base, block, window, mode,
                        F32 if dtype == torch.float32 else BF16, F32, 0, 1.0)
    need = ctypes.c_size_t()
    _check(lib().lbca_attend_prefill_backward_workspace(ctypes.byref(a), ctypes.byref(need)),
           "lbca_attend_prefill_backward_workspace")
    return need.value


def _check_index(q_idx, head_w, keys, pos):
    B, HI, dI = q_idx.shape
    dev = q_idx.device
    _expect(q_idx, "q_idx", (B, HI, dI), strided=True)
    _expect(head_w, "head_w", (B, HI), (torch.float32,), dev)
    _expect(keys, "keys", (B, keys.shape[1], dI), (q_idx.dtype,), dev, strided=True)
    _expect(pos, "pos", (B,), (torch.int64,), dev)


def index_workspace_bytes(q_idx, head_w, keys, pos, block, k):
    """csa_index_topk_workspace: bytes of workspace csa_index_topk needs for these shapes
    (the query's buffer stands in for the output, which the size does not depend on)."""
    _need(keys, "keys", 3)
    _check_index(q_idx, head_w, keys, pos)
    B, HI, dI = q_idx.shape
    a = IndexArgs(_p(q_idx), _p(head_w), _p(keys), _p(pos), _p(q_idx), None,
                  B, HI, dI, keys.shape[1], k, block, _dt(q_idx))
    _set_st(a, q_idx=q_idx, keys=keys)
    need = ctypes.c_size_t()
    _check(lib().csa_index_topk_workspace(ctypes.byref(a), ctypes.byref(need)), "csa_index_topk_workspace")
    return need.value


def csa_index_topk(q_idx, head_w, keys, pos, block, k, out_idx=None, out_score=None,
                   workspace=None, stream=None):
    """csa_index_topk: q_idx [B,HI,dI], head_w [B,HI], keys [B,N,dI]; returns (idx, score)."""
    for t, n, nd in ((q_idx, "q_idx", 3), (keys, "keys", 3)):
        _need(t, n, nd)
    B, HI, dI = q_idx.shape
    if out_idx is None:
        out_idx = torch.empty((B, k), dtype=torch.int32, device=q_idx.device)
    if out_score is None:
        out_score = torch.empty((B, k), dtype=torch.float32, device=q_idx.device)
    _check_index(q_idx, head_w, keys, pos)
    _expect(out_idx, "out_idx", (B, k), (torch.int32,), q_idx.device)
    _expect(out_score, "out_score", (B, k), (torch.float32,), q_idx.device)
    a = IndexArgs(_p(q_idx), _p(head_w), _p(keys), _p(pos), _p(out_idx), _p(out_score),
                  B, HI, dI, keys.shape[1], k, block, _dt(q_idx))
    _set_st(a, q_idx=q_idx, keys=keys)
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
    for t, n, nd in ((q_idx, "q_idx", 4), (q, "q", 4), (entries, "entries", 3), (raw, "raw", 3)):
        _need(t, n, nd)
    B, Tq, Hq, d = q.shape
    HI, dI = q_idx.shape[2], q_idx.shape[3]
    N, R, dev, qt = entries.shape[1], raw.shape[1], q.device, (q.dtype,)
    _expect(q, "q", (B, Tq, Hq, d), strided=True)
    _expect(q_idx, "q_idx", (B, Tq, HI, dI), qt, dev, strided=True)
    _expect(head_w, "head_w", (B, Tq, HI), (torch.float32,), dev)
    _expect(idx_keys, "idx_keys", (B, N, dI), qt, dev, strided=True)
    _expect(entries, "entries", (B, N, d), qt, dev, strided=True)
    _expect(raw, "raw", (B, R, d), qt, dev, strided=True)
    _expect(sink, "sink", (Hq,), (torch.float32,), dev)
    if out is not q:  # the workspace query passes q in place of an absent output
        _expect(out, "out", (B, Tq, Hq, d), (torch.float32,), dev, strided=True)
    _expect(lse, "lse", (B, Tq, Hq), (torch.float32,), dev)
    _expect(out_idx, "out_idx", (B, Tq, k), (torch.int32,), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    a = CsaPrefillArgs(_p(q_idx), _p(head_w), _p(idx_keys), _p(q), _p(entries), _p(raw), _p(sink), _p(out),
                       _p(lse), _p(out_idx), B, Tq, HI, dI, Hq, d, entries.shape[1], raw.shape[1], k,
                       q_pos0, raw_pos_base, block, window, _dt(q), float(scale),
                       -1.0 if rmsnorm_eps is None else float(rmsnorm_eps), int(rope_dims), float(rope_base))
    return _set_st(a, q_idx=q_idx, idx_keys=idx_keys, q=q, entries=entries, raw=raw,
                   out=None if out is q else out)


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


# ---------------------------------------------------------------------------
def grouped_gemm(a, w, out=None, out_dtype=None, groups=1, stream=None):
    """lbca_grouped_gemm on dense tensors: a [M, groups * K] (or [M, K] with groups = 1),
    w [groups, N, K] bf16 ([out, in] per group); returns out [M, groups * N] with group g's
    projection in columns g*N .. (g+1)*N - 1 (fp32 accumulation)."""
    if w.dim() == 2:
        w = w.unsqueeze(0)
    G, N, K = w.shape
    if G != groups:
        raise ValueError(f"w holds {G} groups, {groups} requested")
    _need(a, "a", 2)
    M = a.shape[0]
    _expect(a, "a", (M, G * K))
    _expect(w, "w", (G, N, K), (torch.bfloat16,), a.device)
    if out is None:
        out = torch.empty((M, G * N), dtype=out_dtype or torch.bfloat16, device=a.device)
    _expect(out, "out", (M, G * N), device=a.device)
    args = GemmArgs(_p(a), _p(w), _p(out), G, M, N, K, G * K, K, G * N, K, N * K, N, _dt(a), _dt(out))
    _check(lib().lbca_grouped_gemm(ctypes.byref(args), _stream(stream)), "lbca_grouped_gemm")
    return out


def indexer_queries(c_q, w_uq, heads, out=None, stream=None):
    """Low-rank indexer queries: c_q [..., d_c], w_uq [heads * d_I, d_c] bf16 ->
    [..., heads, d_I] bf16 (one grouped_gemm call with one group)."""
    lead = c_q.shape[:-1]
    flat = c_q.reshape(-1, c_q.shape[-1])
    res = grouped_gemm(flat, w_uq, out=out, stream=stream)
    return res.reshape(*lead, heads, w_uq.shape[0] // heads)


def pooling_logits(h, w_z, dim, out=None, stream=None):
    """Pooling logits of the series: h [..., d_model] (fp32 or bf16), w_z [series * dim,
    d_model] bf16 (series stacked) -> fp32 [..., series, dim] (one grouped_gemm call)."""
    lead = h.shape[:-1]
    flat = h.reshape(-1, h.shape[-1])
    z = grouped_gemm(flat, w_z, out=out, out_dtype=torch.float32, stream=stream)
    return z.reshape(*lead, w_z.shape[0] // dim, dim)


def output_projection(o, w_groups, w_out, mid=None, out=None, out_dtype=torch.float32, stream=None):
    """Grouped output projection: o [T, H, c] (fp32 or bf16, heads consecutive),
    w_groups [g, d_g, (H/g) * c] bf16, w_out [d_model, g * d_g] bf16 -> [T, d_model]
    (two grouped_gemm calls: the g group maps, then the model-width map)."""
    T = o.shape[0]
    g = w_groups.shape[0]
    flat = o.reshape(T, -1)
    mid = grouped_gemm(flat, w_groups, out=mid, groups=g, stream=stream)
    return grouped_gemm(mid, w_out, out=out, out_dtype=out_dtype, stream=stream)
