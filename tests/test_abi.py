"""C-ABI boundary tests that need no GPU.

* liblbca.so loads and exports every entry point include/lbca.h declares;
* the host visibility rule equals the oracle's bit for bit;
* every argument error returns its documented status before any device work
  (fake, never dereferenced pointers are used; each case fails validation).
"""
import ctypes
import subprocess

import pytest

from block_compressed_kv_amd import lbca
from oracle import lbca_oracle as O

FAKE = 0x10000  # 16-byte aligned, never dereferenced (validation fails first)

try:
    import torch

    _GPU = torch.cuda.is_available()
except Exception:  # pragma: no cover
    _GPU = False
# The fake-pointer cases are host-validation tests; on a machine with a GPU a
# case that slipped through validation would launch a kernel on fake pointers.
fake_ptr = pytest.mark.skipif(_GPU, reason="fake-pointer validation cases run on CPU-only machines")


def test_every_declared_symbol_is_exported():
    names = lbca.exported_names()
    assert {"lbca_pool_blocks", "lbca_attend_decode", "lbca_attend_prefill", "csa_index_topk",
            "lbca_visible_range", "lbca_attend_decode_workspace", "csa_index_topk_workspace",
            "lbca_status_string", "lbca_abi_version"} <= set(names)
    L = lbca.lib()
    for n in names:
        assert hasattr(L, n)
    out = subprocess.run(["nm", "-D", "--defined-only", lbca.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(names) <= exported
    # nothing but the C ABI leaks out of the library
    assert all(s.startswith(("lbca_", "csa_")) or s in ("_init", "_fini") for s in exported), exported


def test_status_strings():
    L = lbca.lib()
    for code in (0, -1, -2, -3, -4, 7):
        assert L.lbca_status_string(code)


@pytest.mark.parametrize("mode", [O.EXCLUSIVE, O.OVERLAP])
def test_host_visibility_matches_oracle(mode):
    for m in (1, 3, 4, 16, 64, 128):
        for W in (1, 7, 128):
            for t in list(range(0, 300)) + [32767, 2 ** 20 - 1, 2 ** 17 - 1, 10 ** 9]:
                assert lbca.visible_range(t, m, W, mode) == O.visible_range(t, m, W, mode)


def test_visibility_errors():
    for args in [(-1, 4, 8, 0), (3, 0, 8, 0), (3, 4, 0, 0), (3, 4, 8, 2)]:
        with pytest.raises(lbca.LbcaError) as e:
            lbca.visible_range(*args)
        assert e.value.status == lbca.ERR_INVALID_ARG


def _pool(**kw):
    a = dict(x=FAKE, v=None, z=FAKE, bias=FAKE, xb=None, zb=None, bias_b=None, out_x=FAKE, out_v=None,
             batch=1, heads=2, tokens=64, dim=128, block=16, entries=4, block_begin=0, block_end=4,
             pos_base=0, x_dtype=1, z_dtype=0, rmsnorm_eps=-1.0, rope_dims=0, rope_base=10000.0)
    a.update(kw)
    s = lbca.PoolArgs(**a)
    return lbca.lib().lbca_pool_blocks(ctypes.byref(s), None)


@fake_ptr
@pytest.mark.parametrize("kw,code", [
    (dict(x=None), -1), (dict(z=None), -1), (dict(bias=None), -1), (dict(out_x=None), -1),
    (dict(v=FAKE), -1),                                   # v without out_v
    (dict(xb=FAKE), -1),                                  # partial dual args
    (dict(xb=FAKE, zb=FAKE, bias_b=FAKE, v=FAKE, out_v=FAKE), -2),  # dual with values
    (dict(x_dtype=5), -1), (dict(heads=0), -1), (dict(block=0), -1),
    (dict(dim=96), -2), (dict(dim=1024), -2), (dict(dim=0), -1),
    (dict(block_end=5), -1), (dict(block_begin=3, block_end=2), -1),
    (dict(tokens=63), -1), (dict(pos_base=16), -1),       # token rows outside the buffer
    (dict(rope_dims=24), -2), (dict(rope_dims=256), -1), (dict(rmsnorm_eps=float("nan")), -1),
    (dict(rope_dims=64, rope_base=0.5), -1),
    (dict(v=FAKE, out_v=FAKE, rmsnorm_eps=1e-6), -2),     # treatment needs a shared series
    (dict(x=FAKE + 8), -1),                               # misaligned
    (dict(xb=FAKE, zb=FAKE, bias_b=FAKE, block_begin=1, pos_base=16), -1),  # dual needs block i-1
])
def test_pool_validation(kw, code):
    assert _pool(**kw) == code


@fake_ptr
def test_pool_empty_range_is_ok_without_gpu():
    assert _pool(block_begin=2, block_end=2) == 0
    assert _pool(batch=0) == 0


def _pgrad(ws=None, ws_bytes=0, **kw):
    a = dict(x=FAKE, v=FAKE, z=FAKE, bias=FAKE, grad_x=FAKE, grad_v=FAKE, dx=FAKE, dv=FAKE, dz=FAKE,
             dbias=FAKE, batch=2, heads=8, tokens=4096, dim=128, block=64, entries=64, block_begin=0,
             block_end=64, pos_base=0, x_dtype=1, z_dtype=0, rmsnorm_eps=-1.0, rope_dims=0, rope_base=10000.0)
    a.update(kw)
    s = lbca.PoolGradArgs(**a)
    n = ctypes.c_size_t()
    st_ws = lbca.lib().lbca_pool_blocks_backward_workspace(ctypes.byref(s), ctypes.byref(n))
    st = lbca.lib().lbca_pool_blocks_backward(ctypes.byref(s), ws, ws_bytes, None)
    return st_ws, st, n.value


@fake_ptr
@pytest.mark.parametrize("kw,code", [
    (dict(x=None), -1), (dict(z=None), -1), (dict(bias=None), -1), (dict(grad_x=None), -1),
    (dict(dx=None), -1), (dict(dz=None), -1), (dict(dbias=None), -1),
    (dict(v=None), -1), (dict(grad_v=None), -1), (dict(dv=None), -1),    # values all or none
    (dict(x_dtype=2), -1), (dict(heads=0), -1), (dict(block=0), -1), (dict(tokens=-1), -1),
    (dict(dim=96), -2), (dict(dim=1024), -2), (dict(dim=0), -1),
    (dict(block=128), -2),                                                # block * dim > 8192
    (dict(heads=70000, batch=1), -2),
    (dict(block_end=65), -1), (dict(block_begin=3, block_end=2), -1),
    (dict(tokens=4095), -1), (dict(pos_base=64), -1),                     # rows outside the buffer
    (dict(dz=FAKE + 4), -1),                                              # misaligned
    (dict(rmsnorm_eps=1e-6), -2),                                         # treatment needs a shared series
    (dict(v=None, grad_v=None, dv=None, rope_dims=24), -2),
    (dict(v=None, grad_v=None, dv=None, xb=FAKE), -1),                    # partial dual arguments
    (dict(xb=FAKE, zb=FAKE, bias_b=FAKE, dxb=FAKE, dzb=FAKE, dbias_b=FAKE), -2),   # dual with values
    (dict(v=None, grad_v=None, dv=None, xb=FAKE, zb=FAKE, bias_b=FAKE, dxb=FAKE, dzb=FAKE, dbias_b=FAKE),
     -2),                                                                 # dual: 2 * block * dim > 8192
    (dict(v=None, grad_v=None, dv=None, xb=FAKE, zb=FAKE, bias_b=FAKE, dxb=FAKE, dzb=FAKE, dbias_b=FAKE,
          block=32, block_begin=1, block_end=64, pos_base=32), -1),       # dual reads block begin-1
])
def test_pool_grad_validation(kw, code):
    st_ws, st, _ = _pgrad(**kw)
    assert st_ws == code and st == code


@fake_ptr
def test_pool_grad_workspace_required():
    st_ws, st, need = _pgrad()
    assert st_ws == 0 and need > 0
    assert st == -3                                                       # no workspace
    assert _pgrad(ws=FAKE, ws_bytes=need - 1)[1] == -3
    assert _pgrad(ws=FAKE + 8, ws_bytes=need)[1] == -3                    # misaligned
    st_ws, _, need0 = _pgrad(block_begin=5, block_end=5)
    assert st_ws == 0 and need0 == 0                                      # empty range: no partials


def _cache(**kw):
    a = dict(x_new=FAKE, v_new=FAKE, z_new=FAKE, raw_x=FAKE, raw_v=FAKE, raw_z=FAKE, bias=FAKE, out_x=FAKE,
             out_v=FAKE, pos=FAKE, raw_pos_base=FAKE, batch=2, heads=8, dim=128, block=64, window=128,
             ring=192, entries=512, mode=0, x_dtype=1, z_dtype=0, rmsnorm_eps=-1.0, rope_dims=0,
             rope_base=10000.0)
    a.update(kw)
    s = lbca.CacheArgs(**a)
    return lbca.lib().lbca_cache_append(ctypes.byref(s), None)


@fake_ptr
@pytest.mark.parametrize("kw,code", [
    (dict(x_new=None), -1), (dict(z_new=None), -1), (dict(raw_x=None), -1), (dict(raw_z=None), -1),
    (dict(bias=None), -1), (dict(out_x=None), -1), (dict(pos=None), -1), (dict(raw_pos_base=None), -1),
    (dict(v_new=None), -1), (dict(raw_v=None), -1), (dict(out_v=None), -1),  # values all or none
    (dict(mode=2), -1), (dict(x_dtype=3), -1), (dict(heads=0), -1), (dict(block=0), -1),
    (dict(window=0), -1), (dict(entries=-1), -1), (dict(ring=0), -1),
    (dict(dim=96), -2), (dict(dim=1024), -2), (dict(dim=0), -1),
    (dict(ring=191), -1),                                   # EXCLUSIVE needs ring >= W + m
    (dict(mode=1, ring=127), -1),                           # OVERLAP needs ring >= max(W, m)
    (dict(mode=1, window=16, ring=63), -1),
    (dict(rmsnorm_eps=1e-6), -2),                           # treatment needs a shared series
    (dict(v_new=None, raw_v=None, out_v=None, rope_dims=24), -2),
    (dict(v_new=None, raw_v=None, out_v=None, rope_dims=64, rope_base=0.5), -1),
    (dict(raw_z=FAKE + 4), -1),                             # misaligned
    (dict(v_new=None, raw_v=None, out_v=None, xb_new=FAKE), -1),   # partial dual arguments
    (dict(xb_new=FAKE, zb_new=FAKE, raw_xb=FAKE, raw_zb=FAKE, bias_b=FAKE), -2),  # dual with values
    (dict(v_new=None, raw_v=None, out_v=None, xb_new=FAKE, zb_new=FAKE, raw_xb=FAKE, raw_zb=FAKE,
          bias_b=FAKE, ring=255), -1),                      # dual EXCLUSIVE needs ring >= W + 2m
    (dict(v_new=None, raw_v=None, out_v=None, xb_new=FAKE, zb_new=FAKE, raw_xb=FAKE, raw_zb=FAKE,
          bias_b=FAKE, mode=1, window=16, ring=127), -1),   # dual OVERLAP needs ring >= 2m
])
def test_cache_validation(kw, code):
    assert _cache(**kw) == code


@fake_ptr
def test_cache_empty_batch_is_ok_without_gpu():
    assert _cache(batch=0) == 0
    assert _cache(batch=0, mode=1, ring=128) == 0


def _decode(ws=None, ws_bytes=0, **kw):
    a = dict(q=FAKE, pooled_k=FAKE, pooled_v=FAKE, raw_k=FAKE, raw_v=FAKE, pos=FAKE, raw_pos_base=None,
             sel_idx=None, sink=None, out=FAKE, lse=None, batch=2, q_heads=24, kv_heads=8, dim=128,
             entries=510, raw_rows=256, k_sel=0, block=64, window=128, mode=0, dtype=1, scale=0.08,
             rmsnorm_eps=-1.0, rope_dims=0, rope_base=10000.0)
    a.update(kw)
    s = lbca.DecodeArgs(**a)
    L = lbca.lib()
    n = ctypes.c_size_t()
    st = L.lbca_attend_decode_workspace(ctypes.byref(s), ctypes.byref(n))
    st2 = L.lbca_attend_decode(ctypes.byref(s), ws, ws_bytes, None)
    return st, st2, n.value


@fake_ptr
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(pos=None), -1), (dict(out=None), -1), (dict(raw_v=None), -1),
    (dict(q_heads=25), -1), (dict(kv_heads=0), -1), (dict(raw_rows=0), -1), (dict(window=0), -1),
    (dict(mode=3), -1), (dict(dtype=9), -1), (dict(scale=float("inf")), -1),
    (dict(sel_idx=FAKE, k_sel=0), -1),
    (dict(dim=96), -2), (dict(dim=1024), -2), (dict(q_heads=8 * 65), -2),
    (dict(rmsnorm_eps=1e-6), -2),                              # treatment with separate V
    (dict(pooled_v=None, raw_v=None, rope_dims=32), -2),       # MFMA path rope dims
    (dict(dtype=0, dim=96), -2),
    (dict(dtype=0, pooled_v=None, raw_v=None, rmsnorm_eps=1e-6), -2),
    (dict(out=FAKE + 4), -1),
    (dict(entries=1 << 23), -2),                               # pooled slice of 2 GiB at 128 dims
    (dict(raw_rows=1 << 23), -2),
    (dict(batch=65536), -2),
])
def test_decode_validation(kw, code):
    st, st2, _ = _decode(**kw)
    assert st == code and st2 == code


@fake_ptr
def test_decode_selection_split_limit():
    # The selected ids of one workgroup's row range are staged in LDS (1024 ids)
    # and at most 64 splits are merged, so a selection plus raw span beyond
    # 64 x 1024 rows has no launch shape: rejected, not silently truncated.
    sel = dict(sel_idx=FAKE, k_sel=2048, mode=1, raw_rows=70000)
    wide = dict(q_heads=64, kv_heads=1, dim=512, pooled_v=None, raw_v=None, entries=4096)
    for kw in (dict(sel), dict(sel, **wide)):
        st, st2, _ = _decode(window=64000, **kw)          # 64 + 2000 tiles of 32 rows: 65 ranges
        assert st == st2 == lbca.ERR_UNSUPPORTED, kw
        st, _, need = _decode(window=63488, **kw)         # 64 + 1984 tiles: exactly 64 ranges
        assert st == 0 and need > 0, kw
    assert _csap(k=2048, window=64000, raw_rows=70000, q_pos0=69000, raw_pos_base=0,
                 n_entries=20000)[0] == lbca.ERR_UNSUPPORTED
    assert _csap(k=2048, window=63488, raw_rows=70000, q_pos0=69000, raw_pos_base=0,
                 n_entries=20000)[0] == 0


@fake_ptr
def test_decode_workspace_required():
    big = dict(entries=8192)                            # long row lists are split over workgroups
    st, st2, need = _decode(**big)
    assert st == 0 and need > 0
    assert st2 == lbca.ERR_WORKSPACE                    # no workspace given
    _, st3, _ = _decode(ws=FAKE, ws_bytes=need - 1, **big)
    assert st3 == lbca.ERR_WORKSPACE
    _, st4, _ = _decode(ws=FAKE + 8, ws_bytes=need, **big)
    assert st4 == lbca.ERR_WORKSPACE                    # misaligned workspace
    st5, _, need5 = _decode()                           # 510 entries: one workgroup per unit
    assert st5 == 0 and need5 == 0


def _prefill(**kw):
    a = dict(q=FAKE, pooled_k=FAKE, pooled_v=FAKE, raw_k=FAKE, raw_v=FAKE, sink=None, out=FAKE,
             lse=None, batch=1, q_len=2048, q_heads=24, kv_heads=8, dim=128, entries=1016,
             raw_rows=16384, q_pos0=14336, raw_pos_base=0, block=16, window=128, mode=0, dtype=1,
             out_dtype=1, scale=0.08)
    a.update(kw)
    return lbca.lib().lbca_attend_prefill(ctypes.byref(lbca.PrefillArgs(**a)), None)


@fake_ptr
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(out=None), -1), (dict(pooled_v=None), -1),
    (dict(q_heads=23), -1), (dict(q_pos0=-1), -1), (dict(mode=2), -1), (dict(out_dtype=4), -1),
    (dict(entries=1015), -1),                 # last query needs 1016 pooled entries
    (dict(raw_rows=16383), -1),               # last query's position leaves the raw buffer
    (dict(raw_pos_base=14300), -1),           # first query's raw span (from 14208) starts before the buffer
    (dict(dim=256), -2), (dict(dtype=0, dim=96), -2),
    (dict(scale=-0.1), -2), (dict(scale=0.0), -2),   # MFMA path folds a positive scale into the exponent
])
def test_prefill_validation(kw, code):
    assert _prefill(**kw) == code


@fake_ptr
def test_prefill_empty_is_ok_without_gpu():
    assert _prefill(q_len=0) == 0
    assert _prefill(batch=0) == 0


def _prefill_grad(ws_query=False, **kw):
    a = dict(q=FAKE, pooled_k=FAKE, pooled_v=FAKE, raw_k=FAKE, raw_v=FAKE, sink=None, out=FAKE, lse=FAKE,
             grad_out=FAKE, grad_q=FAKE, grad_pooled_k=FAKE, grad_pooled_v=FAKE, grad_raw_k=FAKE,
             grad_raw_v=FAKE, grad_sink=None, batch=1, q_len=2048, q_heads=24, kv_heads=8, dim=128,
             entries=1016, raw_rows=16384, q_pos0=14336, raw_pos_base=0, block=16, window=128, mode=0,
             dtype=1, out_dtype=0, accumulate=0, scale=0.08)
    a.update(kw)
    s = lbca.PrefillGradArgs(**a)
    n = ctypes.c_size_t()
    L = lbca.lib()
    if ws_query:
        return L.lbca_attend_prefill_backward_workspace(ctypes.byref(s), ctypes.byref(n)), n.value
    return L.lbca_attend_prefill_backward(ctypes.byref(s), None, 0, None), 0


@fake_ptr
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(out=None), -1), (dict(lse=None), -1), (dict(grad_out=None), -1),
    (dict(grad_q=None), -1), (dict(grad_pooled_k=None), -1), (dict(grad_raw_k=None), -1),
    (dict(pooled_v=None), -1),                # V shared on one series only
    (dict(grad_raw_v=None), -1),              # separate V needs its gradient buffer
    (dict(pooled_v=None, raw_v=None), -1),    # shared series takes no value-gradient buffers
    (dict(grad_sink=FAKE), -1),               # a sink gradient needs the sink
    (dict(accumulate=2), -1), (dict(q_heads=23), -1), (dict(mode=2), -1), (dict(out_dtype=5), -1),
    (dict(entries=1015), -1), (dict(raw_rows=16383), -1), (dict(raw_pos_base=14300), -1),
    (dict(grad_q=FAKE + 4), -1),              # fp32 buffers 16-byte aligned
    (dict(dim=256), -2), (dict(dtype=0), -2), (dict(scale=0.0), -2),
    (dict(batch=9000), -2),                   # batch * kv_heads above 65535
])
def test_prefill_backward_validation(kw, code):
    assert _prefill_grad(ws_query=True, **kw)[0] == code
    assert _prefill_grad(**kw)[0] == code


@fake_ptr
def test_prefill_backward_workspace_and_empty_calls():
    st, n = _prefill_grad(ws_query=True)
    # D per query row, then the pooled partials: 8 KV heads x 8 tiles of 128 entries
    # (1016 seen by the last query) x 4 runs of 512 positions x 128 x (K, V) x 128 dims
    assert st == 0 and n == 2048 * 24 * 4 + 8 * 8 * 4 * 128 * 2 * 128 * 4
    st, n = _prefill_grad(ws_query=True, pooled_v=None, raw_v=None, grad_pooled_v=None, grad_raw_v=None)
    assert st == 0 and n == 2048 * 24 * 4 + 8 * 8 * 4 * 128 * 1 * 128 * 4
    assert lbca.attend_prefill_backward_workspace_bytes((1, 2048, 24, 128), 14336, 8, 1016, 16384, 0, 16, 128,
                                                        0) == 2048 * 24 * 4 + 8 * 8 * 4 * 128 * 2 * 128 * 4
    assert _prefill_grad()[0] == -3                                  # no workspace given
    assert _prefill_grad(batch=0)[0] == 0
    assert _prefill_grad(q_len=0, accumulate=1)[0] == 0               # nothing to add
    ok = _prefill_grad(pooled_v=None, raw_v=None, grad_pooled_v=None, grad_raw_v=None, ws_query=True)
    assert ok[0] == 0


def _step(ws_query=False, **kw):
    a = dict(q=FAKE, k_new=FAKE, v_new=FAKE, z_new=FAKE, raw_k=FAKE, raw_v=FAKE, raw_z=FAKE, bias=FAKE,
             pooled_k=FAKE, pooled_v=FAKE, pos=FAKE, raw_pos_base=FAKE, sink=None, out=FAKE, lse=FAKE, batch=16,
             q_heads=24, kv_heads=8, dim=128, block=64, window=128, ring=192, entries=520, dtype=1, z_dtype=0,
             scale=0.088)
    a.update(kw)
    s = lbca.StepArgs(**a)
    n = ctypes.c_size_t()
    L = lbca.lib()
    if ws_query:
        return L.lbca_decode_step_workspace(ctypes.byref(s), ctypes.byref(n)), n.value
    return L.lbca_decode_step(ctypes.byref(s), None, 0, None), 0


@fake_ptr
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(k_new=None), -1), (dict(z_new=None), -1), (dict(raw_z=None), -1),
    (dict(bias=None), -1), (dict(raw_pos_base=None), -1), (dict(out=None), -1),
    (dict(v_new=None), -1), (dict(pooled_v=None, raw_v=None), -1),   # the fused step has K and V series
    (dict(ring=191), -1),                     # ring below window + block
    (dict(ring=0), -1), (dict(q_heads=23), -1), (dict(z_dtype=3), -1),
    (dict(dim=256), -2), (dict(dim=48), -2), (dict(dtype=0), -2),
])
def test_decode_step_validation(kw, code):
    assert _step(ws_query=True, **kw)[0] == code
    assert _step(**kw)[0] == code


@fake_ptr
def test_decode_step_workspace():
    # batch 16 at the 32K layer shape: one workgroup pair per (sequence, KV head), no split partials
    assert _step(ws_query=True) == (0, 0)
    assert _step(batch=0)[0] == 0
    # one sequence with room for 1300 entries: the rows are split (merge partials in the workspace)
    st, n = _step(ws_query=True, batch=1, entries=1300)
    assert st == 0 and n > 0


def _index(ws=None, ws_bytes=0, **kw):
    a = dict(q_idx=FAKE, head_w=FAKE, keys=FAKE, pos=FAKE, out_idx=FAKE, out_score=None, batch=2,
             heads=8, dim=64, entries=32768, k=512, block=4, dtype=1)
    a.update(kw)
    s = lbca.IndexArgs(**a)
    n = ctypes.c_size_t()
    L = lbca.lib()
    return (L.csa_index_topk_workspace(ctypes.byref(s), ctypes.byref(n)),
            L.csa_index_topk(ctypes.byref(s), ws, ws_bytes, None), n.value)


@fake_ptr
@pytest.mark.parametrize("kw,code", [
    (dict(q_idx=None), -1), (dict(head_w=None), -1), (dict(pos=None), -1), (dict(out_idx=None), -1),
    (dict(k=0), -1), (dict(block=0), -1), (dict(heads=0), -1), (dict(dtype=7), -1),
    (dict(dim=48), -2), (dict(heads=17), -2), (dict(k=4096), -2), (dict(entries=1 << 17), -2),
    (dict(dtype=0), -2),
])
def test_index_validation(kw, code):
    st, st2, _ = _index(**kw)
    assert st == code and st2 == code


@fake_ptr
def test_index_workspace_required():
    # 32768 entries: 8 slices of 4096, k = 512 -> two stages: scores plus 8 x 512 (key, id) pairs
    st, st2, need = _index()
    assert st == 0 and need == 2 * 32768 * 4 + 2 * 8 * 512 * 8
    assert st2 == lbca.ERR_WORKSPACE
    # one stage: too few slices, or k above a quarter of a slice
    assert _index(entries=8192)[2] == 2 * 8192 * 4
    assert _index(entries=8193)[2] == 2 * 8196 * 4 + 2 * 3 * 512 * 8
    assert _index(k=1025)[2] == 2 * 32768 * 4
    assert _index(entries=32768, k=3)[2] == 2 * 32768 * 4 + 2 * 24 * 8


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(lbca, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(lbca, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        lbca.lib()


def _csap(ws_query=True, **kw):
    a = dict(q_idx=FAKE, head_w=FAKE, idx_keys=FAKE, q=FAKE, entries=FAKE, raw=FAKE, sink=None, out=FAKE,
             lse=None, out_idx=FAKE, batch=2, q_len=100, idx_heads=8, idx_dim=64, q_heads=64, dim=512,
             n_entries=1000, raw_rows=500, k=64, q_pos0=3000, raw_pos_base=2800, block=4, window=128, dtype=1,
             scale=0.05, rmsnorm_eps=1e-6, rope_dims=64, rope_base=10000.0)
    a.update(kw)
    s = lbca.CsaPrefillArgs(**a)
    if ws_query:
        n = ctypes.c_size_t()
        return lbca.lib().csa_sparse_prefill_workspace(ctypes.byref(s), ctypes.byref(n)), n.value
    return lbca.lib().csa_sparse_prefill(ctypes.byref(s), ctypes.c_void_p(FAKE), 16, None), 0


@fake_ptr
@pytest.mark.parametrize("kw,code", [
    (dict(), 0),
    (dict(q_idx=None), -1), (dict(head_w=None), -1), (dict(idx_keys=None), -1), (dict(q=None), -1),
    (dict(entries=None), -1), (dict(raw=None), -1), (dict(out=None), -1),
    (dict(dtype=3), -1), (dict(dtype=0), -2), (dict(k=0), -1), (dict(k=4096), -2),
    (dict(idx_dim=48), -2), (dict(idx_heads=17), -2), (dict(idx_heads=0), -1), (dict(n_entries=70000), -2),
    (dict(dim=128), -2), (dict(q_heads=48), -2), (dict(q_heads=128), -2),
    (dict(batch=700), -2),                                   # batch * q_len rows above 65535
    (dict(q_len=600), -1),                                   # last query (t = 3599) past the raw buffer
    (dict(q_pos0=3950), -1),                                 # last query sees 1012 entries > 1000
    (dict(raw_pos_base=2900), -1),                           # first query's window starts below the base
    (dict(raw_rows=299), -1),                                # last query's row (t = 3099) past the buffer
    (dict(rope_dims=24), -2), (dict(rope_base=1.0), -1), (dict(scale=float("nan")), -1),
    (dict(out=FAKE + 4), -1), (dict(q_pos0=-1), -1), (dict(window=0), -1), (dict(block=0), -1),
])
def test_csa_sparse_prefill_validation(kw, code):
    st, n = _csap(**kw)
    assert st == code, kw
    if code == 0:
        assert n > 0


@fake_ptr
def test_csa_sparse_prefill_workspace_layout():
    st, with_idx = _csap()
    st2, without = _csap(out_idx=None)
    assert st == st2 == 0
    rows = 2 * 100
    assert without - with_idx == (rows * 64 * 4 + 255) // 256 * 256   # the internal selection rows
    st, big = _csap(n_entries=2000)
    assert st == 0 and big - with_idx >= rows * 1000 * 4               # fp32 scores per row and entry
    # a short workspace fails before any launch
    assert _csap(ws_query=False)[0] == -3
    st, empty = _csap(q_len=0)
    assert st == 0


def _gemm(**kw):
    a = dict(a=FAKE, w=FAKE, c=FAKE, groups=2, m=300, n=200, k=512, lda=1024, ldw=512, ldc=400,
             a_group_stride=512, w_group_stride=200 * 512, c_group_stride=200, a_dtype=1, c_dtype=0)
    a.update(kw)
    return lbca.lib().lbca_grouped_gemm(ctypes.byref(lbca.GemmArgs(**a)), None)


@fake_ptr
@pytest.mark.parametrize("kw,code", [
    (dict(a=None), -1), (dict(w=None), -1), (dict(c=None), -1), (dict(c=FAKE + 8), -1),
    (dict(a_dtype=5), -1), (dict(k=0), -1), (dict(m=-1), -1), (dict(lda=500), -1), (dict(ldc=199), -1),
    (dict(ldw=511), -1),
    (dict(k=500, lda=1000, ldw=500, a_group_stride=500, w_group_stride=100000), -2),   # k not a multiple of 8
    (dict(a_group_stride=516), -2), (dict(w_group_stride=100004), -2), (dict(groups=70000), -2),
    (dict(lda=1 << 24), -2),                                                            # 128-row band of 2 GiB
])
def test_gemm_validation(kw, code):
    assert _gemm(**kw) == code


@fake_ptr
def test_gemm_empty_is_ok_without_gpu():
    assert _gemm(groups=0) == 0 and _gemm(m=0) == 0 and _gemm(n=0) == 0


# --- element strides (lbca_strides) ------------------------------------------
def _st(*s):
    st = lbca.Strides()
    for i, v in enumerate(s):
        st.s[i] = v
    return st


@fake_ptr
@pytest.mark.parametrize("kw,code", [
    (dict(), 0),
    # q as the query part of a fused [batch, 40 heads, 128] projection output
    (dict(q_st=_st(40 * 128, 128)), 0),
    # caches as slices of longer [batch, kv_heads, 4096, 128] buffers, and a
    # head-interleaved raw cache [batch, rows, kv_heads, 128]
    (dict(pooled_k_st=_st(8 * 4096 * 128, 4096 * 128, 128), raw_k_st=_st(256 * 8 * 128, 128, 8 * 128)), 0),
    (dict(out_st=_st(24 * 256, 256)), 0),                 # output rows padded to 256
    (dict(q_st=_st(24 * 128, 4)), -1),                    # 8-byte stride: rows not 16-byte aligned
    (dict(raw_v_st=_st(-256 * 8 * 128, 128, 8 * 128)), -1),  # negative stride
    (dict(out_st=_st(24 * 128, 0)), -1),                  # every head of a sequence on one row
    (dict(out_st=_st(128, 128)), -1),                     # sequences overlap each other's heads
    (dict(out_st=_st(24 * 128, 64)), -1),                 # heads overlap (64 < 128 dims)
    (dict(q_st=_st(0, 128)), 0),                          # an input may repeat across sequences
    (dict(pooled_k_st=_st(0, 0, 1 << 23)), -2),           # a pooled slice beyond 2 GiB at this row stride
])
def test_decode_strides(kw, code):
    st, _, _ = _decode(**kw)
    assert st == code, kw


@fake_ptr
@pytest.mark.parametrize("kw,code", [
    (dict(), 0),
    (dict(q_st=_st(2048 * 40 * 128, 40 * 128, 128), out_st=_st(2048 * 24 * 128, 24 * 128, 128)), 0),
    (dict(raw_k_st=_st(16384 * 8 * 128, 128, 8 * 128)), 0),                 # head-interleaved raw rows
    (dict(raw_k_st=_st(0, 0, 1 << 20)), -2),                                # raw slice beyond 2 GiB
    (dict(out_st=_st(2048 * 24 * 128, 24 * 128, 24 * 128)), -1),            # heads of a query share a row
    (dict(pooled_v_st=_st(1016 * 128, 1016 * 128 * 8, 12)), -1),            # 24-byte row stride
])
def test_prefill_strides(kw, code):
    if code == 0:  # a call with no queries validates the inputs' strides and launches nothing
        assert _prefill(q_len=0, **kw) == 0
    else:
        assert _prefill(**kw) == code


@fake_ptr
def test_pool_and_cache_strides():
    assert _pool(batch=0, out_x_st=_st(0, 0, 0)) == 0
    assert _pool(out_x_st=_st(2 * 4 * 128, 4 * 128, 64)) == -1     # entries overlap
    assert _pool(z_st=_st(2 * 64 * 128, 64 * 128, 2)) == -1         # z rows 8 bytes apart (fp32): misaligned
    assert _cache(raw_x_st=_st(1, 0, 0)) == -1
    assert _index(keys_st=_st(-1, 64))[0] == -1
    assert _csap(entries_st=_st(0, 1 << 21))[0] == -2               # entry slice beyond 2 GiB
    assert _csap(out_st=_st(100 * 64 * 512, 64 * 512, 0))[0] == -1  # heads of a query share a row


def test_binding_passes_view_strides():
    x = torch.zeros((2, 5, 3, 16))
    v = x.permute(0, 2, 1, 3)                                        # [2, 3, 5, 16] head-interleaved view
    st = lbca._st(v)
    assert list(st.s) == [5 * 3 * 16, 16, 3 * 16]
    assert list(lbca._st(x[:, :1]).s) == [5 * 3 * 16, 0, 16]         # extent-1 dims carry stride 0
    with pytest.raises(ValueError, match="contiguous last"):
        lbca._expect(x.transpose(2, 3), "x", (2, 5, 16, 3), strided=True)
    with pytest.raises(ValueError, match="repeats one row"):
        lbca._expect(torch.zeros(16).expand(2, 3, 16), "x", (2, 3, 16), strided=True)
    lbca._expect(v, "v", (2, 3, 5, 16), strided=True)
    with pytest.raises(ValueError, match="contiguous"):
        lbca._expect(v, "lse", (2, 3, 5, 16))                        # dense-only arguments stay dense
