"""The Python binding checks every buffer's shape, dtype and device before the
library sees a pointer (the C ABI gets raw pointers and sizes only, so a short
output or key buffer would be written or read past its end).  Each case here
fails in the binding with ValueError; no library call is made."""
import pytest
import torch

from block_compressed_kv_amd import lbca

f32, bf16, i32, i64 = torch.float32, torch.bfloat16, torch.int32, torch.int64


def z(*shape, dtype=bf16):
    return torch.zeros(shape, dtype=dtype)


def _decode_kw(**over):
    B, Hq, Hkv, N, R, d = 2, 4, 2, 8, 16, 64
    kw = dict(q=z(B, Hq, d), pooled_k=z(B, Hkv, N, d), raw_k=z(B, Hkv, R, d), pos=z(B, dtype=i64),
              block=4, window=8, mode=0, pooled_v=z(B, Hkv, N, d), raw_v=z(B, Hkv, R, d),
              out=z(B, Hq, d, dtype=f32), lse=z(B, Hq, dtype=f32))
    kw.update(over)
    return kw


@pytest.mark.parametrize("over", [
    dict(out=z(2, 4, 32, dtype=f32)),          # short output rows
    dict(out=z(2, 4, 64)),                     # bf16 output (kernels write fp32)
    dict(lse=z(2, 3, dtype=f32)),
    dict(pooled_v=z(2, 2, 7, 64)),             # V shorter than K
    dict(raw_v=z(2, 2, 16, 64, dtype=f32)),    # dtype differs from q
    dict(pos=z(2, dtype=i32)),
    dict(pos=z(3, dtype=i64)),
    dict(sel_idx=z(2, 5, dtype=i64)),
    dict(sel_idx=z(1, 5, dtype=i32)),
    dict(sink=z(3, dtype=f32)),
    dict(raw_pos_base=z(1, dtype=i64)),
    dict(raw_k=z(2, 2, 16, 64)[:, :, ::2]),    # not contiguous
])
def test_decode_rejects(over):
    with pytest.raises(ValueError):
        lbca.attend_decode(**_decode_kw(**over))


def _prefill_kw(**over):
    B, Tq, Hq, Hkv, N, R, d = 1, 8, 4, 2, 4, 64, 64
    kw = dict(q=z(B, Tq, Hq, d), q_pos0=40, pooled_k=z(B, Hkv, N, d), raw_k=z(B, Hkv, R, d), raw_pos_base=0,
              block=4, window=8, mode=0, pooled_v=z(B, Hkv, N, d), raw_v=z(B, Hkv, R, d),
              out=z(B, Tq, Hq, d, dtype=f32), lse=z(B, Tq, Hq, dtype=f32))
    kw.update(over)
    return kw


@pytest.mark.parametrize("over", [
    dict(out=z(1, 7, 4, 64, dtype=f32)),
    dict(lse=z(1, 8, 4)),
    dict(pooled_v=z(1, 2, 3, 64)),
    dict(raw_v=z(1, 1, 64, 64)),
    dict(sink=z(4)),
])
def test_prefill_rejects(over):
    with pytest.raises(ValueError):
        lbca.attend_prefill(**_prefill_kw(**over))


@pytest.mark.parametrize("over", [
    dict(out_idx=z(2, 15, dtype=i32)),         # fewer than k slots
    dict(out_idx=z(2, 16, dtype=i64)),
    dict(out_score=z(2, 16)),                  # bf16 scores
    dict(head_w=z(2, 8)),
    dict(keys=z(2, 100, 32)),                  # key dim differs from the query's
    dict(keys=z(1, 100, 64)),
    dict(pos=z(2, dtype=f32)),
])
def test_index_rejects(over):
    kw = dict(q_idx=z(2, 8, 64), head_w=z(2, 8, dtype=f32), keys=z(2, 100, 64), pos=z(2, dtype=i64), block=4,
              k=16)
    kw.update(over)
    with pytest.raises(ValueError):
        lbca.csa_index_topk(**kw)


def _csap_kw(**over):
    B, Tq, HI, dI, Hq, d, N, R, k = 1, 4, 8, 64, 32, 512, 64, 200, 16
    kw = dict(q_idx=z(B, Tq, HI, dI), head_w=z(B, Tq, HI, dtype=f32), idx_keys=z(B, N, dI), q=z(B, Tq, Hq, d),
              entries=z(B, N, d), raw=z(B, R, d), q_pos0=150, raw_pos_base=0, block=4, window=16, k=k,
              out=z(B, Tq, Hq, d, dtype=f32), lse=z(B, Tq, Hq, dtype=f32), out_idx=z(B, Tq, k, dtype=i32))
    kw.update(over)
    return kw


@pytest.mark.parametrize("over", [
    dict(out_idx=z(1, 4, 8, dtype=i32)),       # narrower than k
    dict(out=z(1, 4, 32, 512)),                # bf16 output
    dict(lse=z(1, 4, 31, dtype=f32)),
    dict(idx_keys=z(1, 63, 64)),               # fewer key rows than entries
    dict(head_w=z(1, 4, 8)),
    dict(sink=z(16, dtype=f32)),
    dict(q_idx=z(1, 4, 8, 64, dtype=f32)),
])
def test_csa_sparse_prefill_rejects(over):
    with pytest.raises(ValueError):
        lbca.csa_sparse_prefill(**_csap_kw(**over))


def test_pool_and_cache_reject():
    B, H, T, d, m = 1, 2, 64, 64, 16
    x, zz, bias = z(B, H, T, d), z(B, H, T, d, dtype=f32), z(H, m, d, dtype=f32)
    with pytest.raises(ValueError):
        lbca.pool_blocks(x, zz, bias, m, 0, 4, z(B, H, 4, d), v=x, out_v=z(B, H, 3, d))
    with pytest.raises(ValueError):
        lbca.pool_blocks(x, zz, z(H, m, d), m, 0, 4, z(B, H, 4, d))     # bf16 bias
    with pytest.raises(ValueError):
        lbca.pool_blocks(x, z(B, H, T - 1, d), bias, m, 0, 4, z(B, H, 4, d))
    with pytest.raises(ValueError):
        lbca.pool_blocks_backward(x, zz, bias, m, 0, 4, z(B, H, 4, d), dz=z(B, H, T, d))  # dz dtype
    ring = 48
    with pytest.raises(ValueError):
        lbca.cache_append(z(B, H, d), z(B, H, d, dtype=f32), z(B, H, 2 * ring, d), z(B, H, 2 * ring, d, dtype=f32),
                          bias, z(B, dtype=i64), z(B, dtype=i32), m, 16, 0, z(B, H, 4, d))
    with pytest.raises(ValueError):
        lbca.cache_append(z(B, H, d), z(B, H, d, dtype=f32), z(B, H, 2 * ring, d), z(B, H, 2 * ring - 2, d, dtype=f32),
                          bias, z(B, dtype=i64), z(B, dtype=i64), m, 16, 0, z(B, H, 4, d))


@pytest.mark.skipif(torch.cuda.is_available(), reason="valid host tensors would reach a launch on a GPU machine")
def test_valid_arguments_pass_the_binding_checks():
    # the unmodified arguments of each case above get past every shape check
    # (and then fail only for want of a GPU stream), so each rejection above is
    # due to the one buffer that case changes
    calls = [(lbca.attend_decode, _decode_kw()), (lbca.attend_prefill, _prefill_kw()),
             (lbca.csa_sparse_prefill, _csap_kw()),
             (lbca.csa_index_topk, dict(q_idx=z(2, 8, 64), head_w=z(2, 8, dtype=f32), keys=z(2, 100, 64),
                                        pos=z(2, dtype=i64), block=4, k=16))]
    for fn, kw in calls:
        with pytest.raises(Exception) as e:
            fn(**kw)
        assert not isinstance(e.value, ValueError), (fn.__name__, e.value)
