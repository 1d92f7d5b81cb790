"""The allocation-free decode entry point, tq_attn_decode_static (split
partials in the library's own device array), against tq_attn_decode (the
same kernels with a caller workspace): two calls in a row, the second on a
smaller input, each bit-identical to the workspace call and within the
attention bar of the float64 oracle; a call whose partials exceed the array
is refused without running."""

import math

import numpy as np
import pytest

import oracle as o
from quantized_kv_cache_tq_amd import inputs

pytestmark = pytest.mark.gpu


def _setup(seed, kv, n_q, n_kv):
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import cuda
    q, k, v = inputs.outlier_decode(seed=seed, kv_len=kv, n_q=n_q, n_kv=n_kv)
    idx = np.arange(kv)
    kc, vc = b.new_cache(3, 128, n_kv, kv), b.new_cache(3, 128, n_kv, kv)
    b.tq_set_rows(kc, cuda(k), cuda(idx))
    b.tq_set_rows(vc, cuda(v), cuda(idx))
    return q, k, v, kc, vc


def test_static_decode_two_calls_second_smaller():
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import assert_attention_close, bf16_cuda
    for seed, kv, n_q, n_kv, tau in [(21, 32768, 32, 4, 0.0), (22, 3000, 8, 2, 0.0), (22, 3000, 8, 2, 5e-3)]:
        print(f"[no-alloc] decode kv={kv} heads={n_q}/{n_kv} tau={tau}", flush=True)
        q, k, v, kc, vc = _setup(seed, kv, n_q, n_kv)
        qt = bf16_cuda(q)
        scale = 1.0 / math.sqrt(128)
        got = b.tq_attn_decode_static(kc, vc, kv, qt, scale, sparse_v_tau=tau)
        want = b.tq_attn_decode(kc, vc, kv, qt, scale, sparse_v_tau=tau)
        torch.cuda.synchronize()
        got = got.cpu().numpy()
        np.testing.assert_array_equal(got, want.cpu().numpy())
        if tau == 0.0:
            ok, ov = o.new_cache(3, 128, n_kv, kv), o.new_cache(3, 128, n_kv, kv)
            o.set_rows(ok, k, np.arange(kv))
            o.set_rows(ov, v, np.arange(kv))
            ref = o.attn_decode(ok, ov, kv, q.astype(np.float64), scale)
            assert_attention_close(got, ref, what=f"static decode kv={kv}")


def test_static_decode_refuses_oversized_partials():
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    # 256-wide K and V heads take splits of at most 256 keys: 1024 splits of
    # 16 q heads x 260 floats over 262144 cells, 17 MB of partials
    kv, n_q, n_kv, d = 262144, 16, 2, 256
    kc, vc = b.new_cache(3, d, n_kv, kv), b.new_cache(3, d, n_kv, kv)
    need = b.tq_attn_decode_workspace(kc, vc, kv, n_q)
    assert need > b.STATIC_SCRATCH_BYTES
    q = torch.zeros((n_q, d), dtype=torch.float32, device="cuda")
    out = torch.full((n_q, d), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(b.TQError) as e:
        b.tq_attn_decode_static(kc, vc, kv, q, 1.0, out=out)
    assert e.value.status == b.TQ_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)          # nothing was enqueued
