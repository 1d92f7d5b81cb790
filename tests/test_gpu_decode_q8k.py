"""GPU parity of the asymmetric cache of the PR36 page, item (b): K in the
8-bit block format (32 int8 codes and a float16 scale per block, not
rotated) beside a turbo V.

* tq_set_rows into such a K cache equals the oracle's quantize_q8 byte for
  byte (codes and scales);
* tq_attn_decode / tq_attn_decode_batch over it equal the oracle's float64
  attention over the dequantized rows at the usual bar (max-abs <= 2e-3,
  relative L2 <= 1e-3).
"""

import math

import numpy as np
import pytest

import oracle as o
from quantized_kv_cache_tq_amd import inputs

pytestmark = pytest.mark.gpu


def _caches(vbits, k, v):
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import cuda
    n, n_kv, dk = k.shape
    dv = v.shape[2]
    idx = np.arange(n)
    kc, vc = b.new_cache(8, dk, n_kv, n), b.new_cache(vbits, dv, n_kv, n)
    b.tq_set_rows(kc, cuda(k), cuda(idx))
    b.tq_set_rows(vc, cuda(v), cuda(idx))
    ok, ov = o.new_cache(8, dk, n_kv, n), o.new_cache(vbits, dv, n_kv, n)
    o.set_rows(ok, k, idx)
    o.set_rows(ov, v, idx)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(kc.codes.cpu().numpy().view(np.int8), ok["codes"])
    np.testing.assert_array_equal(kc.norms.cpu().numpy(), ok["norms"])
    return kc, vc, ok, ov


def test_set_rows_q8_bit_exact_and_scatter():
    """Blocks of every scale (zero, denormal-range and large), scattered to
    permuted cells; the untouched cells stay zero."""
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import cuda
    rng = np.random.default_rng(50)
    x = (rng.standard_normal((300, 3, 256)) * np.exp(rng.standard_normal((300, 3, 8, 1)) * 4).repeat(32, 3)
         .reshape(300, 3, 256)).astype(np.float32)
    x[7, 1, :32] = 0.0
    x[8, 0, 32:64] = 1e-6
    cells = rng.permutation(400)[:300]
    kc = b.new_cache(8, 256, 3, 400)
    b.tq_set_rows(kc, cuda(x), cuda(cells))
    ok = o.new_cache(8, 256, 3, 400)
    o.set_rows(ok, x, cells)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(kc.codes.cpu().numpy().view(np.int8), ok["codes"])
    np.testing.assert_array_equal(kc.norms.cpu().numpy(), ok["norms"])


@pytest.mark.parametrize("vbits", [2, 3, 4])
@pytest.mark.parametrize("dk,dv", [(128, 128), (256, 128), (256, 256)])
def test_q8_k_decode(vbits, dk, dv):
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import assert_attention_close, bf16_cuda
    q, k, v = inputs.outlier_decode(seed=51 + vbits, kv_len=5000, n_q=16, n_kv=2, d=dk, dv=dv)
    kc, vc, ok, ov = _caches(vbits, k, v)
    scale = 1.0 / math.sqrt(dk)
    print(f"[decode-q8k] vbits={vbits} dk={dk} dv={dv}", flush=True)
    got = b.tq_attn_decode(kc, vc, 4999, bf16_cuda(q), scale).cpu().numpy()
    want = o.attn_decode(ok, ov, 4999, q.astype(np.float64), scale)
    assert_attention_close(got, want, what=f"q8 K / turbo{vbits} V {dk}/{dv}")


@pytest.mark.parametrize("kv_len,n_q,n_kv", [(1, 1, 1), (17, 4, 2), (1000, 32, 4), (32768, 32, 4)])
def test_q8_k_decode_shapes(kv_len, n_q, n_kv):
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import assert_attention_close, cuda
    q, k, v = inputs.small_decode(seed=kv_len + n_q, kv_len=max(kv_len, 64), n_q=n_q, n_kv=n_kv)
    kc, vc, ok, ov = _caches(3, k, v)
    scale = 1.0 / math.sqrt(128)
    got = b.tq_attn_decode(kc, vc, kv_len, cuda(q), scale).cpu().numpy()
    want = o.attn_decode(ok, ov, kv_len, q.astype(np.float64), scale)
    assert_attention_close(got, want, what=f"q8 K kv={kv_len} {n_q}/{n_kv}")


def test_q8_k_padded_192_beside_v128():
    """The page's case: 192-wide K heads padded to 256 in the 8-bit format,
    128-wide turbo3 V, GQA 8 over 32K cells, bf16 query padded alike."""
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import assert_attention_close, bf16_cuda
    q, k, v = inputs.outlier_decode(seed=55, kv_len=32768, n_q=16, n_kv=2, d=256, dv=128)
    k[:, :, 192:] = 0.0
    q[:, 192:] = 0.0
    kc, vc, ok, ov = _caches(3, k, v)
    scale = 1.0 / math.sqrt(192)
    got = b.tq_attn_decode(kc, vc, 32768, bf16_cuda(q), scale).cpu().numpy()
    want = o.attn_decode(ok, ov, 32768, q.astype(np.float64), scale)
    (ma, rl) = assert_attention_close(got, want, what="q8 K 192->256 / V 128")
    print(f"    max_abs={ma:.3g} rel_l2={rl:.3g}")


def test_q8_k_batch_two_rows():
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import assert_attention_close, bf16_cuda
    _, k, v = inputs.small_decode(seed=56, kv_len=4000, n_q=1, n_kv=4)
    kc, vc, ok, ov = _caches(3, k, v)
    rng = np.random.default_rng(57)
    q = inputs.bf16_round(rng.standard_normal((3, 2, 32, 128)).astype(np.float32))
    starts, lens = [0, 1500, 3990], [1500, 2490, 1]
    st = torch.tensor(starts, dtype=torch.int64, device="cuda")
    ln = torch.tensor(lens, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(128)
    got = b.tq_attn_decode_batch(kc, vc, st, ln, 2490, bf16_cuda(q), scale).cpu().numpy()
    want = o.attn_decode_batch(ok, ov, starts, lens, q.astype(np.float64), scale)
    for i in range(3):
        for r in range(2):
            if not np.any(want[i, r]):
                np.testing.assert_array_equal(got[i, r], 0.0)
            else:
                assert_attention_close(got[i, r], want[i, r], what=f"q8 K batch seq {i} row {r}")


def test_q8_k_sparse_v_within_bound():
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import bf16_cuda
    q, k, v = inputs.outlier_decode(seed=58, kv_len=8192)
    kc, vc, ok, ov = _caches(3, k, v)
    scale = 1.0 / math.sqrt(128)
    got = b.tq_attn_decode(kc, vc, 8192, bf16_cuda(q), scale, sparse_v_tau=5e-3).cpu().numpy()
    qd = q.astype(np.float64)
    dense = o.attn_decode(ok, ov, 8192, qd, scale)
    bound, n_t = o.sparse_v_bound(ok, ov, 8192, qd, scale, 5e-3)
    assert n_t.sum() > 0
    assert np.all(np.abs(got - dense).max(axis=1) <= bound + 2e-3)
