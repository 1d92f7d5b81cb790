"""GPU parity of tq_attn_decode against the float64 oracle.

Bar: max-abs <= 2e-3 and relative L2 <= 1e-3 on every output.  The GPU reads
caches written by its own tq_set_rows, after checking they equal the
oracle's planes bit for bit; the oracle attends over its own planes.
"""

import math

import numpy as np
import pytest

import oracle as o
from quantized_kv_cache_tq_amd import inputs

pytestmark = pytest.mark.gpu


def _caches(bits, k, v, kv_len=None):
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import cuda
    n_rows, n_kv, d = k.shape
    dv = v.shape[2]
    idx = np.arange(n_rows)
    kc, vc = b.new_cache(bits, d, n_kv, n_rows), b.new_cache(bits, dv, n_kv, n_rows)
    b.tq_set_rows(kc, cuda(k), cuda(idx))
    b.tq_set_rows(vc, cuda(v), cuda(idx))
    ok, ov = o.new_cache(bits, d, n_kv, n_rows), o.new_cache(bits, dv, n_kv, n_rows)
    o.set_rows(ok, k, idx)
    o.set_rows(ov, v, idx)
    torch.cuda.synchronize()
    assert np.array_equal(kc.codes.cpu().numpy(), ok["codes"])
    assert np.array_equal(vc.codes.cpu().numpy(), ov["codes"])
    return kc, vc, ok, ov


def _plan_block(kv, n_kv, dk, dv, n_pairs=8):
    """The keys whose maximum is a key's sparse-V reference, as tq.h states
    the plan for one sequence: 128-wide K and V take blocks of 16 tb keys,
    tb the largest of 4, 2, 1 giving every compute unit a workgroup (counting
    the pair groups of eight), one block per wave while that grid is below
    two rounds (else a running maximum over several blocks: None, no block
    rule); other shapes take 16 T keys, T the largest of 8, 4, 2, 1
    with T (dk + dv) / 128 <= 16 and at least one workgroup per compute unit,
    4 in place of 8 past one round."""
    import torch
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    if dk == 128 and dv == 128:
        wg = n_kv * -(-n_pairs // 8)
        tb = 4
        while tb > 1 and -(-kv // (128 * tb)) * wg < n_cu:
            tb //= 2
        return 16 * tb if -(-kv // (128 * tb)) * wg < 2 * n_cu else None
    groups = (dk + dv) // 128
    tpw = 8
    while tpw > 1 and not (tpw * groups <= 16 and -(-kv // (64 * tpw)) * n_kv >= n_cu):
        tpw //= 2
    if tpw == 8 and -(-kv // 512) * n_kv > n_cu:
        tpw = 4
    return 16 * tpw


def _run(bits, q, k, v, kv_len, q_bf16=False, what=""):
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import assert_attention_close, bf16_cuda, cuda
    d = q.shape[1]
    scale = 1.0 / math.sqrt(d)
    kc, vc, ok, ov = _caches(bits, k, v)
    print(f"[decode] {what} bits={bits} n_q={q.shape[0]} n_kv={k.shape[1]} kv={kv_len} "
          f"dk={k.shape[2]} dv={v.shape[2]}", flush=True)
    qt = bf16_cuda(q) if q_bf16 else cuda(q)
    got = b.tq_attn_decode(kc, vc, kv_len, qt, scale)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    want = o.attn_decode(ok, ov, kv_len, q.astype(np.float64), scale)
    return assert_attention_close(got, want, what=what), got


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_small_decode(bits):
    q, k, v = inputs.small_decode(seed=0)
    _run(bits, q, k, v, 256, what="small")


@pytest.mark.parametrize("kv_len", [1, 2, 17, 64, 65, 1000, 4097])
def test_ragged_lengths(kv_len):
    q, k, v = inputs.small_decode(seed=1, kv_len=4100, n_q=4, n_kv=2)
    _run(3, q, k, v, kv_len, what=f"ragged kv={kv_len}")


@pytest.mark.parametrize("n_q,n_kv", [(1, 1), (2, 1), (4, 2), (8, 1), (12, 3), (32, 4), (32, 2), (16, 1), (40, 2)])
def test_gqa_ratios(n_q, n_kv):
    q, k, v = inputs.small_decode(seed=2, kv_len=3000, n_q=n_q, n_kv=n_kv)
    _run(3, q, k, v, 3000, what=f"gqa {n_q}/{n_kv}")


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("kv_len", [8192, 32768])
def test_turbo2_turbo4_one_head(bits, kv_len):
    q, k, v = inputs.small_decode(seed=3, kv_len=kv_len)
    _run(bits, q, k, v, kv_len, what="turbo2/4 one head")


@pytest.mark.parametrize("kv_len,n_q", [(131072, 8), (100003, 16)])
def test_long_context(kv_len, n_q):
    """128K cells on one kv head (256 splits of 512 keys) and a ragged 100003
    cells with 16 q heads per kv head (sixteen pairs per workgroup, 391
    splits of 256 keys): the 512-thread merge takes several load rounds per
    lane group."""
    q, k, v = inputs.outlier_decode(seed=kv_len % 97, kv_len=kv_len, n_q=n_q, n_kv=1)
    _run(3, q, k, v, kv_len, q_bf16=True, what="long context")


@pytest.mark.parametrize("bits", [3, 2, 4])
def test_outlier_gqa8_32k(bits):
    q, k, v = inputs.outlier_decode(seed=0)
    (ma, rl), _ = _run(bits, q, k, v, 32768, q_bf16=True, what="outlier gqa8 32k")
    print(f"    max_abs={ma:.3g} rel_l2={rl:.3g}")


def test_decode_deterministic():
    q, k, v = inputs.small_decode(seed=4, kv_len=5000, n_q=8, n_kv=1)
    _, a = _run(3, q, k, v, 5000, what="det-1")
    _, b_ = _run(3, q, k, v, 5000, what="det-2")
    np.testing.assert_array_equal(a, b_)


def test_shared_workspace_across_lengths():
    """One workspace serves calls with different split counts: each result
    equals the result of a call with a fresh workspace, bit for bit (eager,
    then under graph replay with eager calls in between)."""
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import bf16_cuda
    q, k, v = inputs.outlier_decode(seed=3, kv_len=32768)
    kc, vc, ok, ov = _caches(3, k, v)
    qt = bf16_cuda(q)
    scale = 1.0 / math.sqrt(q.shape[1])
    lens = [32768, 1000, 17, 32768, 4097]
    fresh = {n: b.tq_attn_decode(kc, vc, n, qt, scale).cpu().numpy() for n in set(lens)}
    nbytes = max(b.tq_attn_decode_workspace(kc, vc, n, q.shape[0]) for n in lens)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for n in lens:
        got = b.tq_attn_decode(kc, vc, n, qt, scale, workspace=ws).cpu().numpy()
        np.testing.assert_array_equal(got, fresh[n], err_msg=f"kv_len={n}")
    want = o.attn_decode(ok, ov, 1000, q.astype(np.float64), scale)
    from gpu_util import assert_attention_close
    assert_attention_close(fresh[1000], want, what="kv 1000")
    # graph capture of two calls on the same workspace, replayed with eager
    # work in between; every replay must reproduce the eager result
    outs = [torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device="cuda") for _ in range(2)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            b.tq_attn_decode(kc, vc, 32768, qt, scale, out=outs[0], workspace=ws, stream=s)
            b.tq_attn_decode(kc, vc, 1000, qt, scale, out=outs[1], workspace=ws, stream=s)
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(outs[0].cpu().numpy(), fresh[32768], err_msg=f"replay {rep}")
        np.testing.assert_array_equal(outs[1].cpu().numpy(), fresh[1000], err_msg=f"replay {rep}")
        eager = b.tq_attn_decode(kc, vc, 17, qt, scale, workspace=ws).cpu().numpy()
        np.testing.assert_array_equal(eager, fresh[17])


@pytest.mark.parametrize("bits,tau", [(2, 1e-2), (3, 5e-3), (4, 5e-3), (3, 0.05)])
def test_sparse_v_within_bound(bits, tau):
    """Sparse V ([PR36] (d) item 3): |out - dense| <= B + 2e-3 per head, with B
    the oracle's bound over every key the kernel may skip."""
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import bf16_cuda
    kv = 8192
    q, k, v = inputs.outlier_decode(seed=5, kv_len=kv)
    kc, vc, ok, ov = _caches(bits, k, v)
    scale = 1.0 / math.sqrt(q.shape[1])
    print(f"[decode] sparse-V bits={bits} tau={tau} kv={kv}", flush=True)
    got = b.tq_attn_decode(kc, vc, kv, bf16_cuda(q), scale, sparse_v_tau=tau).cpu().numpy()
    dense = o.attn_decode(ok, ov, kv, q.astype(np.float64), scale)
    bound, n_t = o.sparse_v_bound(ok, ov, kv, q.astype(np.float64), scale, tau)
    err = np.abs(got - dense).max(axis=1)
    print(f"    keys with weight < tau: {n_t.mean() / kv:.1%}; max err {err.max():.3g}; "
          f"bound {bound.max():.3g}")
    assert n_t.sum() > 0
    assert np.all(err <= bound + 2e-3), (err - bound).max()
    # tight check: the kernel's own rule, a skip against the maximum of each
    # block of keys one wave scores (16 * tiles-per-wave keys, from the plan)
    block = _plan_block(kv, k.shape[1], k.shape[2], v.shape[2])
    if block is not None:
        want = o.attn_decode_sparse_v(ok, ov, kv, q.astype(np.float64), scale, tau, ref_block=block)
        from gpu_util import assert_attention_close
        assert_attention_close(got, want, what=f"sparse-V block rule, block {block}")


def test_sparse_v_limits_on_gpu():
    """tau = 0 is the dense call bit for bit; tau = 2 leaves every key out of
    the value sum (each weight against its range maximum is at most 1)."""
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import bf16_cuda
    q, k, v = inputs.outlier_decode(seed=6, kv_len=3000)
    kc, vc, ok, ov = _caches(3, k, v)
    qt = bf16_cuda(q)
    scale = 1.0 / math.sqrt(q.shape[1])
    dense = b.tq_attn_decode(kc, vc, 3000, qt, scale).cpu().numpy()
    zero_tau = b.tq_attn_decode(kc, vc, 3000, qt, scale, sparse_v_tau=0.0).cpu().numpy()
    np.testing.assert_array_equal(zero_tau, dense)
    allskip = b.tq_attn_decode(kc, vc, 3000, qt, scale, sparse_v_tau=2.0).cpu().numpy()
    assert np.all(allskip == 0)


# ---------------------------------------------------------------- head widths

@pytest.mark.parametrize("dk,dv", [(256, 256), (256, 128), (128, 256)])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_head_widths(bits, dk, dv):
    """K and V heads of 128 or 256 elements, equal or not ([PR36] (b): the
    decode kernel takes a 256-wide K beside a 128-wide V natively), GQA 8
    over 5000 keys (several splits and a ragged last range)."""
    q, k, v = inputs.outlier_decode(seed=20 + bits, kv_len=5000, n_q=16, n_kv=2, d=dk, dv=dv)
    (ma, rl), got = _run(bits, q, k, v, 4999, q_bf16=True, what=f"widths {dk}/{dv}")
    assert got.shape == (16, dv)
    print(f"    max_abs={ma:.3g} rel_l2={rl:.3g}")


@pytest.mark.parametrize("dk,dv", [(256, 256), (256, 128)])
@pytest.mark.parametrize("kv_len,n_q,n_kv", [(1, 1, 1), (17, 4, 2), (65, 8, 8), (1000, 12, 3), (4097, 8, 1)])
def test_head_widths_ragged(dk, dv, kv_len, n_q, n_kv):
    q, k, v = inputs.small_decode(seed=kv_len + n_q, kv_len=4100, n_q=n_q, n_kv=n_kv, d=dk, dv=dv)
    _run(3, q, k, v, kv_len, what=f"widths {dk}/{dv} ragged")


def test_padded_192_key_heads():
    """The case of [PR36] (b): 192-wide K heads zero-padded to 256 (query
    padded the same way) beside 128-wide V heads, turbo3, 32K keys."""
    q, k, v = inputs.outlier_decode(seed=30, kv_len=32768, n_q=16, n_kv=2, d=256, dv=128)
    k[:, :, 192:] = 0.0
    q[:, 192:] = 0.0
    (ma, rl), _ = _run(3, q, k, v, 32768, q_bf16=True, what="K 192->256 / V 128")
    print(f"    max_abs={ma:.3g} rel_l2={rl:.3g}")




@pytest.mark.parametrize("dk,dv,tau", [(256, 256, 5e-3), (256, 128, 5e-3), (256, 256, 0.05)])
def test_sparse_v_wide_heads(dk, dv, tau):
    """Sparse V with two-group heads: within the oracle's bound of the dense
    output, and at the normal bar against the block-reference emulation."""
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import assert_attention_close, bf16_cuda
    kv = 8192
    q, k, v = inputs.outlier_decode(seed=31, kv_len=kv, n_q=16, n_kv=2, d=dk, dv=dv)
    kc, vc, ok, ov = _caches(3, k, v)
    scale = 1.0 / math.sqrt(dk)
    print(f"[decode] sparse-V widths {dk}/{dv} tau={tau} kv={kv}", flush=True)
    got = b.tq_attn_decode(kc, vc, kv, bf16_cuda(q), scale, sparse_v_tau=tau).cpu().numpy()
    qd = q.astype(np.float64)
    dense = o.attn_decode(ok, ov, kv, qd, scale)
    bound, n_t = o.sparse_v_bound(ok, ov, kv, qd, scale, tau)
    err = np.abs(got - dense).max(axis=1)
    assert n_t.sum() > 0
    assert np.all(err <= bound + 2e-3), (err - bound).max()
    block = _plan_block(kv, k.shape[1], dk, dv)
    want = o.attn_decode_sparse_v(ok, ov, kv, qd, scale, tau, ref_block=block)
    assert_attention_close(got, want, what=f"sparse-V {dk}/{dv} block rule, block {block}")


# ---------------------------------------------------------------- Q x centroid table path

def _run_path(bits, q, k, v, kv_len, path, q_bf16=False, what="", tau=0.0):
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import bf16_cuda, cuda
    kc, vc, ok, ov = _caches(bits, k, v)
    scale = 1.0 / math.sqrt(q.shape[1])
    print(f"[decode] {what} path={path} bits={bits} n_q={q.shape[0]} n_kv={k.shape[1]} kv={kv_len}", flush=True)
    qt = bf16_cuda(q) if q_bf16 else cuda(q)
    got = b.tq_attn_decode_path(kc, vc, kv_len, qt, scale, path, sparse_v_tau=tau)
    torch.cuda.synchronize()
    return got.cpu().numpy(), kc, vc, ok, ov, qt, scale


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("n_q,n_kv", [(1, 1), (4, 4), (2, 1), (8, 4), (8, 1)])
@pytest.mark.parametrize("kv_len", [1, 17, 256, 257, 3000, 32768])
def test_table_path(bits, n_q, n_kv, kv_len):
    """The Q x centroid table kernel of [PR36] (c) (TQ_DECODE_TABLE):
    1, 2 and 8 q heads per kv head, outlier-channel K and V, lengths from one
    key to 128 splits with ragged tails, bf16 and f32 queries."""
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import assert_attention_close
    q, k, v = inputs.outlier_decode(seed=40 + bits + n_q, kv_len=max(kv_len, 256), n_q=n_q, n_kv=n_kv)
    got, _, _, ok, ov, _, scale = _run_path(bits, q, k, v, kv_len, b.TQ_DECODE_TABLE, q_bf16=(kv_len % 2 == 0),
                                            what=f"table {n_q}/{n_kv}")
    want = o.attn_decode(ok, ov, kv_len, q.astype(np.float64), scale)
    assert_attention_close(got, want, what=f"table {n_q}/{n_kv} kv={kv_len}")


def test_decode_paths_auto_matrix_and_refusals():
    """TQ_DECODE_AUTO and TQ_DECODE_MATRIX give tq_attn_decode's bits; the
    table path refuses turbo4, 256-wide heads and more than 8 q heads per kv
    head, and an unknown path is an invalid argument."""
    from quantized_kv_cache_tq_amd import binding as b
    q, k, v = inputs.outlier_decode(seed=48, kv_len=5000, n_q=16, n_kv=2)
    got_auto, kc, vc, _, _, qt, scale = _run_path(3, q, k, v, 5000, b.TQ_DECODE_AUTO, q_bf16=True, what="auto")
    got_mat = b.tq_attn_decode_path(kc, vc, 5000, qt, scale, b.TQ_DECODE_MATRIX).cpu().numpy()
    plain = b.tq_attn_decode(kc, vc, 5000, qt, scale).cpu().numpy()
    np.testing.assert_array_equal(got_auto, plain)
    np.testing.assert_array_equal(got_mat, plain)
    with pytest.raises(b.TQError) as e:
        b.tq_attn_decode_path(kc, vc, 5000, qt, scale, 7)
    assert e.value.status == b.TQ_ERR_INVALID_ARG
    for bits, n_q, n_kv, d in [(4, 2, 1, 128), (3, 16, 1, 128), (3, 2, 1, 256)]:
        kc2, vc2 = b.new_cache(bits, d, n_kv, 64), b.new_cache(bits, d, n_kv, 64)
        with pytest.raises(b.TQError) as e:
            b.tq_attn_decode_path_workspace(kc2, vc2, 64, n_q, b.TQ_DECODE_TABLE)
        assert e.value.status == b.TQ_ERR_UNSUPPORTED


@pytest.mark.parametrize("bits,tau", [(2, 1e-2), (3, 5e-3)])
def test_table_sparse_v_within_bound(bits, tau):
    """The table kernel's value skip: within the oracle's bound of the dense
    output (its reference is the maximum of each 256-key split, at most the
    true maximum), and at the bar against the split-block emulation."""
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import assert_attention_close
    kv = 8192
    q, k, v = inputs.outlier_decode(seed=44 + bits, kv_len=kv, n_q=8, n_kv=4)
    got, _, _, ok, ov, _, scale = _run_path(bits, q, k, v, kv, b.TQ_DECODE_TABLE, q_bf16=True, what="table sparse",
                                            tau=tau)
    qd = q.astype(np.float64)
    dense = o.attn_decode(ok, ov, kv, qd, scale)
    bound, n_t = o.sparse_v_bound(ok, ov, kv, qd, scale, tau)
    err = np.abs(got - dense).max(axis=1)
    assert n_t.sum() > 0
    assert np.all(err <= bound + 2e-3), (err - bound).max()
    want = o.attn_decode_sparse_v(ok, ov, kv, qd, scale, tau, ref_block=256)
    assert_attention_close(got, want, what="table sparse-V, 256-key blocks")
