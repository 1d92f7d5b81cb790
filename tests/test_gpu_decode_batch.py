"""GPU parity of tq_attn_decode_batch (several sequences, 1-16 query rows
each, lengths read from device arrays) against the float64 oracle's
attn_decode_batch; bar: max-abs <= 2e-3 and relative L2 <= 1e-3 per row.

The decode case of the "Graph-safe decode" section of the PR28 page: query
batches of at most two rows take the single-row kernel, and a captured graph
replays it with the lengths of each step.
"""

import math

import numpy as np
import pytest

import oracle as o
from quantized_kv_cache_tq_amd import inputs

pytestmark = pytest.mark.gpu


def _caches(bits, k, v):
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import cuda
    n, n_kv, dk = k.shape
    dv = v.shape[2]
    idx = np.arange(n)
    kc, vc = b.new_cache(bits, dk, n_kv, n), b.new_cache(bits, dv, n_kv, n)
    b.tq_set_rows(kc, cuda(k), cuda(idx))
    b.tq_set_rows(vc, cuda(v), cuda(idx))
    ok, ov = o.new_cache(bits, dk, n_kv, n), o.new_cache(bits, dv, n_kv, n)
    o.set_rows(ok, k, idx)
    o.set_rows(ov, v, idx)
    torch.cuda.synchronize()
    return kc, vc, ok, ov


def _seq_arrays(starts, lens):
    import torch
    return (torch.tensor(starts, dtype=torch.int64, device="cuda"),
            torch.tensor(lens, dtype=torch.int32, device="cuda"))


def _check(got, want, what):
    from gpu_util import assert_attention_close
    n_seq, n_rows = want.shape[:2]
    for i in range(n_seq):
        for r in range(n_rows):
            if not np.any(want[i, r]):
                np.testing.assert_array_equal(got[i, r], 0.0, err_msg=f"{what} seq {i} row {r}")
            else:
                assert_attention_close(got[i, r], want[i, r], what=f"{what} seq {i} row {r}")


def _run(bits, n_cells, n_kv, n_q, dk, dv, starts, lens, n_rows, max_len, seed, q_bf16=True, tau=0.0):
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import bf16_cuda, cuda
    _, k, v = inputs.small_decode(seed=seed, kv_len=n_cells, n_q=1, n_kv=n_kv, d=dk, dv=dv)
    rng = np.random.default_rng(seed + 1)
    q = inputs.bf16_round(rng.standard_normal((len(starts), n_rows, n_q, dk)).astype(np.float32))
    kc, vc, ok, ov = _caches(bits, k, v)
    st, ln = _seq_arrays(starts, lens)
    scale = 1.0 / math.sqrt(dk)
    print(f"[decode-batch] bits={bits} heads={n_q}/{n_kv} dk={dk} dv={dv} rows={n_rows} "
          f"starts={starts} lens={lens} max={max_len}", flush=True)
    qt = bf16_cuda(q) if q_bf16 else cuda(q)
    got = b.tq_attn_decode_batch(kc, vc, st, ln, max_len, qt, scale, sparse_v_tau=tau)
    torch.cuda.synchronize()
    return got.cpu().numpy(), q, kc, vc, ok, ov, scale


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("n_rows", [1, 2])
def test_batch_parity(bits, n_rows):
    starts, lens = [0, 1000, 300, 2999, 1500], [1000, 2000, 1, 1, 64]
    got, q, *_, ok, ov, scale = _run(bits, 3000, 2, 8, 128, 128, starts, lens, n_rows, 2000, seed=bits)
    want = o.attn_decode_batch(ok, ov, starts, lens, q.astype(np.float64), scale)
    _check(got, want, f"turbo{bits} rows={n_rows}")


@pytest.mark.parametrize("n_q,n_kv", [(32, 4), (16, 1), (4, 4), (24, 2)])
def test_batch_head_groups(n_q, n_kv):
    """Two rows with 8 or 16 q heads per kv head: 16 or 32 (row, head) pairs,
    two or four head groups over the same cells."""
    starts, lens = [0, 2500, 700], [2500, 1500, 1799]
    got, q, *_, ok, ov, scale = _run(3, 4000, n_kv, n_q, 128, 128, starts, lens, 2, 2500, seed=n_q + n_kv)
    want = o.attn_decode_batch(ok, ov, starts, lens, q.astype(np.float64), scale)
    _check(got, want, f"gqa {n_q}/{n_kv}")


@pytest.mark.parametrize("dk,dv", [(256, 256), (256, 128)])
def test_batch_head_widths(dk, dv):
    starts, lens = [10, 0, 900], [990, 17, 100]
    got, q, *_, ok, ov, scale = _run(3, 1000, 2, 16, dk, dv, starts, lens, 2, 1000, seed=dk + dv, q_bf16=False)
    want = o.attn_decode_batch(ok, ov, starts, lens, q.astype(np.float64), scale)
    _check(got, want, f"widths {dk}/{dv}")


def test_batch_empty_and_clamped_entries():
    """Entries outside the contract are clamped on the device: a length
    beyond max_kv_len or past the cache end is cut, a start past the end
    leaves nothing, and rows that see no cell are zeros."""
    n_cells, max_len = 2000, 1200
    starts, lens = [0, 1500, 2500, -5, 100, 50], [5000, 900, 10, 3, 0, 1]
    eff_s = [min(max(a, 0), n_cells) for a in starts]
    eff_l = [max(0, min(n, max_len, n_cells - a)) for a, n in zip(eff_s, lens)]
    got, q, *_, ok, ov, scale = _run(3, n_cells, 1, 4, 128, 128, starts, lens, 2, max_len, seed=40)
    want = o.attn_decode_batch(ok, ov, eff_s, eff_l, q.astype(np.float64), scale)
    _check(got, want, "clamped")
    assert np.all(got[2] == 0) and np.all(got[4] == 0) and np.all(got[5, 0] == 0)


def test_batch_one_row_equals_single_decode():
    """One sequence of one row from cell 0 is the single-sequence call, bit
    for bit (same plan, same kernels)."""
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import bf16_cuda
    q, k, v = inputs.outlier_decode(seed=41, kv_len=32768)
    kc, vc, ok, ov = _caches(3, k, v)
    scale = 1.0 / math.sqrt(q.shape[1])
    qt = bf16_cuda(q)
    single = b.tq_attn_decode(kc, vc, 32768, qt, scale).cpu().numpy()
    st, ln = _seq_arrays([0], [32768])
    batch = b.tq_attn_decode_batch(kc, vc, st, ln, 32768, qt.reshape(1, 1, *qt.shape), scale).cpu().numpy()
    np.testing.assert_array_equal(batch[0, 0], single)


def test_two_rows_gqa8_32k():
    """Speculative-verify style: two rows over 32K cells, 32 q / 4 kv heads
    (two head groups), one sequence."""
    got, q, *_, ok, ov, scale = _run(3, 32768, 4, 32, 128, 128, [0], [32768], 2, 32768, seed=42)
    want = o.attn_decode_batch(ok, ov, [0], [32768], q.astype(np.float64), scale)
    _check(got, want, "2 rows 32k")


def test_batch_sparse_v_limits():
    """tau = 0 is the dense batched call bit for bit; tau = 2 leaves every
    key out of the value sum."""
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import bf16_cuda
    starts, lens = [0, 500], [500, 1000]
    dense, q, kc, vc, *_ = _run(3, 1500, 2, 8, 128, 128, starts, lens, 2, 1000, seed=43)
    st, ln = _seq_arrays(starts, lens)
    qt = bf16_cuda(q)
    zero = b.tq_attn_decode_batch(kc, vc, st, ln, 1000, qt, 1 / math.sqrt(128), sparse_v_tau=0.0)
    np.testing.assert_array_equal(zero.cpu().numpy(), dense)
    allskip = b.tq_attn_decode_batch(kc, vc, st, ln, 1000, qt, 1 / math.sqrt(128), sparse_v_tau=2.0)
    assert np.all(allskip.cpu().numpy() == 0)


def test_batch_graph_replay_with_new_lengths():
    """A graph captured once replays with the lengths the device arrays hold
    at replay time (updated eagerly between replays, as a serving loop
    would); every replay equals the eager call bit for bit and the oracle at
    the normal bar."""
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import bf16_cuda
    n_cells, max_len = 6000, 3000
    _, k, v = inputs.small_decode(seed=44, kv_len=n_cells, n_q=1, n_kv=2)
    kc, vc, ok, ov = _caches(3, k, v)
    rng = np.random.default_rng(45)
    q = inputs.bf16_round(rng.standard_normal((3, 2, 16, 128)).astype(np.float32))
    qt = bf16_cuda(q)
    scale = 1.0 / math.sqrt(128)
    starts = [0, 3000, 1000]
    st, ln = _seq_arrays(starts, [1, 1, 1])
    ws = torch.empty(b.tq_attn_decode_batch_workspace(kc, vc, 3, 2, max_len, 16), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((3, 2, 16, 128), dtype=torch.float32, device="cuda")
    call = lambda s=None: b.tq_attn_decode_batch(kc, vc, st, ln, max_len, qt, scale, out=out, workspace=ws,
                                                 stream=s)
    call()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call(s)
    torch.cuda.synchronize()
    for step, lens in enumerate([[2, 1, 64], [1000, 3000, 65], [2999, 17, 2000], [3000, 3000, 3000]]):
        ln.copy_(torch.tensor(lens, dtype=torch.int32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replayed = out.cpu().numpy().copy()
        call()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(replayed, out.cpu().numpy(), err_msg=f"step {step}")
        want = o.attn_decode_batch(ok, ov, starts, lens, q.astype(np.float64), scale)
        _check(replayed, want, f"replay step {step}")


@pytest.mark.parametrize("n_rows,n_q,n_kv", [(3, 8, 2), (5, 4, 1), (16, 2, 1), (1, 32, 2), (4, 48, 3)])
def test_batch_many_rows_and_wide_gqa(n_rows, n_q, n_kv):
    """Speculative-verify batches of 3-16 rows and 16 q heads per kv head:
    (row, head) pairs beyond eight take more head groups over the same cells,
    each column masked at its own row's causal limit."""
    starts, lens = [0, 900, 1500], [900, 600, n_rows - 1]
    got, q, *_, ok, ov, scale = _run(3, 2000, n_kv, n_q, 128, 128, starts, lens, n_rows, 900,
                                     seed=60 + n_rows + n_q)
    want = o.attn_decode_batch(ok, ov, starts, lens, q.astype(np.float64), scale)
    _check(got, want, f"rows={n_rows} heads={n_q}/{n_kv}")


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("q_bf16", [True, False])
def test_batch_sixteen_pairs_all_types(bits, q_bf16):
    """Two rows at 8 q heads per kv head: sixteen (row, head) pairs, served
    as two column sets of one workgroup over one decode of the cells, for
    every turbo type and both query dtypes."""
    starts, lens = [0, 1200, 2500], [1200, 1300, 700]
    got, q, *_, ok, ov, scale = _run(bits, 3200, 2, 16, 128, 128, starts, lens, 2, 1300, seed=120 + bits,
                                     q_bf16=q_bf16)
    want = o.attn_decode_batch(ok, ov, starts, lens, q.astype(np.float64), scale)
    _check(got, want, f"16 pairs turbo{bits} bf16={q_bf16}")
