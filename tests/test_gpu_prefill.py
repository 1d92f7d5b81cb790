"""GPU parity of tq_attn_prefill (turbo3, and turbo2/turbo4 on a subset;
head_dim 256, and 128 on a subset) against the float64 oracle; bar: max-abs
<= 2e-3 and relative L2 <= 1e-3.

The grid mirrors the correctness check of the "HIP/turbo3: graph-safe decode
+ inline-dequant TILE prefill" page (section Correctness: turbo3, 256-wide
heads, batches of 3, 4, 6 rows (speculative verify) and 64, 128, 256 rows
(prefill) against 512 and 1024 keys), with the rows aligned to the end of the
keys.
"""

import math

import numpy as np
import pytest

import oracle as o
from quantized_kv_cache_tq_amd import inputs

pytestmark = pytest.mark.gpu


def _run(q, k, v, kv_len, q_pos0, q_bf16=True, what="", out_scale=1.0, bits=3):
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import assert_attention_close, bf16_cuda, cuda
    n_rows, n_q, d = q.shape
    n_cells, n_kv, _ = k.shape
    idx = np.arange(n_cells)
    kc, vc = b.new_cache(bits, d, n_kv, n_cells), b.new_cache(bits, d, n_kv, n_cells)
    b.tq_set_rows(kc, cuda(k), cuda(idx))
    b.tq_set_rows(vc, cuda(v), cuda(idx))
    ok, ov = o.new_cache(bits, d, n_kv, n_cells), o.new_cache(bits, d, n_kv, n_cells)
    o.set_rows(ok, k, idx)
    o.set_rows(ov, v, idx)
    scale = 1.0 / math.sqrt(d)
    print(f"[prefill] {what} bits={bits} rows={n_rows} heads={n_q}/{n_kv} kv={kv_len} q0={q_pos0}", flush=True)
    qt = bf16_cuda(q) if q_bf16 else cuda(q)
    got = b.tq_attn_prefill(kc, vc, kv_len, qt, q_pos0, scale)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    want = o.attn_prefill(ok, ov, kv_len, q.astype(np.float64), q_pos0, scale)
    # out_scale: the bar is stated for unit-scale V; V scaled by c scales the
    # output by c, so both sides are divided by c before the comparison
    return assert_attention_close(got / out_scale, want / out_scale, what=what), got


@pytest.mark.parametrize("kv", [512, 1024])
@pytest.mark.parametrize("nb", [3, 4, 6, 64, 128, 256])
def test_backend_ops_grid(nb, kv):
    q, k, v = inputs.prefill(seed=nb * 7 + kv, rows=nb, kv_len=kv)
    _run(q, k, v, kv, kv - nb, what="grid")


@pytest.mark.parametrize("rows", [512, 2048])
def test_causal_prefill(rows):
    q, k, v = inputs.prefill(seed=0, rows=rows)
    (ma, rl), _ = _run(q, k, v, rows, 0, what="causal")
    print(f"    max_abs={ma:.3g} rel_l2={rl:.3g}")


def test_causal_prefill_4096_sampled_rows():
    """4096 rows at full size; the oracle checks a sample of rows (first,
    last, and a random set) so it finishes in seconds."""
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import assert_attention_close, bf16_cuda, cuda
    rows = 4096
    q, k, v = inputs.prefill(seed=0, rows=rows)
    d = 256
    idx = np.arange(rows)
    kc, vc = b.new_cache(3, d, 8, rows), b.new_cache(3, d, 8, rows)
    b.tq_set_rows(kc, cuda(k), cuda(idx))
    b.tq_set_rows(vc, cuda(v), cuda(idx))
    got = b.tq_attn_prefill(kc, vc, rows, bf16_cuda(q), 0, 1 / 16.0)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    ok, ov = o.new_cache(3, d, 8, rows), o.new_cache(3, d, 8, rows)
    o.set_rows(ok, k, idx)
    o.set_rows(ov, v, idx)
    kd, vd = o.dequant_cache(ok, rows), o.dequant_cache(ov, rows)
    rng = np.random.default_rng(1)
    sample = np.unique(np.concatenate([[0, 1, 63, 64, rows - 1], rng.integers(0, rows, 40)]))
    for r in sample:
        want = o.attention(q[r:r + 1].astype(np.float64), kd, vd, 1 / 16.0, r)
        assert_attention_close(got[r:r + 1], want, what=f"row {r}")


def test_spec_verify_three_rows():
    q, k, v = inputs.prefill(seed=5, rows=3, kv_len=1024)
    _run(q, k, v, 1024, 1021, what="spec-verify")


@pytest.mark.parametrize("n_q,n_kv", [(8, 8), (16, 4), (16, 2), (8, 1)])
def test_gqa_variants(n_q, n_kv):
    q, k, v = inputs.prefill(seed=6, rows=100, kv_len=300, n_q=n_q, n_kv=n_kv)
    _run(q, k, v, 300, 200, what=f"gqa {n_q}/{n_kv}")


@pytest.mark.parametrize("rows,kv,q0", [(1, 1, 0), (1, 77, 76), (33, 33, 0), (65, 200, 100),
                                        (97, 97, 0), (130, 700, 570), (31, 640, 0)])
def test_ragged(rows, kv, q0):
    q, k, v = inputs.prefill(seed=rows + kv, rows=rows, kv_len=kv)
    _run(q, k, v, kv, q0, q_bf16=False, what="ragged f32-q")


def test_prefill_deterministic():
    q, k, v = inputs.prefill(seed=9, rows=200, kv_len=200)
    _, a = _run(q, k, v, 200, 0, what="det-1")
    _, b_ = _run(q, k, v, 200, 0, what="det-2")
    np.testing.assert_array_equal(a, b_)


def test_large_value_norms():
    """V rows with group norms near 45000: float16 P * norm would overflow
    whenever p exceeds about 1.4, so tiles whose score maximum rises take the
    exact-maximum path; outputs are compared at unit V scale."""
    q, k, v = inputs.prefill(seed=10, rows=300, kv_len=300)
    _run(q, k, v * np.float32(4000), 300, 0, what="large norms", out_scale=4000.0)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("rows,kv,q0", [(3, 1024, 1021), (64, 512, 448), (512, 512, 0), (65, 200, 100), (1, 1, 0)])
def test_turbo2_turbo4(bits, rows, kv, q0):
    """The other two cache types of [PR36] (d) through the same kernel (its
    pair table holds 2 or 4-bit code pairs)."""
    q, k, v = inputs.prefill(seed=rows + kv + bits, rows=rows, kv_len=kv)
    (ma, rl), _ = _run(q, k, v, kv, q0, what="turbo2/4", bits=bits)
    print(f"    max_abs={ma:.3g} rel_l2={rl:.3g}")


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("rows,kv,q0,n_q,n_kv", [(3, 1024, 1021, 16, 8), (64, 512, 448, 32, 4),
                                                 (256, 256, 0, 8, 8), (65, 200, 100, 16, 2),
                                                 (1, 1, 0, 8, 1), (130, 700, 570, 32, 8)])
def test_head_dim_128(bits, rows, kv, q0, n_q, n_kv):
    """128-wide heads (one group per key, the head width of the decode
    workload): the same kernel with half the products and half the codes per
    tile."""
    q, k, v = inputs.prefill(seed=rows + kv + 11 * bits, rows=rows, kv_len=kv, n_q=n_q, n_kv=n_kv, d=128)
    (ma, rl), _ = _run(q, k, v, kv, q0, q_bf16=(rows % 2 == 0), what="d128", bits=bits)
    print(f"    max_abs={ma:.3g} rel_l2={rl:.3g}")


def test_head_dim_128_causal_1024():
    q, k, v = inputs.prefill(seed=12, rows=1024, n_q=32, n_kv=8, d=128)
    (ma, rl), _ = _run(q, k, v, 1024, 0, what="d128 causal")
    print(f"    max_abs={ma:.3g} rel_l2={rl:.3g}")


@pytest.mark.parametrize("rows,kv,q0", [(3, 6000, 5997), (17, 6000, 2000), (64, 6000, 5936), (65, 6000, 5935)])
def test_few_rows_after_long_prefix(rows, kv, q0):
    """Calls of at most 64 rows run the split-key kernels (one sequence of
    q_pos0 + n_rows cells), 65 rows the tiled kernel; both against the oracle,
    including a prefix that ends before the cache does (q0 + rows < kv)."""
    q, k, v = inputs.prefill(seed=rows + 7, rows=rows, kv_len=kv)
    _run(q, k, v, kv, q0, what="long prefix")


@pytest.mark.parametrize("d,n_q,n_kv", [(256, 16, 2), (128, 32, 4)])
def test_few_rows_wide_gqa(d, n_q, n_kv):
    """64 rows at 8 q heads per kv head through the split-key kernels: 512
    (row, head) pairs per kv head, 64 head groups of eight (256-wide heads) or
    32 of sixteen (128-wide)."""
    q, k, v = inputs.prefill(seed=d + n_q, rows=64, kv_len=2000, n_q=n_q, n_kv=n_kv, d=d)
    _run(q, k, v, 2000, 1936, what=f"wide gqa {n_q}/{n_kv} d{d}")


def test_few_rows_workspace_rule():
    """The workspace of a split-key call comes from tq_attn_prefill_workspace
    with a kv_len at least q_pos0 + n_rows; a fresh prompt's tiled call needs
    none."""
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import bf16_cuda, cuda
    q, k, v = inputs.prefill(seed=9, rows=5, kv_len=3000, n_q=16, n_kv=8)
    idx = np.arange(3000)
    kc, vc = b.new_cache(3, 256, 8, 3000), b.new_cache(3, 256, 8, 3000)
    b.tq_set_rows(kc, cuda(k), cuda(idx))
    b.tq_set_rows(vc, cuda(v), cuda(idx))
    # 65 rows: the tiled kernel, whose key splits (a few row tiles after a
    # long prefix) also take a workspace of at most 256 MiB
    assert b.tq_attn_prefill_workspace(kc, 65, 16, 3000) <= 256 << 20
    assert b.tq_attn_prefill_workspace(kc, 65, 16, 65) == 0
    # 64 rows at 64 q heads over 65536 cells: the split-key decode path's
    # partials exceed 256 MiB, so the tiled kernel runs (its own partials
    # capped at 256 MiB)
    big = b.new_cache(3, 256, 8, 65536)
    assert b.tq_attn_prefill_workspace(big, 64, 64, 65536) <= 256 << 20
    assert 0 < b.tq_attn_prefill_workspace(big, 64, 64, 2000) <= 256 << 20
    need = b.tq_attn_prefill_workspace(kc, 5, 16, 3000)
    assert need > 0
    assert b.tq_attn_prefill_workspace(kc, 5, 16, 1000) <= need
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = b.tq_attn_prefill(kc, vc, 3000, bf16_cuda(q), 2995, 1.0 / 16.0, workspace=ws)
    torch.cuda.synchronize()
    with pytest.raises(b.TQError):
        b.tq_attn_prefill(kc, vc, 3000, bf16_cuda(q), 2995, 1.0 / 16.0,
                          workspace=torch.empty(64, dtype=torch.uint8, device="cuda"))
    assert np.all(np.isfinite(out.cpu().numpy()))


@pytest.mark.parametrize("rows,kv,q0,d,n_q,n_kv,bits", [
    (100, 6000, 5900, 256, 16, 8, 3), (256, 9000, 8744, 256, 16, 8, 3), (65, 4000, 1000, 256, 16, 8, 3),
    (130, 5000, 4870, 128, 32, 8, 3), (96, 7000, 6904, 256, 16, 2, 2), (80, 3000, 2920, 128, 16, 4, 4)])
def test_key_split_after_long_prefix(rows, kv, q0, d, n_q, n_kv, bits):
    """More than 64 rows after a long prefix: a grid of few row tiles splits
    the key range (power-of-two tiles per split, partials merged by a second
    kernel), including a prefix that ends before the cache does."""
    q, k, v = inputs.prefill(seed=rows + kv, rows=rows, kv_len=kv, n_q=n_q, n_kv=n_kv, d=d)
    _run(q, k, v, kv, q0, q_bf16=(bits != 2), what=f"key split d{d}", bits=bits)


def test_key_split_workspace():
    """The split plan's workspace comes from tq_attn_prefill_workspace (kv_len
    sizes it); fresh prompts and full grids need none."""
    from quantized_kv_cache_tq_amd import binding as b
    kc = b.new_cache(3, 256, 8, 9000)
    assert b.tq_attn_prefill_workspace(kc, 256, 16, 9000) > 0
    assert b.tq_attn_prefill_workspace(kc, 2048, 16, 9000) == 0
    assert b.tq_attn_prefill_workspace(kc, 512, 16, 512) == 0


@pytest.mark.parametrize("rows,kv,q0", [(3, 8192, 7933), (3, 8192, 4100), (40, 16384, 15000)])
def test_few_rows_workspace_for_kv_len(rows, kv, q0):
    """The split-key path runs with the plan for kv_len, the length its
    workspace query was given: a plan for the shorter q_pos0 + n_rows cells
    can pick fewer keys per split (more splits) than the one for kv_len
    (3 rows after 7933 of 8192 cells at 16 q / 8 kv heads), so it would not
    fit the workspace the query returned."""
    q, k, v = inputs.prefill(seed=rows + q0, rows=rows, kv_len=kv)
    _run(q, k, v, kv, q0, what="plan for kv_len")


@pytest.mark.parametrize("rows,kv,q0,d,n_q,n_kv", [
    (200, 300, 100, 256, 24, 8), (130, 130, 0, 256, 12, 2), (150, 400, 250, 128, 5, 1),
    (100, 160, 60, 128, 14, 2), (100, 6000, 5900, 256, 6, 2)])
def test_gqa_not_dividing_tile(rows, kv, q0, d, n_q, n_kv):
    """3, 5, 6 and 7 q heads per kv head in the tiled kernel (more than 64
    rows): a tile holds floor(64 / n_rep) rows of every head and its last
    64 - n_rep floor(64 / n_rep) qrows are idle; the last case also splits
    the key range (few row tiles after a long prefix)."""
    q, k, v = inputs.prefill(seed=rows + n_q, rows=rows, kv_len=kv, n_q=n_q, n_kv=n_kv, d=d)
    _run(q, k, v, kv, q0, q_bf16=(d == 256), what=f"gqa {n_q}/{n_kv} d{d}")
