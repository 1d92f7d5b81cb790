"""GPU parity of tq_attn_int8_prompt against the float64 oracle.

Bar: max-abs <= 1e-4.  The "#1821 qsa_prompt_attn" page (sections Change and
How to check) requires the same output bits whatever the physical placement
of the chunks; that is checked bit for bit between an identity and a random
page table.
"""

import math

import numpy as np
import pytest

import oracle as o
from quantized_kv_cache_tq_amd import inputs

pytestmark = pytest.mark.gpu

TOL = 1e-4


def _gpu(d, ctx_len, q_pos0, q_sel=None):
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import cuda
    dd = d["q"].shape[2]
    out = b.tq_attn_int8_prompt(cuda(d["q"]), cuda(d["k8"]), cuda(d["v8"]), cuda(d["k_scale"]),
                                cuda(d["v_scale"]), cuda(d["page_table"]), ctx_len, q_pos0,
                                1.0 / math.sqrt(dd))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _oracle(d, ctx_len, q_pos0, rows=None):
    q = d["q"] if rows is None else d["q"][rows]
    dd = d["q"].shape[2]
    if rows is None:
        return o.attn_int8_prompt(q, d["k8"], d["v8"], d["k_scale"], d["v_scale"], d["page_table"],
                                  ctx_len, q_pos0, 1.0 / math.sqrt(dd))
    # one query at a time (its own causal horizon)
    outs = [o.attn_int8_prompt(d["q"][r:r + 1], d["k8"], d["v8"], d["k_scale"], d["v_scale"],
                               d["page_table"], ctx_len, q_pos0 + r, 1.0 / math.sqrt(dd))[0]
            for r in rows]
    return np.stack(outs)


def _check(got, want, what):
    err = float(np.abs(got - want).max())
    print(f"[int8] {what}: max_abs={err:.3g}", flush=True)
    assert np.all(np.isfinite(got)) and err <= TOL, f"{what}: max_abs={err:.3g}"


@pytest.mark.parametrize("n_q,ctx,nqh,nkv", [(256, 4096, 8, 1), (100, 2048, 8, 1), (64, 1024, 4, 2),
                                             (50, 640, 1, 1), (33, 960, 16, 1)])
def test_full_compare(n_q, ctx, nqh, nkv):
    d = inputs.int8_prompt(seed=n_q + ctx, ctx=ctx, n_q=n_q, n_q_heads=nqh, n_kv=nkv)
    got = _gpu(d, ctx, ctx - n_q)
    _check(got, _oracle(d, ctx, ctx - n_q), f"full n_q={n_q} ctx={ctx} heads={nqh}/{nkv}")


def test_split_path_few_queries():
    """Three queries: the key range is split across workgroups and merged."""
    d = inputs.int8_prompt(seed=3, ctx=8192, n_q=3)
    _check(_gpu(d, 8192, 8189), _oracle(d, 8192, 8189), "split")


def test_partial_last_page():
    """ctx_len not a multiple of the 32-cell page: the tail page is partly used."""
    d = inputs.int8_prompt(seed=4, ctx=1024, n_q=40)
    _check(_gpu(d, 1000, 960), _oracle(d, 1000, 960), "partial page")


@pytest.mark.parametrize("ctx", [40000, 140000])
def test_prompt_shape_sampled(ctx):
    """2048 queries x 8 heads against 40000 / 140000 cells at full size; the
    oracle checks a sample of queries (each with its own causal horizon)."""
    d = inputs.int8_prompt(seed=0, ctx=ctx)
    n_q = d["q"].shape[0]
    got = _gpu(d, ctx, ctx - n_q)
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([[0, 1, 7, 8, n_q - 1], rng.integers(0, n_q, 11)]))
    _check(got[rows], _oracle(d, ctx, ctx - n_q, rows), f"ctx={ctx} sampled")


def test_page_placement_does_not_change_bits():
    a = inputs.int8_prompt(seed=7, ctx=4096, n_q=128)
    b_ = inputs.int8_prompt(seed=7, ctx=4096, n_q=128, identity_pages=True)
    assert not np.array_equal(a["page_table"], b_["page_table"])
    ga = _gpu(a, 4096, 4096 - 128)
    gb = _gpu(b_, 4096, 4096 - 128)
    np.testing.assert_array_equal(ga, gb)


def test_int8_deterministic():
    d = inputs.int8_prompt(seed=8, ctx=2048, n_q=64)
    np.testing.assert_array_equal(_gpu(d, 2048, 2048 - 64), _gpu(d, 2048, 2048 - 64))


def test_large_scales_and_sharp_scores():
    """V rows scaled by 1e5 (float16 scales near 3000) and K by 4: p * scale
    overflows float16 once p exceeds about 20, so tiles whose score maximum
    rises take the exact-maximum path; compared at unit V scale."""
    d = inputs.int8_prompt(seed=11, ctx=2048, n_q=256, v_mult=1e5, k_mult=4.0)
    got, want = _gpu(d, 2048, 2048 - 256), _oracle(d, 2048, 2048 - 256)
    _check(got / 1e5, want / 1e5, "large scales")


def test_query_rows_of_very_different_size():
    """The query's power-of-two scale is shared by each 32-row block (4
    queries x 8 heads share a block here): queries 1000x smaller and 30x
    larger than unit size sit in the same blocks, so the small rows' low
    float16 parts carry an absolute error bounded by the block's largest
    row.  Their softmax still has to meet the same bar."""
    d = inputs.int8_prompt(seed=12, ctx=2048, n_q=96)
    q = d["q"].copy()
    q[0::3] *= 1e-3
    q[1::3] *= 30.0
    d = dict(d, q=q)
    _check(_gpu(d, 2048, 2048 - 96), _oracle(d, 2048, 2048 - 96), "mixed query magnitudes")
