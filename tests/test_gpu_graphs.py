"""Every entry point under HIP graph capture: a graph captured once and
replayed several times, with new inputs written eagerly between replays (as a
serving loop would), gives on every replay the bits of the eager call on the
same inputs.

The "HIP/turbo3: graph-safe decode + inline-dequant TILE prefill" page
(section Graph-safe decode) traces its failure to work done at capture time
that a replay does not redo; the library allocates nothing and reads every
size from its arguments, so a replay is the eager call.  (Single- and
multi-sequence decode replays are covered in test_gpu_decode.py and
test_gpu_decode_batch.py.)
"""

import math

import numpy as np
import pytest

from quantized_kv_cache_tq_amd import inputs

pytestmark = pytest.mark.gpu


def _capture(fn):
    """fn captured into a graph on a side stream (warmed once first)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn(s)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_set_rows_graph_replay(bits):
    """Quantize into fixed cells from a source buffer refilled between
    replays; codes and norms equal the eager call's bit for bit."""
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    n_cells, n_rows, n_kv, d = 600, 200, 2, 256
    print(f"[graph set_rows] bits={bits}", flush=True)
    rng = np.random.default_rng(70 + bits)
    src = torch.empty((n_rows, n_kv, d), dtype=torch.float32, device="cuda")
    idx = torch.from_numpy(rng.permutation(n_cells)[:n_rows].astype(np.int64)).cuda()
    gc = b.new_cache(bits, d, n_kv, n_cells)
    ec = b.new_cache(bits, d, n_kv, n_cells)
    g = _capture(lambda s=None: b.tq_set_rows(gc, src, idx, stream=s))
    for step in range(3):
        src.copy_(torch.from_numpy(inputs.normal(rng, (n_rows, n_kv, d)) * np.float32(1 + 3 * step)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        b.tq_set_rows(ec, src, idx)
        torch.cuda.synchronize()
        assert torch.equal(gc.codes, ec.codes), f"codes differ at replay {step}"
        assert torch.equal(gc.norms, ec.norms), f"norms differ at replay {step}"


@pytest.mark.parametrize("bits,d", [(3, 256), (2, 256), (4, 128)])
def test_prefill_graph_replay(bits, d):
    """Causal prefill over a fixed cache with the query rows rewritten
    between replays."""
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import cuda
    rows, kv, n_q, n_kv = 300, 300, 8, 4
    print(f"[graph prefill] bits={bits} d={d}", flush=True)
    _, k, v = inputs.prefill(seed=80 + bits, rows=rows, kv_len=kv, n_q=n_q, n_kv=n_kv, d=d)
    idx = torch.arange(kv, dtype=torch.int64, device="cuda")
    kc, vc = b.new_cache(bits, d, n_kv, kv), b.new_cache(bits, d, n_kv, kv)
    b.tq_set_rows(kc, cuda(k), idx)
    b.tq_set_rows(vc, cuda(v), idx)
    q = torch.empty((rows, n_q, d), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((rows, n_q, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, b.tq_attn_prefill_workspace(kc, rows, n_q, kv)), dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(d)
    call = lambda s=None: b.tq_attn_prefill(kc, vc, kv, q, 0, scale, out=out, workspace=ws, stream=s)
    q.copy_(torch.zeros_like(q))
    g = _capture(call)
    rng = np.random.default_rng(90 + bits)
    for step in range(3):
        q.copy_(torch.from_numpy(inputs.bf16_round(inputs.normal(rng, (rows, n_q, d)))).to(torch.bfloat16))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replayed = out.clone()
        call()
        torch.cuda.synchronize()
        assert torch.equal(replayed, out), f"replay {step} differs from the eager call"


@pytest.mark.parametrize("n_q,ctx", [(4096, 4096), (40, 2048)])
def test_int8_prompt_graph_replay(n_q, ctx):
    """Paged int8 prompt attention with the queries rewritten between
    replays: 4096 queries fill the device without key splits; 40 queries
    split the key range and add the merge kernel to the graph."""
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import cuda
    print(f"[graph int8] n_q={n_q} ctx={ctx}", flush=True)
    dd = inputs.int8_prompt(seed=100, ctx=ctx, n_q=n_q, n_q_heads=8, n_kv=1, d=128)
    k8, v8 = cuda(dd["k8"]), cuda(dd["v8"])
    ks, vs, pt = cuda(dd["k_scale"]), cuda(dd["v_scale"]), cuda(dd["page_table"])
    q = torch.empty((n_q, 8, 128), dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    ws = torch.empty(max(1, b.tq_attn_int8_prompt_workspace(n_q, 8, 1, 128, ctx)), dtype=torch.uint8,
                     device="cuda")
    q_pos0 = ctx - n_q
    call = lambda s=None: b.tq_attn_int8_prompt(q, k8, v8, ks, vs, pt, ctx, q_pos0, 1.0 / math.sqrt(128),
                                                out=out, workspace=ws, stream=s)
    q.copy_(torch.zeros_like(q))
    g = _capture(call)
    rng = np.random.default_rng(110)
    for step in range(3):
        q.copy_(torch.from_numpy(inputs.normal(rng, (n_q, 8, 128))))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replayed = out.clone()
        call()
        torch.cuda.synchronize()
        assert torch.equal(replayed, out), f"replay {step} differs from the eager call"
