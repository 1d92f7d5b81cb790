"""GPU parity of tq_set_rows: packed codes and float16 norms must equal the
oracle's bit for bit (called through the C ABI via the ctypes binding)."""

import numpy as np
import pytest

import oracle as o
from quantized_kv_cache_tq_amd import inputs

pytestmark = pytest.mark.gpu


def _gpu_set_rows(bits, src, cell_idx, n_cells):
    import torch
    from quantized_kv_cache_tq_amd import binding as b
    from gpu_util import cuda
    n_rows, n_kv, d = src.shape
    c = b.new_cache(bits, d, n_kv, n_cells)
    b.tq_set_rows(c, cuda(src), cuda(np.asarray(cell_idx, np.int64)))
    torch.cuda.synchronize()
    return c.codes.cpu().numpy(), c.norms.cpu().numpy()


def _oracle_set_rows(bits, src, cell_idx, n_cells):
    n_rows, n_kv, d = src.shape
    c = o.new_cache(bits, d, n_kv, n_cells)
    o.set_rows(c, src, cell_idx)
    return c["codes"], c["norms"]


def _assert_planes_equal(bits, src, cell_idx, n_cells, what):
    gc, gn = _gpu_set_rows(bits, src, cell_idx, n_cells)
    oc, on = _oracle_set_rows(bits, src, cell_idx, n_cells)
    print(f"[set_rows] {what} bits={bits} src={src.shape}", flush=True)
    bad = np.argwhere(gc != oc)
    assert bad.size == 0, f"{what}: {len(bad)} code bytes differ, first at {bad[:4].tolist()}"
    np.testing.assert_array_equal(gn.view(np.uint16), on.view(np.uint16), err_msg=what)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_small_decode_shape(bits):
    q, k, v = inputs.small_decode(seed=0)
    _assert_planes_equal(bits, k, np.arange(256), 256, "cfg-small K")
    _assert_planes_equal(bits, v, np.arange(256), 256, "cfg-small V")


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_scattered_rows_multi_group(bits):
    rng = np.random.default_rng(11)
    src = (rng.standard_normal((77, 3, 384)) * rng.uniform(0.01, 100, (77, 3, 1))).astype(np.float32)
    cells = rng.permutation(200)[:77]
    _assert_planes_equal(bits, src, cells, 200, "scattered")


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_adversarial_groups(bits):
    rows = []
    z = np.zeros(128, np.float32)
    rows.append(z.copy())                                   # zero group
    nz = z.copy(); nz[:] = -0.0; rows.append(nz)            # negative zeros
    for j, a in [(0, -3.0), (77, 1e-3), (127, 7.5)]:        # impulses: |y| = 1 exactly
        e = z.copy(); e[j] = a; rows.append(e)
    rows.append(np.full(128, 2.0 ** -70, np.float32))       # subnormal squares
    rows.append(np.full(128, 2.0 ** -140, np.float32))      # subnormal inputs, squares underflow
    big = np.random.default_rng(1).standard_normal(128).astype(np.float32) * np.float32(1e4)
    rows.append(big)                                        # norm > 65504: float16 inf norm
    rows.append(np.random.default_rng(2).integers(-3, 4, 128).astype(np.float32))  # ties likely
    alt = np.ones(128, np.float32); alt[1::2] = -1; rows.append(alt)
    rng = np.random.default_rng(3)
    for _ in range(6):
        rows.append(rng.standard_normal(128).astype(np.float32) * np.float32(10.0 ** rng.uniform(-30, 30)))
    src = np.stack(rows)[:, None, :]
    _assert_planes_equal(bits, src, np.arange(len(rows)), len(rows), "adversarial")


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_non_finite_groups(bits):
    """Groups holding a NaN, an infinity, both infinities, or finite values
    whose squares overflow: the norm is NaN or +inf, the scale 1/norm is 0
    (the norm is not > 0, or 1/inf), every coordinate is 0 or NaN, so every
    code is +level 0 (comparisons with NaN fail) and the stored norm is the
    float16 NaN or infinity."""
    z = np.random.default_rng(5).standard_normal(128).astype(np.float32)
    rows = []
    for idx, val in [((17,), np.nan), ((3,), np.inf), ((100,), -np.inf), ((5, 6), None)]:
        r = z.copy()
        if val is None:
            r[5], r[6] = np.inf, -np.inf
        else:
            r[list(idx)] = val
        rows.append(r)
    rows.append(np.full(128, np.float32(3e38)))                # squares overflow: norm +inf
    rows.append(z.copy())                                      # a finite neighbour, unaffected
    src = np.stack(rows)[:, None, :]
    n = len(rows)
    gc, gn = _gpu_set_rows(bits, src, np.arange(n), n)
    with np.errstate(all="ignore"):
        oc, on = _oracle_set_rows(bits, src, np.arange(n), n)
    print(f"[set_rows] non-finite bits={bits}", flush=True)
    np.testing.assert_array_equal(gc, oc)
    gh, oh = gn.view(np.uint16).ravel(), on.view(np.uint16).ravel()
    nan_o = np.isnan(on.astype(np.float32).ravel())
    assert np.array_equal(np.isnan(gn.astype(np.float32).ravel()), nan_o)
    np.testing.assert_array_equal(gh[~nan_o], oh[~nan_o])


def test_outlier_decode_shape_turbo3():
    """The 32K x 4-head outlier-channel cache, K and V (2 x 131072 groups)."""
    q, k, v = inputs.outlier_decode(seed=0)
    _assert_planes_equal(3, k, np.arange(k.shape[0]), k.shape[0], "outlier K")
    _assert_planes_equal(3, v, np.arange(v.shape[0]), v.shape[0], "outlier V")


def test_out_of_range_cells_are_dropped():
    rng = np.random.default_rng(4)
    src = rng.standard_normal((4, 1, 128)).astype(np.float32)
    gc, gn = _gpu_set_rows(3, src, [2, -1, 5, 1], 5)        # rows 1 and 2 out of range
    oc, on = _oracle_set_rows(3, src[[0, 3]], [2, 1], 5)
    np.testing.assert_array_equal(gc, oc)
    np.testing.assert_array_equal(gn.view(np.uint16), on.view(np.uint16))


def test_deterministic():
    q, k, v = inputs.small_decode(seed=5, kv_len=300, n_kv=2)
    a = _gpu_set_rows(3, k, np.arange(300), 300)
    b = _gpu_set_rows(3, k, np.arange(300), 300)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1].view(np.uint16), b[1].view(np.uint16))
