"""CPU tests of the C ABI boundary (no GPU needed).

* libtq.so loads and exports every function include/tq.h declares;
* the host-side helpers (plane sizes, codebook, status strings) agree with
  the header's contract and with the oracle's independently derived values;
* every argument error that the host can detect is reported before any HIP
  call (the pointers below are fake and never dereferenced).
"""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle as o

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq.h")
LIB = os.path.join(ROOT, "quantized_kv_cache_tq_amd", "lib", "libtq.so")

needs_lib = pytest.mark.skipif(not os.path.exists(LIB), reason="libtq.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|tq_status|size_t)\s*(tq_\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["tq_set_rows", "tq_attn_decode", "tq_attn_decode_batch", "tq_attn_prefill", "tq_attn_int8_prompt",
              "tq_codebook", "tq_cache_plane_bytes", "tq_version", "tq_status_str"]:
        assert n in names


@needs_lib
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(lib, name), name
    from quantized_kv_cache_tq_amd import binding
    assert set(binding.EXPORTED) == set(declared_functions())


@needs_lib
def test_version_and_status_strings():
    from quantized_kv_cache_tq_amd import binding as b
    assert "gfx950" in b.tq_version()
    assert b.status_str(0) == "ok"
    assert "workspace" in b.status_str(-3)


@needs_lib
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_codebook_matches_oracle(bits):
    from quantized_kv_cache_tq_amd import binding as b
    vals, thr, words = b.tq_codebook(bits)
    np.testing.assert_array_equal(np.array(vals, np.float32), o.code_values(bits))
    np.testing.assert_array_equal(np.array(thr, np.float32), o.mag_thresholds(bits))
    assert words == o.splitmix64(0, 2)


@needs_lib
@pytest.mark.parametrize("bits,per_group", [(2, 32), (3, 48), (4, 64)])
def test_plane_bytes(bits, per_group):
    from quantized_kv_cache_tq_amd import binding as b
    cb, nb = b.tq_cache_plane_bytes(bits, 256, 8, 1000)
    assert cb == 8 * 1000 * 2 * per_group and nb == 8 * 1000 * 2 * 2
    with pytest.raises(b.TQError):
        b.tq_cache_plane_bytes(bits, 192, 8, 1000)      # not a multiple of 128
    with pytest.raises(b.TQError):
        b.tq_cache_plane_bytes(5, 128, 8, 1000)         # no such type


@needs_lib
def test_q8_plane_bytes_and_rules():
    """The 8-bit block K format: one byte per element and a float16 scale
    per 32; it is a K cache for decode only."""
    from quantized_kv_cache_tq_amd import binding as b
    assert b.tq_cache_plane_bytes(8, 256, 4, 100) == (4 * 100 * 256, 4 * 100 * 8 * 2)
    with pytest.raises(b.TQError):
        b.tq_codebook(8)
    lib = b.load_library()
    q8, t3 = _cache(b, type_=8), _cache(b, type_=3)
    dec = lambda k, v: lib.tq_attn_decode(ctypes.byref(k), ctypes.byref(v), 50, FAKE + 8, 1, 32, 0.1, 0.0,
                                          FAKE, FAKE, 1 << 20, None)
    assert dec(t3, q8) == -2                      # V in the 8-bit format: no kernel
    assert dec(q8, q8) == -2
    assert dec(q8, t3) == -1                      # accepted pair; the misaligned q is what fails
    pre = lambda k, v: lib.tq_attn_prefill(ctypes.byref(k), ctypes.byref(v), 50, FAKE, 1, 3, 32, 47, 0.1,
                                           FAKE, FAKE, 1 << 20, None)
    assert pre(q8, t3) == -2
    assert lib.tq_set_rows(ctypes.byref(q8), FAKE, FAKE, 0, None) == 0


# ------------------------------------------------------------ host validation

FAKE = 0x10000000  # aligned, never dereferenced: every call below fails on the host


def _cache(b, type_=3, head_dim=128, n_kv=4, n_cells=100, codes=FAKE, norms=FAKE, reserved=0):
    return b.TQCache(type_, head_dim, n_kv, reserved, n_cells, codes, norms)


@needs_lib
def test_set_rows_rejects_bad_arguments():
    from quantized_kv_cache_tq_amd import binding as b
    lib = b.load_library()
    ok = _cache(b)
    assert lib.tq_set_rows(None, FAKE, FAKE, 1, None) == -1
    assert lib.tq_set_rows(ctypes.byref(_cache(b, type_=5)), FAKE, FAKE, 1, None) == -1
    assert lib.tq_set_rows(ctypes.byref(_cache(b, head_dim=192)), FAKE, FAKE, 1, None) == -1
    assert lib.tq_set_rows(ctypes.byref(_cache(b, codes=FAKE + 4)), FAKE, FAKE, 1, None) == -1
    assert lib.tq_set_rows(ctypes.byref(_cache(b, norms=FAKE + 2)), FAKE, FAKE, 1, None) == -1
    assert lib.tq_set_rows(ctypes.byref(_cache(b, reserved=1)), FAKE, FAKE, 1, None) == -1
    assert lib.tq_set_rows(ctypes.byref(ok), None, FAKE, 1, None) == -1
    assert lib.tq_set_rows(ctypes.byref(ok), FAKE + 4, FAKE, 1, None) == -1
    assert lib.tq_set_rows(ctypes.byref(ok), FAKE, FAKE, -1, None) == -1
    assert lib.tq_set_rows(ctypes.byref(ok), FAKE, FAKE, 0, None) == 0      # empty: no-op


@needs_lib
def test_decode_rejects_bad_arguments():
    from quantized_kv_cache_tq_amd import binding as b
    lib = b.load_library()
    k, v = _cache(b), _cache(b)
    call = lambda k=k, v=v, kv=50, q=FAKE, qd=1, nq=32, sc=0.1, tau=0.0, out=FAKE: lib.tq_attn_decode(
        ctypes.byref(k), ctypes.byref(v), kv, q, qd, nq, sc, tau, out, FAKE, 1 << 20, None)
    assert call(kv=0) == -1
    assert call(kv=101) == -1                     # beyond n_cells
    assert call(nq=30) == -1                      # not a multiple of n_kv_heads
    assert call(v=_cache(b, type_=2)) == -1       # K and V types differ
    assert call(v=_cache(b, n_kv=2)) == -1
    assert call(k=_cache(b, head_dim=384), v=_cache(b, head_dim=384)) == -2   # 3 groups: no kernel
    assert call(v=_cache(b, head_dim=384)) == -2
    assert call(v=_cache(b, n_cells=101)) == -1   # K and V address cells alike
    assert call(v=_cache(b, head_dim=256, type_=4)) == -1
    assert call(q=None) == -1
    assert call(q=FAKE + 2) == -1
    assert call(out=FAKE + 8) == -1
    assert call(qd=7) == -1
    assert call(sc=float("nan")) == -1
    assert call(tau=-1.0) == -1
    assert call(tau=float('nan')) == -1


@needs_lib
def test_decode_batch_rejects_bad_arguments():
    from quantized_kv_cache_tq_amd import binding as b
    lib = b.load_library()
    k, v = _cache(b), _cache(b)
    call = lambda k=k, v=v, ns=3, nr=2, st=FAKE, ln=FAKE, mx=50, q=FAKE, nq=32, tau=0.0, out=FAKE: \
        lib.tq_attn_decode_batch(ctypes.byref(k), ctypes.byref(v), ns, nr, st, ln, mx, q, 1, nq, 0.1, tau, out,
                                 FAKE, 1 << 20, None)
    assert call(ns=-1) == -1
    assert call(ns=65536) == -1
    assert call(nr=0) == -1
    assert call(nr=17) == -1
    assert call(st=None) == -1
    assert call(ln=None) == -1
    assert call(st=FAKE + 4) == -1                # int64 array, 8-byte aligned
    assert call(ln=FAKE + 2) == -1
    assert call(mx=0) == -1
    assert call(mx=101) == -1                     # beyond n_cells
    assert call(nq=30) == -1
    assert call(v=_cache(b, n_cells=99)) == -1
    assert call(k=_cache(b, head_dim=384), v=_cache(b, head_dim=384)) == -2
    assert call(tau=-1.0) == -1
    assert call(q=FAKE + 8) == -1
    assert call(ns=0) == 0                        # no sequences: no-op
    n = ctypes.c_size_t(7)
    assert lib.tq_attn_decode_batch_workspace(ctypes.byref(k), ctypes.byref(v), 0, 1, 50, 32, ctypes.byref(n)) == 0
    assert n.value == 0
    assert lib.tq_attn_decode_batch_workspace(ctypes.byref(k), ctypes.byref(v), 2, 0, 50, 32, ctypes.byref(n)) == -1


@needs_lib
def test_decode_workspace_rejects_bad_arguments():
    from quantized_kv_cache_tq_amd import binding as b
    lib = b.load_library()
    k, v = _cache(b), _cache(b, head_dim=256)
    n = ctypes.c_size_t()
    ws = lambda k=k, v=v, kv=50, nq=32, out=ctypes.byref(n): lib.tq_attn_decode_workspace(
        ctypes.byref(k) if k is not None else None, ctypes.byref(v) if v is not None else None, kv, nq, out)
    assert ws(v=None) == -1
    assert ws(out=None) == -1
    assert ws(kv=0) == -1
    assert ws(v=_cache(b, n_kv=2)) == -1
    assert ws(v=_cache(b, head_dim=512)) == -2


@needs_lib
def test_prefill_rejects_bad_arguments():
    from quantized_kv_cache_tq_amd import binding as b
    lib = b.load_library()
    k = _cache(b, head_dim=256, n_kv=8, n_cells=1024)
    call = lambda k=k, v=k, kv=1024, nrows=3, nq=16, q0=1021, qd=1, sc=0.0625: lib.tq_attn_prefill(
        ctypes.byref(k), ctypes.byref(v), kv, FAKE, qd, nrows, nq, q0, sc, FAKE, FAKE, 1 << 20, None)
    assert call(q0=1022) == -1                    # q_pos0 + n_rows > kv_len
    assert call(q0=-1) == -1
    assert call(nrows=-1) == -1
    assert call(kv=2048) == -1
    assert call(nq=12) == -1
    assert call(v=_cache(b, head_dim=256, n_kv=8, n_cells=2048)) == -1   # n_cells differ
    assert call(v=_cache(b, head_dim=128, n_kv=8, n_cells=1024)) == -1   # widths differ
    d384 = _cache(b, head_dim=384, n_kv=8, n_cells=1024)
    assert call(k=d384, v=d384) == -2             # head_dim 384: no kernel
    d128 = _cache(b, head_dim=128, n_kv=8, n_cells=1024)
    assert call(k=d128, v=_cache(b, head_dim=256, n_kv=8, n_cells=1024)) == -1
    assert call(k=d128, v=d128, nrows=0, q0=0) == 0
    assert call(nrows=0, q0=0) == 0               # empty: no-op


@needs_lib
def test_int8_rejects_bad_arguments():
    from quantized_kv_cache_tq_amd import binding as b
    lib = b.load_library()
    call = lambda nq=2048, nqh=8, nkv=1, d=128, pt=FAKE, npp=1250, ctx=40000, q0=37952, q=FAKE: \
        lib.tq_attn_int8_prompt(q, nq, nqh, FAKE, FAKE, FAKE, FAKE, nkv, d, pt, npp, ctx, q0, 0.08,
                                FAKE, FAKE, 1 << 20, None)
    assert call(q0=37953) == -1
    assert call(nqh=9, nkv=2) == -1              # not a multiple of n_kv_heads
    assert call(d=64) == -2
    assert call(nqh=32) == -2                     # 32 q heads per kv head
    assert call(pt=None) == -1
    assert call(pt=FAKE + 2) == -1
    assert call(npp=0) == -1
    assert call(q=FAKE + 4) == -1
    assert call(nq=0, q0=0) == 0


def test_static_scratch_size_matches_header():
    """The binding's size of the allocation-free decode's device array is the
    header's TQ_STATIC_SCRATCH_BYTES."""
    import re
    from quantized_kv_cache_tq_amd import binding
    hdr = open(os.path.join(ROOT, "include", "tq.h")).read()
    m = re.search(r"#define TQ_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == binding.STATIC_SCRATCH_BYTES
