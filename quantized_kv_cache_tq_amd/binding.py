"""ctypes binding over libtq.so (the C ABI of include/tq.h).

Argument marshalling only: torch supplies device memory and the current
stream; every step of the computation runs in the HIP kernels of libtq.so.
If the library has not been built, the first call raises ``TQError`` (there
is no fallback implementation).
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_int64, c_size_t, c_uint64, c_void_p

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libtq.so")

TQ_TURBO2, TQ_TURBO3, TQ_TURBO4, TQ_Q8 = 2, 3, 4, 8
TQ_F32, TQ_BF16 = 0, 1
TQ_OK, TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_WORKSPACE, TQ_ERR_HIP = 0, -1, -2, -3, -4
TQ_DECODE_AUTO, TQ_DECODE_MATRIX, TQ_DECODE_TABLE = 0, 1, 2
# size of the device array behind tq_attn_decode_static (TQ_STATIC_SCRATCH_BYTES)
STATIC_SCRATCH_BYTES = 16 << 20
TYPE_BY_NAME = {"turbo2": 2, "turbo3": 3, "turbo4": 4, "q8": 8}


class TQError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} ({status})")


class TQCache(ctypes.Structure):
    _fields_ = [("type", c_int32), ("head_dim", c_int32), ("n_kv_heads", c_int32),
                ("reserved", c_int32), ("n_cells", c_int64), ("codes", c_void_p),
                ("norms", c_void_p)]


_lib = None

_SIGS = {
    "tq_version": (c_char_p, []),
    "tq_status_str": (c_char_p, [c_int]),
    "tq_cache_plane_bytes": (c_int, [c_int, c_int32, c_int32, c_int64, POINTER(c_size_t), POINTER(c_size_t)]),
    "tq_codebook": (c_int, [c_int, POINTER(c_float), POINTER(c_float), POINTER(c_uint64)]),
    "tq_set_rows": (c_int, [POINTER(TQCache), c_void_p, c_void_p, c_int64, c_void_p]),
    "tq_attn_decode_workspace": (c_int, [POINTER(TQCache), POINTER(TQCache), c_int64, c_int32,
                                         POINTER(c_size_t)]),
    "tq_attn_decode": (c_int, [POINTER(TQCache), POINTER(TQCache), c_int64, c_void_p, c_int, c_int32,
                               c_float, c_float, c_void_p, c_void_p, c_size_t, c_void_p]),
    "tq_attn_decode_path_workspace": (c_int, [POINTER(TQCache), POINTER(TQCache), c_int64, c_int32, c_int,
                                              POINTER(c_size_t)]),
    "tq_attn_decode_path": (c_int, [POINTER(TQCache), POINTER(TQCache), c_int64, c_void_p, c_int, c_int32,
                                    c_float, c_float, c_int, c_void_p, c_void_p, c_size_t, c_void_p]),
    "tq_attn_decode_static": (c_int, [POINTER(TQCache), POINTER(TQCache), c_int64, c_void_p, c_int, c_int32,
                                      c_float, c_float, c_void_p, c_void_p]),
    "tq_attn_decode_batch_workspace": (c_int, [POINTER(TQCache), POINTER(TQCache), c_int32, c_int32, c_int64,
                                               c_int32, POINTER(c_size_t)]),
    "tq_attn_decode_batch": (c_int, [POINTER(TQCache), POINTER(TQCache), c_int32, c_int32, c_void_p, c_void_p,
                                     c_int64, c_void_p, c_int, c_int32, c_float, c_float, c_void_p, c_void_p,
                                     c_size_t, c_void_p]),
    "tq_attn_prefill_workspace": (c_int, [POINTER(TQCache), c_int64, c_int32, c_int64, POINTER(c_size_t)]),
    "tq_attn_prefill": (c_int, [POINTER(TQCache), POINTER(TQCache), c_int64, c_void_p, c_int, c_int64,
                                c_int32, c_int64, c_float, c_void_p, c_void_p, c_size_t, c_void_p]),
    "tq_attn_int8_prompt_workspace": (c_int, [c_int64, c_int32, c_int32, c_int32, c_int64, POINTER(c_size_t)]),
    "tq_attn_int8_prompt": (c_int, [c_void_p, c_int64, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_int32, c_int32, c_void_p, c_int64, c_int64, c_int64, c_float,
                                    c_void_p, c_void_p, c_size_t, c_void_p]),
}

EXPORTED = tuple(_SIGS)


def load_library(path: str | None = None):
    """Load libtq.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise TQError(-4, f"libtq.so not built at {p} (run __graft_entry__.build())")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def status_str(status: int) -> str:
    try:
        return load_library().tq_status_str(status).decode()
    except Exception:
        return "status"


def _check(status: int, what: str):
    if status != 0:
        raise TQError(status, what)


def tq_version() -> str:
    return load_library().tq_version().decode()


def tq_cache_plane_bytes(type_: int, head_dim: int, n_kv_heads: int, n_cells: int):
    cb, nb = c_size_t(), c_size_t()
    _check(load_library().tq_cache_plane_bytes(type_, head_dim, n_kv_heads, n_cells,
                                               ctypes.byref(cb), ctypes.byref(nb)),
           "tq_cache_plane_bytes")
    return cb.value, nb.value


def tq_codebook(type_: int):
    n = 1 << type_
    vals = (c_float * n)()
    thr = (c_float * max(1, n // 2 - 1))()
    words = (c_uint64 * 2)()
    _check(load_library().tq_codebook(type_, vals, thr, words), "tq_codebook")
    return list(vals), list(thr)[: n // 2 - 1], [words[0], words[1]]


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev_tensor(t: torch.Tensor, dtype, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


class TQCacheTensors:
    """A compressed cache: two torch planes plus the C struct that points at them."""

    def __init__(self, type_: int, head_dim: int, n_kv_heads: int, n_cells: int,
                 device="cuda", codes: torch.Tensor | None = None,
                 norms: torch.Tensor | None = None):
        if isinstance(type_, str):
            type_ = TYPE_BY_NAME[type_]
        g = head_dim // 128
        self.type, self.head_dim, self.n_kv_heads, self.n_cells = type_, head_dim, n_kv_heads, n_cells
        # turbo: [head][cell][group][16 b] code bytes and a norm per group; the
        # 8-bit block format: [head][cell][block][32] int8 bytes and a scale per block
        code_shape = (n_kv_heads, n_cells, head_dim // 32, 32) if type_ == TQ_Q8 else \
            (n_kv_heads, n_cells, g, 16 * type_)
        norm_shape = (n_kv_heads, n_cells, head_dim // 32) if type_ == TQ_Q8 else (n_kv_heads, n_cells, g)
        if codes is None:
            codes = torch.zeros(code_shape, dtype=torch.uint8, device=device)
        if norms is None:
            norms = torch.zeros(norm_shape, dtype=torch.float16, device=device)
        self.codes = _dev_tensor(codes, torch.uint8, "codes")
        self.norms = _dev_tensor(norms, torch.float16, "norms")
        self.struct = TQCache(type_, head_dim, n_kv_heads, 0, n_cells,
                              self.codes.data_ptr(), self.norms.data_ptr())


def new_cache(type_, head_dim: int, n_kv_heads: int, n_cells: int, device="cuda") -> TQCacheTensors:
    return TQCacheTensors(type_, head_dim, n_kv_heads, n_cells, device)


def tq_set_rows(cache: TQCacheTensors, src: torch.Tensor, cell_idx: torch.Tensor, stream=None):
    _dev_tensor(src, torch.float32, "src")
    _dev_tensor(cell_idx, torch.int64, "cell_idx")
    if src.dim() != 3 or src.shape[1] != cache.n_kv_heads or src.shape[2] != cache.head_dim:
        raise ValueError("src must be [n_rows, n_kv_heads, head_dim]")
    if cell_idx.shape != (src.shape[0],):
        raise ValueError("cell_idx must be [n_rows]")
    _check(load_library().tq_set_rows(ctypes.byref(cache.struct), src.data_ptr(), cell_idx.data_ptr(),
                                      src.shape[0], _stream(stream)), "tq_set_rows")


def _q_dtype(q: torch.Tensor) -> int:
    if q.dtype == torch.float32:
        return TQ_F32
    if q.dtype == torch.bfloat16:
        return TQ_BF16
    raise TypeError("q must be float32 or bfloat16")


def _workspace(nbytes: int, device, workspace):
    if workspace is None:
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    _dev_tensor(workspace, torch.uint8, "workspace")
    return workspace


def tq_attn_decode_workspace(k: TQCacheTensors, v: TQCacheTensors, kv_len: int, n_q_heads: int) -> int:
    b = c_size_t()
    _check(load_library().tq_attn_decode_workspace(ctypes.byref(k.struct), ctypes.byref(v.struct), kv_len,
                                                   n_q_heads, ctypes.byref(b)), "tq_attn_decode_workspace")
    return b.value


def tq_attn_decode(k: TQCacheTensors, v: TQCacheTensors, kv_len: int, q: torch.Tensor, scale: float,
                   out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                   sparse_v_tau: float = 0.0, stream=None) -> torch.Tensor:
    qd = _q_dtype(q)
    _dev_tensor(q, q.dtype, "q")
    if q.dim() != 2 or q.shape[1] != k.head_dim:
        raise ValueError("q must be [n_q_heads, k.head_dim]")
    n_q = q.shape[0]
    if out is None:
        out = torch.empty((n_q, v.head_dim), dtype=torch.float32, device=q.device)
    _dev_tensor(out, torch.float32, "out")
    if tuple(out.shape) != (n_q, v.head_dim):
        raise ValueError("out must be [n_q_heads, v.head_dim]")
    ws = _workspace(tq_attn_decode_workspace(k, v, kv_len, n_q), q.device, workspace)
    _check(load_library().tq_attn_decode(ctypes.byref(k.struct), ctypes.byref(v.struct), kv_len,
                                         q.data_ptr(), qd, n_q, scale, sparse_v_tau, out.data_ptr(),
                                         ws.data_ptr(), ws.numel(), _stream(stream)), "tq_attn_decode")
    return out


def tq_attn_decode_path_workspace(k: TQCacheTensors, v: TQCacheTensors, kv_len: int, n_q_heads: int,
                                  path: int) -> int:
    b = c_size_t()
    _check(load_library().tq_attn_decode_path_workspace(ctypes.byref(k.struct), ctypes.byref(v.struct), kv_len,
                                                        n_q_heads, path, ctypes.byref(b)),
           "tq_attn_decode_path_workspace")
    return b.value


def tq_attn_decode_path(k: TQCacheTensors, v: TQCacheTensors, kv_len: int, q: torch.Tensor, scale: float,
                        path: int, out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                        sparse_v_tau: float = 0.0, stream=None) -> torch.Tensor:
    """tq_attn_decode through the kernel `path` names (TQ_DECODE_AUTO,
    TQ_DECODE_MATRIX or TQ_DECODE_TABLE)."""
    qd = _q_dtype(q)
    _dev_tensor(q, q.dtype, "q")
    if q.dim() != 2 or q.shape[1] != k.head_dim:
        raise ValueError("q must be [n_q_heads, k.head_dim]")
    n_q = q.shape[0]
    if out is None:
        out = torch.empty((n_q, v.head_dim), dtype=torch.float32, device=q.device)
    _dev_tensor(out, torch.float32, "out")
    if tuple(out.shape) != (n_q, v.head_dim):
        raise ValueError("out must be [n_q_heads, v.head_dim]")
    ws = _workspace(tq_attn_decode_path_workspace(k, v, kv_len, n_q, path), q.device, workspace)
    _check(load_library().tq_attn_decode_path(ctypes.byref(k.struct), ctypes.byref(v.struct), kv_len,
                                              q.data_ptr(), qd, n_q, scale, sparse_v_tau, path, out.data_ptr(),
                                              ws.data_ptr(), ws.numel(), _stream(stream)), "tq_attn_decode_path")
    return out


def tq_attn_decode_static(k: TQCacheTensors, v: TQCacheTensors, kv_len: int, q: torch.Tensor, scale: float,
                          out: torch.Tensor | None = None, sparse_v_tau: float = 0.0, stream=None) -> torch.Tensor:
    """tq_attn_decode with the split partials in the library's own device
    array (no workspace argument; nothing is allocated but `out` when it is
    not given)."""
    qd = _q_dtype(q)
    _dev_tensor(q, q.dtype, "q")
    if q.dim() != 2 or q.shape[1] != k.head_dim:
        raise ValueError("q must be [n_q_heads, k.head_dim]")
    n_q = q.shape[0]
    if out is None:
        out = torch.empty((n_q, v.head_dim), dtype=torch.float32, device=q.device)
    _dev_tensor(out, torch.float32, "out")
    if tuple(out.shape) != (n_q, v.head_dim):
        raise ValueError("out must be [n_q_heads, v.head_dim]")
    _check(load_library().tq_attn_decode_static(ctypes.byref(k.struct), ctypes.byref(v.struct), kv_len,
                                                q.data_ptr(), qd, n_q, scale, sparse_v_tau, out.data_ptr(),
                                                _stream(stream)), "tq_attn_decode_static")
    return out


def tq_attn_decode_batch_workspace(k: TQCacheTensors, v: TQCacheTensors, n_seq: int, n_rows: int,
                                   max_kv_len: int, n_q_heads: int) -> int:
    b = c_size_t()
    _check(load_library().tq_attn_decode_batch_workspace(ctypes.byref(k.struct), ctypes.byref(v.struct), n_seq,
                                                         n_rows, max_kv_len, n_q_heads, ctypes.byref(b)),
           "tq_attn_decode_batch_workspace")
    return b.value


def tq_attn_decode_batch(k: TQCacheTensors, v: TQCacheTensors, seq_start: torch.Tensor, seq_len: torch.Tensor,
                         max_kv_len: int, q: torch.Tensor, scale: float, out: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None, sparse_v_tau: float = 0.0,
                         stream=None) -> torch.Tensor:
    """q [n_seq, n_rows, n_q_heads, k.head_dim]; seq_start int64 / seq_len int32
    device tensors [n_seq] -> out [n_seq, n_rows, n_q_heads, v.head_dim]."""
    qd = _q_dtype(q)
    _dev_tensor(q, q.dtype, "q")
    _dev_tensor(seq_start, torch.int64, "seq_start")
    _dev_tensor(seq_len, torch.int32, "seq_len")
    if q.dim() != 4 or q.shape[3] != k.head_dim:
        raise ValueError("q must be [n_seq, n_rows, n_q_heads, k.head_dim]")
    n_seq, n_rows, n_q = q.shape[:3]
    if seq_start.shape != (n_seq,) or seq_len.shape != (n_seq,):
        raise ValueError("seq_start and seq_len must be [n_seq]")
    if out is None:
        out = torch.empty((n_seq, n_rows, n_q, v.head_dim), dtype=torch.float32, device=q.device)
    _dev_tensor(out, torch.float32, "out")
    if tuple(out.shape) != (n_seq, n_rows, n_q, v.head_dim):
        raise ValueError("out must be [n_seq, n_rows, n_q_heads, v.head_dim]")
    ws = _workspace(tq_attn_decode_batch_workspace(k, v, n_seq, n_rows, max_kv_len, n_q), q.device, workspace)
    _check(load_library().tq_attn_decode_batch(ctypes.byref(k.struct), ctypes.byref(v.struct), n_seq, n_rows,
                                               seq_start.data_ptr(), seq_len.data_ptr(), max_kv_len,
                                               q.data_ptr(), qd, n_q, scale, sparse_v_tau, out.data_ptr(),
                                               ws.data_ptr(), ws.numel(), _stream(stream)),
           "tq_attn_decode_batch")
    return out


def tq_attn_prefill_workspace(k: TQCacheTensors, n_rows: int, n_q_heads: int, kv_len: int) -> int:
    b = c_size_t()
    _check(load_library().tq_attn_prefill_workspace(ctypes.byref(k.struct), n_rows, n_q_heads, kv_len,
                                                    ctypes.byref(b)), "tq_attn_prefill_workspace")
    return b.value


def tq_attn_prefill(k: TQCacheTensors, v: TQCacheTensors, kv_len: int, q: torch.Tensor, q_pos0: int,
                    scale: float, out: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    qd = _q_dtype(q)
    _dev_tensor(q, q.dtype, "q")
    if q.dim() != 3 or q.shape[2] != k.head_dim:
        raise ValueError("q must be [n_rows, n_q_heads, head_dim]")
    n_rows, n_q = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty((n_rows, n_q, k.head_dim), dtype=torch.float32, device=q.device)
    _dev_tensor(out, torch.float32, "out")
    ws = _workspace(tq_attn_prefill_workspace(k, n_rows, n_q, kv_len), q.device, workspace)
    _check(load_library().tq_attn_prefill(ctypes.byref(k.struct), ctypes.byref(v.struct), kv_len,
                                          q.data_ptr(), qd, n_rows, n_q, q_pos0, scale, out.data_ptr(),
                                          ws.data_ptr(), ws.numel(), _stream(stream)),
           "tq_attn_prefill")
    return out


def tq_attn_int8_prompt_workspace(n_q: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                                  ctx_len: int) -> int:
    b = c_size_t()
    _check(load_library().tq_attn_int8_prompt_workspace(n_q, n_q_heads, n_kv_heads, head_dim, ctx_len,
                                                        ctypes.byref(b)),
           "tq_attn_int8_prompt_workspace")
    return b.value


def tq_attn_int8_prompt(q: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, k_scale: torch.Tensor,
                        v_scale: torch.Tensor, page_table: torch.Tensor, ctx_len: int, q_pos0: int,
                        scale: float, out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    _dev_tensor(q, torch.float32, "q")
    _dev_tensor(k8, torch.int8, "k")
    _dev_tensor(v8, torch.int8, "v")
    _dev_tensor(k_scale, torch.float16, "k_scale")
    _dev_tensor(v_scale, torch.float16, "v_scale")
    _dev_tensor(page_table, torch.int32, "page_table")
    n_q, n_q_heads, d = q.shape
    n_phys, n_kv, d2 = k8.shape
    if d2 != d or v8.shape != k8.shape or k_scale.shape != (n_phys, n_kv) or v_scale.shape != (n_phys, n_kv):
        raise ValueError("int8 cache shape mismatch")
    if n_phys % 32:
        raise ValueError("the int8 cache must hold whole 32-cell pages")
    if page_table.numel() * 32 < ctx_len:
        raise ValueError("page_table too short for ctx_len")
    if out is None:
        out = torch.empty((n_q, n_q_heads, d), dtype=torch.float32, device=q.device)
    _dev_tensor(out, torch.float32, "out")
    ws = _workspace(tq_attn_int8_prompt_workspace(n_q, n_q_heads, n_kv, d, ctx_len), q.device, workspace)
    _check(load_library().tq_attn_int8_prompt(q.data_ptr(), n_q, n_q_heads, k8.data_ptr(), v8.data_ptr(),
                                              k_scale.data_ptr(), v_scale.data_ptr(), n_kv, d,
                                              page_table.data_ptr(), n_phys // 32, ctx_len, q_pos0, scale,
                                              out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream)),
           "tq_attn_int8_prompt")
    return out
