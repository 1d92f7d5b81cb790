"""Seeded synthetic inputs for the five workloads (numpy only).

These generators stand in for the whole-model runs the pages measure (no
weights or datasets are used).  They hold none of the method's arithmetic:
they only draw random tensors with the shapes and value distributions of the
workloads, round them to the dtypes the entry points take, and lay out the
int8 prompt cache.  Both the GPU tests and the CPU oracle tests draw from
here; nothing here calls either side.

Recipe: ``numpy.random.default_rng(seed)`` (PCG64), draws in the order they
are listed, ``standard_normal`` in float64 rounded to float32; bf16 values
are float32 values rounded to bfloat16 (round-to-nearest-even) and kept as
float32 arrays that are exactly representable in bfloat16.
"""

from __future__ import annotations

import numpy as np


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even); returns float32."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32)


def normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float64).astype(np.float32)


def small_decode(seed: int = 0, kv_len: int = 256, n_q: int = 1, n_kv: int = 1, d: int = 128,
                 dv: int | None = None):
    """turbo quantize+decode smoke shape: Q [n_q, d], K [kv_len, n_kv, d] and
    V [kv_len, n_kv, dv] (dv = d unless given), iid N(0,1)."""
    dv = d if dv is None else dv
    rng = np.random.default_rng(seed)
    q = normal(rng, (n_q, d))
    k = normal(rng, (kv_len, n_kv, d))
    v = normal(rng, (kv_len, n_kv, dv))
    return q, k, v


def outlier_decode(seed: int = 0, kv_len: int = 32768, n_q: int = 32, n_kv: int = 4, d: int = 128,
                   dv: int | None = None):
    """GQA decode with outlier channels.

    sigma_K = exp(N(0,1)) per (kv head, channel) [n_kv, d], sigma_V likewise
    [n_kv, dv]; K = N(0,1) * sigma_K [kv_len, n_kv, d], V = N(0,1) * sigma_V
    [kv_len, n_kv, dv] (dv = d unless given); Q = bf16(N(0,1)) [n_q, d].
    """
    dv = d if dv is None else dv
    rng = np.random.default_rng(seed)
    sk = np.exp(rng.standard_normal((n_kv, d))).astype(np.float32)
    sv = np.exp(rng.standard_normal((n_kv, dv))).astype(np.float32)
    k = (normal(rng, (kv_len, n_kv, d)) * sk[None]).astype(np.float32)
    v = (normal(rng, (kv_len, n_kv, dv)) * sv[None]).astype(np.float32)
    q = bf16_round(normal(rng, (n_q, d)))
    return q, k, v


def prefill(seed: int = 0, rows: int = 512, kv_len: int | None = None, n_q: int = 16,
            n_kv: int = 8, d: int = 256):
    """Causal prefill: K, V = N(0,1) [kv_len, n_kv, d]; Q = bf16(N(0,1)) [rows, n_q, d]."""
    kv_len = rows if kv_len is None else kv_len
    rng = np.random.default_rng(seed)
    k = normal(rng, (kv_len, n_kv, d))
    v = normal(rng, (kv_len, n_kv, d))
    q = bf16_round(normal(rng, (rows, n_q, d)))
    return q, k, v


def _int8_rows(rows: np.ndarray):
    """Symmetric per-row int8 with a float16 scale: scale = fp16(max|row|/127)."""
    amax = np.abs(rows).max(axis=-1)
    scale16 = (amax / np.float32(127)).astype(np.float32).astype(np.float16)
    s32 = scale16.astype(np.float32)
    safe = np.where(s32 > 0, s32, np.float32(1))
    q = np.clip(np.rint(rows / safe[..., None]), -127, 127).astype(np.int8)
    return q, scale16


def int8_prompt(seed: int = 0, ctx: int = 40000, n_q: int = 2048, n_q_heads: int = 8,
                n_kv: int = 1, d: int = 128, page: int = 32, identity_pages: bool = False,
                k_mult: float = 1.0, v_mult: float = 1.0):
    """Paged int8 prompt-attention inputs.

    K_f, V_f = N(0,1) [ctx, n_kv, d] in logical order -> int8 with per-row
    float16 scales; page table = rng.permutation(n_chunks) (logical chunk i is
    stored at physical chunk pt[i]); Q = N(0,1) [n_q, n_q_heads, d] float32.
    Returns q, k8, v8, k_scale, v_scale (physical order), page_table, logical
    copies (k8_log, v8_log, ks_log, vs_log) for reference.  k_mult / v_mult
    scale K_f / V_f before the int8 conversion (large-magnitude cases).
    """
    assert ctx % page == 0
    rng = np.random.default_rng(seed)
    kf = normal(rng, (ctx, n_kv, d))
    vf = normal(rng, (ctx, n_kv, d))
    kf = (kf * np.float32(k_mult)).astype(np.float32)
    vf = (vf * np.float32(v_mult)).astype(np.float32)
    n_chunks = ctx // page
    pt = rng.permutation(n_chunks).astype(np.int32)
    if identity_pages:
        pt = np.arange(n_chunks, dtype=np.int32)
    q = normal(rng, (n_q, n_q_heads, d))
    k8l, ksl = _int8_rows(kf)
    v8l, vsl = _int8_rows(vf)
    phys = (pt[np.arange(ctx) // page].astype(np.int64) * page + np.arange(ctx) % page)
    k8 = np.empty_like(k8l); v8 = np.empty_like(v8l)
    ks = np.empty_like(ksl); vs = np.empty_like(vsl)
    k8[phys] = k8l; v8[phys] = v8l; ks[phys] = ksl; vs[phys] = vsl
    return {"q": q, "k8": k8, "v8": v8, "k_scale": ks, "v_scale": vs, "page_table": pt,
            "k8_logical": k8l, "v8_logical": v8l, "ks_logical": ksl, "vs_logical": vsl}
