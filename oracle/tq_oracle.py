"""Plain, slow CPU oracle for attention over a TurboQuant-compressed KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring): the GPU library never
imports or calls this file, and this file imports nothing from it.

Sources, cited by page title and section throughout:

* [PR36] the llama-cpp-turboquant pull request 36 page: four commit messages,
  (a) the SET_ROWS butterfly moved to warp shuffles, (b) the asymmetric-K
  head-dim fix, (c) the decode Q x centroid lookup table, (d) the four VEC
  flash-attention optimisations and their results table.
* [PR28] "HIP/turbo3: graph-safe decode + inline-dequant TILE prefill on
  gfx1201 (RDNA4)": sections "Graph-safe decode", "Inline-dequant TILE
  prefill", the prefill table, "Correctness", "Scope / honesty".
* [QSA1821] "#1821 qsa_prompt_attn: int8 K/V prefetched in registers and
  sharing one buffer (Turing / sm_75)": sections What, Why, Change,
  Measured, How to check.

The pages describe kernels, not formulas.  Every point they leave open is
settled by a stated reading (marked "Reading:"), chosen once and used by the
GPU library as well:

* quantizer arithmetic is IEEE float32 with round-to-nearest-even and no
  fused multiply-add, because the packed codes must agree bit for bit and the
  GPU kernel decides them in float32;
* attention truth is float64 over the dequantized cache.

Parity pins (tests that tie each function to something other than itself)
live in ``tests/test_oracle_*.py``; every function below has at least one.
"""

from __future__ import annotations

import numpy as np
from scipy.special import ndtr

GROUP = 128                      # elements per quantization group
LOG2_GROUP = 7
TYPE_BITS = {"turbo2": 2, "turbo3": 3, "turbo4": 4}
INT8_PAGE = 32                   # cells per page of the int8 cache


# --------------------------------------------------------------------------
# O0. Constants
# --------------------------------------------------------------------------

def lloyd_max_normal(n_levels: int, tol: float = 1e-13, max_iter: int = 100000) -> np.ndarray:
    """Lloyd-Max reconstruction levels for a unit normal source, float64, ascending.

    Reading: the pages never print a codebook; [PR36] (c) only says turbo4
    has 16 centroids (and turbo2/3 fewer).  The codebook is the
    minimum-mean-square-error quantizer of N(0,1) with 2^b levels, found by
    Lloyd's alternation: cell edges at the midpoints of neighbouring levels,
    each level at the conditional mean of its cell, which for a normal source
    on (a, b) is (phi(a) - phi(b)) / (Phi(b) - Phi(a)).
    """
    c = np.linspace(-2.5, 2.5, n_levels)
    for _ in range(max_iter):
        edges = np.concatenate(([-np.inf], 0.5 * (c[1:] + c[:-1]), [np.inf]))
        a, b = edges[:-1], edges[1:]
        pdf_a = np.exp(-0.5 * a * a) / np.sqrt(2.0 * np.pi)   # 0 at -inf
        pdf_b = np.exp(-0.5 * b * b) / np.sqrt(2.0 * np.pi)   # 0 at +inf
        new = (pdf_a - pdf_b) / (ndtr(b) - ndtr(a))
        step = np.max(np.abs(new - c))
        c = new
        if step < tol:
            break
    # exact odd symmetry: average the two halves
    half = 0.5 * (c[n_levels // 2:] - c[:n_levels // 2][::-1])
    return np.concatenate((-half[::-1], half))


def code_magnitudes(bits: int) -> np.ndarray:
    """Positive reconstruction magnitudes of a b-bit code, ascending, float32.

    Reading: the levels of ``lloyd_max_normal(2**bits)`` (the Lloyd-Max
    quantizer of a unit normal source), rounded once to float32, the precision
    of the quantizer's own arithmetic.  They are not rounded to any narrower
    type: how a GPU kernel represents a level in its matrix products is that
    kernel's approximation, checked against these values.
    """
    lv = lloyd_max_normal(2 ** bits)
    return lv[2 ** (bits - 1):].astype(np.float32)


def code_values(bits: int) -> np.ndarray:
    """Reconstruction value of every b-bit code, float32, indexed by the code.

    Reading of "qs + sign bits" ([PR36] (c): per 8 elements, qs bytes plus a
    signs byte): a code carries a (b-1)-bit magnitude index ``qs`` in its low
    bits and a sign bit on top (set = negative), so
    value(code) = (-1 if code >> (b-1) else +1) * magnitudes[code & (2^(b-1)-1)].
    """
    mags = code_magnitudes(bits)
    half = 2 ** (bits - 1)
    codes = np.arange(2 ** bits)
    v = mags[codes & (half - 1)]
    return np.where(codes >= half, -v, v).astype(np.float32)


def mag_thresholds(bits: int) -> np.ndarray:
    """Decision thresholds between neighbouring magnitudes, float32.

    Reading: a level's cell ends halfway to its neighbour (the Lloyd-Max
    condition that makes the rule "nearest level"); each threshold is the
    midpoint of the two float64 levels, rounded once to float32.
    """
    lv = lloyd_max_normal(2 ** bits)[2 ** (bits - 1):]
    return (0.5 * (lv[1:] + lv[:-1])).astype(np.float32)


def splitmix64(seed: int, n: int) -> list:
    """First n outputs of the SplitMix64 generator (Steele, Lea, Flood 2014).

    Written from the published definition: the state advances by the golden
    gamma 0x9E3779B97F4A7C15; the output is the state passed through two
    xor-shift-multiply rounds (shifts 30 and 27, multipliers 0xBF58476D1CE4E5B9
    and 0x94D049BB133111EB) and a final xor-shift by 31.
    """
    mask = (1 << 64) - 1
    state = seed & mask
    out = []
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) & mask
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & mask
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & mask
        out.append(z ^ (z >> 31))
    return out


def sign_flips() -> np.ndarray:
    """The fixed random sign vector s (bool[128], True = negate).

    Reading: the pages never show the random sign flip that precedes the
    transform.  It is one fixed vector for every group of K, V and Q:
    element d is negated iff bit (d mod 64) of word floor(d/64) is set, the
    two words being the first two SplitMix64 outputs from state 0.
    """
    w = splitmix64(0, 2)
    return np.array([(w[d // 64] >> (d % 64)) & 1 == 1 for d in range(GROUP)])


# --------------------------------------------------------------------------
# O1. Quantize one group (bit-exact contract, float32)
# --------------------------------------------------------------------------

def wht_butterfly(u: np.ndarray) -> np.ndarray:
    """Unnormalized 128-point Walsh-Hadamard transform along the last axis.

    [PR36] (a): seven butterfly stages h = 1, 2, 4, ..., 64; at each stage
    element j pairs with element j xor h, the lower index of the pair becomes
    the sum and the upper one the lower value minus the upper value.  Stages
    run in that ascending order (it fixes the float32 rounding).  The dtype of
    the input is kept, so float32 input gives the float32 butterfly.
    """
    u = np.array(u, copy=True)
    n = u.shape[-1]
    assert n == GROUP
    lead = u.shape[:-1]
    h = 1
    while h < n:
        v = u.reshape(lead + (n // (2 * h), 2, h))
        lo = v[..., 0, :].copy()
        hi = v[..., 1, :].copy()
        v[..., 0, :] = lo + hi
        v[..., 1, :] = lo - hi
        u = v.reshape(lead + (n,))
        h *= 2
    return u


def sum_squares_tree(x: np.ndarray) -> np.ndarray:
    """Sum of squares of a float32 group, in the butterfly's pairing order.

    Reading: the norm's sum uses the same xor pattern as the transform
    ([PR36] (a)): seven rounds h = 1..64 in which each partial adds the
    partial at index xor h.  That equals summing neighbouring pairs level by
    level, which is what this computes; every add is one float32 rounding.
    """
    v = (x.astype(np.float32) * x.astype(np.float32)).astype(np.float32)
    for _ in range(LOG2_GROUP):
        v = (v[..., 0::2] + v[..., 1::2]).astype(np.float32)
    return v[..., 0]


def quantize_groups(x: np.ndarray, bits: int):
    """Quantize float32 groups [..., 128] to b-bit codes and float16 norms.

    [PR36] (a) and (c) give the kernel's parts (sign flip and butterfly,
    qs + sign bits); the readings fill the rest.  Per group, all float32:

    1. n2 = sum_squares_tree(x); norm = sqrt(n2) (correctly rounded);
       the stored norm is float16(norm), round-to-nearest-even.
    2. inv = 1/norm if norm > 0 else 0 (a zero or NaN norm gives inv = 0).
    3. u = s (.) x (sign flip), then the butterfly of ``wht_butterfly``.
    4. y = u * inv.  y is the orthonormal transform of x scaled to unit
       variance: H/sqrt(128) applied to s (.) x, times sqrt(128)/||x||; the two
       sqrt(128) cancel, so no 1/sqrt(128) multiply appears.
    5. sign bit = (y < 0); qs = number of thresholds t_k with |y| > t_k.
       This is the nearest stored level; a tie goes to the smaller
       magnitude and y = 0 (or NaN) codes as +magnitudes[0].
    """
    x = np.asarray(x, dtype=np.float32)
    assert x.shape[-1] == GROUP
    n2 = sum_squares_tree(x)
    norm = np.sqrt(n2).astype(np.float32)
    with np.errstate(over="ignore"):
        norm16 = norm.astype(np.float16)
    pos = norm > np.float32(0)
    safe = np.where(pos, norm, np.float32(1))
    inv = np.where(pos, (np.float32(1) / safe).astype(np.float32), np.float32(0)).astype(np.float32)
    s = sign_flips()
    u = np.where(s, -x, x).astype(np.float32)
    u = wht_butterfly(u)
    with np.errstate(invalid="ignore"):
        y = (u * inv[..., None]).astype(np.float32)
        neg = y < np.float32(0)
        a = np.abs(y)
        qs = np.zeros(y.shape, dtype=np.uint8)
        for t in mag_thresholds(bits):
            qs += (a > t).astype(np.uint8)
    code = qs | (neg.astype(np.uint8) << (bits - 1))
    return code.astype(np.uint8), norm16


def group_bytes(bits: int) -> int:
    """Packed code bytes per 128-element group: 128*b bits."""
    return GROUP * bits // 8


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack codes [..., 128] into [..., 16*b] bytes.

    Reading of the block layout ([PR36] (c) says only that 8 elements take
    2 qs bytes and 1 signs byte for turbo3): the group is one little-endian
    bit stream, element e's b-bit code at stream bits b*e .. b*e+b-1, the
    least significant code bit first; stream bit k is bit (k mod 8) of byte
    k div 8.  That is 3 bytes per 8 elements for turbo3 as on the page, and
    34 bytes per group with the norm for turbo2, the 7.5x of [PR36] (d).
    """
    codes = np.asarray(codes, dtype=np.uint8)
    lead = codes.shape[:-1]
    bitplanes = ((codes[..., :, None] >> np.arange(bits, dtype=np.uint8)) & 1).astype(np.uint8)
    stream = bitplanes.reshape(lead + (GROUP * bits,))
    return np.packbits(stream, axis=-1, bitorder="little")


def unpack_codes(packed: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of ``pack_codes``."""
    packed = np.asarray(packed, dtype=np.uint8)
    lead = packed.shape[:-1]
    stream = np.unpackbits(packed, axis=-1, bitorder="little")
    b = stream.reshape(lead + (GROUP, bits)).astype(np.uint8)
    return (b << np.arange(bits, dtype=np.uint8)).sum(axis=-1).astype(np.uint8)


# --------------------------------------------------------------------------
# O2. Dequantize (float64)
# --------------------------------------------------------------------------

def dequant_rotated(codes: np.ndarray, norm16: np.ndarray, bits: int) -> np.ndarray:
    """Rotated-domain values: level(code) * norm16 / sqrt(128), float64.

    Reading: each level is a unit-variance coordinate, so the dequantized
    coordinate of the orthonormal transform is level * ||x|| / sqrt(128).
    """
    vals = code_values(bits).astype(np.float64)[codes]
    return vals * (norm16.astype(np.float64)[..., None] / np.sqrt(GROUP))


def dequant(codes: np.ndarray, norm16: np.ndarray, bits: int) -> np.ndarray:
    """Original-domain group: x_hat = s (.) H w_hat / sqrt(128), float64.

    H is symmetric with H H = 128 I, so this inverts step 3-4 of
    ``quantize_groups`` exactly when every code hits its value.
    """
    w = dequant_rotated(codes, norm16, bits)
    s = sign_flips()
    t = wht_butterfly(w) / np.sqrt(GROUP)
    return np.where(s, -t, t)


# --------------------------------------------------------------------------
# O2b. The 8-bit block format for an asymmetric K cache
# --------------------------------------------------------------------------
#
# [PR36] (b): the fork can keep K in q8_0 (8-bit blocks) beside a turbo V,
# "auto-asymmetric".  The page names the format only; reading: a row is cut
# into blocks of 32 elements, each stored as 32 signed 8-bit codes and one
# float16 scale d = fp16(max|x| / 127); code = clamp(rint(x / d), -127, 127)
# with the division in float32 and ties to even; a block whose scale is 0 or
# not finite stores zero codes.  The element is code * d.  This K is not
# rotated.

Q8_BLOCK = 32
Q8_BITS = 8                      # the "bits" tag of a cache in this format


def quantize_q8(x: np.ndarray):
    """float32 [..., 32] -> (codes int8 [..., 32], scales float16 [...])."""
    x = np.asarray(x, dtype=np.float32)
    assert x.shape[-1] == Q8_BLOCK
    amax = np.abs(x).max(axis=-1)
    d16 = (amax / np.float32(127)).astype(np.float32).astype(np.float16)
    d32 = d16.astype(np.float32)
    ok = np.isfinite(d32) & (d32 > 0)
    safe = np.where(ok, d32, np.float32(1))
    q = np.clip(np.rint(x / safe[..., None]), -127, 127)
    return np.where(ok[..., None], q, 0).astype(np.int8), d16


def dequant_q8(codes: np.ndarray, d16: np.ndarray) -> np.ndarray:
    """codes int8 [..., 32], scales float16 [...] -> float64 [..., 32]."""
    return codes.astype(np.float64) * d16.astype(np.float64)[..., None]


# --------------------------------------------------------------------------
# The compressed cache (two planes per K or V cache)
# --------------------------------------------------------------------------

def new_cache(bits: int, head_dim: int, n_kv_heads: int, n_cells: int) -> dict:
    """Zero-filled cache planes.

    codes : uint8 [n_kv_heads, n_cells, head_dim/128, 16*b]
    norms : float16 [n_kv_heads, n_cells, head_dim/128]
    head_dim must be a multiple of 128 ([PR36] (b) pads a 192-wide head to 256
    rather than quantizing a partial group).
    """
    assert head_dim % GROUP == 0
    g = head_dim // GROUP
    if bits == Q8_BITS:
        # the 8-bit block format: codes int8 [n_kv_heads, n_cells, head_dim/32,
        # 32], scales float16 [n_kv_heads, n_cells, head_dim/32]
        nb = head_dim // Q8_BLOCK
        return {"bits": bits, "head_dim": head_dim,
                "codes": np.zeros((n_kv_heads, n_cells, nb, Q8_BLOCK), np.int8),
                "norms": np.zeros((n_kv_heads, n_cells, nb), np.float16)}
    return {
        "bits": bits,
        "head_dim": head_dim,
        "codes": np.zeros((n_kv_heads, n_cells, g, group_bytes(bits)), np.uint8),
        "norms": np.zeros((n_kv_heads, n_cells, g), np.float16),
    }


def set_rows(cache: dict, src: np.ndarray, cell_idx: np.ndarray) -> None:
    """SET_ROWS ([PR36] (a)): quantize rows src[r] into cells cell_idx[r].

    src is float32 [n_rows, n_kv_heads, head_dim]; every 128-element group
    of every head is quantized independently.  cell_idx values are unique.
    """
    bits = cache["bits"]
    src = np.asarray(src, dtype=np.float32)
    n_rows, n_kv, d = src.shape
    idx = np.asarray(cell_idx, dtype=np.int64)
    if bits == Q8_BITS:
        q, d16 = quantize_q8(src.reshape(n_rows, n_kv, d // Q8_BLOCK, Q8_BLOCK))
        cache["codes"][:, idx] = q.transpose(1, 0, 2, 3)
        cache["norms"][:, idx] = d16.transpose(1, 0, 2)
        return
    g = d // GROUP
    codes, norm16 = quantize_groups(src.reshape(n_rows, n_kv, g, GROUP), bits)
    packed = pack_codes(codes, bits)
    cache["codes"][:, idx] = packed.transpose(1, 0, 2, 3)
    cache["norms"][:, idx] = norm16.transpose(1, 0, 2)


def dequant_cache(cache: dict, kv_len: int) -> np.ndarray:
    """Original-domain float64 rows [n_kv_heads, kv_len, head_dim]."""
    bits = cache["bits"]
    if bits == Q8_BITS:
        x = dequant_q8(cache["codes"][:, :kv_len], cache["norms"][:, :kv_len])
        return x.reshape(x.shape[0], x.shape[1], -1)
    packed = cache["codes"][:, :kv_len]
    codes = unpack_codes(packed, bits)
    x = dequant(codes, cache["norms"][:, :kv_len], bits)
    n_kv, L, g, _ = x.shape
    return x.reshape(n_kv, L, g * GROUP)


# --------------------------------------------------------------------------
# O3. Attention (float64)
# --------------------------------------------------------------------------

def kv_head_of(n_q_heads: int, n_kv_heads: int) -> np.ndarray:
    """Reading of grouped-query attention: q head h uses kv head h // (n_q/n_kv)."""
    assert n_q_heads % n_kv_heads == 0
    return np.arange(n_q_heads) // (n_q_heads // n_kv_heads)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              q_pos0: int, block: int = 512) -> np.ndarray:
    """Causal softmax attention, float64.

    q: [n_rows, n_q_heads, D_K]; k: [n_kv_heads, L, D_K]; v: [n_kv_heads, L,
    D_V].  Query row r sits at absolute position q_pos0 + r and sees keys
    j <= q_pos0 + r (reading: the query block is aligned to the end of the keys
    it was appended after, the prefill/spec-verify case of [PR28]
    "Inline-dequant TILE prefill").
    out[r, h] = sum_j softmax_j(scale * <q[r,h], k[g(h), j]>) v[g(h), j], of
    V's width: the key and value widths may differ ([PR36] (b): 192-wide keys,
    padded to 256, beside 128-wide values).
    """
    q = np.asarray(q, dtype=np.float64)
    n_rows, n_q, d = q.shape
    n_kv, L, _ = k.shape
    assert k.shape[2] == d and v.shape[:2] == k.shape[:2]
    g_of = kv_head_of(n_q, n_kv)
    out = np.zeros((n_rows, n_q, v.shape[2]))
    for h in range(n_q):
        kh = k[g_of[h]]
        vh = v[g_of[h]]
        for r0 in range(0, n_rows, block):
            r1 = min(n_rows, r0 + block)
            s = scale * (q[r0:r1, h] @ kh.T)
            last = q_pos0 + np.arange(r0, r1)
            s = np.where(np.arange(L)[None, :] <= last[:, None], s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            out[r0:r1, h] = (p @ vh) / p.sum(axis=1, keepdims=True)
    return out


def attn_decode(kc: dict, vc: dict, kv_len: int, q: np.ndarray, scale: float) -> np.ndarray:
    """One query row over the whole cache: q [n_q_heads, D_K] -> [n_q_heads, D_V] float64.

    The decode case of [PR36] (c)/(d) and [PR28] "Graph-safe decode".
    """
    k = dequant_cache(kc, kv_len)
    v = dequant_cache(vc, kv_len)
    return attention(np.asarray(q)[None], k, v, scale, kv_len - 1)[0]


def attn_decode_batch(kc: dict, vc: dict, seq_start, seq_len, q: np.ndarray,
                      scale: float) -> np.ndarray:
    """Several sequences and one or two query rows each, in one call: the
    decode case of [PR28] "Graph-safe decode" (query batches of at most two
    rows take the single-row kernel) for a batch of sequences.

    Reading: sequence i owns cells [seq_start[i], seq_start[i] + seq_len[i])
    of every kv head; its n_rows query rows are the last n_rows positions, so
    row r sees its sequence's cells j <= seq_len[i] - n_rows + r (causal, as
    in attention()).  q [n_seq, n_rows, n_q_heads, D_K] -> [n_seq, n_rows,
    n_q_heads, D_V] float64; a row that sees no cell is zero.
    """
    q = np.asarray(q, dtype=np.float64)
    n_seq, n_rows = q.shape[:2]
    out = np.zeros((n_seq, n_rows, q.shape[2], vc["head_dim"]))
    for i in range(n_seq):
        a, n = int(seq_start[i]), int(seq_len[i])
        if n < 1:
            continue
        k = dequant_cache(kc, a + n)[:, a:]
        v = dequant_cache(vc, a + n)[:, a:]
        first = n - n_rows                        # position of row 0
        lo = max(0, -first)                       # rows that see no cell stay zero
        if lo < n_rows:
            out[i, lo:] = attention(q[i, lo:], k, v, scale, first + lo)
    return out


def attn_prefill(kc: dict, vc: dict, kv_len: int, q: np.ndarray, q_pos0: int,
                 scale: float) -> np.ndarray:
    """Multi-row causal attention ([PR28] "Inline-dequant TILE prefill").

    q [n_rows, n_q_heads, D] -> [n_rows, n_q_heads, D] float64.
    """
    k = dequant_cache(kc, kv_len)
    v = dequant_cache(vc, kv_len)
    return attention(q, k, v, scale, q_pos0)


# --------------------------------------------------------------------------
# O4. Sparse-V decode (float64): value skip and its error bound
# --------------------------------------------------------------------------
#
# [PR36] (d), the VEC flash-attention optimisations, item 3: the sparse-V
# threshold is raised to 5e-3 for turbo3/turbo4 and 1e-2 for turbo2.
# Reading (the page does not define the weight it compares): the weight of key
# j is p_j = e^(S_j - m) with m a running reference no larger than the true
# maximum m*; a key whose p_j < tau is left out of the value sum only, and the
# normalizer keeps every key.  A kernel's reference depends on its key order,
# so the GPU result is checked against the bound below rather than one exact
# skipped set.

def decode_scores(kc: dict, kv_len: int, q: np.ndarray, scale: float) -> np.ndarray:
    """Natural-log scores S[h, j] = scale <q_h, k_{g(h), j}> over the dequantized cache."""
    k = dequant_cache(kc, kv_len)
    q = np.asarray(q, dtype=np.float64)
    g_of = kv_head_of(q.shape[0], k.shape[0])
    return scale * np.einsum("hd,hjd->hj", q, k[g_of])


def attn_decode_sparse_v(kc: dict, vc: dict, kv_len: int, q: np.ndarray, scale: float,
                         tau: float, ref_block: int | None = None) -> np.ndarray:
    """Decode with the value skip:
    out_h = sum_{j: e^(S_hj - r_hj) >= tau} w_hj v_j / sum_j w_hj, w_hj = e^(S_hj - m*_h),
    where the reference r_hj is the true maximum m*_h (ref_block None: the
    largest reference, so the largest skipped set) or the maximum over the
    aligned block of ref_block keys holding j (a kernel that scores the keys
    in blocks and takes each block's own maximum)."""
    s = decode_scores(kc, kv_len, q, scale)
    v = dequant_cache(vc, kv_len)
    g_of = kv_head_of(s.shape[0], v.shape[0])
    m = s.max(axis=1, keepdims=True)
    if ref_block is None:
        ref = np.broadcast_to(m, s.shape)
    else:
        ref = np.empty_like(s)
        for j0 in range(0, kv_len, ref_block):
            ref[:, j0:j0 + ref_block] = s[:, j0:j0 + ref_block].max(axis=1, keepdims=True)
    w = np.exp(s - m)
    keep = np.where(np.exp(s - ref) >= tau, w, 0.0)
    return np.einsum("hj,hjd->hd", keep, v[g_of]) / w.sum(axis=1)[:, None]


def sparse_v_bound(kc: dict, vc: dict, kv_len: int, q: np.ndarray, scale: float, tau: float):
    """The error bound of any value skip whose reference is <= m*.

    T_h = {j : e^(S_hj - m*_h) < tau} holds every key such a kernel can skip
    (its weight against a smaller reference is even larger, so it is skipped
    only if its weight against m* is below tau).  Leaving a set S of keys out
    of the value sum changes the output by - sum_{j in S} (p_j / L) v_j, whose
    largest element is at most its 2-norm, at most
    B_h = sum_{j in T_h} (p_j / L_h) ||v_j||_2.
    Returns (B [n_q], |T_h| [n_q])."""
    s = decode_scores(kc, kv_len, q, scale)
    v = dequant_cache(vc, kv_len)
    g_of = kv_head_of(s.shape[0], v.shape[0])
    p = np.exp(s - s.max(axis=1, keepdims=True))
    w = p / p.sum(axis=1, keepdims=True)
    small = p < tau
    vnorm = np.linalg.norm(v, axis=2)[g_of]          # [n_q, kv_len]
    return (w * vnorm * small).sum(axis=1), small.sum(axis=1)


# --------------------------------------------------------------------------
# O5. int8 paged prompt attention (float64)
# --------------------------------------------------------------------------

def int8_logical_rows(page_table: np.ndarray, ctx_len: int) -> np.ndarray:
    """Physical row of each logical cell 0..ctx_len-1.

    [QSA1821] "Why": the kernel walks 32-cell chunks whose K and V rows are
    scattered.  Reading: a page table maps logical chunk i to physical chunk
    page_table[i]; logical cell j lives at physical row
    page_table[j // 32] * 32 + j % 32.
    """
    j = np.arange(ctx_len)
    return np.asarray(page_table, dtype=np.int64)[j // INT8_PAGE] * INT8_PAGE + j % INT8_PAGE


def int8_dequant(rows8: np.ndarray, scale16: np.ndarray) -> np.ndarray:
    """int8 value times its row's float16 scale, float64 (symmetric, no zero point)."""
    return rows8.astype(np.float64) * scale16.astype(np.float64)[..., None]


def attn_int8_prompt(q: np.ndarray, k8: np.ndarray, v8: np.ndarray, k_scale: np.ndarray,
                     v_scale: np.ndarray, page_table: np.ndarray, ctx_len: int,
                     q_pos0: int, scale: float) -> np.ndarray:
    """Prompt attention over a paged int8 K/V cache ([QSA1821] What/Change).

    q: [n_q, n_q_heads, D]; k8, v8: int8 [n_phys_cells, n_kv_heads, D];
    k_scale, v_scale: float16 [n_phys_cells, n_kv_heads]; causal as in
    ``attention`` over the logical order.  The physical placement of the
    chunks does not enter the result ([QSA1821] Change: the same bytes in the
    same places give the same output).
    """
    rows = int8_logical_rows(page_table, ctx_len)
    k = int8_dequant(k8[rows], k_scale[rows]).transpose(1, 0, 2)
    v = int8_dequant(v8[rows], v_scale[rows]).transpose(1, 0, 2)
    return attention(q, k, v, scale, q_pos0)
