"""fp64 CPU oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline may import or run anything in this package; the product library never
does.  It shares no code with the HIP path: no kernels, headers, helpers or
tables.  It is deliberately plain and slow.

What it computes, and where each step comes from:

* Cache layout, block table and slot arithmetic: "AI Infra入门干货总结：大模型是
  如何高效推理的" (github QianJinGuo/wiki), section "Paged Attention": one layer
  is ``[2, num_blocks, block_size, num_kv_heads, head_dim]`` with K at index 0
  and V at index 1 of the second dimension; ``block_table[r]`` lists request
  ``r``'s physical blocks; a slot ``s`` names block ``s // block_size`` and
  offset ``s % block_size`` inside it.
* Q is ``[query_lens, num_heads, head_dim]``; K/V are read per request as
  ``[seq_lens, num_kv_heads, head_dim]``; a group of query heads shares one KV
  head by index (same page, section "LLM 推理全流程", 3. Transformer Block,
  "Attention (FlashAttention)").
* ``num_computed_tokens`` counts tokens already in the cache (same page,
  section "连续批处理"), so the step's query ``i`` sits at absolute position
  ``num_computed_tokens + i`` and, being causal, sees keys ``0 .. that position``
  (chunked prefill is a prompt split into pieces run step by step:
  lpnh.cn/news/2436702, section 2.3).
* The attention itself is the plain definition printed as the naive
  ``scaled_dot_product_attention`` in lpnh.cn/news/2669538, section 2.1:
  ``softmax(q kᵀ · scale + mask) v`` (the page's extraction lost the ``=``
  signs; the reading is the textbook one).  Tiling, online softmax and
  split-KV are ways to reach this same value, so the oracle computes the value
  directly, in float64.

Every function here is pinned by tests (``tests/test_oracle.py``) to facts that
do not come from the oracle itself: a scalar brute force over independently
drawn contiguous K/V, PyTorch's fp64 CPU SDPA, closed forms, and hand-worked
fixtures under ``tests/golden/``.
"""
from __future__ import annotations

from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

BLOCK_SIZE = 16


# ---------------------------------------------------------------------------
# Storage formats.

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64, exactly.

    A bf16 number is the top 16 bits of an IEEE float32, so shifting the
    pattern left by 16 gives the float32 with the same value."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f64":   # values already decoded (e.g. a dequantised cache)
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# INT8 KV cache: online quantisation of each new token as it is written
# (lpnh.cn/news/2436702, section 4.2: the KV cache is produced at run time, so
# it is quantised and dequantised online; FP16 -> INT8 halves its size).
# Readings (the page gives no scheme): symmetric, one float32 scale per
# (token, kv head) row of head_dim values, scale = max|x| / 127 (float32
# division), code = round-half-even(x / scale) in float32, clamped to
# [-127, 127]; an all-zero row has scale 0 and codes 0.  A value is read back
# as code * scale.  Both divisions are float32 so that the codes, integers
# decided by floating point, are taken in one stated precision.

def quantize_int8(x: np.ndarray, dtype: str) -> Tuple[np.ndarray, np.ndarray]:
    """``x [..., D]`` storage values -> (int8 codes ``[..., D]``, float32 scales ``[...]``)."""
    xf = to_f64(x, dtype).astype(np.float32)          # exact: bf16 and f32 values are float32
    amax = np.abs(xf).max(axis=-1)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = np.rint((xf / safe[..., None]).astype(np.float32))
    codes = np.clip(q, -127, 127).astype(np.int8)
    codes[scale == 0] = 0
    return codes, scale


def dequantize_int8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    return codes.astype(np.float64) * scales.astype(np.float64)[..., None]


def kv_write_int8(codes: np.ndarray, scales: np.ndarray, k: np.ndarray, v: np.ndarray,
                  slot_mapping: np.ndarray, dtype: str) -> Tuple[np.ndarray, np.ndarray]:
    """INT8 cache write: ``codes [2, NB, 16, Hkv, D]`` int8 and ``scales
    [2, NB, 16, Hkv]`` float32 get token ``t``'s quantised K and V at
    ``slot_mapping[t]`` (-1 = skip), as ``kv_write`` places bf16 / fp32 rows."""
    kc, ks = quantize_int8(k, dtype)
    vc, vs = quantize_int8(v, dtype)
    codes = kv_write(codes, kc, vc, slot_mapping)
    scales = kv_write(scales[..., None], ks[..., None], vs[..., None], slot_mapping)[..., 0]
    return codes, scales


# FP8 KV cache: the same online quantisation per (token, K or V, kv head) row
# as INT8 (lpnh.cn/news/2436702, section 4.2, "KV Cache 量化"), with codes in
# the OCP 8-bit floating-point format E4M3 (1 sign, 4 exponent bits with bias
# 7, 3 mantissa bits; exponent field 0 holds the subnormals m/8 * 2^-6; no
# infinities; S.1111.111 is NaN, so the largest finite magnitude is
# 1.75 * 2^8 = 448).  Reading: scale = max|x| / 448 and code = the E4M3 value
# nearest to x / scale (float32 quotient, magnitude clipped at 448), ties to
# the even code; an all-zero row has scale 0 and codes 0.

def fp8_e4m3_magnitudes() -> np.ndarray:
    """Values of the finite non-negative codes 0x00 .. 0x7e, in code order
    (increasing), from the format's definition."""
    out = []
    for code in range(0x7f):
        e, m = code >> 3, code & 7
        out.append(m / 8.0 * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(out, np.float64)


def fp8_e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values (NaN for 0x7f / 0xff)."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    mags = np.append(fp8_e4m3_magnitudes(), np.nan)
    v = mags[c & 0x7F]
    return np.where(c & 0x80, -v, v)


def fp8_e4m3_encode(y: np.ndarray) -> np.ndarray:
    """float32 values -> uint8 codes: the nearest finite E4M3 value to y (|y|
    clipped at 448), ties to the even code; the sign bit is y's sign bit."""
    yf = np.asarray(y, np.float32)
    a = np.minimum(np.abs(yf).astype(np.float64), 448.0)
    mags = fp8_e4m3_magnitudes()
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, len(mags) - 1)
    lo = np.clip(hi - 1, 0, len(mags) - 1)
    dlo, dhi = a - mags[lo], mags[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return code | np.where(np.signbit(yf), np.uint8(0x80), np.uint8(0))


def quantize_fp8(x: np.ndarray, dtype: str) -> Tuple[np.ndarray, np.ndarray]:
    """``x [..., D]`` storage values -> (uint8 E4M3 codes ``[..., D]``, float32 scales ``[...]``)."""
    xf = to_f64(x, dtype).astype(np.float32)          # exact: bf16 and f32 values are float32
    amax = np.abs(xf).max(axis=-1)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    codes = fp8_e4m3_encode((xf / safe[..., None]).astype(np.float32))
    codes[scale == 0] = 0
    return codes, scale


def dequantize_fp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    return fp8_e4m3_decode(codes) * scales.astype(np.float64)[..., None]


def kv_write_fp8(codes: np.ndarray, scales: np.ndarray, k: np.ndarray, v: np.ndarray,
                 slot_mapping: np.ndarray, dtype: str) -> Tuple[np.ndarray, np.ndarray]:
    """FP8 cache write: ``codes [2, NB, 16, Hkv, D]`` uint8 and ``scales
    [2, NB, 16, Hkv]`` float32, as ``kv_write_int8``."""
    kc, ks = quantize_fp8(k, dtype)
    vc, vs = quantize_fp8(v, dtype)
    codes = kv_write(codes, kc, vc, slot_mapping)
    scales = kv_write(scales[..., None], ks[..., None], vs[..., None], slot_mapping)[..., 0]
    return codes, scales


# ---------------------------------------------------------------------------
# paged_kv_write: place each new token's K and V at its slot.

def kv_write(pool: np.ndarray, k: np.ndarray, v: np.ndarray,
             slot_mapping: np.ndarray, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Return a copy of ``pool`` with token ``t``'s K/V stored at ``slot_mapping[t]``.

    ``pool``: ``[2, num_blocks, block_size, Hkv, D]``; ``k``, ``v``:
    ``[T, Hkv, D]``.  Slot ``-1`` marks a padding token and is skipped.  The
    stored values are the input bits unchanged (pure copy).  Slot -> (block,
    offset) follows the page's slot formula (section "Paged Attention")."""
    out = pool.copy()
    num_blocks = pool.shape[1]
    for t in range(int(slot_mapping.shape[0])):
        s = int(slot_mapping[t])
        if s == -1:
            continue
        if s < 0 or s >= num_blocks * block_size:
            raise ValueError(f"slot {s} of token {t} is outside the pool")
        block_idx = s // block_size
        block_offset = s % block_size
        out[0, block_idx, block_offset] = k[t]
        out[1, block_idx, block_offset] = v[t]
    return out


def rope(x: np.ndarray, positions: np.ndarray, cos_sin_cache: np.ndarray, rotary_dim: int,
         is_neox: bool, dtype: str) -> np.ndarray:
    """Rotary position embedding of ``x [T, H, D]`` (storage values), in float64.

    "AI Infra入门干货总结", section "LLM 推理全流程" / "RoPE": a token's position is
    encoded as rotation angles, read from a precomputed ``cos_sin_cache`` of shape
    ``[max_position_embeddings, rotary_dim]``.  Readings (the page gives only that
    much): row ``p`` holds ``cos`` of the ``rotary_dim/2`` angles of position ``p``
    followed by their ``sin``; angle ``i`` rotates the pair (``i``, ``i + rotary_dim/2``)
    when ``is_neox`` (the two halves of the rotary dims) and (``2i``, ``2i+1``)
    otherwise, as ``x' = x cos - y sin``, ``y' = y cos + x sin``; dims from
    ``rotary_dim`` on pass through.  Returns float64; the caller rounds to storage."""
    v = to_f64(x, dtype).copy()
    half = rotary_dim // 2
    cs = np.asarray(cos_sin_cache, dtype=np.float32).astype(np.float64)[np.asarray(positions, dtype=np.int64)]
    c, s = cs[:, None, :half], cs[:, None, half:rotary_dim]
    if is_neox:
        ix, iy = np.arange(half), np.arange(half) + half
    else:
        ix, iy = 2 * np.arange(half), 2 * np.arange(half) + 1
    xs, ys = v[:, :, ix].copy(), v[:, :, iy].copy()
    v[:, :, ix] = xs * c - ys * s
    v[:, :, iy] = ys * c + xs * s
    return v


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> storage values: float32 (IEEE nearest even), or bf16 bit
    patterns.  bf16 keeps the top 16 bits of the float32, rounded to nearest
    with ties to even (a float32 whose low 16 bits are exactly 0x8000 is a
    tie); the float64 value is first rounded to float32, as the product's own
    float32 arithmetic does.  A carry out of the mantissa bumps the exponent
    (so the largest finite float32 rounds to infinity); NaN becomes the quiet
    NaN 0x7FC0."""
    with np.errstate(over="ignore", invalid="ignore"):     # beyond float32 -> +-inf
        f = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return f
    u = f.view(np.uint32).astype(np.uint64)            # no wrap-around in the addition
    r = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)).astype(np.uint16)
    return np.where(np.isnan(f), np.uint16(0x7FC0), r).astype(np.uint16)


def copy_blocks(pool: np.ndarray, copies) -> np.ndarray:
    """Return a copy of ``pool`` where each destination block holds its source
    block's K and V (every slot, every head): the copy step of copy-on-write
    prefix sharing (lpnh.cn/news/2436702, section 2.2).  ``copies``: pairs
    (source, destination); no block is both, or twice a destination."""
    out = pool.copy()
    for src, dst in np.asarray(copies, dtype=np.int64).reshape(-1, 2):
        out[:, dst] = pool[:, src]
    return out


# ---------------------------------------------------------------------------
# Reading one request's K/V through its block table.

def gather_kv(pool: np.ndarray, block_table_row: np.ndarray, seq_len: int,
              dtype: str, block_size: int = BLOCK_SIZE) -> Tuple[np.ndarray, np.ndarray]:
    """Logical ``K, V [seq_len, Hkv, D]`` (float64) of one request.

    Logical token ``t`` lives in physical block ``block_table_row[t // block_size]``
    at offset ``t % block_size`` (section "Paged Attention")."""
    pos = np.arange(seq_len)
    blocks = np.asarray(block_table_row)[pos // block_size]
    offs = pos % block_size
    K = to_f64(pool[0, blocks, offs], dtype)
    V = to_f64(pool[1, blocks, offs], dtype)
    return K, V


# ---------------------------------------------------------------------------
# Attention.

def _softmax_rows(scores: np.ndarray, visible: np.ndarray) -> np.ndarray:
    """Row softmax of ``scores`` over the ``visible`` entries (others get weight 0)."""
    s = np.where(visible, scores, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    w = np.where(visible, np.exp(s - m), 0.0)
    return w / w.sum(axis=-1, keepdims=True)


def _check_request(r: int, seq_len: int, computed: int, qlen: int) -> None:
    if qlen < 0 or seq_len != computed + qlen:
        raise ValueError(f"request {r}: seq_len {seq_len} != computed {computed} + query {qlen}")


def request_weights(q_rows: np.ndarray, K: np.ndarray, computed: int, scale: float,
                    num_q_heads: int) -> np.ndarray:
    """Softmax weights ``[ql, Hq, L]`` of one request (float64).

    Query row ``i`` is at absolute position ``computed + i`` and sees keys
    ``t <= computed + i``.  Query head ``h`` reads KV head ``h // (Hq // Hkv)``,
    so the scores are formed one KV head at a time: its ``G = Hq // Hkv``
    query heads, all rows, times that head's keys (one matrix product)."""
    ql, _, D = q_rows.shape
    L, Hkv, _ = K.shape
    G = num_q_heads // Hkv
    scores = np.empty((ql, num_q_heads, L))
    for g in range(Hkv):
        heads = slice(g * G, (g + 1) * G)
        qg = q_rows[:, heads, :].reshape(ql * G, D)
        scores[:, heads, :] = (np.matmul(qg, K[:, g, :].T) * scale).reshape(ql, G, L)
    visible = (np.arange(L)[None, :] <= (computed + np.arange(ql))[:, None])[:, None, :]
    return _softmax_rows(scores, visible)


def weighted_values(w: np.ndarray, V: np.ndarray) -> np.ndarray:
    """``out [ql, Hq, D] = sum_t w[i, h, t] V[t, h // G]`` (float64), one KV
    head at a time (its G query heads share that head's values)."""
    ql, Hq, L = w.shape
    _, Hkv, D = V.shape
    G = Hq // Hkv
    out = np.empty((ql, Hq, D))
    for g in range(Hkv):
        heads = slice(g * G, (g + 1) * G)
        out[:, heads, :] = np.matmul(w[:, heads, :].reshape(ql * G, L), V[:, g, :]).reshape(ql, G, D)
    return out


def attention(q: np.ndarray, pool: np.ndarray, block_table: np.ndarray,
              seq_lens: np.ndarray, query_start_loc: np.ndarray,
              num_computed_tokens: np.ndarray, scale: float, dtype: str,
              requests: Optional[Iterable[int]] = None) -> np.ndarray:
    """Paged attention for one step, float64 ``out [T, Hq, D]``.

    ``requests`` restricts the work to some requests (other rows stay NaN)."""
    T, Hq, D = q.shape
    Hkv = pool.shape[3]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    out = np.full((T, Hq, D), np.nan)
    R = int(seq_lens.shape[0])
    for r in (range(R) if requests is None else requests):
        qs, qe = int(query_start_loc[r]), int(query_start_loc[r + 1])
        L, c = int(seq_lens[r]), int(num_computed_tokens[r])
        _check_request(r, L, c, qe - qs)
        if qe == qs:
            continue
        K, V = gather_kv(pool, block_table[r], L, dtype)
        qf = to_f64(q[qs:qe], dtype)
        out[qs:qe] = weighted_values(request_weights(qf, K, c, scale, Hq), V)
    return out


def attention_int8(q: np.ndarray, codes: np.ndarray, scales: np.ndarray, block_table: np.ndarray,
                   seq_lens: np.ndarray, query_start_loc: np.ndarray,
                   num_computed_tokens: np.ndarray, scale: float, dtype: str,
                   requests: Optional[Iterable[int]] = None) -> np.ndarray:
    """``attention`` over an INT8 cache: the keys and values are the
    dequantised ``code * scale`` (q in ``dtype``)."""
    return attention(to_f64(q, dtype), dequantize_int8(codes, scales), block_table, seq_lens,
                     query_start_loc, num_computed_tokens, scale, "f64", requests=requests)


def attention_fp8(q: np.ndarray, codes: np.ndarray, scales: np.ndarray, block_table: np.ndarray,
                  seq_lens: np.ndarray, query_start_loc: np.ndarray,
                  num_computed_tokens: np.ndarray, scale: float, dtype: str,
                  requests: Optional[Iterable[int]] = None) -> np.ndarray:
    """``attention`` over an FP8 cache: the keys and values are the
    dequantised ``decode(code) * scale`` (q in ``dtype``)."""
    return attention(to_f64(q, dtype), dequantize_fp8(codes, scales), block_table, seq_lens,
                     query_start_loc, num_computed_tokens, scale, "f64", requests=requests)


def attention_rows(q: np.ndarray, pool: np.ndarray, block_table: np.ndarray,
                   seq_lens: np.ndarray, query_start_loc: np.ndarray,
                   num_computed_tokens: np.ndarray, scale: float, dtype: str,
                   tokens: Sequence[int], max_run: int = 256) -> np.ndarray:
    """``out[t]`` (all heads, float64) for the chosen token rows only.

    Consecutive chosen rows of one request (at most ``max_run`` of them) are
    computed together: row ``t`` of request ``r`` is at absolute position
    ``p = computed + (t - query_start)`` and sees keys ``0 .. p``, so a run
    starting at row ``t0`` is the request's attention with ``computed + (t0 -
    query_start)`` tokens before it."""
    Hq = q.shape[1]
    tokens = [int(t) for t in tokens]
    res = np.empty((len(tokens), Hq, q.shape[2]))
    i = 0
    while i < len(tokens):
        t0 = tokens[i]
        r = int(np.searchsorted(query_start_loc, t0, side="right") - 1)
        qs, qe = int(query_start_loc[r]), int(query_start_loc[r + 1])
        L, c = int(seq_lens[r]), int(num_computed_tokens[r])
        _check_request(r, L, c, qe - qs)
        n = 1
        while i + n < len(tokens) and n < max_run and tokens[i + n] == t0 + n and t0 + n < qe:
            n += 1
        p0 = c + (t0 - qs)                      # absolute position of the run's first query
        K, V = gather_kv(pool, block_table[r], p0 + n, dtype)
        w = request_weights(to_f64(q[t0:t0 + n], dtype), K, p0, scale, Hq)   # [n, Hq, p0+n]
        res[i:i + n] = weighted_values(w, V)
        i += n
    return res


# ---------------------------------------------------------------------------
# Split-KV (Flash-Decoding, named in lpnh.cn/news/2436702 section 6; the pages
# give no algorithm).  Reading taken: cut the visible keys into partitions,
# keep for each the running max m, the sum l of exp(s - m) and the
# un-normalised o = sum exp(s - m) v, then merge with the log-sum-exp rule.
# Online softmax (section "Attention (FlashAttention)") is what makes the
# merge exact.

def partition_state(scores: np.ndarray, values: np.ndarray) -> Tuple[float, float, np.ndarray]:
    """(m, l, o) of one partition: scores ``[n]``, values ``[n, D]``."""
    m = float(scores.max())
    e = np.exp(scores - m)
    return m, float(e.sum()), e @ values


def merge_states(states: Sequence[Tuple[float, float, np.ndarray]]) -> np.ndarray:
    """Attention output from partition states: sum_p e^{m_p-M} o_p / sum_p e^{m_p-M} l_p."""
    M = max(m for m, _, _ in states)
    num = sum(np.exp(m - M) * o for m, _, o in states)
    den = sum(np.exp(m - M) * l for m, l, _ in states)
    return num / den


def split_kv_row(q_row: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                 partition: int) -> np.ndarray:
    """One query head's output computed partition by partition and merged.

    ``q_row [D]``, ``K, V [n, D]`` (the visible keys of that head's KV head)."""
    n = K.shape[0]
    scores = (K @ q_row) * scale
    states = [partition_state(scores[a:a + partition], V[a:a + partition])
              for a in range(0, n, partition)]
    return merge_states(states)


# ---------------------------------------------------------------------------
# Dense brute force, for tiny inputs only: contiguous K/V, scalar loops.

def dense_brute_force(q: Sequence, K: Sequence, V: Sequence, scale: float,
                      computed: int) -> List:
    """Scalar-loop attention of one request over contiguous K/V.

    ``q[i][h][d]``, ``K[t][g][d]``, ``V[t][g][d]`` as nested sequences of
    Python floats.  Returns ``out[i][h][d]``."""
    import math
    ql, Hq, D = len(q), len(q[0]), len(q[0][0])
    Hkv = len(K[0])
    G = Hq // Hkv
    out = []
    for i in range(ql):
        row = []
        for h in range(Hq):
            g = h // G
            last = computed + i
            s = []
            for t in range(last + 1):
                acc = 0.0
                for d in range(D):
                    acc += q[i][h][d] * K[t][g][d]
                s.append(acc * scale)
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            tot = sum(e)
            o = []
            for d in range(D):
                acc = 0.0
                for t in range(last + 1):
                    acc += e[t] * V[t][g][d]
                o.append(acc / tot)
            row.append(o)
        out.append(row)
    return out
