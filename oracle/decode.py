"""FP64 CPU oracle for single-token paged GQA decode attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
this module: only the test suite, the smoke check in ``__graft_entry__`` and
the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code, constants
or helpers with the HIP library, and the HIP library never falls back to it.

What it computes, and where the pages define it
------------------------------------------------
* "Qwen 3" (TensorSharp docs), section 3 "Forward graph": every query head is
  multiplied by 1/sqrt(head_dim) and attends, after the new token has been
  appended to the cache, to every cached position of its sequence with a full
  softmax: GQA, no sliding window (section 4.1 "Attention": no sinks, no SWA).
* "Qwen3-14B" (pypto-lib models page), section "decode_fwd": the attention
  stage reads flat paged K/V pools whose bytes are ordered
  [page, token, kv_head, dim]; Q and O are "active TND" tensors, i.e. one row
  per sequence in decode, shape [B, Hq, D].
* "Qwen 3" (TensorSharp docs), section 11 "Batched / paged forward": the K/V of
  a sequence are gathered from the block tables and the sequence lengths, and a
  token lives at ``block_id * block_size + offset`` of the layer buffer.
* "Qwen3-14B" (pypto-lib), "Deployment configuration" table: 40 query heads
  over 8 KV heads (GQA), head_dim 128, 128-token pages, context <= 4096.

So for every sequence b, query head hq and its KV head h:

    out[b, hq, :] = softmax_t( scale * q[b, hq, :] . K_b[t, h, :] ) @ V_b[:, h, :]

over t in [0, context_lens[b]), with K_b / V_b the sequence's gathered pages.

Readings of points the pages leave open
---------------------------------------
R1  Query head hq uses KV head ``hq // G`` with G = Hq // Hkv (consecutive
    grouping), the layout the fused QKV row order [qDim | kvDim | kvDim] and
    the per-KV-head padding of query heads on the orcarouter page imply.
R2  ``scale`` is handed over as an FP32 value; the oracle uses that FP32 value
    widened exactly to FP64 and applies it to the dot product.
R3  ``context_lens[b]`` counts every cached token including the current one
    (the KV write precedes attention), and decode has no extra causal mask.
R4  ``context_lens[b] == 0`` gives an output row of exact zeros (the orcarouter
    page's convention for fully masked and empty rows).
R5  Block-table entries at or past ceil(ctx / page_size) are never read; they
    may hold -1 or anything else.
R6  Slots at or past ctx inside the last page are excluded before any
    arithmetic; they may hold NaN.

All arithmetic is FP64. Inputs are BF16 values (held in any float array; a BF16
value widens exactly to FP64). The output is FP64; a GPU result rounded to BF16
is compared against it.

``paged_kv_write`` is the plain index write that stores a step's new K/V rows
into the pools before attention reads them. ``paged_decode_attention_fp8``
dequantises FP8-E4M3 pools (``decode_fp8_e4m3`` times a per-tensor scale) and
then computes the same attention. ``paged_multi_query_attention`` handles
several causal query tokens per sequence (chunked prefill, multi-token decode).

Parity pins (checked by tests/test_oracle_pins.py, tests/test_oracle_kv_write.py,
tests/test_oracle_fp8.py and tests/test_oracle_multi_query.py against things
other than this file): a pure-Python scalar brute force, torch's CPU scaled-dot-product
attention in FP64, closed forms (context 1, uniform scores, a one-hot limit,
hand-derived two-token values), paged == contiguous layouts, invariance under
a permutation of the page pool, shared physical pages, the [K,V]/[q,0]
embedding identity, and a split/LSE-merge partition identity.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "attend",
    "paged_decode_attention",
    "contiguous_decode_attention",
    "gather_sequence",
    "partial_attention",
    "lse_merge",
    "paged_kv_write",
    "decode_fp8_e4m3",
    "encode_fp8_e4m3",
    "quantize_fp8_e4m3",
    "paged_kv_write_fp8",
    "paged_decode_attention_fp8",
    "paged_multi_query_attention",
]


def _as_f64(x) -> np.ndarray:
    """Widen to float64 (exact for BF16/FP32 inputs)."""
    if hasattr(x, "detach"):  # a torch tensor: go through float32, exact for bf16
        x = x.detach().to("cpu").float().numpy()
    return np.asarray(x, dtype=np.float64)


def _as_i64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    return np.asarray(x, dtype=np.int64)


def attend(qv: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
           return_weights: bool = False):
    """Softmax attention of one query vector over n keys and values.

    ``qv`` is [D], ``K`` and ``V`` are [n, D], all FP64, n >= 1.
    Logit t is ``scale * (qv . K[t])``; the weights are the softmax of the
    logits ("Qwen 3", TensorSharp docs, section 3: Q is scaled by
    1/sqrt(head_dim) before attention) and the result is ``weights @ V``.
    The subtraction of the maximum logit only guards exp() against overflow;
    it cancels exactly in real arithmetic.
    """
    K = np.ascontiguousarray(K, dtype=np.float64)
    V = np.ascontiguousarray(V, dtype=np.float64)
    logits = (K @ np.ascontiguousarray(qv, dtype=np.float64)) * scale
    w = np.exp(logits - logits.max())
    w = w / w.sum()
    out = w @ V
    if return_weights:
        return out, w
    return out


def gather_sequence(cache: np.ndarray, block_table_row: np.ndarray, n: int) -> np.ndarray:
    """Gather the first ``n`` tokens of one sequence from a paged pool.

    ``cache`` is [num_pages, page_size, Hkv, D] (the [page, token, kv_head,
    dim] byte order of the "Qwen3-14B" pypto-lib page, "decode_fwd" section).
    Token t of the sequence sits in page ``block_table_row[t // page_size]`` at
    slot ``t % page_size`` ("Qwen 3" TensorSharp docs, section 11: block id
    times block size plus offset). Only the first ceil(n / page_size) table
    entries are read (reading R5); slots past n are dropped (R6).
    Returns [n, Hkv, D].
    """
    page_size = cache.shape[1]
    npages = -(-n // page_size)
    pages = [int(block_table_row[j]) for j in range(npages)]
    gathered = cache[pages]                      # [npages, P, Hkv, D]
    gathered = gathered.reshape(npages * page_size, *cache.shape[2:])
    return gathered[:n]


def paged_decode_attention(q, k_cache, v_cache, block_table, context_lens, scale,
                           return_weights: bool = False):
    """Decode attention over a paged K/V pool, in FP64.

    q            [B, Hq, D]               (BF16 values)
    k_cache      [N, P, Hkv, D]           (BF16 values)
    v_cache      [N, P, Hkv, D]           (BF16 values; may be the same array)
    block_table  [B, W] int               (row b lists the pages of sequence b)
    context_lens [B] int                  (tokens cached for sequence b)
    scale        float, handed over as FP32 (reading R2)

    Returns out [B, Hq, D] FP64, and with ``return_weights`` also a dict
    {(b, hq): weights[n]}.
    """
    q = _as_f64(q)
    k_cache = _as_f64(k_cache)
    v_cache = _as_f64(v_cache)
    block_table = _as_i64(block_table)
    context_lens = _as_i64(context_lens)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    G = Hq // Hkv
    s64 = float(np.float32(scale))               # reading R2
    out = np.zeros((B, Hq, D), dtype=np.float64)
    weights = {}
    for b in range(B):
        n = int(context_lens[b])
        if n == 0:                               # reading R4
            continue
        K = gather_sequence(k_cache, block_table[b], n)
        V = gather_sequence(v_cache, block_table[b], n)
        for hq in range(Hq):
            h = hq // G                          # reading R1
            res = attend(q[b, hq], K[:, h, :], V[:, h, :], s64, return_weights)
            if return_weights:
                out[b, hq], weights[(b, hq)] = res
            else:
                out[b, hq] = res
    if return_weights:
        return out, weights
    return out


def contiguous_decode_attention(q, k_seq, v_seq, context_lens, scale):
    """The same attention over a contiguous per-sequence cache.

    ``k_seq`` / ``v_seq`` are [B, Hkv, max_seq, D]: per sequence, the
    [NumKVHeads, maxSeqLen, headDim] cache layout of "Qwen 3" (TensorSharp
    docs), section 10 "Memory and KV cache strategy". Used to check that the
    paged gather changes nothing.
    """
    q = _as_f64(q)
    k_seq = _as_f64(k_seq)
    v_seq = _as_f64(v_seq)
    context_lens = _as_i64(context_lens)
    B, Hq, D = q.shape
    Hkv = k_seq.shape[1]
    G = Hq // Hkv
    s64 = float(np.float32(scale))
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        n = int(context_lens[b])
        if n == 0:
            continue
        for hq in range(Hq):
            h = hq // G
            out[b, hq] = attend(q[b, hq], k_seq[b, h, :n, :], v_seq[b, h, :n, :], s64)
    return out


def partial_attention(qv, K, V, scale):
    """Unnormalised softmax partial over one token range, in base e.

    Returns (acc[D], m, l) with m = max logit, l = sum exp(logit - m) and
    acc = sum exp(logit - m) * V[t]. An empty range gives (0, -inf, 0).
    This is the plain definition of a softmax over a sub-range; merging such
    partials with ``lse_merge`` reproduces ``attend`` over the union.
    """
    D = V.shape[1]
    if K.shape[0] == 0:
        return np.zeros(D), -math.inf, 0.0
    logits = (np.ascontiguousarray(K, dtype=np.float64)
              @ np.ascontiguousarray(qv, dtype=np.float64)) * scale
    m = float(logits.max())
    e = np.exp(logits - m)
    return e @ np.ascontiguousarray(V, dtype=np.float64), m, float(e.sum())


def lse_merge(parts):
    """Merge (acc, m, l) partials of disjoint token ranges into one output.

    With M = max m_i: out = sum_i exp(m_i - M) acc_i / sum_i exp(m_i - M) l_i.
    Partials of empty ranges (m = -inf) carry zero weight; if every range is
    empty the output is zeros (reading R4).
    """
    ms = [m for (_, m, _) in parts if m != -math.inf]
    if not ms:
        return np.zeros_like(parts[0][0])
    M = max(ms)
    num = np.zeros_like(parts[0][0])
    den = 0.0
    for acc, m, l in parts:
        if m == -math.inf:
            continue
        w = math.exp(m - M)
        num = num + w * acc
        den += w * l
    return num / den


def paged_kv_write(k_cache, v_cache, k_new, v_new, slot_mapping):
    """Scatter new K/V rows into the paged pools; returns new (k_cache, v_cache).

    "Qwen 3" (TensorSharp docs), section 11 "Batched / paged forward": the
    layer's K and V of every token are written at block_id * block_size +
    offset of the paged buffer. Here ``slot_mapping[t]`` is that flat slot for
    token t: page ``slot // P``, position ``slot % P``. A negative slot marks a
    padding token that writes nothing (reading of the pages' -1 padding);
    slots at or past ``num_pages * P`` are caller errors and are skipped too,
    so nothing outside the pool is written.

    k_cache, v_cache  [N, P, Hkv, D]      (any dtype; copied, not modified)
    k_new, v_new      [T, Hkv, D]
    slot_mapping      [T] int
    """
    k = np.array(k_cache, copy=True)
    v = np.array(v_cache, copy=True)
    N, P = k.shape[0], k.shape[1]
    slots = _as_i64(slot_mapping)
    kn = np.asarray(k_new)
    vn = np.asarray(v_new)
    for t, slot in enumerate(slots.tolist()):
        if slot < 0 or slot >= N * P:
            continue
        page, pos = divmod(slot, P)
        k[page, pos] = kn[t]
        v[page, pos] = vn[t]
    return k, v


def decode_fp8_e4m3(codes) -> np.ndarray:
    """FP8 E4M3 (the OCP "FN" variant) bytes to FP64 values.

    Definition: sign bit s, 4 exponent bits e (bias 7), 3 mantissa bits m.
    e = 0 is subnormal: (-1)^s * m * 2^-9; otherwise (-1)^s * (1 + m/8) *
    2^(e-7); the two codes with e = 15, m = 7 are NaN; there is no infinity.
    The KV-cache dtype choice is the one the orcarouter page measures
    (fp8_e4m3 KV against NVFP4 KV in decode) and "Qwen 3" section 10 lists KV
    dtype options for.
    """
    b = np.asarray(codes).astype(np.int64) & 0xFF
    s = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = s * val
    return np.where((e == 15) & ((b & 7) == 7), np.nan, val)


def encode_fp8_e4m3(y) -> np.ndarray:
    """FP32 values to FP8 E4M3 ("FN") bytes: saturate, round to nearest even.

    The value set is the one ``decode_fp8_e4m3`` defines. |y| is first limited
    to 448, the largest finite value (the format has no infinity, so overflow
    saturates); the result is the code of the nearest value, and of the two
    neighbours of an exact midpoint the one whose code (hence mantissa) is
    even. The sign bit is y's, so -0.0 gives 0x80. NaN gives 0x7F. Reading: the
    pages name the dtype but not its rounding; nearest-even with saturation is
    the plainest one for a cache that must hold every finite input.
    """
    y = np.asarray(y, dtype=np.float32).astype(np.float64)       # exact widening
    pos = decode_fp8_e4m3(np.arange(0x7F))                         # codes 0..0x7E, increasing
    a = np.minimum(np.abs(y), pos[-1])
    hi = np.clip(np.searchsorted(pos, a, side="left"), 1, 0x7E)   # first value >= a
    lo = hi - 1
    d_lo = a - pos[lo]
    d_hi = pos[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo) | (np.signbit(y).astype(np.int64) << 7)
    code = np.where(np.isnan(y), 0x7F, code)
    return code.astype(np.uint8)


def quantize_fp8_e4m3(x, scale) -> np.ndarray:
    """Codes of x / scale: x widened to FP32, the quotient taken in FP32
    (IEEE division, round to nearest even), then ``encode_fp8_e4m3``. The
    stored code stands for code * scale, as ``paged_decode_attention_fp8``
    reads it."""
    x32 = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        q = x32 / np.float32(scale)
    return encode_fp8_e4m3(q)


def paged_kv_write_fp8(k_codes, v_codes, k_new, v_new, k_scale, v_scale, slot_mapping):
    """``paged_kv_write`` into FP8-E4M3 pools: the rows written are
    ``quantize_fp8_e4m3(k_new, k_scale)`` and ``quantize_fp8_e4m3(v_new,
    v_scale)``; the same slot rules (negative or past the pool: nothing
    written). Returns new (k_codes, v_codes) uint8 arrays."""
    with np.errstate(invalid="ignore"):                 # signalling NaN inputs widen quietly
        kq = quantize_fp8_e4m3(_as_f64(k_new), k_scale)
        vq = quantize_fp8_e4m3(_as_f64(v_new), v_scale)
    return paged_kv_write(np.asarray(k_codes, dtype=np.uint8), np.asarray(v_codes, dtype=np.uint8),
                          kq, vq, slot_mapping)


def paged_decode_attention_fp8(q, k_codes, v_codes, k_scale, v_scale, block_table,
                               context_lens, scale):
    """Decode attention over FP8-E4M3 K/V pools with per-tensor FP32 scales.

    K = decode(k_codes) * k_scale and V = decode(v_codes) * v_scale (each
    scale handed over as FP32, used exactly in FP64), then the same attention
    as ``paged_decode_attention``. Reading: the pages do not fix the scale
    granularity; one scale per tensor is the plainest one.
    """
    k = decode_fp8_e4m3(k_codes) * float(np.float32(k_scale))
    v = decode_fp8_e4m3(v_codes) * float(np.float32(v_scale))
    return paged_decode_attention(q, k, v, block_table, context_lens, scale)


def paged_multi_query_attention(q, k_cache, v_cache, block_table, context_lens, query_start,
                                scale):
    """Several query tokens per sequence (chunked prefill, multi-token decode).

    q [T, Hq, D] holds the query tokens of all sequences packed token-major,
    sequence b owning rows query_start[b] .. query_start[b+1]-1 ("Qwen3-14B"
    pypto-lib page, prefill_fwd: inputs packed token-major, T = sum of chunk
    lengths, no batch padding). The Lq_b query tokens are the last Lq_b
    tokens of sequence b's context_lens[b] cached tokens (their K/V were
    written first, as in decode), so query i (position ctx - Lq + i) attends
    causally to tokens [0, ctx - Lq + i] ("Qwen 3" TensorSharp docs, section
    4.1: standard causal attention). A query that sees no token (ctx < Lq)
    is a fully masked row and gives zeros, the convention the orcarouter
    Qwen4-Exp QSA prefill page keeps for such rows ("operational details"
    list, size-limits item). Returns out [T, Hq, D] FP64.
    """
    q = _as_f64(q)
    k_cache = _as_f64(k_cache)
    v_cache = _as_f64(v_cache)
    block_table = _as_i64(block_table)
    context_lens = _as_i64(context_lens)
    qs = _as_i64(query_start)
    T, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    G = Hq // Hkv
    s64 = float(np.float32(scale))
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for b in range(len(context_lens)):
        lq = int(qs[b + 1] - qs[b])
        ctx = int(context_lens[b])
        if lq == 0 or ctx <= 0:
            continue
        K = gather_sequence(k_cache, block_table[b], ctx)
        V = gather_sequence(v_cache, block_table[b], ctx)
        for i in range(lq):
            n = ctx - lq + i + 1                 # tokens query i may see
            if n <= 0:
                continue
            r = int(qs[b]) + i
            for hq in range(Hq):
                h = hq // G
                out[r, hq] = attend(q[r, hq], K[:n, h, :], V[:n, h, :], s64)
    return out


def paged_multi_query_attention_fp8(q, k_codes, v_codes, k_scale, v_scale, block_table,
                                    context_lens, query_start, scale):
    """Multi-query attention over FP8-E4M3 K/V pools with per-tensor FP32 scales.

    K = decode(k_codes) * k_scale and V = decode(v_codes) * v_scale, as in
    ``paged_decode_attention_fp8``, then ``paged_multi_query_attention``: a
    cache kept in fp8_e4m3 (the KV dtype the orcarouter page measures) is read
    by chunked prefill and multi-token decode as well as by single-token
    decode.
    """
    k = decode_fp8_e4m3(k_codes) * float(np.float32(k_scale))
    v = decode_fp8_e4m3(v_codes) * float(np.float32(v_scale))
    return paged_multi_query_attention(q, k, v, block_table, context_lens, query_start, scale)
