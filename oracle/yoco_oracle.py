"""Float64 CPU oracle for the YOCO cross-decoder hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the library calls this module: only the
tests, the package smoke check and the benchmark's CPU-baseline leg import it.
It shares no code, tables or helpers with the HIP path, and it never reads a
value that the HIP path produced: every input it sees comes from the seeded
generators or from the pages.

It is the plain, slow definition of what the library's calls compute,
written with NumPy in float64 (bf16 and fp32 inputs convert to float64
exactly).  Loops run over requests, heads and tokens; a matrix product is the
only library primitive used.  Where the pages leave a step open, the reading
taken is named in the docstring of the function it affects.

Pages cited (by title and section):
  [vLLM]  "You Only Cache Once, in vLLM" (yhshin.com), section
          "Implementation in vLLM": the scheduling walk-through (R1 with a
          6-token prompt, R2 with a 2-token prompt) and the statement that the
          cross-decoder keeps only the last scheduled token of each request;
          the metadata builder's query_start_loc / seq_lens / slot_mapping /
          block_table fields.
  [YOCO]  "YOCO_论文与推理数据流详解" (yuyanqi.com), §3 architecture flowchart
          (shared projection K̂ = LN(M)W_K, V̂ = LN(M)W_V; one K/V pair appended
          per token; every cross layer reads the same K̂, V̂), §7.4 (only the last
          position goes through the cross-decoder), §10.3 (one append per token,
          not per layer), §10.4 (query differs per layer, K/V are shared),
          §13.2 (query length 1 against KV length t), §4.1-4.2 (the
          self-decoder's gated retention: a gated linear recurrence over a
          fixed-size state, with parallel, recurrent and chunkwise forms).
  [KV]    "KV cache memory systems" (blog.ecitis.org), section "Cache contents"
          (decode attention softmax(q_t K_{<=t}^T / sqrt(d_h)) V_{<=t}) and
          section "Contiguous allocation wastes capacity" (every logical block
          is resolved through the block table).

Parity pins: every function here is pinned by tests that do not re-run its own
formula (closed forms, invariants, library routines, the pages' worked
examples); none is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "logical_kv",
    "attention_one_query",
    "cross_attention",
    "rms_norm",
    "kv_project",
    "kv_append",
    "gather_last",
    "cross_metadata",
    "gather_rows",
    "query_positions",
    "cross_attention_varlen",
    "e4m3_decode",
    "e4m3_encode",
    "quantize_rows",
    "dequantize_cache",
    "kv_scatter",
    "kv_append_fp8",
    "gated_retention",
]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Paged cache addressing  ([KV] "Contiguous allocation wastes capacity")
# ---------------------------------------------------------------------------

def logical_kv(k_cache, v_cache, table_row, n: int):
    """Return the first ``n`` logical K̂ and V̂ rows of one request.

    The cache tensors are laid out ``[num_blocks][num_kv_heads][block_size]
    [head_dim]``.  Logical position ``j`` lives in physical block
    ``table_row[j // block_size]`` at offset ``j % block_size``: the block
    table maps logical token blocks to arbitrary physical pages ([KV],
    "Contiguous allocation wastes capacity").

    Returns two float64 arrays of shape ``[n, num_kv_heads, head_dim]``.
    """
    bs = k_cache.shape[2]
    table_row = np.asarray(table_row)
    keys = []
    values = []
    for j in range(n):
        block = int(table_row[j // bs])
        offset = j % bs
        keys.append(_f64(k_cache[block, :, offset, :]))
        values.append(_f64(v_cache[block, :, offset, :]))
    if n == 0:
        hkv, d = k_cache.shape[1], k_cache.shape[3]
        return np.zeros((0, hkv, d)), np.zeros((0, hkv, d))
    return np.stack(keys), np.stack(values)


# ---------------------------------------------------------------------------
# Causal cross-attention, one query per request  ([KV] "Cache contents";
# [YOCO] §10.4, §13.2)
# ---------------------------------------------------------------------------

def attention_one_query(q_vec, keys, values, scale: float) -> np.ndarray:
    """softmax(scale * keys @ q) @ values for one query vector.

    ``keys`` and ``values`` are ``[n, d]``; the query attends to every one of
    the n rows (query length 1, KV length n, [YOCO] §13.2).  The maximum score
    is subtracted before exponentiating; this leaves the softmax unchanged and
    keeps float64 in range.
    """
    q_vec = _f64(q_vec)
    keys = _f64(keys)
    values = _f64(values)
    scores = scale * (keys @ q_vec)
    weights = np.exp(scores - scores.max())
    return (weights @ values) / weights.sum()


def cross_attention(q, k_cache, v_cache, block_table, seq_lens, scale: float):
    """One cross layer's attention for every request and query head.

    q: ``[R][Hq][D]``; caches ``[num_blocks][Hkv][block_size][D]``;
    block_table: ``[R][max_blocks]``; seq_lens: ``[R]``.  Returns float64
    ``[R][Hq][D]``.

    Readings of the pages taken here:
      * the context is inclusive: request r's query attends to all
        ``seq_lens[r]`` cached tokens, its own among them ([KV] writes
        K_{<=t}; [YOCO] §10.3 appends K̂_t before the cross layers run);
      * query head h reads KV head ``h // (Hq // Hkv)`` (contiguous GQA groups);
      * ``scale`` is passed in; the pages' value is 1/sqrt(head_dim);
      * a request with an empty context yields a zero output row.
    """
    q = np.asarray(q)
    num_reqs, num_q_heads, head_dim = q.shape
    num_kv_heads = k_cache.shape[1]
    group = num_q_heads // num_kv_heads
    out = np.zeros((num_reqs, num_q_heads, head_dim), dtype=np.float64)
    for r in range(num_reqs):
        n = int(seq_lens[r])
        if n == 0:
            continue
        keys, values = logical_kv(k_cache, v_cache, block_table[r], n)
        for h in range(num_q_heads):
            g = h // group
            out[r, h] = attention_one_query(q[r, h], keys[:, g, :], values[:, g, :], scale)
    return out


# ---------------------------------------------------------------------------
# Shared K/V projection and append  ([YOCO] §3 flowchart, §7.3, §10.3)
# ---------------------------------------------------------------------------

def rms_norm(x, weight, eps: float) -> np.ndarray:
    """Row-wise RMSNorm: x / sqrt(mean(x^2) + eps) * weight.

    The pages write the normalisation before the shared projection as "LN";
    the self-decoder blocks use RMSNorm, and RMSNorm is the reading taken here
    (no mean subtraction, no bias, weight multiplies the normalised row).
    """
    x = _f64(x)
    weight = _f64(weight)
    out = np.empty_like(x)
    for t in range(x.shape[0]):
        row = x[t]
        out[t] = row / np.sqrt(np.mean(row * row) + eps) * weight
    return out


def kv_project(x, rms_weight, eps: float, w_k, w_v, num_kv_heads: int, head_dim: int):
    """K̂ = LN(M) W_K and V̂ = LN(M) W_V for every row of M ([YOCO] §3, §10.3).

    ``x`` is ``[T][hidden]``; ``w_k``/``w_v`` are ``[num_kv_heads*head_dim]
    [hidden]`` (output features by input features), so K̂_t = W_K @ x̂_t.  No
    bias, no positional rotation (the pages' formula has neither).

    Returns ``(k, v, bound_k, bound_v)``, each float64 ``[T][Hkv][D]``.  The
    bounds are |x̂| @ |W|^T element by element: the scale of the terms summed
    into each output, which floating-point error bounds are stated against.
    """
    xh = rms_norm(x, rms_weight, eps)
    wk = _f64(w_k)
    wv = _f64(w_v)
    t = xh.shape[0]
    k = (xh @ wk.T).reshape(t, num_kv_heads, head_dim)
    v = (xh @ wv.T).reshape(t, num_kv_heads, head_dim)
    bk = (np.abs(xh) @ np.abs(wk).T).reshape(t, num_kv_heads, head_dim)
    bv = (np.abs(xh) @ np.abs(wv).T).reshape(t, num_kv_heads, head_dim)
    return k, v, bk, bv


def kv_append(x, rms_weight, eps: float, w_k, w_v, slot_mapping, k_cache, v_cache):
    """Project every scheduled token once and write it into its paged slot.

    Returns float64 copies of both caches with the new rows written.  Token t
    with ``slot_mapping[t] >= 0`` goes to block ``slot // block_size``, offset
    ``slot % block_size``, for every KV head; tokens with a negative slot
    (graph padding) are skipped and write nothing ([vLLM] metadata builder:
    slot_mapping passes through to the attention layers; [YOCO] §10.3: one
    K/V pair per token, not one per cross layer).
    """
    num_blocks, num_kv_heads, bs, head_dim = k_cache.shape
    k, v, _, _ = kv_project(x, rms_weight, eps, w_k, w_v, num_kv_heads, head_dim)
    k_out = _f64(k_cache).copy()
    v_out = _f64(v_cache).copy()
    for t, slot in enumerate(np.asarray(slot_mapping)):
        slot = int(slot)
        if slot < 0:
            continue
        block, offset = divmod(slot, bs)
        k_out[block, :, offset, :] = k[t]
        v_out[block, :, offset, :] = v[t]
    return k_out, v_out


# ---------------------------------------------------------------------------
# Last scheduled token of each request  ([vLLM] "Implementation in vLLM";
# [YOCO] §7.4)
# ---------------------------------------------------------------------------

def gather_last(hidden, cu_seqlens):
    """Select each request's last scheduled row of a token-major batch.

    ``hidden`` is ``[T][...]`` (any dtype; rows are copied bit for bit) and
    ``cu_seqlens`` is ``[R+1]`` with request r owning rows
    ``cu_seqlens[r] .. cu_seqlens[r+1]-1``.  Returns ``(rows, index)``:
    ``rows[r] = hidden[cu_seqlens[r+1]-1]`` and ``index[r]`` that row number.
    A request with no scheduled rows gets a zero row and index -1 (a reading:
    the pages assume every scheduled request has a current token).
    """
    hidden = np.asarray(hidden)
    cu = [int(c) for c in np.asarray(cu_seqlens)]
    num_reqs = len(cu) - 1
    rows = np.zeros((num_reqs,) + hidden.shape[1:], dtype=hidden.dtype)
    index = np.full(num_reqs, -1, dtype=np.int32)
    for r in range(num_reqs):
        if cu[r + 1] > cu[r]:
            index[r] = cu[r + 1] - 1
            rows[r] = hidden[cu[r + 1] - 1]
    return rows, index


# ---------------------------------------------------------------------------
# Several logits positions per request  ([vLLM] "Implementation in vLLM":
# the cross-decoder metadata builder and its printed example)
# ---------------------------------------------------------------------------

def cross_metadata(logits_indices, query_start_loc):
    """Rebuild the cross-decoder's query_start_loc from the logits positions.

    ``query_start_loc`` ``[R+1]``: request r owns token rows
    ``query_start_loc[r] .. query_start_loc[r+1]-1`` of the step's batch.
    ``logits_indices`` lists the token rows whose logits are needed (graph
    padding already cut off).  As in the page's builder, each index is assigned
    to the request whose row range holds it, the indices of each request are
    counted, and the counts are summed into a new ``[R+1]`` offset array.

    Returns ``(request_ids, counts, cross_query_start_loc, max_query_len)``.
    An index outside ``[query_start_loc[0], query_start_loc[R])`` belongs to
    no request: its request id is -1 and it is not counted (a reading; the
    page assumes every index lies inside the batch).
    """
    qsl = [int(c) for c in np.asarray(query_start_loc)]
    num_reqs = len(qsl) - 1
    request_ids = np.full(len(np.asarray(logits_indices)), -1, dtype=np.int64)
    counts = np.zeros(num_reqs, dtype=np.int64)
    for i, idx in enumerate(np.asarray(logits_indices)):
        idx = int(idx)
        for r in range(num_reqs):
            if qsl[r] <= idx < qsl[r + 1]:
                request_ids[i] = r
                counts[r] += 1
                break
    cross_qsl = np.zeros(num_reqs + 1, dtype=np.int64)
    for r in range(num_reqs):
        cross_qsl[r + 1] = cross_qsl[r] + counts[r]
    max_query_len = int(counts.max()) if num_reqs else 0
    return request_ids, counts, cross_qsl, max_query_len


def gather_rows(hidden, logits_indices):
    """``rows[i] = hidden[logits_indices[i]]`` bit for bit; an index outside
    ``[0, T)`` gives a zero row (the cross-decoder's batch is the selected
    rows, [vLLM] "Implementation in vLLM")."""
    hidden = np.asarray(hidden)
    idx = [int(i) for i in np.asarray(logits_indices)]
    rows = np.zeros((len(idx),) + hidden.shape[1:], dtype=hidden.dtype)
    for i, t in enumerate(idx):
        if 0 <= t < hidden.shape[0]:
            rows[i] = hidden[t]
    return rows


def query_positions(seq_len: int, num_queries: int):
    """Logical positions of a request's queries in the cross-decoder.

    The metadata the page builds keeps ``seq_lens`` and marks the attention
    causal, so a request with n cached tokens and q query rows has its queries
    at the last q positions n-q .. n-1 (for the page's example, request 1 with
    seq_len 31 and logits rows 18, 19 queries positions 29 and 30).  A
    position below zero (more queries than cached tokens) has no keys.
    """
    return [seq_len - num_queries + i for i in range(num_queries)]


def cross_attention_varlen(q, k_cache, v_cache, block_table, seq_lens, query_start_loc, scale: float,
                           window: int = 0):
    """One cross layer with any number of query rows per request.

    q: ``[Nq][Hq][D]`` where request r's rows are ``query_start_loc[r] ..
    query_start_loc[r+1]-1``; caches and block table as in
    :func:`cross_attention`.  The query at position p (:func:`query_positions`)
    attends causally to positions ``j <= p`` of the request's context; with
    ``window > 0`` only to the last ``window`` of them, ``p - window < j <= p``
    (a sliding-window cross layer reading a shared sliding-window cache, as
    Gemma 3n's cross layers reuse the 19th layer's sliding-window cache, [vLLM]
    "Gemma 3n").  A query with no keys yields a zero row.  Returns float64
    ``[Nq][Hq][D]``.
    """
    q = np.asarray(q)
    num_rows, num_q_heads, head_dim = q.shape
    num_kv_heads = k_cache.shape[1]
    group = num_q_heads // num_kv_heads
    qsl = [int(c) for c in np.asarray(query_start_loc)]
    out = np.zeros((num_rows, num_q_heads, head_dim), dtype=np.float64)
    for r in range(len(qsl) - 1):
        n = int(seq_lens[r])
        rows = list(range(qsl[r], qsl[r + 1]))
        if not rows or n <= 0:
            continue
        keys, values = logical_kv(k_cache, v_cache, block_table[r], n)
        for row, p in zip(rows, query_positions(n, len(rows))):
            lo = 0 if window <= 0 else max(0, p - window + 1)
            if p < 0:
                continue
            for h in range(num_q_heads):
                g = h // group
                out[row, h] = attention_one_query(q[row, h], keys[lo:p + 1, g, :], values[lo:p + 1, g, :], scale)
    return out


# ---------------------------------------------------------------------------
# 8-bit shared cache  ("KV cache memory systems", section "Quantized cache
# changes attention inputs"; [YOCO] §18.2: build compression or quantization
# of the shared K/V once and reuse it in every cross layer)
# ---------------------------------------------------------------------------
#
# Readings taken (the pages fix none of these):
#   * format: FP8 E4M3 in the finite-only variant (1 sign bit, 4 exponent bits
#     with bias 7, 3 mantissa bits; exponent field 15 with mantissa 7 is NaN;
#     no infinities; largest finite 448; subnormals m * 2^-9);
#   * one fp32 scale per (token, KV head), separately for K and for V (the
#     page: keys and values may need different calibration), chosen when the
#     token is appended as s = max|x| / 448, so the row's largest value maps
#     to the format's largest; a stored value means code * s;
#   * the scale and the division x / s are fp32 operations (IEEE, rounded to
#     nearest even), and x / s is rounded to E4M3 to nearest even -- the
#     precision the kernel takes this integer decision in.

E4M3_MAX = 448.0


def _e4m3_value(c: int) -> float:
    """Value of one FP8 E4M3 (finite-only) code."""
    sign = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return np.nan
    if e == 0:
        return sign * m * 2.0 ** -9                    # subnormal: 0.mmm * 2^-6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# every code's value, from the formula above (a cache holds millions of codes)
_E4M3_VALUES = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes) -> np.ndarray:
    """Value of every FP8 E4M3 (finite-only) code, as float64."""
    return _E4M3_VALUES[np.asarray(codes, dtype=np.uint8).astype(np.intp)]


def e4m3_encode(x) -> np.ndarray:
    """Round each value to the nearest FP8 E4M3 value, ties to the even code
    (mantissa bit 0 clear); magnitudes above 448 saturate to 448; NaN gives the
    NaN code 0x7F with the value's sign bit.  Enumerates the 127 non-negative
    finite values and picks by distance, which is the definition itself."""
    grid = e4m3_decode(np.arange(0x7F, dtype=np.uint8))          # codes 0x00..0x7E: 0 .. 448, increasing
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    for idx, v in np.ndenumerate(x):
        if np.isnan(v):
            out[idx] = 0xFF if np.signbit(v) else 0x7F
            continue
        a = min(abs(v), E4M3_MAX)
        j = int(np.searchsorted(grid, a))                          # grid[j-1] < a <= grid[j]
        if j < len(grid) and grid[j] == a:
            code = j
        else:
            lo, hi = j - 1, j
            dl, dh = a - grid[lo], grid[hi] - a
            code = lo if dl < dh else hi if dh < dl else (lo if lo % 2 == 0 else hi)
        out[idx] = code | (0x80 if np.signbit(v) else 0)
    return out


def quantize_rows(rows):
    """Quantize each row (last axis) of fp32 values to (codes, scale).

    scale = max|row| / 448 and code = E4M3(row / scale), both divisions in
    fp32; a row of zeros gets scale 0 and zero codes.  Returns uint8 codes
    shaped like ``rows`` and fp32 scales with the last axis dropped.
    """
    rows = np.asarray(rows, dtype=np.float32)
    codes = np.zeros(rows.shape, dtype=np.uint8)
    scales = np.zeros(rows.shape[:-1], dtype=np.float32)
    for idx in np.ndindex(rows.shape[:-1]):
        row = rows[idx]
        amax = np.float32(np.max(np.abs(row))) if not np.isnan(row).any() else np.float32(np.nan)
        s = np.float32(amax / np.float32(E4M3_MAX))
        scales[idx] = s
        if s == 0:
            continue
        codes[idx] = e4m3_encode(np.float32(row / s) if np.isfinite(s) else np.full(row.shape, np.nan, np.float32))
    return codes, scales


def dequantize_cache(codes, scales) -> np.ndarray:
    """The values an 8-bit cache holds: code value times its row's scale
    (exact in float64).  codes ``[..., D]``, scales ``[...]``."""
    return e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[..., None]


def kv_scatter(rows_k, rows_v, slot_mapping, k_cache, v_cache, k_scale=None, v_scale=None):
    """Write given K/V rows ``[T][Hkv][D]`` into their slots ([vLLM]
    slot_mapping; slot s is block s // block_size, row s % block_size;
    negative slots are skipped).  Without scales the rows are copied as they
    are; with scales (an 8-bit cache) each (token, KV head) row is quantized
    with :func:`quantize_rows`.  Returns updated copies of the cache arrays
    (and of the scales)."""
    bs = np.asarray(k_cache).shape[2]
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    quant = k_scale is not None
    if quant:
        ks, vs = np.array(k_scale, copy=True), np.array(v_scale, copy=True)
        ck, sk = quantize_rows(rows_k)
        cv, sv = quantize_rows(rows_v)
    for t, slot in enumerate(np.asarray(slot_mapping)):
        slot = int(slot)
        if slot < 0:
            continue
        block, offset = divmod(slot, bs)
        if quant:
            kc[block, :, offset, :], ks[block, :, offset] = ck[t], sk[t]
            vc[block, :, offset, :], vs[block, :, offset] = cv[t], sv[t]
        else:
            kc[block, :, offset, :] = rows_k[t]
            vc[block, :, offset, :] = rows_v[t]
    return (kc, vc, ks, vs) if quant else (kc, vc)


def kv_append_fp8(x, rms_weight, eps: float, w_k, w_v, slot_mapping, num_kv_heads: int, head_dim: int):
    """The shared projection (:func:`kv_project`, float64) of every scheduled
    token, quantized per (token, KV head) as :func:`quantize_rows` does after
    rounding the projected values to fp32.  Returns, per token, float64 K/V
    ``[T][Hkv][D]``, their fp32-rounded codes and scales, and the error-bound
    scales of :func:`kv_project` (the slots are the caller's to apply)."""
    k, v, bk, bv = kv_project(x, rms_weight, eps, w_k, w_v, num_kv_heads, head_dim)
    ck, sk = quantize_rows(k.astype(np.float32))
    cv, sv = quantize_rows(v.astype(np.float32))
    return k, v, (ck, sk), (cv, sv), bk, bv


# ---------------------------------------------------------------------------
# Self-decoder gated retention  ([YOCO] §4.1-4.2)
# ---------------------------------------------------------------------------
#
# The page describes gated retention as a linear recurrence with a
# data-dependent forget gate gamma_t: a fixed-size state S compresses the
# history, K_t^T V_t writes the current token into it, and the query reads
# from it; parallel, recurrent and chunkwise forms compute the same thing.
# Its formulas did not survive extraction.  Reading taken: per head,
#     S_t = gamma_t * S_{t-1} + k_t^T v_t      (S: [d_k][d_v], k_t^T v_t the outer product)
#     o_t = q_t S_t                           (the current token included)
# with gamma_t in (0, 1] given per (token, head) (how the model computes it
# from the input is not on the page), no output normalisation, no scale.

def gated_retention(q, k, v, gamma, cu_seqlens, state, state_indices):
    """The recurrent form, token by token, for a batch of requests.

    q, k: ``[T][H][Dk]``; v: ``[T][H][Dv]``; gamma: ``[T][H]``; request r owns
    rows ``cu_seqlens[r] .. cu_seqlens[r+1]-1`` in order; state: ``[slots][H]
    [Dk][Dv]``, request r starting from slot ``state_indices[r]`` (a negative
    index starts from zeros and stores nothing).  Returns float64 ``(out
    [T][H][Dv], new_state)``: every request's final state written to its slot.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    gamma = _f64(gamma)
    out = np.zeros(v.shape, dtype=np.float64)
    new_state = _f64(state).copy()
    cu = [int(c) for c in np.asarray(cu_seqlens)]
    num_heads = q.shape[1]
    for r in range(len(cu) - 1):
        slot = int(state_indices[r])
        for h in range(num_heads):
            s = new_state[slot, h].copy() if slot >= 0 else np.zeros((k.shape[2], v.shape[2]))
            for t in range(cu[r], cu[r + 1]):
                s = gamma[t, h] * s + np.outer(k[t, h], v[t, h])
                out[t, h] = q[t, h] @ s
            if slot >= 0:
                new_state[slot, h] = s
    return out, new_state
