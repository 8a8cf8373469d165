"""Algorithmic bytes and flops of the hot path (what the roofline is priced on).

Storage follows the KV-cache storage formula of "KV cache memory systems"
(section "Cache contents"): M_KV = 2 L S H_kv D B bytes per sequence for L
caching layers.  A YOCO model caches once ("YOCO_论文与推理数据流详解" §6:
one global K/V), so L = 1 for the shared cache, while each of the L cross
layers reads all of it in turn (§11 and §17.2: the global K/V is written once
and read by every cross layer).

Algorithmic bytes count every input byte the definition needs once and every
output byte once; workspace traffic (split-KV partials) is not counted.
"""

from __future__ import annotations

import numpy as np


def kv_bytes(layers: int, sequence: int, kv_heads: int, head_dim: int, bytes_per_scalar: int) -> int:
    """Cache storage per sequence: keys and values of every caching layer."""
    return 2 * layers * sequence * kv_heads * head_dim * bytes_per_scalar


def attn_ranges(seq_lens, query_lens=None, window: int = 0):
    """Per request, the context range [lo, n) its query rows read: the whole
    context, or with a window of W tokens and q rows at the last q positions,
    from n - q - W + 1 on."""
    seq = np.asarray(seq_lens, dtype=np.int64)
    ql = np.ones_like(seq) if query_lens is None else np.asarray(query_lens, dtype=np.int64)
    lo = np.zeros_like(seq) if window <= 0 else np.maximum(0, seq - ql - window + 1)
    lo = np.where(ql > 0, lo, seq)           # a request without rows reads nothing
    return lo, seq


def attn_layer_bytes(seq_lens, num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                     elem_bytes: int, query_lens=None, window: int = 0, q_bytes=None, scale_bytes: int = 0) -> int:
    """One cross-attention call: every K/V row of the range each request reads
    once (with an 8-bit cache: 1-byte elements plus the row's K and V scales,
    scale_bytes per token and KV head), q in and fp32 out for every query row,
    the block-table entries the ranges span, seq_lens (and query_start_loc
    when there are several rows)."""
    lo, n = attn_ranges(seq_lens, query_lens, window)
    kv = int(sum(kv_bytes(1, int(b - a), num_kv_heads, head_dim, elem_bytes) for a, b in zip(lo, n)))
    kv += int(np.sum(n - lo)) * num_kv_heads * scale_bytes
    r = len(n)
    rows = r if query_lens is None else int(np.sum(query_lens))
    q_out = rows * num_q_heads * head_dim * ((elem_bytes if q_bytes is None else q_bytes) + 4)
    spanned = np.where(n > lo, (np.maximum(n, 1) - 1) // block_size - lo // block_size + 1, 0)
    table = int(np.sum(spanned)) * 4
    return kv + q_out + table + 4 * r + (0 if query_lens is None else 4 * (r + 1))


def attn_layer_flops(seq_lens, num_q_heads: int, head_dim: int) -> int:
    """q.k and p.v multiply-adds (2 flops each) per context token and query head."""
    return int(np.sum(np.asarray(seq_lens, dtype=np.int64))) * num_q_heads * 4 * head_dim


def append_bytes(num_tokens: int, hidden: int, num_kv_heads: int, head_dim: int, elem_bytes: int,
                 written_rows: int) -> int:
    """yoco_kv_append: x, RMS weight and both weight matrices read once; each
    written row's K and V stored once; slot_mapping read."""
    out = 2 * num_kv_heads * head_dim
    return (num_tokens * hidden + hidden + out * hidden) * elem_bytes + written_rows * out * elem_bytes + 4 * num_tokens


def append_flops(num_tokens: int, hidden: int, num_kv_heads: int, head_dim: int) -> int:
    return 2 * num_tokens * hidden * 2 * num_kv_heads * head_dim


def gather_bytes(num_reqs: int, row_bytes: int) -> int:
    return 2 * num_reqs * row_bytes + 4 * (num_reqs + 1) + 4 * num_reqs


def retention_layer_bytes(lens, state_slots, num_heads: int, head_dim: int, qkv_bytes: int = 2) -> int:
    """One gated-retention layer over a batch: every row's q, k, v, gate (fp32)
    and output (fp32) once, and the fp32 [D][D] state of each head read and
    written once for every request that has rows and a state slot
    ("YOCO_论文与推理数据流详解" §18.1: the fixed-size self-decoder state is
    read and written back at every token step); plus the int32 offsets and
    slot numbers."""
    lens = np.asarray(lens, dtype=np.int64)
    slots = np.asarray(state_slots, dtype=np.int64)
    rows = int(lens.sum())
    per_row = num_heads * (3 * head_dim * qkv_bytes + 4 + 4 * head_dim)
    stateful = int(((lens > 0) & (slots >= 0)).sum())
    return rows * per_row + stateful * num_heads * 2 * head_dim * head_dim * 4 + 4 * (2 * len(lens) + 1)


def retention_layer_flops(lens, num_heads: int, head_dim: int) -> int:
    """The recurrence's own multiply-adds, 2 flops each: per row and head,
    gamma S + k^T v (D^2) and q S (D^2)."""
    return int(np.asarray(lens, dtype=np.int64).sum()) * num_heads * 4 * head_dim * head_dim
