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


def attn_layer_bytes(seq_lens, num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                     elem_bytes: int) -> int:
    """One yoco_cross_attn call: every context K/V row once, q in, fp32 out,
    the block-table entries the contexts use, and seq_lens."""
    seq = np.asarray(seq_lens, dtype=np.int64)
    kv = int(sum(kv_bytes(1, int(n), num_kv_heads, head_dim, elem_bytes) for n in seq))
    r = len(seq)
    q_out = r * num_q_heads * head_dim * (elem_bytes + 4)
    table = int(np.sum(-(-seq // block_size))) * 4
    return kv + q_out + table + 4 * r


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
