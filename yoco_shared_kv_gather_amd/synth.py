"""Seeded synthetic workloads for the YOCO cross-decoder hot path.

This module only draws inputs: request lengths, block placement, slot
numbers and random tensors.  It holds none of the method's arithmetic (no
normalisation, projection, softmax or gather), so the tests can hand the same
buffers to the library and to the float64 checker.

Workloads (all synthetic, seeded):
  1 "tiny"   the scheduling walk-through of "You Only Cache Once, in vLLM"
             (R1 with a 6-token prompt, R2 with a 2-token prompt), step 1:
             R1 decodes token 6, R2 prefills tokens 0-1.  fp32, 1 KV head x 64,
             block 4, 8 physical blocks in random order, 8 cross layers of 4
             query heads, hidden 256.
  2 "decode64"   64 decodes, context U{1024..8192}, bf16 2 KV heads x 256,
             block 16, 10 layers x 8 query heads, hidden 2048.
  3 "decode32x32k" 32 decodes at 32768, bf16 8 x 128, block 16, 16 layers x 32
             query heads, hidden 3072; 0.1% of key vectors scaled by 20.
  4 "mixed48"  16 prefills (log-uniform 512..16384) + 32 decodes (U{2048..
             32768}) in shuffled order, bf16 8 x 128, block 16, 16 layers x 32
             query heads, hidden 3072, ~5% graph-padding rows (slot -1).
  5 "long512k" one request at 524288 tokens, bf16 8 x 128, block 32 in random
             placement, 24 layers x 32 query heads, hidden 3072.

Shapes follow YOCO-3B where the pages give them ("YOCO_论文与推理数据流详解",
§16.1: hidden 3072, 24 query heads, 8 KV heads, so head_dim 128).

Cache pools hold about 1.25x the blocks the contexts need; blocks are handed
out in a seeded random order, and free blocks, tail slots past each context
and unused block-table entries are poisoned with NaN so that any read outside
a context shows up in the output.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

SEED_BASE = 2024

# Child-stream indices of the per-workload SeedSequence (one per drawn item).
_S_LENGTHS, _S_PERM, _S_K, _S_V, _S_OUTLIER, _S_Q, _S_X, _S_WK, _S_WV, _S_ORDER, _S_RMS = range(11)


@dataclasses.dataclass(frozen=True)
class Geometry:
    name: str
    dtype: str            # "f32" or "bf16": cache, q, x and weight dtype
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_layers: int
    hidden: int

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


GEOMETRIES: Dict[int, Geometry] = {
    1: Geometry("tiny", "f32", 4, 1, 64, 4, 8, 256),
    2: Geometry("decode64", "bf16", 8, 2, 256, 16, 10, 2048),
    3: Geometry("decode32x32k", "bf16", 32, 8, 128, 16, 16, 3072),
    4: Geometry("mixed48", "bf16", 32, 8, 128, 16, 16, 3072),
    5: Geometry("long512k", "bf16", 32, 8, 128, 32, 24, 3072),
}


@dataclasses.dataclass
class Metadata:
    """Scheduling metadata of one step (host numpy arrays)."""
    config_id: int
    size: str
    geom: Geometry
    seq_lens: np.ndarray        # int32 [R]  cached tokens per request, current one included
    query_lens: np.ndarray      # int32 [R]  tokens scheduled this step per request
    cu_seqlens: np.ndarray      # int32 [R+1]
    num_tokens: int             # T, padding rows included
    slot_mapping: np.ndarray    # int32 [T], -1 for padding rows
    block_table: np.ndarray     # int32 [R][max_blocks]
    num_blocks: int
    poison_block: int           # a free block every unused table entry points at
    outlier_prob: float = 0.0
    outlier_scale: float = 1.0

    @property
    def num_reqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_reqs else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])


def _seed_seq(config_id: int, size: str, seed: int) -> np.random.SeedSequence:
    size_tag = {"full": 0, "small": 1, "edge": 2}[size]
    return np.random.SeedSequence([seed, config_id, size_tag])


def custom_geometry(dtype: str, num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                    hidden: int = 256, num_layers: int = 1) -> Geometry:
    return Geometry(f"custom_{dtype}_{num_q_heads}x{num_kv_heads}x{head_dim}_bs{block_size}", dtype, num_q_heads,
                    num_kv_heads, head_dim, block_size, num_layers, hidden)


def _child_seed(ss: np.random.SeedSequence, index: int) -> int:
    """A 63-bit integer seed for child stream ``index`` of ``ss``."""
    child = np.random.SeedSequence(entropy=ss.entropy, spawn_key=ss.spawn_key + (index,))
    return int(child.generate_state(2, dtype=np.uint64)[0] >> np.uint64(1))


def _rng(ss: np.random.SeedSequence, index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(_child_seed(ss, index)))


def _requests(config_id: int, size: str, ss: np.random.SeedSequence):
    """Per-request (context length, scheduled tokens) and padding rows."""
    rng = _rng(ss, _S_LENGTHS)
    pad = 0
    if size == "edge":
        # an empty context, a single token, exact block multiples and ragged tails
        return [(0, 0), (1, 1)] + [(c, 1) for c in (2, 31, 32, 33, 64, 97)], 0
    if config_id == 1:
        # step 1 of the walk-through: R1 decodes its token 6, R2 prefills 2 tokens
        reqs = [(7, 1), (2, 2)]
    elif config_id == 2:
        if size == "full":
            ctx = rng.integers(1024, 8192, size=64, endpoint=True)
        else:
            ctx = np.array([1, 15, 16, 17, 300, 1024, 2049, 2500])
        reqs = [(int(c), 1) for c in ctx]
    elif config_id == 3:
        if size == "full":
            reqs = [(32768, 1)] * 32
        else:
            reqs = [(33, 1), (4101, 1), (1, 1), (2048, 1)]
    elif config_id == 4:
        if size == "full":
            prompts = np.rint(np.exp(rng.uniform(math.log(512), math.log(16384), size=16))).astype(np.int64)
            decodes = rng.integers(2048, 32768, size=32, endpoint=True)
        else:
            prompts = np.array([37, 600])
            decodes = np.array([1, 2048, 3001, 50])
        reqs = [(int(p), int(p)) for p in prompts] + [(int(c), 1) for c in decodes]
        order = _rng(ss, _S_ORDER).permutation(len(reqs))
        reqs = [reqs[i] for i in order]
        scheduled = sum(q for _, q in reqs)
        pad = max(1, int(round(0.05 * scheduled)))
    elif config_id == 5:
        ctx = 524288 if size == "full" else 20000
        reqs = [(ctx, 1)]
    else:
        raise ValueError(f"unknown workload {config_id}")
    return reqs, pad


def make_metadata(config_id: int, size: str = "full", seed: int = SEED_BASE) -> Metadata:
    """Build the scheduling metadata of one synthetic step."""
    geom = GEOMETRIES[config_id]
    ss = _seed_seq(config_id, size, seed)
    reqs, pad = _requests(config_id, size, ss)
    bs = geom.block_size
    seq_lens = np.array([c for c, _ in reqs], dtype=np.int32)
    query_lens = np.array([q for _, q in reqs], dtype=np.int32)
    blocks_needed = [(-(-int(c) // bs)) for c in seq_lens]
    total_needed = int(sum(blocks_needed))
    if config_id == 1 and size != "edge":
        num_blocks = 8
    else:
        num_blocks = int(math.ceil(1.25 * total_needed)) + 1
    perm = _rng(ss, _S_PERM).permutation(num_blocks).astype(np.int32)
    used = perm[:total_needed]
    free = perm[total_needed:]
    poison = int(free[0])
    max_blocks = max(1, max(blocks_needed) + 1)    # one spare entry per row
    table = np.full((len(reqs), max_blocks), poison, dtype=np.int32)
    cursor = 0
    for r, nb in enumerate(blocks_needed):
        table[r, :nb] = used[cursor:cursor + nb]
        cursor += nb
    cu = np.zeros(len(reqs) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(query_lens)
    scheduled = int(cu[-1])
    slots = np.full(scheduled + pad, -1, dtype=np.int32)
    for r in range(len(reqs)):
        n, ql = int(seq_lens[r]), int(query_lens[r])
        for i in range(ql):
            pos = n - ql + i            # the newest ql positions of the context
            slots[cu[r] + i] = table[r, pos // bs] * bs + pos % bs
    meta = Metadata(
        config_id=config_id, size=size, geom=geom, seq_lens=seq_lens, query_lens=query_lens,
        cu_seqlens=cu, num_tokens=scheduled + pad, slot_mapping=slots, block_table=table,
        num_blocks=num_blocks, poison_block=poison,
    )
    if config_id == 3:
        meta.outlier_prob, meta.outlier_scale = 0.001, 20.0
    return meta


def make_custom_metadata(geom: Geometry, seq_lens, seed: int = SEED_BASE, spare_table_entries: int = 1,
                         tag: int = 99) -> Metadata:
    """A decode batch of any head geometry: one scheduled token per request
    (none for an empty context), blocks handed out in seeded random order
    from a pool ~1.25x the need, NaN-poisoned spare blocks."""
    ss = np.random.SeedSequence([seed, tag, len(seq_lens)])
    bs = geom.block_size
    seq = np.asarray(seq_lens, dtype=np.int32)
    qlens = (seq > 0).astype(np.int32)
    need = [(-(-int(c) // bs)) for c in seq]
    total = int(sum(need))
    num_blocks = int(math.ceil(1.25 * total)) + 1
    perm = _rng(ss, _S_PERM).permutation(num_blocks).astype(np.int32)
    poison = int(perm[total])
    table = np.full((len(seq), max(1, max(need) + spare_table_entries)), poison, dtype=np.int32)
    cursor = 0
    for r, nb in enumerate(need):
        table[r, :nb] = perm[cursor:cursor + nb]
        cursor += nb
    cu = np.zeros(len(seq) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(qlens)
    slots = np.full(int(cu[-1]), -1, dtype=np.int32)
    for r in range(len(seq)):
        if qlens[r]:
            pos = int(seq[r]) - 1
            slots[cu[r]] = table[r, pos // bs] * bs + pos % bs
    return Metadata(config_id=tag, size="small", geom=geom, seq_lens=seq, query_lens=qlens, cu_seqlens=cu,
                    num_tokens=int(cu[-1]), slot_mapping=slots, block_table=table, num_blocks=num_blocks,
                    poison_block=poison)


def make_varlen_metadata(geom: Geometry, seq_lens, query_lens, seed: int = SEED_BASE, tag: int = 98) -> Metadata:
    """A batch where request r has query_lens[r] query rows (its newest
    positions, as under speculative decoding) over seq_lens[r] cached tokens;
    blocks handed out as in make_custom_metadata.  A request may have more
    rows than cached tokens or none at all."""
    base = make_custom_metadata(geom, seq_lens, seed=seed, tag=tag)
    qlens = np.asarray(query_lens, dtype=np.int32)
    cu = np.zeros(len(qlens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(qlens)
    bs = geom.block_size
    slots = np.full(int(cu[-1]), -1, dtype=np.int32)
    for r in range(len(qlens)):
        n = int(base.seq_lens[r])
        for i in range(int(qlens[r])):
            pos = n - int(qlens[r]) + i
            if pos >= 0:
                slots[cu[r] + i] = base.block_table[r, pos // bs] * bs + pos % bs
    base.query_lens = qlens
    base.cu_seqlens = cu
    base.num_tokens = int(cu[-1])
    base.slot_mapping = slots
    return base


def with_query_rows(meta: Metadata, rows: int) -> Metadata:
    """The same batch with `rows` scheduled tokens per request (its newest
    positions, as a speculative-decoding step appends and verifies them):
    slots for those positions, offsets [0, rows, 2*rows, ...], no padding."""
    bs = meta.geom.block_size
    r = meta.num_reqs
    qlens = np.full(r, rows, dtype=np.int32)
    cu = (np.arange(r + 1) * rows).astype(np.int32)
    slots = np.full(r * rows, -1, dtype=np.int32)
    for i in range(r):
        n = int(meta.seq_lens[i])
        for j in range(rows):
            pos = n - rows + j
            if pos >= 0:
                slots[i * rows + j] = meta.block_table[i, pos // bs] * bs + pos % bs
    return dataclasses.replace(meta, query_lens=qlens, cu_seqlens=cu, num_tokens=r * rows, slot_mapping=slots)


def live_slot_mask(meta: Metadata) -> np.ndarray:
    """bool [num_blocks][block_size]: True for slots inside some context."""
    bs = meta.geom.block_size
    mask = np.zeros((meta.num_blocks, bs), dtype=bool)
    for r in range(meta.num_reqs):
        n = int(meta.seq_lens[r])
        nb = -(-n // bs)
        for b in range(nb):
            phys = int(meta.block_table[r, b])
            mask[phys, : min(bs, n - b * bs)] = True
    return mask


# ---------------------------------------------------------------------------
# Tensors (torch; device memory is where the library reads them)
# ---------------------------------------------------------------------------

def torch_dtype(geom: Geometry):
    import torch
    return torch.float32 if geom.dtype == "f32" else torch.bfloat16


def _generator(device, seed: int):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, dtype, device, seed, std=1.0, chunk_rows=None):
    """N(0, std^2) drawn in fp32 from a seeded generator, then cast to ``dtype``.

    Large tensors are drawn ``chunk_rows`` leading rows at a time from one
    generator, so the values depend only on the seed, the shape and the chunk
    size.
    """
    import torch
    g = _generator(device, seed)
    out = torch.empty(shape, dtype=dtype, device=device)
    rows = shape[0]
    step = rows if chunk_rows is None else chunk_rows
    for start in range(0, rows, step):
        stop = min(rows, start + step)
        part = torch.randn((stop - start,) + tuple(shape[1:]), generator=g, dtype=torch.float32, device=device)
        if std != 1.0:
            part.mul_(std)
        out[start:stop].copy_(part)
    return out


def make_cache(meta: Metadata, device="cpu", seed: int = SEED_BASE):
    """Two cache tensors ``[num_blocks][Hkv][block_size][D]`` in the workload dtype.

    Live slots hold N(0,1) values (key vectors optionally scaled as outliers
    before rounding); free blocks and tail slots hold NaN.
    """
    import torch
    geom = meta.geom
    ss = _seed_seq(meta.config_id, meta.size, seed)
    shape = (meta.num_blocks, geom.num_kv_heads, geom.block_size, geom.head_dim)
    dt = torch_dtype(geom)
    chunk = max(1, (1 << 26) // (geom.num_kv_heads * geom.block_size * geom.head_dim))
    k = torch.empty(shape, dtype=dt, device=device)
    v = torch.empty(shape, dtype=dt, device=device)
    gk = _generator(device, _child_seed(ss, _S_K))
    gv = _generator(device, _child_seed(ss, _S_V))
    go = _generator(device, _child_seed(ss, _S_OUTLIER))
    for start in range(0, meta.num_blocks, chunk):
        stop = min(meta.num_blocks, start + chunk)
        sub = (stop - start,) + shape[1:]
        kk = torch.randn(sub, generator=gk, dtype=torch.float32, device=device)
        if meta.outlier_prob > 0:
            sel = torch.rand(sub[:-1], generator=go, dtype=torch.float32, device=device) < meta.outlier_prob
            kk = torch.where(sel.unsqueeze(-1), kk * meta.outlier_scale, kk)
        k[start:stop].copy_(kk)
        v[start:stop].copy_(torch.randn(sub, generator=gv, dtype=torch.float32, device=device))
    live = torch.from_numpy(live_slot_mask(meta)).to(device)          # [NB][bs]
    dead = (~live).view(meta.num_blocks, 1, geom.block_size, 1)
    k.masked_fill_(dead, float("nan"))
    v.masked_fill_(dead, float("nan"))
    return k, v


def make_fp8_cache(meta: Metadata, device="cpu", seed: int = SEED_BASE):
    """An 8-bit (FP8 E4M3) cache: codes ``uint8 [num_blocks][Hkv][block_size]
    [D]`` and fp32 scales ``[num_blocks][Hkv][block_size]`` for K and for V.
    Live slots hold codes drawn uniformly from the 254 finite codes and
    scales from U(0.002, 0.02) (stored values of magnitude up to ~9); free
    blocks and tail slots hold the NaN code 0x7F and NaN scales."""
    import torch
    geom = meta.geom
    ss = _seed_seq(meta.config_id, meta.size, seed)
    shape = (meta.num_blocks, geom.num_kv_heads, geom.block_size, geom.head_dim)
    live = torch.from_numpy(live_slot_mask(meta)).to(device).view(meta.num_blocks, 1, geom.block_size)
    out = []
    for stream in (_S_K, _S_V):
        g = _generator(device, _child_seed(ss, stream))
        codes = torch.randint(0, 254, shape, generator=g, device=device, dtype=torch.int32)
        codes = torch.where(codes >= 0x7F, codes + 1, codes).to(torch.uint8)         # skip 0x7F; 0xFF is > 253 + 1
        scales = torch.rand(shape[:-1], generator=g, device=device, dtype=torch.float32) * 0.018 + 0.002
        codes.masked_fill_(~live.unsqueeze(-1), 0x7F)
        scales.masked_fill_(~live, float("nan"))
        out += [codes, scales]
    return tuple(out)          # k_codes, k_scale, v_codes, v_scale


def make_queries(meta: Metadata, device="cpu", seed: int = SEED_BASE, num_layers: Optional[int] = None,
                 rows: Optional[int] = None):
    """q for every cross layer: ``[L][rows][Hq][D]`` N(0,1) in the workload
    dtype; rows defaults to one per request."""
    geom = meta.geom
    ss = _seed_seq(meta.config_id, meta.size, seed)
    layers = geom.num_layers if num_layers is None else num_layers
    shape = (layers, meta.num_reqs if rows is None else rows, geom.num_q_heads, geom.head_dim)
    return _randn(shape, torch_dtype(geom), device, _child_seed(ss, _S_Q))


def make_append_inputs(meta: Metadata, device="cpu", seed: int = SEED_BASE, rms_weight: str = "ones"):
    """Inputs of the shared K/V projection.

    x ``[T][hidden]`` ~ N(0,1); W_K, W_V ``[Hkv*D][hidden]`` ~ N(0, 1/hidden);
    RMSNorm weight ones (``rms_weight="ones"``) or U(0.5, 1.5)
    (``"random"``).  All in the workload dtype.
    """
    import torch
    geom = meta.geom
    ss = _seed_seq(meta.config_id, meta.size, seed)
    dt = torch_dtype(geom)
    out_features = geom.num_kv_heads * geom.head_dim
    x = _randn((meta.num_tokens, geom.hidden), dt, device, _child_seed(ss, _S_X), chunk_rows=8192)
    std = 1.0 / math.sqrt(geom.hidden)
    w_k = _randn((out_features, geom.hidden), dt, device, _child_seed(ss, _S_WK), std=std)
    w_v = _randn((out_features, geom.hidden), dt, device, _child_seed(ss, _S_WV), std=std)
    if rms_weight == "ones":
        w = torch.ones(geom.hidden, dtype=dt, device=device)
    else:
        g = _generator(device, _child_seed(ss, _S_RMS))
        w = (torch.rand(geom.hidden, generator=g, dtype=torch.float32, device=device) + 0.5).to(dt)
    return x, w, w_k, w_v


@dataclasses.dataclass
class RetentionInputs:
    """One self-decoder retention layer's inputs for a batch of requests."""
    lens: np.ndarray            # int64 [R] rows per request
    cu_seqlens: np.ndarray      # int32 [R + 1]
    state_indices: np.ndarray   # int32 [R] (distinct; -1 = start from zeros)
    q: object                   # bf16 [T][H][D]
    k: object                   # bf16 [T][H][D], drawn with std D^-1/2
    v: object                   # bf16 [T][H][D]
    gamma: object               # fp32 [T][H], uniform in gamma_range
    state: object               # fp32 [slots][H][D][D], N(0, 1/D)


def retention_lengths(name: str, seed: int = SEED_BASE) -> np.ndarray:
    """Rows per request of a retention workload: "mixed48" is the mixed step's
    request mix (16 prefills, prompts log-uniform in [512, 16384], and 32
    one-token decodes); "decode64" is 64 one-token decodes."""
    if name == "mixed48":
        meta = make_metadata(4, "full", seed)
        return np.diff(meta.cu_seqlens).astype(np.int64)
    if name == "decode64":
        return np.ones(64, dtype=np.int64)
    raise ValueError(name)


def make_retention_inputs(lens, num_heads: int, head_dim: int, device="cpu", seed: int = SEED_BASE,
                          gamma_range=(0.85, 1.0), num_slots: Optional[int] = None, zero_state_every: int = 0,
                          tag: int = 77) -> RetentionInputs:
    """Seeded q, k, v (bf16), gates, initial states and slot numbers for the
    requests' rows ``lens``.  Slots are a random injective map into
    ``num_slots`` (default 1.25x the requests); with ``zero_state_every`` = m,
    every m-th request gets slot -1 (it starts from a zero state)."""
    import torch
    lens = np.asarray(lens, dtype=np.int64)
    num_reqs = len(lens)
    ss = np.random.SeedSequence([seed, tag, num_reqs, num_heads, head_dim])
    rng = _rng(ss, 0)
    cu = np.zeros(num_reqs + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    total = int(cu[-1])
    slots = num_slots if num_slots is not None else max(1, (5 * num_reqs + 3) // 4)
    idx = rng.permutation(slots)[:num_reqs].astype(np.int32)
    if zero_state_every > 0:
        idx[::zero_state_every] = -1
    shape = (total, num_heads, head_dim)
    bf = torch.bfloat16
    chunk = 1 << 14
    q = _randn(shape, bf, device, _child_seed(ss, 1), chunk_rows=chunk)
    k = _randn(shape, bf, device, _child_seed(ss, 2), std=head_dim ** -0.5, chunk_rows=chunk)
    v = _randn(shape, bf, device, _child_seed(ss, 3), chunk_rows=chunk)
    lo, hi = gamma_range
    g = _generator(device, _child_seed(ss, 4))
    gamma = torch.rand((total, num_heads), generator=g, dtype=torch.float32, device=device).mul_(hi - lo).add_(lo)
    state = _randn((slots, num_heads, head_dim, head_dim), torch.float32, device, _child_seed(ss, 5),
                   std=head_dim ** -0.5, chunk_rows=64)
    return RetentionInputs(lens, cu, idx, q, k, v, gamma, state)


def describe(meta: Metadata) -> dict:
    """Small JSON-able summary of a workload."""
    return {
        "workload": meta.geom.name,
        "config_id": meta.config_id,
        "size": meta.size,
        "num_reqs": meta.num_reqs,
        "num_tokens": meta.num_tokens,
        "context_tokens": int(meta.seq_lens.sum()),
        "max_seq_len": meta.max_seq_len,
        "num_q_heads": meta.geom.num_q_heads,
        "num_kv_heads": meta.geom.num_kv_heads,
        "head_dim": meta.geom.head_dim,
        "block_size": meta.geom.block_size,
        "num_layers": meta.geom.num_layers,
        "hidden": meta.geom.hidden,
        "dtype": meta.geom.dtype,
    }


def config_ids() -> List[int]:
    return sorted(GEOMETRIES)
