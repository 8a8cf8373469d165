"""yoco_cross_attn on head geometries and block sizes the five workloads do not
use: every supported head_dim, group size (query heads per KV head) and dtype,
block sizes from 1 to 256, contexts that end on and just past block and
partition boundaries, an empty context, and out-of-range block ids."""

import math

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import ATTN_ATOL, dev, host, say
from yoco_shared_kv_gather_amd import binding as yb
from yoco_shared_kv_gather_amd import synth

pytestmark = pytest.mark.gpu

CTX = [0, 1, 63, 64, 65, 127, 128, 129, 300]


def _run(geom, ctx, partition_tokens, seed=7):
    meta = synth.make_custom_metadata(geom, ctx, seed=seed)
    d = dev()
    k, v = synth.make_cache(meta, d, seed)
    q = synth.make_queries(meta, d, seed, num_layers=1)[0]
    table = torch.from_numpy(meta.block_table).to(d)
    seq = torch.from_numpy(meta.seq_lens).to(d)
    out = yb.cross_attn(q, k, v, table, seq, meta.max_seq_len, partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    ref = oracle.cross_attention(host(q), host(k), host(v), meta.block_table, meta.seq_lens,
                                 1.0 / math.sqrt(geom.head_dim))
    got = host(out)
    assert np.isfinite(got).all()
    return float(np.abs(got - ref).max())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("head_dim", [64, 128, 256])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_head_geometries(dtype, head_dim, group):
    geom = synth.custom_geometry(dtype, 2 * group, 2, head_dim, 16)
    for part in (0, 64):
        say(f"shapes: {dtype} D={head_dim} G={group} partition {part}")
        err = _run(geom, CTX, part)
        assert err <= ATTN_ATOL, err


@pytest.mark.parametrize("block_size", [1, 2, 8, 32, 64, 128, 256])
def test_block_sizes(block_size):
    geom = synth.custom_geometry("bf16", 8, 2, 128, block_size)
    for part in (0, 64, 192):
        say(f"shapes: block size {block_size} partition {part}")
        err = _run(geom, CTX + [block_size - 1, block_size, block_size + 1, 3 * block_size + 5], part)
        assert err <= ATTN_ATOL, err


@pytest.mark.parametrize("lost_blocks", [(1, 2), (0,), (0, 1, 2, 3, 4, 5, 6)])
def test_out_of_range_block_ids_are_skipped(lost_blocks):
    """A table entry outside [0, num_blocks) inside a context is a broken
    precondition: the kernel must stay in bounds, leave those tokens out of
    the softmax wherever the entry sits (inside a partition, at the start of
    one, or every entry of the context: a zero row), and leave the other
    requests' outputs exact.  Free blocks hold NaN, so a masked row that
    leaked into the sums would show."""
    say(f"shapes: out-of-range block ids at {lost_blocks} of request 0")
    geom = synth.custom_geometry("bf16", 8, 2, 128, 16)
    meta = synth.make_custom_metadata(geom, [100, 40, 70], seed=3)
    d = dev()
    k, v = synth.make_cache(meta, d, 3)
    q = synth.make_queries(meta, d, 3, num_layers=1)[0]
    bad = meta.block_table.copy()
    for i, b in enumerate(lost_blocks):
        bad[0, b] = meta.num_blocks + 5 if i % 2 == 0 else -3
    table = torch.from_numpy(bad).to(d)
    seq = torch.from_numpy(meta.seq_lens).to(d)
    scale = 1.0 / math.sqrt(geom.head_dim)
    keep = np.ones(100, dtype=bool)
    for b in lost_blocks:
        keep[16 * b:16 * (b + 1)] = False
    kk, vv = oracle.logical_kv(host(k), host(v), meta.block_table[0], 100)
    for part in (0, 64):
        out = host(yb.cross_attn(q, k, v, table, seq, meta.max_seq_len, partition_tokens=part))
        torch.cuda.synchronize()
        ref = oracle.cross_attention(host(q), host(k), host(v), meta.block_table, meta.seq_lens, scale)
        assert np.isfinite(out).all()
        np.testing.assert_allclose(out[1:], ref[1:], atol=ATTN_ATOL, rtol=0)
        # request 0 equals attention over its remaining tokens (none: zeros)
        for h in range(geom.num_q_heads):
            g = h // 4
            if keep.any():
                r0 = oracle.attention_one_query(host(q)[0, h], kk[keep, g], vv[keep, g], scale)
            else:
                r0 = np.zeros(geom.head_dim)
            np.testing.assert_allclose(out[0, h], r0, atol=ATTN_ATOL, rtol=0)


def test_seq_lens_beyond_the_table_are_clamped():
    """seq_lens larger than max_blocks*block_size (or than max_seq_len) are
    clamped to what the table covers; no read leaves the table row."""
    say("shapes: seq_lens clamped to the table")
    geom = synth.custom_geometry("bf16", 4, 1, 128, 16)
    meta = synth.make_custom_metadata(geom, [40, 33], seed=5, spare_table_entries=0)
    d = dev()
    k, v = synth.make_cache(meta, d, 5)
    q = synth.make_queries(meta, d, 5, num_layers=1)[0]
    table = torch.from_numpy(meta.block_table).to(d)
    cap = meta.block_table.shape[1] * geom.block_size          # 48
    seq_big = torch.tensor([10_000, 33], dtype=torch.int32, device=d)
    out = host(yb.cross_attn(q, k, v, table, seq_big, cap, partition_tokens=64))
    torch.cuda.synchronize()
    live = synth.live_slot_mask(meta)
    assert live.sum() == 73
    # request 0 reads all 48 table slots: the 8 past its context hold NaN
    assert np.isnan(out[0]).all()
    ref = oracle.cross_attention(host(q), host(k), host(v), meta.block_table, meta.seq_lens,
                                 1.0 / math.sqrt(geom.head_dim))
    np.testing.assert_allclose(out[1], ref[1], atol=ATTN_ATOL, rtol=0)
