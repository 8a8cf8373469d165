"""Host replay of the matrix-core attention kernel's row addressing (no GPU).

The kernel streams 16-key tiles of each work item from 16-aligned positions;
a tile past the item's end reads a stand-in tile (masked) so that its loads
need no branch.  This test repeats that index arithmetic for every item of
windowed and unwindowed batches (partition sizes from the library itself) and
checks that every row a tile touches -- K and V rows, and the FP8 scale rows
at the same indices -- lies inside the (block, KV head) slice it starts in,
hence inside a cache of exactly num_blocks * Hkv * block_size rows.  It also
shows that the earlier stand-in (the item's own first key, not 16-aligned)
leaves that slice on the same batches.
"""

import numpy as np
import pytest

from yoco_shared_kv_gather_amd import binding as yb

WAVES = 4                      # wavefronts per workgroup
MAX_SLICE = 512                # block-table entries one item may span


def keys_per_iteration(elem_bytes, head_dim):
    if elem_bytes == 2 and head_dim == 256:
        return 32                  # the four head_dim slices of a workgroup share 32-key iterations
    budget = 4096 if elem_bytes == 1 else 8192
    n = budget // (2 * head_dim * elem_bytes)
    return min(max(n, 16), 64)


def range_lo(n, ql, window):
    return 0 if window <= 0 else max(n - ql - window + 1, 0)


def partitions(m, split):
    """(start, length) of every partition of a key range of m tokens under the
    library's split (P, Ps, T): full partitions of P tokens, then the rest in
    pieces of Ps tokens."""
    P, Ps, T = split
    big = (m - T) // P if m > T else 0
    rest = m - big * P
    small = 1 if m <= 0 else -(-rest // Ps)
    return [(p * P, P) if p < big else (big * P + (p - big) * Ps, Ps) for p in range(big + small)]


def tiles_of_batch(seq_lens, ql, window, split, bs, num_kv_heads, nk, aligned_standin=True):
    """Yield (first row, slice entry, entries in slice, row within block) of
    every 16-row tile load of every item, as the kernel computes them."""
    shift = bs.bit_length() - 1
    for n in seq_lens:
        lo = range_lo(n, ql, window)
        for off, size in partitions(n - lo, split):
            start = lo + off
            end = min(start + size, n)
            if end <= start:
                continue
            first_blk = start >> shift
            num_blk = ((end - 1) >> shift) - first_blk + 1
            base0 = start & ~15
            iters = -(-(end - base0) // nk)
            # each wavefront also requests the iteration after its last one
            for it in range(iters + 2 * WAVES):
                for t in range(nk // 16):
                    p0 = base0 + it * nk + 16 * t
                    if p0 < end:
                        pos = p0
                    else:
                        pos = (start & ~15) if aligned_standin else start
                    yield pos & (bs - 1), (pos >> shift) - first_blk, num_blk


BATCHES = [
    # (seq_lens, query rows per request, window, block size, elem bytes, head_dim)
    ([300, 40, 700, 5, 129, 2049], 1, 37, 16, 2, 128),
    ([300, 40, 700, 5, 129, 2049], 4, 100, 16, 1, 128),
    ([1000, 17, 64, 65], 3, 1, 32, 2, 64),
    ([5000, 33], 1, 1000, 16, 1, 256),
    ([5000, 33, 1, 700], 1, 1000, 16, 2, 256),
    ([8192, 1024, 77], 4, 0, 16, 2, 256),
    ([524288], 1, 8192, 32, 2, 128),
    ([32768] * 4, 4, 0, 16, 2, 128),
]


@pytest.mark.parametrize("seq_lens,ql,window,bs,eb,d", BATCHES)
def test_every_tile_stays_in_its_block(seq_lens, ql, window, bs, eb, d):
    hkv = 8
    span = max(seq_lens) if window <= 0 else min(max(seq_lens), window + ql - 1)
    dtype = yb.DTYPE_FP8_E4M3 if eb == 1 else yb.DTYPE_BF16
    P, Ps, T, _ = yb.cross_attn_partition_split(len(seq_lens), hkv, d, max(seq_lens), bs, 0, dtype, ql, window)
    assert P > 0 and P % 64 == 0 and Ps % 64 == 0 and 0 < Ps <= P and T >= 0
    nk = keys_per_iteration(eb, d)
    for row, entry, entries in tiles_of_batch(seq_lens, ql, window, (P, Ps, T), bs, hkv, nk):
        assert 0 <= entry < entries <= MAX_SLICE
        assert row % 16 == 0 and row + 15 < bs


def test_unaligned_standin_would_leave_the_block():
    """With the item's own start as the stand-in, a windowed batch has tiles
    whose 16 rows run past the end of their block."""
    seq_lens, ql, window, bs, eb, d = BATCHES[0]
    split = yb.cross_attn_partition_split(len(seq_lens), 8, d, max(seq_lens), bs, 0,
                                          yb.DTYPE_FP8_E4M3 if eb == 1 else yb.DTYPE_BF16, ql, window)[:3]
    rows = [row for row, _, _ in tiles_of_batch(seq_lens, ql, window, split, bs, 8, keys_per_iteration(eb, d),
                                                aligned_standin=False)]
    assert max(rows) + 15 >= bs
