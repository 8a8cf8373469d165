"""yoco_cross_attn on the GPU against the float64 oracle.

Small and edge workloads are compared element by element on every output;
full-size workloads, in the launch configuration the benchmark uses, on every
output of two layers.  Tolerance: 2e-3 absolute on every output.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import ATTN_ATOL, DeviceWorkload, dev, host, oracle_attention_full, say
from yoco_shared_kv_gather_amd import binding as yb
from yoco_shared_kv_gather_amd import synth

pytestmark = pytest.mark.gpu


def _max_err(got, ref):
    got = got.detach().cpu().double().numpy()
    assert np.isfinite(got).all()
    return float(np.abs(got - ref).max()) if got.size else 0.0


@pytest.mark.parametrize("cid,size", [(1, "full"), (2, "small"), (3, "small"), (4, "small"), (5, "small"),
                                      (1, "edge"), (2, "edge"), (3, "edge")])
@pytest.mark.parametrize("partition_tokens", [0, 64])
@pytest.mark.parametrize("kernel", ["default", "vector"])
def test_parity_small(cid, size, partition_tokens, kernel):
    """Every output, with the kernel the library picks (the vector kernel, or
    the matrix-core kernel at head_dim 256) and with the vector kernel forced."""
    say(f"cross_attn parity: workload {cid} {size} partition {partition_tokens} {kernel}")
    w = DeviceWorkload(cid, size, layers=2)
    force = yb.FLAG_VECTOR_KERNEL if kernel == "vector" else 0
    for layer in range(2):
        out = w.attn(layer, partition_tokens=partition_tokens, flags=(layer & 1) | force)
        torch.cuda.synchronize()
        ref = oracle_attention_full(w, layer)
        err = _max_err(out, ref)
        say(f"  layer {layer}: max abs err {err:.3e}")
        assert err <= ATTN_ATOL


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_parity_full_size_every_output(cid):
    """Full-size workloads in the benchmark's launch configuration (default
    partitions; layer 0 in the default work order, layer 1 reversed): every
    output of both layers -- each request, each query head -- against the
    oracle, fetching one request's blocks at a time."""
    say(f"cross_attn full size, every output: workload {cid}")
    w = DeviceWorkload(cid, "full", layers=2)
    meta, geom = w.meta, w.geom
    outs = [w.attn(layer, flags=layer & 1).cpu().double().numpy() for layer in range(2)]
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(geom.head_dim)
    bs = geom.block_size
    worst = 0.0
    for r in range(meta.num_reqs):
        n = int(meta.seq_lens[r])
        nb = -(-n // bs)
        blocks = torch.from_numpy(meta.block_table[r, :max(nb, 1)].astype(np.int64)).to(dev())
        kc = host(w.k.index_select(0, blocks))                       # [nb][Hkv][bs][D], table order
        vc = host(w.v.index_select(0, blocks))
        for layer in range(2):
            ref = oracle.cross_attention(host(w.q[layer, r:r + 1]), kc, vc, np.arange(max(nb, 1))[None, :],
                                         np.array([n]), scale)[0]
            assert np.isfinite(outs[layer][r]).all()
            worst = max(worst, float(np.abs(outs[layer][r] - ref).max()))
        assert worst <= ATTN_ATOL, (r, worst)
    say(f"  {meta.num_reqs} requests x {geom.num_q_heads} heads x 2 layers: max abs err {worst:.3e}")


def test_deterministic_and_order_independent():
    say("cross_attn determinism: workload 2 small, partitions of 64, both orders")
    w = DeviceWorkload(2, "small", layers=1)
    a = w.attn(0, partition_tokens=64, flags=0).clone()
    b = w.attn(0, partition_tokens=64, flags=0).clone()
    c = w.attn(0, partition_tokens=64, flags=yb.FLAG_REVERSE_ORDER).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(a.view(torch.int32), c.view(torch.int32))


def test_block_table_permutation_gives_same_bits():
    """Moving every physical block (and its table entries) leaves the output
    unchanged bit for bit."""
    say("cross_attn: physical block permutation")
    w = DeviceWorkload(4, "small", layers=1)
    a = w.attn(0, partition_tokens=128).clone()
    perm = torch.randperm(w.meta.num_blocks, generator=torch.Generator().manual_seed(5)).to(w.k.device)
    k2 = torch.empty_like(w.k)
    v2 = torch.empty_like(w.v)
    k2[perm] = w.k
    v2[perm] = w.v
    table2 = perm[w.block_table.long()].to(torch.int32)
    b = yb.cross_attn(w.q[0], k2, v2, table2, w.seq_lens, w.meta.max_seq_len, partition_tokens=128)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_many_partitions_long_context():
    """One request split into more than 256 partitions (the merge kernel's
    multi-wave path) still matches."""
    say("cross_attn: 313 partitions on workload 5 small")
    w = DeviceWorkload(5, "small", layers=1)
    out = w.attn(0, partition_tokens=64)
    torch.cuda.synchronize()
    ref = oracle_attention_full(w, 0)
    err = _max_err(out, ref)
    say(f"  max abs err {err:.3e}")
    assert err <= ATTN_ATOL


def _custom(geom, ctx, seed):
    meta = synth.make_custom_metadata(geom, ctx, seed=seed)
    d = dev()
    k, v = synth.make_cache(meta, d, seed)
    q = synth.make_queries(meta, d, seed, num_layers=1)[0]
    table = torch.from_numpy(meta.block_table).to(d)
    seq = torch.from_numpy(meta.seq_lens).to(d)
    return meta, q, k, v, table, seq


def _oracle(meta, q, k, v):
    return oracle.cross_attention(host(q), host(k), host(v), meta.block_table, meta.seq_lens,
                                  1.0 / math.sqrt(meta.geom.head_dim))


def test_queue_counters_left_zero_between_calls():
    """The persistent schedule's work-queue counters are zero again after each
    call, so one workspace serves call after call with the same bits."""
    say("cross_attn: work-queue counters across calls on one workspace")
    w = DeviceWorkload(2, "small", layers=1)
    g = w.geom
    need = yb.cross_attn_workspace_size(w.meta.num_reqs, g.num_q_heads, g.num_kv_heads, g.head_dim,
                                        w.meta.max_seq_len, g.block_size, 64)
    ws = torch.zeros(need, dtype=torch.uint8, device=w.k.device)
    ref = oracle_attention_full(w, 0)
    first = None
    for i in range(4):
        out = yb.cross_attn(w.q[0], w.k, w.v, w.block_table, w.seq_lens, w.meta.max_seq_len, partition_tokens=64,
                            flags=i & 1, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[:yb.CROSS_ATTN_QUEUE_BYTES].count_nonzero()) == 0
        assert _max_err(out, ref) <= ATTN_ATOL
        if first is None:
            first = out.clone()
        assert torch.equal(first.view(torch.int32), out.view(torch.int32))


@pytest.mark.parametrize("ctx", [[5], [5, 0, 17], [0], [0, 0, 1]])
@pytest.mark.parametrize("head_dim", [128, 256])
def test_fewer_work_items_than_queues(ctx, head_dim):
    """One to three work items: the grid shrinks to the item count and only
    that many queues are used (vector kernel at head_dim 128, matrix-core
    kernel with four head_dim slices at 256)."""
    say(f"cross_attn: contexts {ctx} with one KV head, head_dim {head_dim}")
    geom = synth.custom_geometry("bf16", 4, 1, head_dim, 16)
    meta, q, k, v, table, seq = _custom(geom, ctx, seed=11)
    out = yb.cross_attn(q, k, v, table, seq, meta.max_seq_len)
    torch.cuda.synchronize()
    assert _max_err(out, _oracle(meta, q, k, v)) <= ATTN_ATOL


@pytest.mark.parametrize("num_reqs", [2048, 2049])
@pytest.mark.parametrize("head_dim", [64, 256])
def test_request_count_at_the_schedule_switch(num_reqs, head_dim):
    """2048 requests fill the persistent schedule's prefix exactly; one more
    takes the one-workgroup-per-item schedule (at head_dim 256 also the
    switch from the matrix-core kernel to the vector kernel).  Both match
    the oracle."""
    say(f"cross_attn: {num_reqs} requests, head_dim {head_dim}")
    rng = np.random.default_rng(num_reqs)
    ctx = [int(c) for c in rng.integers(0, 48, size=num_reqs)]
    geom = synth.custom_geometry("bf16", 2, 1, head_dim, 16)
    meta, q, k, v, table, seq = _custom(geom, ctx, seed=13)
    ref = _oracle(meta, q, k, v)
    # a max_seq_len far past what the table rows span: partitions beyond the
    # rows must not touch the table
    for max_len in (meta.max_seq_len, 40 * meta.max_seq_len):
        for part in (0, 64):
            out = yb.cross_attn(q, k, v, table, seq, max_len, partition_tokens=part)
            torch.cuda.synchronize()
            err = _max_err(out, ref)
            say(f"  max_seq_len {max_len} partition {part}: max abs err {err:.3e}")
            assert err <= ATTN_ATOL


def test_tail_pieces_every_output_both_orders():
    """A batch whose default split ends every context in tail pieces (full
    partitions of P tokens, then the last T or more tokens in pieces of P/4),
    with contexts from 1 to 4096 tokens: every output against the oracle, and
    the reverse order -- the full partitions and the pieces each reversed,
    the pieces still last -- gives the same bits."""
    rng = np.random.default_rng(77)
    ctx = [4096] * 4 + [int(c) for c in rng.integers(1, 4097, size=28)]
    geom = synth.custom_geometry("bf16", 32, 8, 128, 16)
    meta, q, k, v, table, seq = _custom(geom, ctx, seed=21)
    P, Ps, T, most = yb.cross_attn_partition_split(len(ctx), 8, 128, meta.max_seq_len, 16)
    say(f"cross_attn: 32 requests up to 4096 tokens, P {P}, pieces of {Ps} over the last {T}")
    assert T > 0 and Ps < P
    ref = _oracle(meta, q, k, v)
    a = yb.cross_attn(q, k, v, table, seq, meta.max_seq_len)
    b = yb.cross_attn(q, k, v, table, seq, meta.max_seq_len, flags=yb.FLAG_REVERSE_ORDER)
    torch.cuda.synchronize()
    err = _max_err(a, ref)
    say(f"  max abs err {err:.3e}")
    assert err <= ATTN_ATOL
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("mode", ["fp8", "several_rows", "fp8_matrix"])
def test_tail_pieces_varlen_both_orders(mode):
    """Tail pieces through yoco_cross_attn_varlen: on the vector-ALU kernel
    (forced with YOCO_FLAG_VECTOR_KERNEL) with an FP8 cache and one row per
    request, or a bf16 cache with up to four rows per request; and on the
    matrix-core kernel with an FP8 cache (8 requests up to 32K tokens, whose
    split there has pieces).  Every output against the oracle, and both
    orders give the same bits."""
    rng = np.random.default_rng(79)
    if mode == "fp8_matrix":
        ctx = [32768, 32768] + [int(c) for c in rng.integers(1, 32769, size=6)]
    else:
        ctx = [4096] * 4 + [int(c) for c in rng.integers(1, 4097, size=28)]
    force = 0 if mode == "fp8_matrix" else yb.FLAG_VECTOR_KERNEL
    qlens = [min(c, 1 + i % 4) for i, c in enumerate(ctx)] if mode == "several_rows" else [1] * len(ctx)
    geom = synth.custom_geometry("bf16", 32, 8, 128, 16)
    meta = synth.make_varlen_metadata(geom, ctx, qlens, seed=23)
    d = dev()
    rows = int(meta.cu_seqlens[-1])
    q = synth.make_queries(meta, d, 23, num_layers=1, rows=rows)[0]
    table = torch.from_numpy(meta.block_table).to(d)
    seq = torch.from_numpy(meta.seq_lens).to(d)
    qsl = torch.from_numpy(meta.cu_seqlens).to(d)
    ql = max(qlens)
    if mode.startswith("fp8"):
        kc, ks, vc, vs = synth.make_fp8_cache(meta, d, 23)
        kd = oracle.dequantize_cache(kc.cpu().numpy(), ks.cpu().numpy())
        vd = oracle.dequantize_cache(vc.cpu().numpy(), vs.cpu().numpy())
        dtype, extra = yb.DTYPE_FP8_E4M3, dict(k_scale=ks, v_scale=vs)
    else:
        kc, vc = synth.make_cache(meta, d, 23)
        kd, vd = host(kc), host(vc)
        dtype, extra = yb.DTYPE_BF16, {}
    P, Ps, T, most = yb.cross_attn_partition_split(len(ctx), 8, 128, meta.max_seq_len, 16, 0, dtype, ql, 0, force)
    say(f"cross_attn_varlen {mode}: P {P}, pieces of {Ps} over the last {T}")
    assert T > 0 and Ps < P
    ref = oracle.cross_attention_varlen(host(q), kd, vd, meta.block_table, meta.seq_lens, meta.cu_seqlens,
                                        1.0 / math.sqrt(128), 0)
    outs = [yb.cross_attn_varlen(q, kc, vc, table, seq, meta.max_seq_len, query_start_loc=qsl, max_query_len=ql,
                                 flags=force | f, **extra) for f in (0, yb.FLAG_REVERSE_ORDER)]
    torch.cuda.synchronize()
    err = _max_err(outs[0], ref)
    say(f"  max abs err {err:.3e}")
    assert err <= ATTN_ATOL
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))


@pytest.mark.parametrize("several", [False, True])
def test_matrix_kernel_many_items_both_orders(several):
    """The matrix-core kernel with more work items than resident workgroups
    (FP8 cache, 32 requests x 8 KV heads up to 4096 tokens, some contexts
    empty), so every workgroup hands items over with the next item's first
    tile already requested: every output against the oracle over the
    dequantized cache, and the reverse order gives the same bits."""
    rng = np.random.default_rng(78)
    ctx = [4096, 0, 4096, 1] + [int(c) for c in rng.integers(0, 4097, size=28)]
    qlens = [min(c, 1 + i % 4) for i, c in enumerate(ctx)] if several else [1 if c > 0 else 0 for c in ctx]
    geom = synth.custom_geometry("bf16", 32, 8, 128, 16)
    meta = synth.make_varlen_metadata(geom, ctx, qlens, seed=22)
    d = dev()
    kc, ks, vc, vs = synth.make_fp8_cache(meta, d, 22)
    rows = int(meta.cu_seqlens[-1])
    q = synth.make_queries(meta, d, 22, num_layers=1, rows=rows)[0]
    table = torch.from_numpy(meta.block_table).to(d)
    seq = torch.from_numpy(meta.seq_lens).to(d)
    qsl = torch.from_numpy(meta.cu_seqlens).to(d)
    ql = max(qlens)
    say(f"cross_attn_varlen FP8: 32 requests up to 4096 tokens, up to {ql} rows each")
    kd = oracle.dequantize_cache(kc.cpu().numpy(), ks.cpu().numpy())
    vd = oracle.dequantize_cache(vc.cpu().numpy(), vs.cpu().numpy())
    ref = oracle.cross_attention_varlen(host(q), kd, vd, meta.block_table, meta.seq_lens, meta.cu_seqlens,
                                        1.0 / math.sqrt(128), 0)
    outs = [yb.cross_attn_varlen(q, kc, vc, table, seq, meta.max_seq_len, query_start_loc=qsl, max_query_len=ql,
                                 k_scale=ks, v_scale=vs, flags=f) for f in (0, yb.FLAG_REVERSE_ORDER)]
    torch.cuda.synchronize()
    err = _max_err(outs[0], ref)
    say(f"  max abs err {err:.3e}")
    assert err <= ATTN_ATOL
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))


@pytest.mark.gpu
def test_kernel_query_names_the_kernel_that_runs():
    """yoco_cross_attn_kernel names the kernel a call launches, checked through
    the results on decode64's full size (bf16 at head_dim 256): where it
    reports the vector ALUs, forcing the vector kernel gives the same bits;
    where it reports the matrix cores, the outputs differ (the kernels sum in
    different orders), and both agree with the oracle."""
    w = DeviceWorkload(2, "full", layers=1)
    g = w.geom
    for window in (0, 512):
        kind = yb.cross_attn_kernel(w.meta.num_reqs, g.num_kv_heads, g.head_dim, w.meta.max_seq_len, g.block_size,
                                    dtype=yb.DTYPE_BF16, window=window)
        say(f"decode64 full, window {window}: {kind} kernel")

        def run(flags):
            if window == 0:
                return w.attn(0, flags=flags)
            return yb.cross_attn_varlen(w.q[0], w.k, w.v, w.block_table, w.seq_lens, w.meta.max_seq_len,
                                        window=window, flags=flags)

        default, forced = run(0), run(yb.FLAG_VECTOR_KERNEL)
        torch.cuda.synchronize()
        assert kind == ("matrix" if window == 0 else "vector")
        assert torch.equal(default, forced) == (kind == "vector")
        ref = oracle.cross_attention_varlen(host(w.q[0]), host(w.k), host(w.v), w.meta.block_table,
                                            w.meta.seq_lens, np.arange(w.meta.num_reqs + 1),
                                            1.0 / math.sqrt(g.head_dim), window)
        for out in (default, forced):
            assert _max_err(out, ref) <= ATTN_ATOL
