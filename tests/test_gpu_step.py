"""One whole step of the hot path on the tiny workload (fp32): append the
scheduled tokens, gather the last rows, run every cross layer; compared with
the oracle run the same way from the same inputs."""

import math

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import ATTN_ATOL, DeviceWorkload, host, say
from yoco_shared_kv_gather_amd import binding as yb

pytestmark = pytest.mark.gpu


def test_tiny_step_chain():
    say("step: workload 1, append -> gather -> 8 cross layers")
    w = DeviceWorkload(1, "full", with_append=True)
    meta, geom = w.meta, w.geom
    k_host, v_host = host(w.k), host(w.v)
    yb.kv_append(w.x, w.w_rms, 1e-6, w.w_k, w.w_v, w.slot_mapping, w.k, w.v)
    rows, idx = yb.gather_last(w.x, w.cu_seqlens)
    outs = [w.attn(l) for l in range(geom.num_layers)]
    torch.cuda.synchronize()

    kc, vc = oracle.kv_append(host(w.x), host(w.w_rms), 1e-6, host(w.w_k), host(w.w_v), meta.slot_mapping,
                              k_host, v_host)
    rref, iref = oracle.gather_last(host(w.x), meta.cu_seqlens)
    assert np.array_equal(idx.cpu().numpy(), iref) and np.array_equal(host(rows), rref)
    scale = 1.0 / math.sqrt(geom.head_dim)
    for l in range(geom.num_layers):
        ref = oracle.cross_attention(host(w.q[l]), kc, vc, meta.block_table, meta.seq_lens, scale)
        err = float(np.abs(host(outs[l]) - ref).max())
        say(f"  layer {l}: max abs err {err:.3e}")
        assert err <= ATTN_ATOL


def _step_buffers(w, q_rows):
    """Preallocated outputs and workspaces of one decode step (a captured
    graph must not allocate)."""
    g = w.geom
    d = w.k.device
    code = yb.DTYPE_BF16 if g.dtype == "bf16" else yb.DTYPE_F32
    return dict(
        outs=torch.empty((g.num_layers, q_rows, g.num_q_heads, g.head_dim), dtype=torch.float32, device=d),
        rows=torch.empty((w.meta.num_reqs, g.hidden), dtype=w.x.dtype, device=d),
        idx=torch.empty(w.meta.num_reqs, dtype=torch.int32, device=d),
        ws=torch.zeros(yb.cross_attn_workspace_size(w.meta.num_reqs, g.num_q_heads, g.num_kv_heads, g.head_dim,
                                                    w.meta.max_seq_len, g.block_size, 64), dtype=torch.uint8, device=d),
        ws_append=torch.zeros(max(16, yb.kv_append_workspace_size(code, g.hidden, g.num_kv_heads, g.head_dim)),
                              dtype=torch.uint8, device=d),
    )


@pytest.mark.parametrize("cid", [2, 4])
def test_step_in_a_hip_graph(cid):
    """A whole step (append, gather, every cross layer, split into partitions
    so the merge kernel and the work-queue counters are used) captured in a
    HIP graph and replayed three times, with other eager work between the
    replays: every replay gives the eager step's bits (the calls allocate
    nothing, write no memsets, and leave the queue counters at zero)."""
    say(f"step in a HIP graph: workload {cid} small")
    w = DeviceWorkload(cid, "small", with_append=True)
    layers = w.geom.num_layers
    k0, v0 = w.k.clone(), w.v.clone()
    b = _step_buffers(w, w.meta.num_reqs)
    stream = torch.cuda.Stream()

    def step():
        s = torch.cuda.current_stream()
        yb.kv_append(w.x, w.w_rms, 1e-6, w.w_k, w.w_v, w.slot_mapping, w.k, w.v, workspace=b["ws_append"], stream=s)
        yb.gather_last(w.x, w.cu_seqlens, out=b["rows"], out_index=b["idx"], stream=s)
        for l in range(layers):
            yb.cross_attn(w.q[l], w.k, w.v, w.block_table, w.seq_lens, w.meta.max_seq_len, partition_tokens=64,
                          flags=l & 1, out=b["outs"][l], workspace=b["ws"], stream=s)

    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    eager_out, eager_rows = b["outs"].clone(), b["rows"].clone()
    eager_k = w.k.clone()

    graph = torch.cuda.CUDAGraph()
    w.k.copy_(k0)
    w.v.copy_(v0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        step()
    for replay in range(3):
        b["outs"].fill_(float("nan"))
        b["rows"].zero_()
        w.k.copy_(k0)
        w.v.copy_(v0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(b["outs"].view(torch.int32), eager_out.view(torch.int32)), replay
        assert torch.equal(b["rows"].view(torch.uint8), eager_rows.view(torch.uint8)), replay
        assert torch.equal(w.k.view(torch.uint8), eager_k.view(torch.uint8)), replay   # NaN-poisoned slots: compare bytes
        assert int(b["ws"][:yb.CROSS_ATTN_QUEUE_BYTES].count_nonzero()) == 0
        # eager work on the default stream between replays
        yb.cross_attn(w.q[0], w.k, w.v, w.block_table, w.seq_lens, w.meta.max_seq_len, partition_tokens=64)
        torch.cuda.synchronize()
    say("  3 replays identical to the eager step")
