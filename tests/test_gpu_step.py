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
