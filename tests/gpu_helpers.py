"""Shared pieces of the GPU parity tests: device workloads, host copies for the
float64 oracle, and the tolerances."""

from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from yoco_shared_kv_gather_amd import binding as yb
from yoco_shared_kv_gather_amd import synth

U_BF16 = 2.0 ** -8      # unit roundoff of bf16 (8 significant bits, nearest even)
U_F32 = 2.0 ** -24      # unit roundoff of fp32
ATTN_ATOL = 2e-3        # cross-attention tolerance, fp32 outputs (bf16 or fp32 K/V)


def dev():
    return torch.device("cuda", 0)


def say(msg):
    print(msg, flush=True)


class DeviceWorkload:
    """A workload's metadata and tensors on the GPU."""

    def __init__(self, config_id, size="small", seed=synth.SEED_BASE, layers=None, with_append=False,
                 rms_weight="ones"):
        self.meta = synth.make_metadata(config_id, size, seed)
        self.geom = self.meta.geom
        d = dev()
        self.k, self.v = synth.make_cache(self.meta, d, seed)
        self.q = synth.make_queries(self.meta, d, seed, num_layers=layers)
        self.block_table = torch.from_numpy(self.meta.block_table).to(d)
        self.seq_lens = torch.from_numpy(self.meta.seq_lens).to(d)
        self.cu_seqlens = torch.from_numpy(self.meta.cu_seqlens).to(d)
        self.slot_mapping = torch.from_numpy(self.meta.slot_mapping).to(d)
        if with_append:
            self.x, self.w_rms, self.w_k, self.w_v = synth.make_append_inputs(self.meta, d, seed, rms_weight)

    def attn(self, layer=0, partition_tokens=0, flags=0, out=None):
        return yb.cross_attn(self.q[layer], self.k, self.v, self.block_table, self.seq_lens, self.meta.max_seq_len,
                             partition_tokens=partition_tokens, flags=flags, out=out)


def host(t):
    """Exact float copy of a device tensor on the host (bf16 -> fp32 is exact)."""
    return t.detach().float().cpu().numpy()


def oracle_attention_full(w: DeviceWorkload, layer=0):
    scale = 1.0 / math.sqrt(w.geom.head_dim)
    return oracle.cross_attention(host(w.q[layer]), host(w.k), host(w.v), w.meta.block_table, w.meta.seq_lens, scale)


def append_tolerance(ref, bound, hidden, dtype):
    """Per-element bound on |gpu - ref| for yoco_kv_append.

    bf16: the folded weight is rounded once (u_b relative), the H products
    are exact in fp32 and their sum carries at most H u_f relative to the
    absolute sum, the fp32 row scale rsqrt(mean(x^2)+eps) is off by at most
    (H+8) u_f, its multiplication adds u_f, and the final store rounds to bf16
    (u_b relative to the computed value).  With B = |xhat| . |W|:
        |gpu - ref| <= u_b |ref| + (1+u_b) (u_b + (2H+9) u_f)(1+u_b) B.
    fp32: no bf16 roundings: (2H+10) u_f B + u_f |ref|.
    """
    ref = np.abs(ref)
    if dtype == "bf16":
        delta = (U_BF16 + (2 * hidden + 9) * U_F32) * (1 + U_BF16) * bound
        return U_BF16 * ref + (1 + U_BF16) * delta
    return (2 * hidden + 10) * U_F32 * bound + U_F32 * ref


def bf16_rne(a):
    """Round float64 values to the nearest bf16 (ties to even), as float64."""
    f = np.asarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)
