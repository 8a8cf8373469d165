"""yoco_gather_logits and yoco_cross_attn_varlen on the GPU against the float64
oracle: several query rows per request (aligned to the end of each context,
causal) and sliding windows.

Row gathers and rebuilt offsets are compared bit for bit; attention outputs
element by element within 2e-3 absolute (small and edge sizes, and every
output at full size).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import ATTN_ATOL, DeviceWorkload, dev, host, say
from tests.oracle_pins import load_golden
from yoco_shared_kv_gather_amd import binding as yb
from yoco_shared_kv_gather_amd import synth

pytestmark = pytest.mark.gpu


def _max_err(got, ref):
    got = got.detach().cpu().double().numpy()
    assert np.isfinite(got).all()
    return float(np.abs(got - ref).max()) if got.size else 0.0


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to(dev())


# ---- yoco_gather_logits -------------------------------------------------------------

def test_gather_logits_page_example():
    """The page's printed example: rows [14,18,19,27] of a 28-row batch with
    query_start_loc [0,15,20,28] give offsets [0,1,3,4], largest count 2."""
    fx = load_golden("vllm_logits_indices_example.json")["printed"]
    say("gather_logits: the page's example")
    hidden = torch.arange(28 * 8, dtype=torch.float32, device=dev()).reshape(28, 8)
    rows, qsl, mx = yb.gather_logits(hidden, _i32(fx["logits_indices"]), _i32(fx["query_start_loc"]))
    torch.cuda.synchronize()
    assert qsl.cpu().tolist() == fx["decode_query_start_loc"]
    assert int(mx.item()) == max(fx["num_decode_tokens"])
    assert torch.equal(rows, hidden[torch.tensor(fx["logits_indices"], device=dev())])


@pytest.mark.parametrize("num_reqs", [0, 1, 7, 300, 8192])
def test_gather_logits_random(num_reqs):
    """Random batches (empty requests, positions on request boundaries, a few
    positions outside the batch) against the oracle, bit for bit."""
    say(f"gather_logits: {num_reqs} requests")
    rng = np.random.default_rng(num_reqs + 3)
    lens = rng.integers(0, 6, size=num_reqs)
    qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(qsl[-1])
    idx = np.sort(rng.integers(-2, total + 3, size=max(1, total // 2)))
    bits = rng.integers(0, 2 ** 31, size=(max(total, 1), 12), dtype=np.int64).astype(np.int32)
    hidden = torch.from_numpy(bits).to(dev())
    rows, out_qsl, mx = yb.gather_logits(hidden[:total] if total else hidden[:0], _i32(idx), _i32(qsl))
    torch.cuda.synchronize()
    _, counts, ref_qsl, ref_max = oracle.cross_metadata(idx, qsl)
    ref_rows = oracle.gather_rows(bits[:total], idx)
    assert out_qsl.cpu().numpy().tolist() == ref_qsl.tolist()
    assert int(mx.item()) == ref_max
    assert np.array_equal(rows.cpu().numpy(), ref_rows)


# ---- yoco_cross_attn_varlen ---------------------------------------------------------

class VarlenCase:
    """A batch with query_lens[r] rows per request on the GPU."""

    def __init__(self, geom, seq_lens, query_lens, seed):
        self.meta = synth.make_varlen_metadata(geom, seq_lens, query_lens, seed=seed)
        self.geom = geom
        d = dev()
        self.k, self.v = synth.make_cache(self.meta, d, seed)
        self.rows = int(self.meta.cu_seqlens[-1])
        self.q = synth.make_queries(self.meta, d, seed, num_layers=1, rows=self.rows)[0]
        self.table = torch.from_numpy(self.meta.block_table).to(d)
        self.seq = torch.from_numpy(self.meta.seq_lens).to(d)
        self.qsl = torch.from_numpy(self.meta.cu_seqlens).to(d)
        self.max_qlen = int(np.max(query_lens)) if len(query_lens) else 0

    def run(self, window=0, partition_tokens=0, flags=0, qsl=True):
        return yb.cross_attn_varlen(self.q, self.k, self.v, self.table, self.seq, self.meta.max_seq_len,
                                    query_start_loc=self.qsl if qsl else None,
                                    max_query_len=self.max_qlen if qsl else 1, window=window,
                                    partition_tokens=partition_tokens, flags=flags)

    def oracle(self, window=0):
        return oracle.cross_attention_varlen(host(self.q), host(self.k), host(self.v), self.meta.block_table,
                                             self.meta.seq_lens, self.meta.cu_seqlens,
                                             1.0 / math.sqrt(self.geom.head_dim), window)


GEOMS = [("bf16", 4, 1, 128), ("bf16", 8, 2, 256), ("bf16", 8, 8, 64), ("bf16", 8, 1, 128), ("bf16", 2, 1, 64),
         ("f32", 4, 2, 64), ("f32", 16, 2, 128)]


@pytest.mark.parametrize("dtype,hq,hkv,d", GEOMS)
@pytest.mark.parametrize("window", [0, 1, 37])
@pytest.mark.parametrize("partition_tokens", [0, 64])
@pytest.mark.parametrize("kernel", ["default", "vector"])
def test_varlen_rows_and_window(dtype, hq, hkv, d, window, partition_tokens, kernel):
    """Several rows per request, including more rows than cached tokens, no
    rows, an empty context, exact block multiples and ragged tails; with the
    kernel the library picks (matrix cores for bf16) and the vector kernel."""
    say(f"cross_attn_varlen: {dtype} {hq}x{hkv}x{d} window {window} partition {partition_tokens} {kernel}")
    geom = synth.custom_geometry(dtype, hq, hkv, d, 16)
    ctx = [5, 300, 1, 0, 64, 129, 3, 700, 2]
    ql = [3, 4, 1, 2, 5, 1, 6, 2, 0]
    case = VarlenCase(geom, ctx, ql, seed=hq * 7 + d + window)
    out = case.run(window=window, partition_tokens=partition_tokens,
                   flags=yb.FLAG_VECTOR_KERNEL if kernel == "vector" else 0)
    torch.cuda.synchronize()
    err = _max_err(out, case.oracle(window))
    say(f"  max abs err {err:.3e}")
    assert err <= ATTN_ATOL


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
@pytest.mark.parametrize("window", [1, 100, 1000, 5000])
def test_window_one_row_per_request(cid, window):
    """A window with one query row per request (the decode kernel with a
    shorter range) on each workload's small size."""
    say(f"cross_attn_varlen window {window}: workload {cid} small")
    w = DeviceWorkload(cid, "small", layers=1)
    for part in (0, 64):
        out = yb.cross_attn_varlen(w.q[0], w.k, w.v, w.block_table, w.seq_lens, w.meta.max_seq_len, window=window,
                                   partition_tokens=part)
        torch.cuda.synchronize()
        ref = oracle.cross_attention_varlen(host(w.q[0]), host(w.k), host(w.v), w.meta.block_table,
                                            w.meta.seq_lens, np.arange(w.meta.num_reqs + 1),
                                            1.0 / math.sqrt(w.geom.head_dim), window)
        err = _max_err(out, ref)
        say(f"  partition {part}: max abs err {err:.3e}")
        assert err <= ATTN_ATOL


def test_varlen_one_row_matches_decode_call():
    """query_start_loc [0,1,..,R] with one row each and no window gives the
    decode call's result within the attention tolerance; without
    query_start_loc the varlen call is the decode call, bit for bit."""
    say("cross_attn_varlen vs cross_attn: workload 2 small")
    w = DeviceWorkload(2, "small", layers=1)
    base = w.attn(0, partition_tokens=64).clone()
    same = yb.cross_attn_varlen(w.q[0], w.k, w.v, w.block_table, w.seq_lens, w.meta.max_seq_len,
                                partition_tokens=64)
    qsl = torch.arange(w.meta.num_reqs + 1, dtype=torch.int32, device=dev())
    rows = yb.cross_attn_varlen(w.q[0], w.k, w.v, w.block_table, w.seq_lens, w.meta.max_seq_len,
                                query_start_loc=qsl, max_query_len=1, partition_tokens=64)
    torch.cuda.synchronize()
    assert torch.equal(base.view(torch.int32), same.view(torch.int32))
    assert float((rows - base).abs().max()) <= 1e-5


@pytest.mark.parametrize("kernel", [0, yb.FLAG_VECTOR_KERNEL])
def test_varlen_deterministic_and_order_independent(kernel):
    say(f"cross_attn_varlen determinism: both work orders, kernel flag {kernel}")
    geom = synth.custom_geometry("bf16", 8, 2, 128, 16)
    case = VarlenCase(geom, [900, 40, 1500, 7], [4, 2, 3, 1], seed=21)
    a = case.run(window=300, partition_tokens=64, flags=kernel).clone()
    b = case.run(window=300, partition_tokens=64, flags=kernel | yb.FLAG_REVERSE_ORDER).clone()
    c = case.run(window=300, partition_tokens=64, flags=kernel).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(a.view(torch.int32), c.view(torch.int32))
    assert _max_err(a, case.oracle(300)) <= ATTN_ATOL


def test_spec_decode_step_chain():
    """A speculative-decoding step end to end: the logits rows of each request
    gathered with the offsets rebuilt on the device, then attention with those
    offsets (the device-side max_query_len bound is checked too)."""
    say("gather_logits -> cross_attn_varlen chain")
    geom = synth.custom_geometry("bf16", 8, 2, 128, 16)
    rng = np.random.default_rng(5)
    ctx = [int(c) for c in rng.integers(50, 3000, size=12)]
    sched = [int(s) for s in rng.integers(1, 6, size=12)]        # scheduled rows per request
    kept = [int(rng.integers(1, s + 1)) for s in sched]          # its last rows produce logits
    case = VarlenCase(geom, ctx, kept, seed=6)
    sched_qsl = np.concatenate([[0], np.cumsum(sched)]).astype(np.int32)
    logits_idx = np.concatenate([np.arange(sched_qsl[r + 1] - kept[r], sched_qsl[r + 1]) for r in range(12)])
    # the step's hidden rows: the query rows placed at the logits positions
    hidden = torch.zeros((int(sched_qsl[-1]), geom.num_q_heads, geom.head_dim), dtype=torch.bfloat16, device=dev())
    hidden[torch.from_numpy(logits_idx).to(dev())] = case.q
    q, qsl, mx = yb.gather_logits(hidden, _i32(logits_idx), _i32(sched_qsl))
    torch.cuda.synchronize()
    assert qsl.cpu().tolist() == case.meta.cu_seqlens.tolist()
    assert int(mx.item()) == max(kept)
    out = yb.cross_attn_varlen(q, case.k, case.v, case.table, case.seq, case.meta.max_seq_len, query_start_loc=qsl,
                               max_query_len=max(kept))
    torch.cuda.synchronize()
    assert _max_err(out, case.oracle()) <= ATTN_ATOL


@pytest.mark.parametrize("cid,ql,window", [(3, 4, 0), (4, 3, 2048), (5, 2, 0), (5, 1, 8192), (2, 4, 0), (2, 1, 512)])
def test_varlen_full_size_every_output(cid, ql, window):
    """Full-size workloads with ql query rows per request (every request) and
    an optional window: every output row and head against the oracle, one
    request's blocks fetched at a time (from the first block its window
    reaches)."""
    say(f"cross_attn_varlen full size: workload {cid}, {ql} rows per request, window {window}")
    meta = synth.make_metadata(cid, "full")
    geom = meta.geom
    d = dev()
    k, v = synth.make_cache(meta, d)
    rows = meta.num_reqs * ql
    q = synth.make_queries(meta, d, num_layers=1, rows=rows)[0]
    qsl_np = (np.arange(meta.num_reqs + 1) * ql).astype(np.int32)
    table = torch.from_numpy(meta.block_table).to(d)
    seq = torch.from_numpy(meta.seq_lens).to(d)
    out = yb.cross_attn_varlen(q, k, v, table, seq, meta.max_seq_len, query_start_loc=_i32(qsl_np),
                               max_query_len=ql, window=window)
    torch.cuda.synchronize()
    got_all = out.cpu().double().numpy()
    bs = geom.block_size
    worst = 0.0
    for r in range(meta.num_reqs):
        n = int(meta.seq_lens[r])
        lo = 0 if window == 0 else max(0, n - ql - window + 1)
        b0, b1 = lo // bs, -(-n // bs)
        blocks = torch.from_numpy(meta.block_table[r, b0:b1].astype(np.int64)).to(d)
        kc = host(k.index_select(0, blocks))
        vc = host(v.index_select(0, blocks))
        # the same request over the blocks from b0 on: positions shift by b0*bs
        ref = oracle.cross_attention_varlen(host(q[r * ql:(r + 1) * ql]), kc, vc, np.arange(b1 - b0)[None, :],
                                            np.array([n - b0 * bs]), np.array([0, ql]),
                                            1.0 / math.sqrt(geom.head_dim), window)
        got = got_all[r * ql:(r + 1) * ql]
        assert np.isfinite(got).all()
        worst = max(worst, float(np.abs(got - ref).max()))
        assert worst <= ATTN_ATOL, (r, worst)
    say(f"  {rows} rows x {geom.num_q_heads} heads: max abs err {worst:.3e}")


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("ql,window", [(3, 37), (1, 37), (4, 100), (2, 1)])
def test_window_start_in_last_block_of_exact_pool(fp8, ql, window):
    """A windowed item whose first block is the pool's last physical block,
    read for every KV head (the last one included), with a pool of exactly
    the blocks the context needs and a window start that is not 16-aligned:
    the matrix-core kernel's stand-in tiles past the item's end stay inside
    that block.  Checked against the oracle."""
    say(f"window start in the last block: fp8 {fp8}, {ql} rows, window {window}")
    hq, hkv, d, bs, n = 8, 2, 128, 16, 300
    nb = -(-n // bs)
    lo = max(0, n - ql - window + 1)
    assert lo % 16 != 0
    rng = np.random.default_rng(ql * 100 + window)
    table = rng.permutation(nb).astype(np.int32)
    j = int(np.where(table == nb - 1)[0][0])
    table[j], table[lo // bs] = table[lo // bs], table[j]           # the window's first block is physical nb-1
    assert table[lo // bs] == nb - 1
    tail = n - (nb - 1) * bs                                        # rows used in the last logical block
    d_ = dev()
    if fp8:
        shape = (nb, hkv, bs, d)
        codes = rng.integers(0, 254, size=(2,) + shape)
        codes = np.where(codes >= 0x7F, codes + 1, codes).astype(np.uint8)
        scales = rng.uniform(0.002, 0.02, size=(2,) + shape[:-1]).astype(np.float32)
        last = table[nb - 1]
        codes[:, last, :, tail:] = 0x7F
        scales[:, last, :, tail:] = np.nan
        kc, vc = (torch.from_numpy(codes[i].copy()).to(d_) for i in range(2))
        ks, vs = (torch.from_numpy(scales[i].copy()).to(d_) for i in range(2))
        kref, vref = (oracle.dequantize_cache(codes[i], scales[i]) for i in range(2))
    else:
        kv = rng.standard_normal((2, nb, hkv, bs, d)).astype(np.float32)
        kv[:, table[nb - 1], :, tail:] = np.nan
        kc, vc = (torch.from_numpy(kv[i].copy()).to(d_).to(torch.bfloat16) for i in range(2))
        ks = vs = None
        kref, vref = host(kc), host(vc)
    q = torch.from_numpy(rng.standard_normal((ql, hq, d)).astype(np.float32)).to(d_).to(torch.bfloat16)
    qsl = np.array([0, ql], dtype=np.int32)
    out = yb.cross_attn_varlen(q, kc, vc, _i32(table[None, :]), _i32([n]), n, query_start_loc=_i32(qsl),
                               max_query_len=ql, window=window, partition_tokens=64, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    ref = oracle.cross_attention_varlen(host(q), kref, vref, table[None, :], np.array([n]), qsl,
                                        1.0 / math.sqrt(d), window)
    err = _max_err(out, ref)
    say(f"  max abs err {err:.3e}")
    assert err <= ATTN_ATOL
