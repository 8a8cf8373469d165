"""The 8-bit (FP8 E4M3) shared cache on the GPU against the float64 oracle.

* yoco_kv_scatter: codes and scales bit for bit equal to the oracle's
  quantizer fed with the same fp32 (or bf16) rows; copies into bf16 / fp32
  caches bit for bit; untouched cache bytes keep their bits.
* yoco_kv_append_fp8: every stored value within a derived bound of the
  float64 projection (the append's own floating-point error plus half an
  E4M3 step), scales within the same error.
* yoco_cross_attn_varlen over FP8 caches: within 2e-3 of the oracle's
  attention over the dequantized cache.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import ATTN_ATOL, U_BF16, U_F32, dev, host, say
from yoco_shared_kv_gather_amd import binding as yb
from yoco_shared_kv_gather_amd import synth

pytestmark = pytest.mark.gpu


def _codes_equal(a, b):
    return np.array_equal(np.asarray(a, dtype=np.uint8), np.asarray(b, dtype=np.uint8))


def _scales_equal(a, b):
    return np.array_equal(np.asarray(a, dtype=np.float32).view(np.uint32)[np.isfinite(a)],
                          np.asarray(b, dtype=np.float32).view(np.uint32)[np.isfinite(b)]) and \
        np.array_equal(np.isfinite(a), np.isfinite(b))


@pytest.mark.parametrize("src", ["f32", "bf16"])
@pytest.mark.parametrize("hkv,d,bs", [(1, 64, 4), (2, 128, 16), (8, 128, 16), (2, 256, 32)])
def test_scatter_quantizes_bit_exact(src, hkv, d, bs):
    say(f"kv_scatter -> FP8: {src} rows, {hkv} KV heads x {d}, block {bs}")
    rng = np.random.default_rng(hkv * 1000 + d + bs)
    t, nb = 37, 40
    rows = rng.standard_normal((2, t, hkv, d)).astype(np.float32)
    rows[0, 3] *= 40.0                                   # large rows
    rows[1, 5] *= 1e-4                                   # codes in the subnormal range
    rows[0, 7, 0] = 0.0                                  # a zero row
    rows[1, 9, 0, 3] = np.nan                            # a row holding NaN
    rows[0, 11, 0, 1] = -np.inf
    # values on and next to E4M3 rounding midpoints (ties to even decide):
    # scale 1/8 exactly (row max 56), and a scale that is no power of two
    mids = _e4m3_midpoints()
    for row, scale in ((rows[0, 13, 0], 0.125), (rows[1, 13, 0], np.float32(0.3))):
        vals = (np.resize(mids, d) * np.float32(scale)).astype(np.float32)
        vals[1::3] = np.nextafter(vals[1::3], np.float32(np.inf))
        vals[2::3] = np.nextafter(vals[2::3], np.float32(-np.inf))
        vals[::2] *= -1
        vals[0] = np.float32(448.0) * np.float32(scale)
        row[:] = vals
    rows[1, 15, -1] = rows[1, 15, -1] * np.float32(1e-39)   # a scale whose reciprocal overflows
    if src == "bf16":
        rows_t = torch.from_numpy(rows).to(torch.bfloat16)
        rows = rows_t.float().numpy()                    # exact widening: what the kernel reads
    else:
        rows_t = torch.from_numpy(rows)
    slots = rng.permutation(nb * bs)[:t].astype(np.int32)
    slots[4] = -1
    codes0 = np.full((nb, hkv, bs, d), 0x5A, dtype=np.uint8)
    sc0 = np.full((nb, hkv, bs), 7.0, dtype=np.float32)
    kc, vc = torch.from_numpy(codes0).to(dev()), torch.from_numpy(codes0).to(dev())
    ks, vs = torch.from_numpy(sc0).to(dev()), torch.from_numpy(sc0).to(dev())
    kr, vr = rows_t[0].contiguous().to(dev()), rows_t[1].contiguous().to(dev())
    yb.kv_scatter(kr, vr, torch.from_numpy(slots).to(dev()), kc, vc, ks, vs)
    torch.cuda.synchronize()
    ref_k, ref_v, ref_ks, ref_vs = oracle.kv_scatter(rows[0], rows[1], slots, codes0, codes0, sc0, sc0)
    assert _codes_equal(kc.cpu().numpy(), ref_k) and _codes_equal(vc.cpu().numpy(), ref_v)
    assert _scales_equal(ks.cpu().numpy(), ref_ks) and _scales_equal(vs.cpu().numpy(), ref_vs)


def _e4m3_midpoints():
    """Every point halfway between two neighbouring E4M3 magnitudes below 448
    (exact in fp32): (k + 1/2) 2^-9 among the subnormals, (1 + (2k+1)/16) 2^e
    among the normals."""
    sub = [(k + 0.5) * 2.0 ** -9 for k in range(8)]
    nrm = [(1 + (2 * k + 1) / 16) * 2.0 ** e for e in range(-6, 9) for k in range(8)]
    return np.array([m for m in sub + nrm if m < 448], dtype=np.float32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scatter_copies_bit_exact(dtype):
    say(f"kv_scatter copy: {dtype}")
    rng = np.random.default_rng(7)
    t, nb, hkv, bs, d = 21, 9, 2, 8, 64
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    rows = torch.from_numpy(rng.standard_normal((2, t, hkv, d)).astype(np.float32)).to(tdt)
    slots = rng.permutation(nb * bs)[:t].astype(np.int32)
    slots[[2, 6]] = -1
    cache0 = torch.full((nb, hkv, bs, d), -2.75, dtype=tdt)
    kc, vc = cache0.clone().to(dev()), cache0.clone().to(dev())
    yb.kv_scatter(rows[0].contiguous().to(dev()), rows[1].contiguous().to(dev()), torch.from_numpy(slots).to(dev()),
                  kc, vc)
    torch.cuda.synchronize()
    ref_k, ref_v = oracle.kv_scatter(rows[0].float().numpy(), rows[1].float().numpy(), slots,
                                     cache0.float().numpy(), cache0.float().numpy())
    assert np.array_equal(kc.float().cpu().numpy(), ref_k) and np.array_equal(vc.float().cpu().numpy(), ref_v)


def _append_error(bound, hidden, dtype):
    """The append's error before the final store (see gpu_helpers.append_tolerance):
    bf16: (u_b + (2H+9) u_f)(1+u_b) B; fp32: (2H+10) u_f B."""
    if dtype == "bf16":
        return (U_BF16 + (2 * hidden + 9) * U_F32) * (1 + U_BF16) * bound
    return (2 * hidden + 10) * U_F32 * bound


@pytest.mark.parametrize("cid,size,sample", [(1, "full", 0), (2, "small", 0), (4, "small", 0), (3, "full", 0),
                                             (4, "full", 128)])
def test_append_fp8_within_bound(cid, size, sample):
    """Every written row: |code*s - ref| <= err + half an E4M3 step of the
    stored value (2^-4 relative, s*2^-10 in the subnormal range), and the
    scale times 448 within the append error of the row's largest |ref|."""
    meta = synth.make_metadata(cid, size)
    say(f"kv_append_fp8: workload {cid} {size}, {meta.num_tokens} tokens")
    _check_append_fp8(meta, sample)


@pytest.mark.parametrize("hkv,d", [(1, 64), (3, 64), (2, 256), (1, 256)])
def test_append_fp8_head_dims_tiled(hkv, d):
    """The tiled bf16 GEMM (more than 64 tokens) at head_dim 64 (two heads per
    wavefront; an odd head count leaves half a tile of features) and 256 (a
    head across both column halves of the tile), 150 tokens in a partial
    128-token tile, every seventh row unscheduled (slot -1)."""
    geom = synth.custom_geometry("bf16", 2 * hkv, hkv, d, 16, hidden=512)
    lens = np.random.default_rng(d + hkv).integers(1, 60, size=160)
    lens[::16] = 0
    meta = synth.make_custom_metadata(geom, lens, tag=70 + hkv)
    meta.slot_mapping[::7] = -1
    say(f"kv_append_fp8: {meta.num_tokens} tokens, hidden 512 -> {hkv} x {d}")
    assert meta.num_tokens > 64
    _check_append_fp8(meta, 0)


@pytest.mark.parametrize("num_tokens", [40, 150])
def test_append_fp8_special_rows(num_tokens):
    """Activation rows holding NaN or inf project to non-finite K/V rows:
    every code of such a (token, KV head) row is the NaN code 0x7F and its
    scale is NaN; a row of zeros projects to zeros: zero codes, scale 0.  At
    most 64 tokens the rows go through the quantizing scatter, beyond that the
    tiled GEMM quantizes them in its epilogue; both against the oracle."""
    geom = synth.custom_geometry("bf16", 4, 2, 128, 16, hidden=512)
    lens = np.random.default_rng(num_tokens).integers(1, 60, size=num_tokens)
    meta = synth.make_custom_metadata(geom, lens, tag=80)
    say(f"kv_append_fp8 special rows: {meta.num_tokens} tokens")
    d = dev()
    x, w_rms, w_k, w_v = synth.make_append_inputs(meta, d, rms_weight="random")
    nan_t, inf_t, zero_t = 3, 5, 7
    x[nan_t, 17] = float("nan")
    x[inf_t, 300] = float("inf")
    x[zero_t] = 0
    shape = (meta.num_blocks, geom.num_kv_heads, geom.block_size, geom.head_dim)
    kc = torch.full(shape, 0x5A, dtype=torch.uint8, device=d)
    vc = kc.clone()
    ks = torch.full(shape[:-1], 7.0, dtype=torch.float32, device=d)
    vs = ks.clone()
    yb.kv_append_fp8(x, w_rms, 1e-6, w_k, w_v, torch.from_numpy(meta.slot_mapping).to(d), kc, vc, ks, vs)
    torch.cuda.synchronize()
    tokens = [nan_t, inf_t, zero_t, 0, num_tokens - 1]
    _, _, (ck, sk), (cv, sv), _, _ = oracle.kv_append_fp8(host(x)[tokens], host(w_rms), 1e-6, host(w_k), host(w_v),
                                                       meta.slot_mapping[tokens], geom.num_kv_heads, geom.head_dim)
    kq, vq = kc.cpu().numpy(), vc.cpu().numpy()
    ksn, vsn = ks.cpu().numpy(), vs.cpu().numpy()
    bs = geom.block_size
    for i, t in enumerate(tokens):
        blk, off = divmod(int(meta.slot_mapping[t]), bs)
        for codes, scales, rc, rs in ((kq, ksn, ck, sk), (vq, vsn, cv, sv)):
            got_c, got_s = codes[blk, :, off], scales[blk, :, off]
            if t in (nan_t, inf_t):
                assert (got_c == 0x7F).all() and np.isnan(got_s).all()
                assert (rc[i] == 0x7F).all() and not np.isfinite(rs[i]).any()
            elif t == zero_t:
                assert (got_c == 0).all() and (got_s == 0).all()
                assert (rc[i] == 0).all() and (rs[i] == 0).all()
            else:
                assert np.isfinite(got_s).all() and (got_s > 0).all()


@pytest.mark.parametrize("num_tokens", [1, 10, 130])
def test_append_fp8_hidden_not_multiple_of_256(num_tokens):
    """hidden 320 (a multiple of 64 but not of 256) sends even a single token
    through the tiled GEMM: a 128-token tile of mostly repeated rows,
    quantized in its epilogue."""
    geom = synth.custom_geometry("bf16", 4, 2, 128, 16, hidden=320)
    lens = np.random.default_rng(num_tokens + 5).integers(1, 40, size=num_tokens)
    meta = synth.make_custom_metadata(geom, lens, tag=90)
    say(f"kv_append_fp8: {meta.num_tokens} tokens, hidden 320 -> 2 x 128")
    _check_append_fp8(meta, 0)


def _check_append_fp8(meta, sample):
    geom = meta.geom
    d = dev()
    x, w_rms, w_k, w_v = synth.make_append_inputs(meta, d, rms_weight="random")
    shape = (meta.num_blocks, geom.num_kv_heads, geom.block_size, geom.head_dim)
    kc = torch.full(shape, 0x5A, dtype=torch.uint8, device=d)
    vc = kc.clone()
    ks = torch.full(shape[:-1], 7.0, dtype=torch.float32, device=d)
    vs = ks.clone()
    slots = torch.from_numpy(meta.slot_mapping).to(d)
    yb.kv_append_fp8(x, w_rms, 1e-6, w_k, w_v, slots, kc, vc, ks, vs)
    torch.cuda.synchronize()
    tokens = list(range(meta.num_tokens))
    if sample:
        # full size: one random row of every `sample`-row tile of the GEMM
        # (each row covers every feature tile), plus the last row (the
        # oracle's quantizer runs in Python)
        rng = np.random.default_rng(meta.config_id)
        tokens = sorted({min(t0 + int(rng.integers(0, sample)), meta.num_tokens - 1)
                         for t0 in range(0, meta.num_tokens, sample)} | {meta.num_tokens - 1})
    k, v, _, _, bk, bv = oracle.kv_append_fp8(host(x)[tokens], host(w_rms), 1e-6, host(w_k), host(w_v),
                                             meta.slot_mapping[tokens], geom.num_kv_heads, geom.head_dim)
    kq, vq = kc.cpu().numpy(), vc.cpu().numpy()
    ksn, vsn = ks.cpu().numpy(), vs.cpu().numpy()
    bs = geom.block_size
    worst = 0.0
    same = total = 0
    for i, t in enumerate(tokens):
        slot = meta.slot_mapping[t]
        if slot < 0:
            continue
        blk, off = divmod(int(slot), bs)
        for ref, bound, codes, scales in ((k[i], bk[i], kq, ksn), (v[i], bv[i], vq, vsn)):
            err = _append_error(bound, geom.hidden, geom.dtype)                 # [Hkv][D]
            s = scales[blk, :, off].astype(np.float64)                          # [Hkv]
            got = oracle.e4m3_decode(codes[blk, :, off]) * s[:, None]
            step = np.maximum((np.abs(ref) + err) * 2.0 ** -4, s[:, None] * 2.0 ** -10)
            assert (np.abs(got - ref) <= err + step * (1 + 1e-6)).all()
            amax = np.abs(ref).max(axis=1)
            assert (np.abs(s * 448.0 - amax) <= err.max(axis=1) + amax * 2.0 ** -22).all()
            # the row's own largest value is what the scale was taken from: it
            # divides to 448 up to one fp32 rounding, so every row holds +-448
            assert ((codes[blk, :, off] & 0x7F) == 0x7E).any(axis=1).all()
            worst = max(worst, float((np.abs(got - ref) / (err + step)).max()))
            same += int((codes[blk, :, off] == oracle.quantize_rows(ref.astype(np.float32))[0]).sum())
            total += ref.size
    live = meta.slot_mapping[meta.slot_mapping >= 0]
    untouched = np.ones((meta.num_blocks, bs), dtype=bool)
    untouched[live // bs, live % bs] = False
    assert (kq.transpose(0, 2, 1, 3)[untouched] == 0x5A).all() and (ksn.transpose(0, 2, 1)[untouched] == 7.0).all()
    say(f"  worst error / bound {worst:.3f}; codes equal to the float64 reference's {same / total:.4%}")


def _fp8_case(geom, ctx, qlens, seed):
    meta = synth.make_varlen_metadata(geom, ctx, qlens, seed=seed)
    d = dev()
    kc, ks, vc, vs = synth.make_fp8_cache(meta, d, seed)
    rows = int(meta.cu_seqlens[-1])
    q = synth.make_queries(meta, d, seed, num_layers=1, rows=rows)[0]
    return meta, q, kc, ks, vc, vs


@pytest.mark.parametrize("hq,hkv,d", [(4, 1, 64), (8, 2, 128), (8, 2, 256), (8, 8, 128), (16, 2, 64), (32, 8, 128)])
@pytest.mark.parametrize("several", [False, True])
@pytest.mark.parametrize("window", [0, 50])
@pytest.mark.parametrize("kernel", ["default", "vector"])
def test_attention_fp8(hq, hkv, d, several, window, kernel):
    say(f"cross_attn_varlen FP8: {hq}x{hkv}x{d} several rows {several} window {window} {kernel}")
    geom = synth.custom_geometry("bf16", hq, hkv, d, 16)
    ctx = [5, 300, 1, 0, 64, 129, 3, 700, 2]
    qlens = [3, 4, 1, 2, 5, 1, 6, 2, 0] if several else [1 if c > 0 else 0 for c in ctx]
    meta, q, kc, ks, vc, vs = _fp8_case(geom, ctx, qlens, seed=hq + d + window)
    table = torch.from_numpy(meta.block_table).to(dev())
    seq = torch.from_numpy(meta.seq_lens).to(dev())
    kd = oracle.dequantize_cache(kc.cpu().numpy(), ks.cpu().numpy())
    vd = oracle.dequantize_cache(vc.cpu().numpy(), vs.cpu().numpy())
    ref = oracle.cross_attention_varlen(host(q), kd, vd, meta.block_table, meta.seq_lens, meta.cu_seqlens,
                                        1.0 / math.sqrt(d), window)
    for part in (0, 64):
        qsl = torch.from_numpy(meta.cu_seqlens).to(dev()) if several else None
        qq = q if several else q[:0]
        if not several:
            # one row per request, no offsets: requests with an empty context still own a row
            qq = torch.zeros((meta.num_reqs, hq, d), dtype=torch.bfloat16, device=dev())
            qq[torch.from_numpy(np.nonzero(np.asarray(qlens))[0]).to(dev())] = q
        out = yb.cross_attn_varlen(qq, kc, vc, table, seq, meta.max_seq_len, query_start_loc=qsl,
                                   max_query_len=max(qlens) if several else 1, window=window, partition_tokens=part,
                                   k_scale=ks, v_scale=vs, flags=yb.FLAG_VECTOR_KERNEL if kernel == "vector" else 0)
        torch.cuda.synchronize()
        got = out.cpu().double().numpy()
        if not several:
            got = got[np.nonzero(np.asarray(qlens))[0]]
        assert np.isfinite(got).all()
        err = float(np.abs(got - ref).max())
        say(f"  partition {part}: max abs err {err:.3e}")
        assert err <= ATTN_ATOL


@pytest.mark.parametrize("cid,ql", [(2, 1), (3, 1), (5, 1), (3, 4)])
def test_attention_fp8_full_size_every_output(cid, ql):
    """Full-size workloads over an 8-bit cache (codes and scales drawn as in
    make_fp8_cache), ql query rows per request: every output row and head
    against the oracle over the dequantized values (the oracle's decoder
    applied to all 256 codes, times each row's scale)."""
    meta = synth.make_metadata(cid, "full")
    geom = meta.geom
    say(f"cross_attn_varlen FP8 full size: workload {cid}, {ql} rows per request")
    d = dev()
    kc, ks, vc, vs = synth.make_fp8_cache(meta, d)
    rows = meta.num_reqs * ql
    q = synth.make_queries(meta, d, num_layers=1, rows=rows)[0]
    qsl = (np.arange(meta.num_reqs + 1) * ql).astype(np.int32)
    table = torch.from_numpy(meta.block_table).to(d)
    seq = torch.from_numpy(meta.seq_lens).to(d)
    out = yb.cross_attn_varlen(q, kc, vc, table, seq, meta.max_seq_len,
                               query_start_loc=torch.from_numpy(qsl).to(d) if ql > 1 else None, max_query_len=ql,
                               k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    got_all = out.cpu().double().numpy()
    value = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    bs = geom.block_size
    worst = 0.0
    for r in range(meta.num_reqs):
        n = int(meta.seq_lens[r])
        nb = -(-n // bs)
        blocks = torch.from_numpy(meta.block_table[r, :nb].astype(np.int64)).to(d)
        kd = value[kc.index_select(0, blocks).cpu().numpy()] * ks.index_select(0, blocks).cpu().numpy()[..., None]
        vd = value[vc.index_select(0, blocks).cpu().numpy()] * vs.index_select(0, blocks).cpu().numpy()[..., None]
        ref = oracle.cross_attention_varlen(host(q[r * ql:(r + 1) * ql]), kd, vd, np.arange(nb)[None, :],
                                            np.array([n]), np.array([0, ql]), 1.0 / math.sqrt(geom.head_dim))
        got = got_all[r * ql:(r + 1) * ql]
        assert np.isfinite(got).all()
        worst = max(worst, float(np.abs(got - ref).max()))
        assert worst <= ATTN_ATOL, (r, worst)
    say(f"  {rows} rows x {geom.num_q_heads} heads: max abs err {worst:.3e}")


def test_scatter_then_attention_chain():
    """The product chain -- quantize a bf16 cache's rows with yoco_kv_scatter,
    then attend over the FP8 cache -- against the oracle's quantizer and
    attention on the same bf16 rows."""
    say("kv_scatter(FP8) -> cross_attn_varlen chain, workload 2 small")
    meta = synth.make_metadata(2, "small")
    geom = meta.geom
    d = dev()
    k, v = synth.make_cache(meta, d)
    q = synth.make_queries(meta, d, num_layers=1)[0]
    bs = geom.block_size
    # every context position as a row to scatter
    slots, rows_k, rows_v = [], [], []
    for r in range(meta.num_reqs):
        for j in range(int(meta.seq_lens[r])):
            b = int(meta.block_table[r, j // bs])
            slots.append(b * bs + j % bs)
    slots = np.array(slots, dtype=np.int32)
    blk = torch.from_numpy(slots // bs).long().to(d)
    off = torch.from_numpy(slots % bs).long().to(d)
    rk = k[blk, :, off].contiguous()           # [T][Hkv][D] bf16
    rv = v[blk, :, off].contiguous()
    shape = (meta.num_blocks, geom.num_kv_heads, bs, geom.head_dim)
    kc = torch.full(shape, 0x7F, dtype=torch.uint8, device=d)
    vc = kc.clone()
    ks = torch.full(shape[:-1], float("nan"), dtype=torch.float32, device=d)
    vs = ks.clone()
    yb.kv_scatter(rk, rv, torch.from_numpy(slots).to(d), kc, vc, ks, vs)
    table = torch.from_numpy(meta.block_table).to(d)
    seq = torch.from_numpy(meta.seq_lens).to(d)
    out = yb.cross_attn_varlen(q, kc, vc, table, seq, meta.max_seq_len, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    codes0 = np.full(shape, 0x7F, dtype=np.uint8)
    sc0 = np.full(shape[:-1], np.nan, dtype=np.float32)
    ok_, ov_, oks, ovs = oracle.kv_scatter(host(rk), host(rv), slots, codes0, codes0, sc0, sc0)
    ref = oracle.cross_attention(host(q), oracle.dequantize_cache(ok_, oks), oracle.dequantize_cache(ov_, ovs),
                                 meta.block_table, meta.seq_lens, 1.0 / math.sqrt(geom.head_dim))
    err = float(np.abs(out.cpu().double().numpy() - ref).max())
    say(f"  max abs err {err:.3e}")
    assert err <= ATTN_ATOL
