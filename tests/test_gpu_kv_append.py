"""yoco_kv_append on the GPU against the float64 oracle.

Written slots must match the oracle's projection within the floating-point
bound derived in tests/gpu_helpers.append_tolerance; every other byte of the
cache must keep its bits."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import DeviceWorkload, append_tolerance, bf16_rne, host, say
from yoco_shared_kv_gather_amd import binding as yb
from yoco_shared_kv_gather_amd import synth

pytestmark = pytest.mark.gpu
EPS = 1e-6


def _check_rows(w, k_before, v_before, tokens, dtype):
    """Compare the cache rows written for `tokens` and require every other
    slot to be unchanged."""
    meta, geom = w.meta, w.geom
    x = host(w.x[tokens])
    kref, vref, kb, vb = oracle.kv_project(x, host(w.w_rms), EPS, host(w.w_k), host(w.w_v),
                                           geom.num_kv_heads, geom.head_dim)
    slots = meta.slot_mapping[tokens]
    bs = geom.block_size
    worst = 0.0
    match = []
    for i, s in enumerate(slots):
        if s < 0:
            continue
        for cache, ref, bound in ((w.k, kref[i], kb[i]), (w.v, vref[i], vb[i])):
            got = host(cache[s // bs, :, s % bs, :]).astype(np.float64)
            tol = append_tolerance(ref, bound, geom.hidden, dtype)
            err = np.abs(got - ref)
            assert (err <= tol).all(), (i, float(err.max()), float(tol[err > tol].min()))
            worst = max(worst, float((err / tol).max()))
            if dtype == "bf16":
                match.append((got == bf16_rne(ref)).mean())
    say(f"  worst error / bound {worst:.3f}" + (f", bf16-equal to RNE(ref): {np.mean(match):.4f}" if match else ""))
    return match


def _untouched_equal(w, k_before, v_before):
    live = torch.zeros(w.meta.num_blocks * w.geom.block_size, dtype=torch.bool, device=w.k.device)
    sm = w.slot_mapping[w.slot_mapping >= 0].long()
    live[sm] = True
    live = live.view(w.meta.num_blocks, 1, w.geom.block_size, 1).expand_as(w.k)
    ib = torch.int16 if w.k.element_size() == 2 else torch.int32
    for after, before in ((w.k, k_before), (w.v, v_before)):
        assert torch.equal(after.view(ib)[~live], before.view(ib)[~live])


@pytest.mark.parametrize("cid,size,rms", [(1, "full", "ones"), (1, "full", "random"), (2, "small", "ones"),
                                          (2, "small", "random"), (2, "full", "random"), (3, "small", "ones"),
                                          (4, "small", "ones"), (4, "small", "random"), (5, "small", "ones")])
def test_append_parity(cid, size, rms):
    say(f"kv_append parity: workload {cid} {size} rms weight {rms}")
    w = DeviceWorkload(cid, size, layers=1, with_append=True, rms_weight=rms)
    k0, v0 = w.k.clone(), w.v.clone()
    yb.kv_append(w.x, w.w_rms, EPS, w.w_k, w.w_v, w.slot_mapping, w.k, w.v)
    torch.cuda.synchronize()
    _untouched_equal(w, k0, v0)
    match = _check_rows(w, k0, v0, np.arange(w.meta.num_tokens), w.geom.dtype)
    if w.geom.dtype == "bf16" and rms == "ones":
        assert np.mean(match) > 0.99


def test_append_full_size_mixed_step():
    """Workload 4 at full size (67,387 rows, 64,178 of them written, through
    the tiled MFMA GEMM): every untouched byte keeps its bits; one random row
    of every 128-row GEMM tile (each row spans every feature tile), every
    request's last row and the batch's last row match the oracle."""
    say("kv_append full size: workload 4")
    w = DeviceWorkload(4, "full", layers=1, with_append=True)
    k0, v0 = w.k.clone(), w.v.clone()
    yb.kv_append(w.x, w.w_rms, EPS, w.w_k, w.w_v, w.slot_mapping, w.k, w.v)
    torch.cuda.synchronize()
    _untouched_equal(w, k0, v0)
    rng = np.random.default_rng(4)
    t_count = w.meta.num_tokens
    per_tile = [min(t0 + int(rng.integers(0, 128)), t_count - 1) for t0 in range(0, t_count, 128)]
    last = w.meta.cu_seqlens[1:] - 1
    sample = np.unique(np.concatenate([per_tile, last, [t_count - 1]]))
    say(f"  {len(sample)} rows checked ({len(per_tile)} tiles of 128)")
    match = _check_rows(w, k0, v0, sample, "bf16")
    assert np.mean(match) > 0.99


def test_append_twice_is_idempotent():
    say("kv_append: same call twice gives the same bits")
    w = DeviceWorkload(2, "small", layers=1, with_append=True)
    yb.kv_append(w.x, w.w_rms, EPS, w.w_k, w.w_v, w.slot_mapping, w.k, w.v)
    k1 = w.k.clone()
    yb.kv_append(w.x, w.w_rms, EPS, w.w_k, w.w_v, w.slot_mapping, w.k, w.v)
    torch.cuda.synchronize()
    assert torch.equal(k1.view(torch.int16), w.k.view(torch.int16))


@pytest.mark.parametrize("num_tokens", [1, 16, 17, 33, 64, 65, 300])
def test_append_token_counts_both_paths(num_tokens):
    """Token counts on both sides of the 64-token switch between the decode
    (skinny) and prefill (tiled GEMM) bf16 paths, with partial 16-row tiles,
    a padding row and a random RMS weight."""
    say(f"kv_append: {num_tokens} tokens, hidden 3072 -> 8 x 128")
    w = DeviceWorkload(3, "small", layers=1, with_append=True, rms_weight="random")
    meta = w.meta
    rng = np.random.default_rng(num_tokens)
    live = np.flatnonzero(synth.live_slot_mask(meta).reshape(-1))
    slots = rng.choice(live, size=num_tokens, replace=False).astype(np.int32)
    if num_tokens > 2:
        slots[num_tokens // 2] = -1                         # a graph-padding row
    meta.slot_mapping = slots
    meta.num_tokens = num_tokens
    w.slot_mapping = torch.from_numpy(slots).to(w.k.device)
    w.x = torch.randn(num_tokens, meta.geom.hidden, device=w.k.device).to(torch.bfloat16)
    k0, v0 = w.k.clone(), w.v.clone()
    yb.kv_append(w.x, w.w_rms, EPS, w.w_k, w.w_v, w.slot_mapping, w.k, w.v)
    torch.cuda.synchronize()
    _untouched_equal(w, k0, v0)
    _check_rows(w, k0, v0, np.arange(num_tokens), "bf16")


@pytest.mark.parametrize("num_tokens", [1, 10, 130])
def test_append_hidden_not_multiple_of_256(num_tokens):
    """hidden 320 (a multiple of 64 but not of 256): every token count goes
    through the tiled GEMM, down to one token in a 128-token tile."""
    from tests.gpu_helpers import dev
    geom = synth.custom_geometry("bf16", 4, 2, 128, 16, hidden=320)
    lens = np.random.default_rng(num_tokens + 7).integers(1, 40, size=num_tokens)
    meta = synth.make_custom_metadata(geom, lens, tag=91)
    say(f"kv_append: {meta.num_tokens} tokens, hidden 320 -> 2 x 128")
    d = dev()
    x, w_rms, w_k, w_v = synth.make_append_inputs(meta, d, rms_weight="random")
    shape = (meta.num_blocks, geom.num_kv_heads, geom.block_size, geom.head_dim)
    k = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=d)
    v = k.clone()
    slots = torch.from_numpy(meta.slot_mapping).to(d)
    yb.kv_append(x, w_rms, EPS, w_k, w_v, slots, k, v)
    torch.cuda.synchronize()
    kref, vref, kb, vb = oracle.kv_project(host(x), host(w_rms), EPS, host(w_k), host(w_v),
                                           geom.num_kv_heads, geom.head_dim)
    bs = geom.block_size
    for t, s in enumerate(meta.slot_mapping):
        for cache, ref, bound in ((k, kref[t], kb[t]), (v, vref[t], vb[t])):
            got = host(cache[s // bs, :, s % bs, :]).astype(np.float64)
            assert (np.abs(got - ref) <= append_tolerance(ref, bound, geom.hidden, "bf16")).all()
    written = torch.zeros(meta.num_blocks * bs, dtype=torch.bool, device=d)
    written[slots.long()] = True
    untouched = ~written.view(meta.num_blocks, 1, bs, 1).expand_as(k)
    assert torch.isnan(k[untouched].float()).all() and torch.isnan(v[untouched].float()).all()
