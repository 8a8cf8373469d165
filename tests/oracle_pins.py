"""Pins of the float64 oracle against facts that do not come from the oracle.

Each ``check_*`` function takes the function under test as an argument and
raises AssertionError when it disagrees with a closed form, an invariant, a
library routine or a worked example from the pages.  ``test_oracle_pins``
runs them on the oracle; ``test_oracle_mutants`` runs them on copies of the
oracle with a plausible mistake planted in each, and requires every mutant to
fail at least one check.
"""

from __future__ import annotations

import json
import os
from decimal import Decimal, getcontext

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# helpers that build paged caches from logical K/V (test-side only)
# ---------------------------------------------------------------------------

def paged_from_logical(keys_list, values_list, block_size, tables, num_blocks):
    """Place each request's logical K/V ``[n][Hkv][D]`` into a NaN-filled pool."""
    hkv, d = keys_list[0].shape[1], keys_list[0].shape[2]
    kc = np.full((num_blocks, hkv, block_size, d), np.nan)
    vc = np.full((num_blocks, hkv, block_size, d), np.nan)
    for keys, values, table in zip(keys_list, values_list, tables):
        for j in range(keys.shape[0]):
            kc[table[j // block_size], :, j % block_size, :] = keys[j]
            vc[table[j // block_size], :, j % block_size, :] = values[j]
    return kc, vc


def random_problem(rng, lens, hq, hkv, d, bs, spare_blocks=3):
    """Random logical K/V per request, placed in randomly permuted blocks."""
    keys = [rng.standard_normal((n, hkv, d)) for n in lens]
    values = [rng.standard_normal((n, hkv, d)) for n in lens]
    need = [-(-n // bs) for n in lens]
    num_blocks = sum(need) + spare_blocks
    perm = rng.permutation(num_blocks)
    width = max(max(need), 1) + 1
    tables = np.full((len(lens), width), perm[-1], dtype=np.int64)   # spare: NaN block
    cursor = 0
    for r, nb in enumerate(need):
        tables[r, :nb] = perm[cursor:cursor + nb]
        cursor += nb
    kc, vc = paged_from_logical(keys, values, bs, tables, num_blocks)
    q = rng.standard_normal((len(lens), hq, d))
    return q, kc, vc, tables, np.array(lens), keys, values


# ---------------------------------------------------------------------------
# attention checks
# ---------------------------------------------------------------------------

def check_attn_sdpa(attn):
    """Library routine: torch SDPA in float64 (its default scale is 1/sqrt(D),
    its GQA mapping repeats each KV head over a contiguous group of query
    heads) on the logical K/V of every request."""
    rng = np.random.default_rng(11)
    for hq, hkv, d, bs, lens in [(4, 1, 8, 4, [7, 2, 13]), (8, 2, 16, 16, [1, 40, 17]), (6, 6, 4, 2, [5, 9])]:
        q, kc, vc, tables, seq, keys, values = random_problem(rng, lens, hq, hkv, d, bs)
        got = attn(q, kc, vc, tables, seq, 1.0 / np.sqrt(d))
        for r, n in enumerate(lens):
            qt = torch.from_numpy(q[r]).reshape(1, hq, 1, d)
            kt = torch.from_numpy(keys[r]).permute(1, 0, 2).reshape(1, hkv, n, d).contiguous()
            vt = torch.from_numpy(values[r]).permute(1, 0, 2).reshape(1, hkv, n, d).contiguous()
            ref = F.scaled_dot_product_attention(qt, kt, vt, enable_gqa=(hq != hkv)).reshape(hq, d).numpy()
            np.testing.assert_allclose(got[r], ref, rtol=0, atol=1e-12)


def check_attn_block_table_replay(attn):
    """The pages' Replay figure: logical blocks 0,1,2,3 on physical pages
    0,2,1,4 with pages 3 and 5 free gives the same output as contiguous
    placement, bit for bit."""
    fx = load_golden("kv_block_table_replay.json")
    table = np.array(fx["block_table"])
    rng = np.random.default_rng(12)
    bs, hkv, d, hq = 4, 2, 8, 4
    n = 4 * bs - 1                      # four logical blocks, the last one partial
    keys = rng.standard_normal((n, hkv, d))
    values = rng.standard_normal((n, hkv, d))
    kc, vc = paged_from_logical([keys], [values], bs, [table], len(fx["physical_pages"]))
    for free in fx["free_pages"]:
        assert np.isnan(kc[free]).all()
    kc2, vc2 = paged_from_logical([keys], [values], bs, [np.arange(4)], 4)
    q = rng.standard_normal((1, hq, d))
    a = attn(q, kc, vc, table[None, :], np.array([n]), 0.3)
    b = attn(q, kc2, vc2, np.arange(4)[None, :], np.array([n]), 0.3)
    assert np.isfinite(a).all()
    assert np.array_equal(a, b)


def check_attn_random_permutation(attn):
    """Any physical permutation of the blocks (table permuted with them) leaves
    the output unchanged."""
    rng = np.random.default_rng(13)
    q, kc, vc, tables, seq, _, _ = random_problem(rng, [9, 30, 3], 4, 2, 8, 4)
    base = attn(q, kc, vc, tables, seq, 0.25)
    perm = rng.permutation(kc.shape[0])          # new position of old block b is perm[b]
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    tables2 = perm[tables]
    assert np.array_equal(attn(q, kc2, vc2, tables2, seq, 0.25), base)


def check_attn_closed_forms(attn):
    """Closed forms: identical keys or a zero query give the mean of V; a
    context of one token returns that token's V; a key aligned with the query
    and scaled up dominates."""
    rng = np.random.default_rng(14)
    bs, d = 4, 8
    # identical keys -> mean of V, for any query
    n = 11
    keys = np.repeat(rng.standard_normal((1, 1, d)), n, axis=0)
    values = rng.standard_normal((n, 1, d))
    kc, vc = paged_from_logical([keys], [values], bs, [np.array([2, 0, 1])], 3)
    q = rng.standard_normal((1, 2, d)) * 3.0
    out = attn(q, kc, vc, np.array([[2, 0, 1]]), np.array([n]), 0.7)
    np.testing.assert_allclose(out[0, 0], values[:, 0].mean(axis=0), atol=1e-13)
    np.testing.assert_allclose(out[0, 1], values[:, 0].mean(axis=0), atol=1e-13)
    # zero query -> mean of V with arbitrary keys
    keys = rng.standard_normal((n, 1, d))
    kc, vc = paged_from_logical([keys], [values], bs, [np.array([1, 2, 0])], 3)
    out = attn(np.zeros((1, 1, d)), kc, vc, np.array([[1, 2, 0]]), np.array([n]), 0.7)
    np.testing.assert_allclose(out[0, 0], values[:, 0].mean(axis=0), atol=1e-13)
    # context of one token -> exactly that V row
    out = attn(q[:, :1], kc, vc, np.array([[1, 2, 0]]), np.array([1]), 0.7)
    assert np.array_equal(out[0, 0], values[0, 0])
    # one key = lambda * q, the others small -> that row's V
    keys = rng.standard_normal((n, 1, d)) * 0.01
    qv = rng.standard_normal(d)
    keys[5, 0] = 40.0 * qv / np.linalg.norm(qv)
    kc, vc = paged_from_logical([keys], [values], bs, [np.array([0, 1, 2])], 3)
    out = attn((qv / np.linalg.norm(qv) * 40.0).reshape(1, 1, d), kc, vc, np.array([[0, 1, 2]]), np.array([n]), 1.0)
    np.testing.assert_allclose(out[0, 0], values[5, 0], atol=1e-12)


def check_attn_invariants(attn):
    """Shifting every key by one vector leaves the output unchanged; an affine
    map of V maps the output the same way; identical queries in one GQA group
    give identical outputs; a request with an empty context gives zeros."""
    rng = np.random.default_rng(15)
    q, kc, vc, tables, seq, keys, values = random_problem(rng, [10, 6], 4, 2, 8, 4)
    base = attn(q, kc, vc, tables, seq, 0.4)
    shift = rng.standard_normal(8)
    live = ~np.isnan(kc)
    kc2 = np.where(live, kc + shift, kc)
    np.testing.assert_allclose(attn(q, kc2, vc, tables, seq, 0.4), base, atol=1e-12)
    vc2 = np.where(live, 2.5 * vc + 0.75, vc)
    np.testing.assert_allclose(attn(q, kc, vc2, tables, seq, 0.4), 2.5 * base + 0.75, atol=1e-12)
    q2 = q.copy()
    q2[:, 1] = q2[:, 0]                 # heads 0 and 1 share KV head 0 (group of 2)
    out = attn(q2, kc, vc, tables, seq, 0.4)
    assert np.array_equal(out[:, 0], out[:, 1])
    assert not np.allclose(out[:, 0], out[:, 2])
    empty = attn(q, kc, vc, tables, np.array([0, 6]), 0.4)
    assert np.array_equal(empty[0], np.zeros_like(empty[0]))
    np.testing.assert_allclose(empty[1], base[1], atol=0)


def check_attn_aliased_prefix(attn):
    """Two requests whose tables share a physical prefix block give the same
    outputs as with private copies of that block."""
    rng = np.random.default_rng(16)
    bs, d = 4, 8
    shared_k = rng.standard_normal((bs, 1, d))
    shared_v = rng.standard_normal((bs, 1, d))
    ka = np.concatenate([shared_k, rng.standard_normal((3, 1, d))])
    va = np.concatenate([shared_v, rng.standard_normal((3, 1, d))])
    kb = np.concatenate([shared_k, rng.standard_normal((2, 1, d))])
    vb = np.concatenate([shared_v, rng.standard_normal((2, 1, d))])
    q = rng.standard_normal((2, 2, d))
    private_tables = np.array([[0, 1], [2, 3]])
    kc, vc = paged_from_logical([ka, kb], [va, vb], bs, private_tables, 4)
    alias_tables = np.array([[0, 1], [0, 3]])
    kc2, vc2 = paged_from_logical([ka, kb], [va, vb], bs, alias_tables, 4)
    seq = np.array([7, 6])
    assert np.array_equal(attn(q, kc, vc, private_tables, seq, 0.5), attn(q, kc2, vc2, alias_tables, seq, 0.5))


def _dec_attention(qv, keys, values, scale):
    getcontext().prec = 50
    s = [Decimal(scale) * sum(Decimal(float(a)) * Decimal(float(b)) for a, b in zip(qv, k)) for k in keys]
    mx = max(s)
    w = [(x - mx).exp() for x in s]
    tot = sum(w)
    return [float(sum(wi * Decimal(float(v[c])) for wi, v in zip(w, values)) / tot) for c in range(len(values[0]))]


def check_attn_decimal(attn):
    """Brute force in 50-digit decimal arithmetic on tiny inputs."""
    rng = np.random.default_rng(17)
    for trial in range(4):
        lens = [int(x) for x in rng.integers(1, 13, size=2)]
        q, kc, vc, tables, seq, keys, values = random_problem(rng, lens, 2, 1, int(rng.integers(2, 9)), 4)
        d = q.shape[2]
        got = attn(q, kc, vc, tables, seq, 1.0 / np.sqrt(d))
        for r in range(len(lens)):
            for h in range(2):
                ref = _dec_attention(q[r, h], keys[r][:, 0], values[r][:, 0], 1.0 / np.sqrt(d))
                np.testing.assert_allclose(got[r, h], ref, rtol=0, atol=1e-13)


ATTN_CHECKS = [
    check_attn_sdpa,
    check_attn_block_table_replay,
    check_attn_random_permutation,
    check_attn_closed_forms,
    check_attn_invariants,
    check_attn_aliased_prefix,
    check_attn_decimal,
]


# ---------------------------------------------------------------------------
# projection / append checks
# ---------------------------------------------------------------------------

def check_proj_torch(project):
    """Library routine: torch.nn.functional.rms_norm then linear, in float64."""
    rng = np.random.default_rng(21)
    t, hidden, hkv, d = 5, 24, 2, 4
    x = rng.standard_normal((t, hidden)) * rng.uniform(0.1, 5.0, size=(t, 1))
    w = rng.uniform(0.5, 1.5, size=hidden)
    wk = rng.standard_normal((hkv * d, hidden))
    wv = rng.standard_normal((hkv * d, hidden))
    for eps in (1e-6, 0.3):
        k, v, bk, bv = project(x, w, eps, wk, wv, hkv, d)
        xt = F.rms_norm(torch.from_numpy(x), (hidden,), torch.from_numpy(w), eps=eps)
        np.testing.assert_allclose(k.reshape(t, -1), F.linear(xt, torch.from_numpy(wk)).numpy(), atol=1e-12)
        np.testing.assert_allclose(v.reshape(t, -1), F.linear(xt, torch.from_numpy(wv)).numpy(), atol=1e-12)
        assert (bk >= np.abs(k) - 1e-12).all() and (bv >= np.abs(v) - 1e-12).all()


def check_proj_closed_forms(project):
    """A constant row c gives xhat = c / sqrt(c^2 + eps) * w; weight rows that
    are unit vectors select entries of xhat into [Hkv][D] order; with eps = 0
    scaling a row leaves the result unchanged."""
    rng = np.random.default_rng(22)
    hidden, hkv, d = 12, 2, 3
    w = rng.uniform(0.5, 1.5, size=hidden)
    perm_k = rng.permutation(hidden)[: hkv * d]
    perm_v = rng.permutation(hidden)[: hkv * d]
    wk = np.eye(hidden)[perm_k]
    wv = np.eye(hidden)[perm_v]
    c, eps = -1.7, 0.25
    x = np.full((1, hidden), c)
    k, v, _, _ = project(x, w, eps, wk, wv, hkv, d)
    xhat = c / np.sqrt(c * c + eps) * w
    np.testing.assert_allclose(k[0], xhat[perm_k].reshape(hkv, d), atol=1e-14)
    np.testing.assert_allclose(v[0], xhat[perm_v].reshape(hkv, d), atol=1e-14)
    x = rng.standard_normal((3, hidden))
    k1, v1, _, _ = project(x, w, 0.0, wk, wv, hkv, d)
    k2, v2, _, _ = project(7.5 * x, w, 0.0, wk, wv, hkv, d)
    np.testing.assert_allclose(k1, k2, atol=1e-13)
    np.testing.assert_allclose(v1, v2, atol=1e-13)


def check_proj_decimal(project):
    """Brute force in 50-digit decimal on a tiny projection."""
    getcontext().prec = 50
    rng = np.random.default_rng(23)
    t, hidden, hkv, d = 2, 6, 1, 3
    x = rng.standard_normal((t, hidden))
    w = rng.uniform(0.5, 1.5, size=hidden)
    wk = rng.standard_normal((hkv * d, hidden))
    wv = rng.standard_normal((hkv * d, hidden))
    eps = 1e-6
    k, v, _, _ = project(x, w, eps, wk, wv, hkv, d)
    for i in range(t):
        xs = [Decimal(float(a)) for a in x[i]]
        ms = sum(a * a for a in xs) / hidden
        inv = 1 / (ms + Decimal(eps)).sqrt()
        xh = [a * inv * Decimal(float(b)) for a, b in zip(xs, w)]
        for o in range(hkv * d):
            rk = float(sum(Decimal(float(wk[o, j])) * xh[j] for j in range(hidden)))
            rv = float(sum(Decimal(float(wv[o, j])) * xh[j] for j in range(hidden)))
            assert abs(k[i].reshape(-1)[o] - rk) < 1e-13
            assert abs(v[i].reshape(-1)[o] - rv) < 1e-13


PROJ_CHECKS = [check_proj_torch, check_proj_closed_forms, check_proj_decimal]


def check_append_scatter(append):
    """Slot s lands in block s // block_size at offset s % block_size for
    every KV head; negative slots write nothing; every other cache entry keeps
    its bits.  Hand-worked: block size 4, slot 10 -> block 2, offset 2."""
    rng = np.random.default_rng(31)
    nb, hkv, bs, d, hidden = 5, 2, 4, 3, 8
    sentinel = np.full((nb, hkv, bs, d), -7.25)
    x = rng.standard_normal((4, hidden))
    w = np.ones(hidden)
    wk = np.eye(hidden)[: hkv * d]
    wv = -np.eye(hidden)[2: 2 + hkv * d]
    slots = np.array([10, -1, 0, 17])
    kc, vc = append(x, w, 1e-6, wk, wv, slots, sentinel, sentinel)
    xhat = x / np.sqrt((x * x).mean(axis=1, keepdims=True) + 1e-6)
    expected_k = sentinel.copy()
    expected_v = sentinel.copy()
    for t, (blk, off) in {0: (2, 2), 2: (0, 0), 3: (4, 1)}.items():
        expected_k[blk, :, off, :] = xhat[t, : hkv * d].reshape(hkv, d)
        expected_v[blk, :, off, :] = -xhat[t, 2: 2 + hkv * d].reshape(hkv, d)
    np.testing.assert_allclose(kc, expected_k, atol=1e-14)
    np.testing.assert_allclose(vc, expected_v, atol=1e-14)
    changed = (kc != sentinel).any(axis=(1, 3))
    assert changed.sum() == 3


APPEND_CHECKS = [check_append_scatter]


# ---------------------------------------------------------------------------
# gather checks
# ---------------------------------------------------------------------------

def check_gather_pages(gather):
    """The pages' worked examples: query_start_loc [0,15,20,28] keeps rows
    14, 19 and 27; the three scheduling steps keep rows [5], [0,2], [0,1]."""
    fx = load_golden("vllm_logits_indices_example.json")
    cu = np.array(fx["printed"]["query_start_loc"])
    hidden = np.arange(28 * 3, dtype=np.float32).reshape(28, 3)
    rows, idx = gather(hidden, cu)
    assert idx.tolist() == fx["derived_for_last_token_gather"]["last_index"]
    assert np.array_equal(rows, hidden[idx])
    # the printed request_ids: the largest logits index of each request
    li = np.array(fx["printed"]["logits_indices"])
    rid = np.array(fx["printed"]["request_ids"])
    assert [int(li[rid == r].max()) for r in range(fx["printed"]["num_reqs"])] == idx.tolist()
    sched = load_golden("vllm_schedule_example.json")
    for step in sched["steps"]:
        cu = np.array(step["cu_seqlens"])
        h = np.random.default_rng(step["step"]).standard_normal((int(cu[-1]), 5))
        rows, idx = gather(h, cu)
        assert idx.tolist() == step["last_row"]
        assert np.array_equal(rows, h[idx])


def check_gather_bits(gather):
    """Rows are copied bit for bit (NaN payloads included); a request with no
    scheduled rows gets a zero row and index -1."""
    rng = np.random.default_rng(41)
    bits = rng.integers(0, 2 ** 32, size=(9, 6), dtype=np.uint64).astype(np.uint32)
    bits[3, 0] = 0x7FC01234
    cu = np.array([0, 2, 2, 4, 9])
    rows, idx = gather(bits, cu)
    assert idx.tolist() == [1, -1, 3, 8]
    assert np.array_equal(rows[0], bits[1]) and np.array_equal(rows[2], bits[3])
    assert np.array_equal(rows[3], bits[8]) and not rows[1].any()


GATHER_CHECKS = [check_gather_pages, check_gather_bits]
