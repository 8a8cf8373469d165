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


# ---------------------------------------------------------------------------
# several query rows per request, sliding window  (varlen attention)
# ---------------------------------------------------------------------------

def _band_mask(n, positions, window):
    """bool [len(positions)][n]: query at p sees j <= p, and j > p - window
    when window > 0 (built here directly from the statement, test side)."""
    m = np.zeros((len(positions), n), dtype=bool)
    for i, p in enumerate(positions):
        for j in range(n):
            m[i, j] = j <= p and (window <= 0 or j > p - window)
    return m


def check_varlen_decode_reduction(attn_varlen):
    """One query row per request and no window is the decode attention of
    every request's whole context: the pinned single-query oracle."""
    import oracle
    rng = np.random.default_rng(51)
    q, kc, vc, tables, seq, _, _ = random_problem(rng, [9, 1, 30], 4, 2, 8, 4)
    qsl = np.arange(4)
    got = attn_varlen(q, kc, vc, tables, seq, qsl, 0.3, 0)
    np.testing.assert_allclose(got, oracle.cross_attention(q, kc, vc, tables, seq, 0.3), rtol=0, atol=1e-13)


def check_varlen_sdpa(attn_varlen):
    """Library routine: torch SDPA in float64 with an explicit boolean mask
    (queries on the last positions, causal, optional window) and GQA."""
    rng = np.random.default_rng(52)
    for hq, hkv, d, bs, lens, qlens, window in [
            (4, 2, 8, 4, [11, 6, 17], [3, 1, 2], 0),
            (4, 1, 8, 4, [13, 5], [4, 2], 5),
            (2, 2, 16, 8, [40, 3, 9], [1, 3, 9], 7),
            (8, 2, 4, 2, [2, 21], [5, 1], 1)]:
        _, kc, vc, tables, seq, keys, values = random_problem(rng, lens, hq, hkv, d, bs)
        qsl = np.concatenate([[0], np.cumsum(qlens)])
        q = rng.standard_normal((int(qsl[-1]), hq, d))
        got = attn_varlen(q, kc, vc, tables, seq, qsl, 1.0 / np.sqrt(d), window)
        for r, n in enumerate(lens):
            ql = qlens[r]
            pos = [n - ql + i for i in range(ql)]
            mask = _band_mask(n, pos, window)
            qt = torch.from_numpy(q[qsl[r]:qsl[r + 1]]).permute(1, 0, 2).reshape(1, hq, ql, d).contiguous()
            kt = torch.from_numpy(keys[r]).permute(1, 0, 2).reshape(1, hkv, n, d).contiguous()
            vt = torch.from_numpy(values[r]).permute(1, 0, 2).reshape(1, hkv, n, d).contiguous()
            live = mask.any(axis=1)
            ref = F.scaled_dot_product_attention(qt[:, :, live], kt, vt, attn_mask=torch.from_numpy(mask[live]),
                                                 enable_gqa=(hq != hkv))
            ref = ref.reshape(hq, int(live.sum()), d).permute(1, 0, 2).numpy()
            np.testing.assert_allclose(got[qsl[r]:qsl[r + 1]][live], ref, rtol=0, atol=1e-12)
            assert not got[qsl[r]:qsl[r + 1]][~live].any()


def check_varlen_closed_forms(attn_varlen):
    """A window of one returns each query's own V row exactly; a window as
    long as the context changes nothing; with more queries than cached tokens
    the queries before position 0 give zeros; the last query of a request
    sees the whole context."""
    import oracle
    rng = np.random.default_rng(53)
    lens, qlens = [10, 4, 7], [3, 6, 1]
    _, kc, vc, tables, seq, keys, values = random_problem(rng, lens, 4, 2, 8, 4)
    qsl = np.concatenate([[0], np.cumsum(qlens)])
    q = rng.standard_normal((int(qsl[-1]), 4, 8))
    one = attn_varlen(q, kc, vc, tables, seq, qsl, 0.5, 1)
    for r, n in enumerate(lens):
        for i in range(qlens[r]):
            p = n - qlens[r] + i
            row = one[qsl[r] + i]
            if p < 0:
                assert not row.any()
            else:
                for h in range(4):
                    assert np.array_equal(row[h], values[r][p, h // 2])
    full = attn_varlen(q, kc, vc, tables, seq, qsl, 0.5, 0)
    np.testing.assert_allclose(attn_varlen(q, kc, vc, tables, seq, qsl, 0.5, 10), full, rtol=0, atol=0)
    assert not full[qsl[1]:qsl[1] + 2].any()           # request 1: positions -2, -1
    last = q[qsl[1:] - 1]
    np.testing.assert_allclose(full[qsl[1:] - 1], oracle.cross_attention(last, kc, vc, tables, seq, 0.5),
                               rtol=0, atol=1e-13)


def check_varlen_decimal(attn_varlen):
    """Brute force in 50-digit decimal: each query over its own causal window."""
    rng = np.random.default_rng(54)
    for window in (0, 3):
        lens, qlens = [7, 5], [3, 2]
        _, kc, vc, tables, seq, keys, values = random_problem(rng, lens, 2, 1, 4, 4)
        qsl = np.concatenate([[0], np.cumsum(qlens)])
        q = rng.standard_normal((int(qsl[-1]), 2, 4))
        got = attn_varlen(q, kc, vc, tables, seq, qsl, 0.5, window)
        for r, n in enumerate(lens):
            for i in range(qlens[r]):
                p = n - qlens[r] + i
                lo = 0 if window == 0 else max(0, p - window + 1)
                for h in range(2):
                    ref = _dec_attention(q[qsl[r] + i, h], keys[r][lo:p + 1, 0], values[r][lo:p + 1, 0], 0.5)
                    np.testing.assert_allclose(got[qsl[r] + i, h], ref, rtol=0, atol=1e-13)


VARLEN_CHECKS = [check_varlen_decode_reduction, check_varlen_sdpa, check_varlen_closed_forms, check_varlen_decimal]


def check_metadata_page_example(meta_fn):
    """The page's printed example: logits rows [14,18,19,27] of a batch with
    query_start_loc [0,15,20,28] belong to requests [0,1,1,2], counted
    [1,2,1], giving the cross-decoder query_start_loc [0,1,3,4]."""
    fx = load_golden("vllm_logits_indices_example.json")["printed"]
    rid, counts, qsl, mx = meta_fn(np.array(fx["logits_indices"]), np.array(fx["query_start_loc"]))
    assert rid.tolist() == fx["request_ids"]
    assert counts.tolist() == fx["num_decode_tokens"]
    assert qsl.tolist() == fx["decode_query_start_loc"]
    assert mx == max(fx["num_decode_tokens"])


def check_metadata_torch(meta_fn):
    """Library routines: torch.bucketize(right=True) over query_start_loc[1:],
    bincount and cumsum on random batches (indices inside the batch), with
    empty requests and indices on request boundaries."""
    rng = np.random.default_rng(55)
    for trial in range(20):
        lens = rng.integers(0, 6, size=int(rng.integers(1, 7)))
        qsl = np.concatenate([[0], np.cumsum(lens)])
        total = int(qsl[-1])
        if total == 0:
            continue
        idx = np.sort(rng.choice(total, size=int(rng.integers(1, total + 1)), replace=False))
        idx = np.unique(np.concatenate([idx, qsl[1:-1][qsl[1:-1] < total]]))
        rid, counts, cross, mx = meta_fn(idx, qsl)
        t_rid = torch.bucketize(torch.from_numpy(idx), torch.from_numpy(qsl[1:]), right=True)
        t_cnt = torch.bincount(t_rid, minlength=len(lens))
        assert rid.tolist() == t_rid.tolist()
        assert counts.tolist() == t_cnt.tolist()
        assert cross.tolist() == [0] + torch.cumsum(t_cnt, 0).tolist()
        assert mx == int(t_cnt.max())


def check_gather_rows_bits(gather_rows_fn):
    """Selected rows are copied bit for bit in the order given; an index
    outside the batch gives a zero row."""
    rng = np.random.default_rng(56)
    bits = rng.integers(0, 2 ** 32, size=(8, 5), dtype=np.uint64).astype(np.uint32)
    bits[6, 2] = 0x7FC0BEEF
    rows = gather_rows_fn(bits, np.array([6, 0, 6, 9, -1, 7]))
    assert np.array_equal(rows[0], bits[6]) and np.array_equal(rows[1], bits[0])
    assert np.array_equal(rows[2], bits[6]) and np.array_equal(rows[5], bits[7])
    assert not rows[3].any() and not rows[4].any()


METADATA_CHECKS = [check_metadata_page_example, check_metadata_torch]
GATHER_ROWS_CHECKS = [check_gather_rows_bits]


# ---------------------------------------------------------------------------
# 8-bit cache: FP8 E4M3 codes, per-row scales
# ---------------------------------------------------------------------------

def check_e4m3_decode(decode):
    """Library routine: torch's float8_e4m3fn interpretation of all 256 codes;
    closed forms: 0x7E = 448 (largest), 0x01 = 2^-9 (smallest subnormal),
    0x08 = 2^-6 (smallest normal), 0x38 = 1, 0x7F and 0xFF are NaN."""
    codes = np.arange(256, dtype=np.uint8)
    got = decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(got, ref, equal_nan=True)
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6 and got[0x38] == 1.0
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and got[0xFE] == -448.0


def check_e4m3_encode(encode):
    """Library routine: torch's round-to-nearest-even conversion to
    float8_e4m3fn on values across the whole range (subnormals included);
    closed forms: ties go to the even code (1 + 1/16 -> 1, 1 + 3/16 -> 1.25),
    448 -> 0x7E, -0.0 -> 0x80, NaN -> 0x7F."""
    rng = np.random.default_rng(61)
    x = np.concatenate([rng.standard_normal(4000) * 60, rng.standard_normal(2000) * 2.0 ** -7,
                        rng.uniform(-448, 448, 2000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(encode(x), ref)
    ties = np.array([1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -10, 448.0, -0.0, np.nan], dtype=np.float32)
    assert encode(ties).tolist() == [0x38, 0x3A, 0xB8, 0x00, 0x02, 0x7E, 0x80, 0x7F]


def check_quantize_rows(quantize):
    """Each row's largest magnitude becomes the code of +-448 and its scale is
    the value that maps back to it; codes equal torch's conversion of the fp32
    quotient; scaling a row by 2^k scales its scale by 2^k and keeps the codes;
    a zero row has scale 0 and zero codes; every value comes back within half
    an E4M3 step."""
    rng = np.random.default_rng(62)
    rows = (rng.standard_normal((5, 3, 16)) * rng.uniform(0.01, 30, size=(5, 3, 1))).astype(np.float32)
    rows[1, 2] = 0.0
    codes, scales = quantize(rows)
    assert codes.dtype == np.uint8 and scales.dtype == np.float32 and scales.shape == (5, 3)
    for idx in np.ndindex(5, 3):
        row = rows[idx]
        if not row.any():
            assert scales[idx] == 0 and not codes[idx].any()
            continue
        j = int(np.argmax(np.abs(row)))
        assert codes[idx][j] == (0xFE if row[j] < 0 else 0x7E)
        quotient = torch.from_numpy(row) / torch.tensor(scales[idx])
        assert np.array_equal(codes[idx], quotient.to(torch.float8_e4m3fn).view(torch.uint8).numpy())
        back = torch.from_numpy(codes[idx]).view(torch.float8_e4m3fn).to(torch.float64).numpy() * float(scales[idx])
        step = np.maximum(np.abs(row) * 2.0 ** -3, float(scales[idx]) * 2.0 ** -9)   # one ulp bound per value
        assert (np.abs(back - row) <= step / 2 * (1 + 1e-6)).all()
        assert abs(float(scales[idx]) * 448.0 - float(np.abs(row).max())) <= float(np.abs(row).max()) * 2.0 ** -23
    c2, s2 = quantize(rows * np.float32(8.0))
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales * np.float32(8.0))


def check_kv_scatter(scatter):
    """Rows land in slot s = block s // block_size, row s % block_size for every
    KV head (hand-worked: block size 4, slot 10 -> block 2 row 2); negative
    slots write nothing; with an 8-bit cache the stored code times the scale
    gives the row back within half an E4M3 step; untouched entries keep their
    bits."""
    rng = np.random.default_rng(63)
    nb, hkv, bs, d = 5, 2, 4, 8
    rows_k = rng.standard_normal((3, hkv, d)).astype(np.float32)
    rows_v = rng.standard_normal((3, hkv, d)).astype(np.float32)
    slots = np.array([10, -1, 17])
    kc0 = np.full((nb, hkv, bs, d), -3.5, dtype=np.float32)
    kc, vc = scatter(rows_k, rows_v, slots, kc0, kc0)
    assert np.array_equal(kc[2, :, 2], rows_k[0]) and np.array_equal(vc[4, :, 1], rows_v[2])
    assert (kc != kc0).any(axis=(1, 3)).sum() == 2
    codes0 = np.full((nb, hkv, bs, d), 0x55, dtype=np.uint8)
    sc0 = np.full((nb, hkv, bs), 9.0, dtype=np.float32)
    kq, vq, ks, vs = scatter(rows_k, rows_v, slots, codes0, codes0, sc0, sc0)
    for t, (blk, off) in {0: (2, 2), 2: (4, 1)}.items():
        for rows, codes, sc in ((rows_k, kq, ks), (rows_v, vq, vs)):
            back = torch.from_numpy(codes[blk, :, off]).view(torch.float8_e4m3fn).to(torch.float64).numpy()
            back = back * sc[blk, :, off][:, None]
            assert (np.abs(back - rows[t]) <= np.abs(rows[t]) * 2.0 ** -4 + sc[blk, :, off][:, None] * 2.0 ** -10).all()
    changed = (kq != codes0).any(axis=(1, 3)) | (ks != sc0).any(axis=1)
    assert changed.sum() == 2


def check_append_fp8_rounding(append_fp8):
    """The 8-bit append quantizes the projection after one rounding to fp32
    (the precision the kernel decides each code in): with x a row of ones and
    eps = 0, xhat is exactly the RMS weight, and unit-vector weight rows copy
    chosen entries of it into K and V.  The entries are built so that the
    fp32-rounded value and the exact value lie on opposite sides of an E4M3
    rounding midpoint (or a bf16 rounding moves the value onto one).  The
    scale is the power of two 2^-3 (the largest entry is 448 * 2^-3), so every
    quotient is exact and the expected codes are hand-worked closed forms;
    torch's float8_e4m3fn conversion of the fp32 quotient (library routine)
    must agree with them and with every other code."""
    e = 2.0 ** -3
    entries = np.array([
        448.0 * e,                              # the largest: code 0x7E, scale 2^-3
        (1.0625 + 2.0 ** -26) * e,              # fp32 -> midpoint 1 + 1/16 -> even 1.0 (0x38); exact -> 1.125
        -(1.1875 - 2.0 ** -26) * e,             # fp32 -> midpoint 1 + 3/16 -> even -1.25 (0xBA); exact -> -1.125
        (1.5 - 2.0 ** -26) * 2.0 ** -9 * e,     # fp32 -> subnormal midpoint 1.5 * 2^-9 -> 2 * 2^-9 (0x02); exact -> 0x01
        (1.0625 + 2.0 ** -9) * e,               # kept by fp32 -> 1.125 (0x39); a bf16 rounding -> 1.0625 -> 0x38
        0.0,
        2.3 * e,
        -300.0 * e,
    ])
    hand = {0: 0x7E, 1: 0x38, 2: 0xBA, 3: 0x02, 4: 0x39, 5: 0x00}
    hidden = len(entries)
    x = np.ones((1, hidden))
    wk = np.eye(hidden)                         # K = xhat
    wv = np.eye(hidden)[::-1].copy()            # V = xhat reversed
    k, v, (ck, sk), (cv, sv), _, _ = append_fp8(x, entries, 0.0, wk, wv, np.array([0]), 1, hidden)
    np.testing.assert_array_equal(np.asarray(k).reshape(-1), entries)
    np.testing.assert_array_equal(np.asarray(v).reshape(-1), entries[::-1])
    assert np.asarray(sk).reshape(-1).tolist() == [e] and np.asarray(sv).reshape(-1).tolist() == [e]
    k32 = torch.from_numpy(entries).to(torch.float32)
    ref = (k32 / torch.tensor(e, dtype=torch.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for i, code in hand.items():
        assert ref[i] == code, (i, hex(int(ref[i])))
    assert np.asarray(ck).reshape(-1).tolist() == ref.tolist()
    assert np.asarray(cv).reshape(-1).tolist() == ref[::-1].tolist()


FP8_DECODE_CHECKS = [check_e4m3_decode]
FP8_ENCODE_CHECKS = [check_e4m3_encode]
QUANT_CHECKS = [check_quantize_rows]
SCATTER_CHECKS = [check_kv_scatter]
APPEND_FP8_CHECKS = [check_append_fp8_rounding]


# ---------------------------------------------------------------------------
# helpers the pinned functions are built from, pinned on their own
# ---------------------------------------------------------------------------

def check_logical_kv(logical_kv):
    """The pages' Replay figure: logical blocks 0,1,2,3 on physical pages
    0,2,1,4 (pages 3 and 5 free) come back in logical order, the last block
    cut at the context length; a context of 0 gives empty arrays."""
    fx = load_golden("kv_block_table_replay.json")
    table = np.array(fx["block_table"])
    bs, hkv, d = 4, 2, 3
    pages = len(fx["physical_pages"])
    kc = np.full((pages, hkv, bs, d), np.nan)
    vc = np.full((pages, hkv, bs, d), np.nan)
    for logical, page in enumerate(table):
        for off in range(bs):
            for g in range(hkv):
                kc[page, g, off] = 100 * logical + 10 * off + g + np.arange(d) / 8
                vc[page, g, off] = -kc[page, g, off]
    n = 14
    keys, values = logical_kv(kc, vc, table, n)
    assert keys.shape == (n, hkv, d) and values.shape == (n, hkv, d)
    for j in range(n):
        for g in range(hkv):
            want = 100 * (j // bs) + 10 * (j % bs) + g + np.arange(d) / 8
            assert np.array_equal(keys[j, g], want) and np.array_equal(values[j, g], -want)
    k0, v0 = logical_kv(kc, vc, table, 0)
    assert k0.shape == (0, hkv, d) and v0.shape == (0, hkv, d)


def check_attention_one_query(attn_one):
    """Library routine: torch SDPA in float64 for one query; closed forms: one
    key gives its value row exactly, identical keys give the mean of the
    values."""
    rng = np.random.default_rng(71)
    for n, d in [(1, 4), (9, 8), (33, 16)]:
        q = rng.standard_normal(d)
        keys = rng.standard_normal((n, d))
        values = rng.standard_normal((n, d))
        got = attn_one(q, keys, values, 0.37)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q).reshape(1, 1, d),
                                             torch.from_numpy(keys).reshape(1, n, d),
                                             torch.from_numpy(values).reshape(1, n, d), scale=0.37).reshape(d)
        np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-12)
    values = rng.standard_normal((1, 5))
    assert np.array_equal(attn_one(rng.standard_normal(5), rng.standard_normal((1, 5)), values, 1.0), values[0])
    keys = np.tile(rng.standard_normal(5), (6, 1))
    values = rng.standard_normal((6, 5))
    np.testing.assert_allclose(attn_one(rng.standard_normal(5), keys, values, 0.5), values.mean(axis=0), atol=1e-14)


def check_rms_norm(rms):
    """Library routine: torch.nn.functional.rms_norm in float64; closed form:
    a constant row c gives c / sqrt(c^2 + eps) * w."""
    rng = np.random.default_rng(72)
    x = rng.standard_normal((4, 10)) * rng.uniform(0.1, 9.0, size=(4, 1))
    w = rng.uniform(0.5, 1.5, size=10)
    for eps in (1e-6, 0.5):
        ref = F.rms_norm(torch.from_numpy(x), (10,), torch.from_numpy(w), eps=eps).numpy()
        np.testing.assert_allclose(rms(x, w, eps), ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(rms(np.full((1, 10), -2.0), w, 0.25), -2.0 / np.sqrt(4.25) * w[None, :], atol=1e-15)


def check_query_positions(positions):
    """The vLLM page's example: request 1 has seq_len 31 and two logits rows,
    which sit at its last two positions, 29 and 30; more query rows than
    context tokens put the first ones below position 0."""
    fx = load_golden("vllm_logits_indices_example.json")["printed"]
    assert positions(fx["seq_lens"][1], fx["num_decode_tokens"][1]) == [29, 30]
    assert positions(fx["seq_lens"][0], 1) == [40]
    assert positions(2, 4) == [-2, -1, 0, 1]
    assert positions(5, 0) == []


HELPER_CHECKS = {
    "logical_kv": check_logical_kv,
    "attention_one_query": check_attention_one_query,
    "rms_norm": check_rms_norm,
    "query_positions": check_query_positions,
}


# ---------------------------------------------------------------------------
# gated retention (self-decoder)
# ---------------------------------------------------------------------------

def _retention_problem(rng, lens, h=2, dk=4, dv=3, slots=4, gamma_range=(0.5, 1.0)):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    t = int(cu[-1])
    q = rng.standard_normal((t, h, dk))
    k = rng.standard_normal((t, h, dk))
    v = rng.standard_normal((t, h, dv))
    g = rng.uniform(*gamma_range, size=(t, h))
    state = rng.standard_normal((slots, h, dk, dv))
    idx = rng.permutation(slots)[:len(lens)]
    return q, k, v, g, cu, state, idx


def check_retention_parallel_form(ret):
    """The parallel form, derived by unrolling the recurrence (written here
    independently as a double sum): o_t = sum_{s<=t} (prod_{s<u<=t} g_u)
    (q_t . k_s) v_s + (prod_{u<=t} g_u) q_t S_0, over each request's rows."""
    rng = np.random.default_rng(71)
    q, k, v, g, cu, state, idx = _retention_problem(rng, [5, 1, 7])
    out, new_state = ret(q, k, v, g, cu, state, idx)
    for r in range(len(cu) - 1):
        a, b = int(cu[r]), int(cu[r + 1])
        for h in range(q.shape[1]):
            for t in range(a, b):
                ref = np.prod(g[a:t + 1, h]) * (q[t, h] @ state[idx[r], h])
                for s_ in range(a, t + 1):
                    ref = ref + np.prod(g[s_ + 1:t + 1, h]) * (q[t, h] @ k[s_, h]) * v[s_, h]
                np.testing.assert_allclose(out[t, h], ref, rtol=0, atol=1e-12)
            fin = np.prod(g[a:b, h]) * state[idx[r], h]
            for s_ in range(a, b):
                fin = fin + np.prod(g[s_ + 1:b, h]) * np.outer(k[s_, h], v[s_, h])
            np.testing.assert_allclose(new_state[idx[r], h], fin, rtol=0, atol=1e-12)


def check_retention_linear_attention(ret):
    """Library routine: with gamma = 1 and a zero state it is causal linear
    attention, tril(Q K^T) V per head (torch matmul + tril in float64)."""
    rng = np.random.default_rng(72)
    q, k, v, g, cu, state, idx = _retention_problem(rng, [9, 4])
    g[:] = 1.0
    state[:] = 0.0
    out, _ = ret(q, k, v, g, cu, state, idx)
    for r in range(len(cu) - 1):
        a, b = int(cu[r]), int(cu[r + 1])
        for h in range(q.shape[1]):
            qt, kt, vt = (torch.from_numpy(x[a:b, h]) for x in (q, k, v))
            ref = torch.tril(qt @ kt.T) @ vt
            np.testing.assert_allclose(out[a:b, h], ref.numpy(), rtol=0, atol=1e-12)


def check_retention_closed_forms(ret):
    """gamma = 0 keeps only the current token: o_t = (q_t . k_t) v_t and the
    final state is k_T^T v_T; a negative slot starts from zeros and leaves
    every slot unchanged."""
    rng = np.random.default_rng(73)
    q, k, v, g, cu, state, idx = _retention_problem(rng, [3, 6])
    g[:] = 0.0
    out, new_state = ret(q, k, v, g, cu, state, idx)
    for t in range(q.shape[0]):
        for h in range(q.shape[1]):
            np.testing.assert_allclose(out[t, h], (q[t, h] @ k[t, h]) * v[t, h], rtol=0, atol=1e-13)
    for r in range(2):
        last = int(cu[r + 1]) - 1
        for h in range(q.shape[1]):
            np.testing.assert_allclose(new_state[idx[r], h], np.outer(k[last, h], v[last, h]), rtol=0, atol=1e-13)
    q, k, v, g, cu, state, idx = _retention_problem(rng, [4])
    out, new_state = ret(q, k, v, g, cu, state, np.array([-1]))
    assert np.array_equal(new_state, state)
    ref, _ = ret(q, k, v, g, cu, np.zeros_like(state), np.array([0]))
    np.testing.assert_allclose(out, ref, rtol=0, atol=0)


def check_retention_carry(ret):
    """Splitting every request's rows into two calls, the state carried in
    its slot, gives the single call's outputs and final state."""
    rng = np.random.default_rng(74)
    lens = [6, 3, 8]
    q, k, v, g, cu, state, idx = _retention_problem(rng, lens)
    out, fin = ret(q, k, v, g, cu, state, idx)
    first = [2, 1, 5]
    rows1 = np.concatenate([np.arange(cu[r], cu[r] + first[r]) for r in range(3)])
    rows2 = np.concatenate([np.arange(cu[r] + first[r], cu[r + 1]) for r in range(3)])
    cu1 = np.concatenate([[0], np.cumsum(first)])
    cu2 = np.concatenate([[0], np.cumsum(np.array(lens) - np.array(first))])
    o1, s1 = ret(q[rows1], k[rows1], v[rows1], g[rows1], cu1, state, idx)
    o2, s2 = ret(q[rows2], k[rows2], v[rows2], g[rows2], cu2, s1, idx)
    np.testing.assert_allclose(o1, out[rows1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o2, out[rows2], rtol=0, atol=1e-12)
    np.testing.assert_allclose(s2, fin, rtol=0, atol=1e-12)


def check_retention_decimal(ret):
    """Brute force in 50-digit decimal on a tiny sequence."""
    getcontext().prec = 50
    rng = np.random.default_rng(75)
    q, k, v, g, cu, state, idx = _retention_problem(rng, [4], h=1, dk=2, dv=2, slots=1)
    out, _ = ret(q, k, v, g, cu, state, np.array([0]))
    S = [[Decimal(float(state[0, 0, i, j])) for j in range(2)] for i in range(2)]
    for t in range(4):
        gt = Decimal(float(g[t, 0]))
        S = [[gt * S[i][j] + Decimal(float(k[t, 0, i])) * Decimal(float(v[t, 0, j])) for j in range(2)] for i in range(2)]
        for j in range(2):
            ref = sum(Decimal(float(q[t, 0, i])) * S[i][j] for i in range(2))
            assert abs(out[t, 0, j] - float(ref)) < 1e-13


RETENTION_CHECKS = [check_retention_parallel_form, check_retention_linear_attention, check_retention_closed_forms,
                    check_retention_carry, check_retention_decimal]
