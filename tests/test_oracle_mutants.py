"""Plant plausible mistakes in copies of the oracle (on the CPU) and require
each one to fail at least one pin: evidence that the pins can tell a wrong
oracle from a right one."""

import numpy as np
import pytest
import torch

import oracle
from oracle import yoco_oracle as yo
from tests import oracle_pins as pins


def _attn_variant(score_fn=None, group_fn=None, n_fn=None, locate=None, combine=None):
    """A copy of the oracle's attention with one step replaced."""
    def attn(q, k_cache, v_cache, block_table, seq_lens, scale):
        q = np.asarray(q)
        nreq, hq, d = q.shape
        hkv = k_cache.shape[1]
        bs = k_cache.shape[2]
        out = np.zeros((nreq, hq, d))
        for r in range(nreq):
            n = int(seq_lens[r]) if n_fn is None else n_fn(int(seq_lens[r]))
            if n <= 0:
                continue
            ks, vs = [], []
            for j in range(n):
                blk, off = (block_table[r][j // bs], j % bs) if locate is None else locate(block_table[r], j, bs)
                ks.append(np.asarray(k_cache[blk, :, off, :], dtype=np.float64))
                vs.append(np.asarray(v_cache[blk, :, off, :], dtype=np.float64))
            ks, vs = np.stack(ks), np.stack(vs)
            for h in range(hq):
                g = h // (hq // hkv) if group_fn is None else group_fn(h, hq, hkv)
                s = scale * (ks[:, g, :] @ q[r, h]) if score_fn is None else score_fn(ks[:, g, :], q[r, h], scale)
                if combine is None:
                    w = np.exp(s - s.max())
                    out[r, h] = (w @ vs[:, g, :]) / w.sum()
                else:
                    out[r, h] = combine(s, ks[:, g, :], vs[:, g, :])
        return out
    return attn


ATTN_MUTANTS = {
    "scale_dropped": _attn_variant(score_fn=lambda k, q, s: k @ q),
    "sign_flipped": _attn_variant(score_fn=lambda k, q, s: -s * (k @ q)),
    "gqa_interleaved": _attn_variant(group_fn=lambda h, hq, hkv: h % hkv),
    "context_exclusive": _attn_variant(n_fn=lambda n: n - 1),
    "block_offset_swapped": _attn_variant(locate=lambda t, j, bs: (t[j % bs], j // bs) if j % bs < len(t) else (t[0], 0)),
    "no_normalisation": _attn_variant(combine=lambda s, k, v: np.exp(s - s.max()) @ v),
    "keys_as_values": _attn_variant(combine=lambda s, k, v: (np.exp(s - s.max()) @ k) / np.exp(s - s.max()).sum()),
    "no_max_subtraction": _attn_variant(combine=lambda s, k, v: (np.exp(s) @ v) / np.exp(s).sum()),
}


def _proj_variant(norm=None, post=None):
    def project(x, rms_weight, eps, w_k, w_v, num_kv_heads, head_dim):
        x = np.asarray(x, dtype=np.float64)
        w = np.asarray(rms_weight, dtype=np.float64)
        xh = yo.rms_norm(x, w, eps) if norm is None else norm(x, w, eps)
        wk = np.asarray(w_k, dtype=np.float64)
        wv = np.asarray(w_v, dtype=np.float64)
        t = x.shape[0]
        k = xh @ wk.T
        v = xh @ wv.T
        if post is not None:
            k, v = post(k, v, num_kv_heads, head_dim)
        k = k.reshape(t, num_kv_heads, head_dim)
        v = v.reshape(t, num_kv_heads, head_dim)
        bk = (np.abs(xh) @ np.abs(wk).T).reshape(t, num_kv_heads, head_dim)
        bv = (np.abs(xh) @ np.abs(wv).T).reshape(t, num_kv_heads, head_dim)
        return k, v, bk, bv
    return project


def _dh_order(k, v, hkv, d):
    t = k.shape[0]
    return (k.reshape(t, d, hkv).transpose(0, 2, 1).reshape(t, -1),
            v.reshape(t, d, hkv).transpose(0, 2, 1).reshape(t, -1))


PROJ_MUTANTS = {
    "sum_not_mean": _proj_variant(norm=lambda x, w, e: x / np.sqrt((x * x).sum(axis=1, keepdims=True) + e) * w),
    "eps_outside_sqrt": _proj_variant(norm=lambda x, w, e: x / (np.sqrt((x * x).mean(axis=1, keepdims=True)) + e) * w),
    "weight_ignored": _proj_variant(norm=lambda x, w, e: x / np.sqrt((x * x).mean(axis=1, keepdims=True) + e)),
    "layernorm_centred": _proj_variant(norm=lambda x, w, e: (x - x.mean(axis=1, keepdims=True))
                                       / np.sqrt(x.var(axis=1, keepdims=True) + e) * w),
    "k_v_swapped": _proj_variant(post=lambda k, v, h, d: (v, k)),
    "head_dim_order": _proj_variant(post=_dh_order),
}


def _append_variant(decompose):
    def append(x, rms_weight, eps, w_k, w_v, slot_mapping, k_cache, v_cache):
        nb, hkv, bs, d = k_cache.shape
        k, v, _, _ = yo.kv_project(x, rms_weight, eps, w_k, w_v, hkv, d)
        kc = np.asarray(k_cache, dtype=np.float64).copy()
        vc = np.asarray(v_cache, dtype=np.float64).copy()
        for t, slot in enumerate(slot_mapping):
            res = decompose(int(slot), bs, nb)
            if res is None:
                continue
            kc[res[0], :, res[1], :] = k[t]
            vc[res[0], :, res[1], :] = v[t]
        return kc, vc
    return append


APPEND_MUTANTS = {
    "offset_block_swapped": _append_variant(lambda s, bs, nb: None if s < 0 else (s % bs, s // bs) if s % bs < nb and s // bs < bs else (0, 0)),
    "padding_not_skipped": _append_variant(lambda s, bs, nb: divmod(s % (nb * bs), bs)),
}


def _gather_variant(pick):
    def gather(hidden, cu_seqlens):
        hidden = np.asarray(hidden)
        cu = [int(c) for c in cu_seqlens]
        rows = np.zeros((len(cu) - 1,) + hidden.shape[1:], dtype=hidden.dtype)
        idx = np.full(len(cu) - 1, -1, dtype=np.int32)
        for r in range(len(cu) - 1):
            i = pick(cu, r)
            if i is not None and 0 <= i < hidden.shape[0]:
                idx[r] = i
                rows[r] = hidden[i]
        return rows, idx
    return gather


GATHER_MUTANTS = {
    "first_token": _gather_variant(lambda cu, r: cu[r] if cu[r + 1] > cu[r] else None),
    "off_by_one": _gather_variant(lambda cu, r: cu[r + 1] if cu[r + 1] > cu[r] else None),
    "empty_not_handled": _gather_variant(lambda cu, r: cu[r + 1] - 1),
}


def _varlen_variant(positions=None, keep=None):
    """A copy of the varlen attention with the query placement or the key
    selection replaced."""
    def attn(q, k_cache, v_cache, block_table, seq_lens, query_start_loc, scale, window=0):
        q = np.asarray(q)
        nrow, hq, d = q.shape
        hkv = k_cache.shape[1]
        qsl = [int(c) for c in query_start_loc]
        out = np.zeros((nrow, hq, d))
        for r in range(len(qsl) - 1):
            n = int(seq_lens[r])
            ql = qsl[r + 1] - qsl[r]
            if ql == 0 or n <= 0:
                continue
            ks, vs = yo.logical_kv(k_cache, v_cache, block_table[r], n)
            pos = [n - ql + i for i in range(ql)] if positions is None else positions(n, ql)
            for i, p in enumerate(pos):
                sel = [j for j in range(n) if (j <= p and (window <= 0 or j > p - window))] if keep is None \
                    else [j for j in range(n) if keep(j, p, window)]
                if not sel:
                    continue
                for h in range(hq):
                    g = h // (hq // hkv)
                    out[qsl[r] + i, h] = yo.attention_one_query(q[qsl[r] + i, h], ks[sel, g], vs[sel, g], scale)
        return out
    return attn


VARLEN_MUTANTS = {
    "queries_at_start": _varlen_variant(positions=lambda n, ql: list(range(ql))),
    "not_causal": _varlen_variant(keep=lambda j, p, w: w <= 0 or j > p - w),
    "window_ignored": _varlen_variant(keep=lambda j, p, w: j <= p),
    "window_one_longer": _varlen_variant(keep=lambda j, p, w: j <= p and (w <= 0 or j >= p - w)),
    "current_token_excluded": _varlen_variant(keep=lambda j, p, w: j < p and (w <= 0 or j > p - w)),
}


def _metadata_variant(owner=None, offsets=None):
    def meta(logits_indices, query_start_loc):
        qsl = [int(c) for c in query_start_loc]
        nreq = len(qsl) - 1
        rid = np.full(len(logits_indices), -1)
        counts = np.zeros(nreq, dtype=np.int64)
        for i, idx in enumerate(logits_indices):
            r = owner(int(idx), qsl) if owner is not None else \
                next((r for r in range(nreq) if qsl[r] <= int(idx) < qsl[r + 1]), -1)
            if 0 <= r < nreq:
                rid[i] = r
                counts[r] += 1
        cross = np.concatenate([[0], np.cumsum(counts)]) if offsets is None else offsets(counts)
        return rid, counts, cross, int(counts.max()) if nreq else 0
    return meta


METADATA_MUTANTS = {
    "boundary_to_previous": _metadata_variant(owner=lambda idx, qsl: next(
        (r for r in range(len(qsl) - 1) if qsl[r] < idx <= qsl[r + 1]), -1)),
    "exclusive_offsets": _metadata_variant(offsets=lambda c: np.concatenate([[0, 0], np.cumsum(c)[:-1]])),
}


def _decode_variant(bias=7, subnormal_as_normal=False):
    def decode(codes):
        codes = np.asarray(codes, dtype=np.uint8)
        out = np.empty(codes.shape)
        for idx, c in np.ndenumerate(codes):
            c = int(c)
            sign = -1.0 if c & 0x80 else 1.0
            e, m = (c >> 3) & 0xF, c & 7
            if e == 15 and m == 7:
                out[idx] = np.nan
            elif e == 0 and not subnormal_as_normal:
                out[idx] = sign * m * 2.0 ** (1 - bias - 3)
            else:
                out[idx] = sign * (1 + m / 8) * 2.0 ** (e - bias)
        return out
    return decode


def _encode_variant(ties_up=False, no_subnormals=False):
    def encode(x):
        grid = yo.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
        x = np.asarray(x, dtype=np.float64)
        out = np.empty(x.shape, dtype=np.uint8)
        for idx, v in np.ndenumerate(x):
            if np.isnan(v):
                out[idx] = 0x7F
                continue
            a = min(abs(v), 448.0)
            if no_subnormals and a < 2.0 ** -6:
                a = 0.0
            j = int(np.searchsorted(grid, a))
            if j < len(grid) and grid[j] == a:
                code = j
            else:
                dl, dh = a - grid[j - 1], grid[j] - a
                code = j - 1 if dl < dh else j if dh < dl else (j if ties_up else (j - 1 if (j - 1) % 2 == 0 else j))
            out[idx] = code | (0x80 if np.signbit(v) else 0)
        return out
    return encode


def _quant_variant(qmax=448.0, scale_from_mean=False):
    def quantize(rows):
        rows = np.asarray(rows, dtype=np.float32)
        codes = np.zeros(rows.shape, dtype=np.uint8)
        scales = np.zeros(rows.shape[:-1], dtype=np.float32)
        for idx in np.ndindex(rows.shape[:-1]):
            row = rows[idx]
            ref = np.abs(row).mean() * 3 if scale_from_mean else np.abs(row).max()
            s = np.float32(np.float32(ref) / np.float32(qmax))
            scales[idx] = s
            if s:
                codes[idx] = yo.e4m3_encode(np.float32(row / s))
        return codes, scales
    return quantize


def _append_fp8_variant(round_projection):
    """The 8-bit append quantizing a differently rounded projection."""
    def append_fp8(x, rms_weight, eps, w_k, w_v, slot_mapping, num_kv_heads, head_dim):
        k, v, bk, bv = yo.kv_project(x, rms_weight, eps, w_k, w_v, num_kv_heads, head_dim)
        return k, v, round_projection(k), round_projection(v), bk, bv
    return append_fp8


def _quantize_float64(rows):
    """Scale and quotient in float64, no fp32 rounding anywhere."""
    rows = np.asarray(rows, dtype=np.float64)
    scales = np.abs(rows).max(axis=-1) / 448.0
    codes = np.zeros(rows.shape, dtype=np.uint8)
    for idx in np.ndindex(rows.shape[:-1]):
        if scales[idx]:
            codes[idx] = yo.e4m3_encode(rows[idx] / scales[idx])
    return codes, scales.astype(np.float32)


def _quantize_bf16(rows):
    """The projection rounded to bf16 first, then the fp32 quantizer."""
    r = torch.from_numpy(np.asarray(rows, dtype=np.float64)).to(torch.bfloat16).to(torch.float32).numpy()
    return yo.quantize_rows(r)


APPEND_FP8_MUTANTS = {
    "quantize_float64_projection": _append_fp8_variant(_quantize_float64),
    "quantize_bf16_projection": _append_fp8_variant(_quantize_bf16),
}


FP8_DECODE_MUTANTS = {"bias_8": _decode_variant(bias=8), "subnormal_as_normal": _decode_variant(subnormal_as_normal=True)}
FP8_ENCODE_MUTANTS = {"ties_up": _encode_variant(ties_up=True), "no_subnormals": _encode_variant(no_subnormals=True)}
QUANT_MUTANTS = {"int8_range": _quant_variant(qmax=127.0), "scale_from_mean": _quant_variant(scale_from_mean=True)}


def _retention_variant(update=None, read_before=False, store=True):
    def ret(q, k, v, gamma, cu_seqlens, state, state_indices):
        q, k, v, gamma = (np.asarray(x, dtype=np.float64) for x in (q, k, v, gamma))
        out = np.zeros(v.shape)
        new = np.asarray(state, dtype=np.float64).copy()
        cu = [int(c) for c in cu_seqlens]
        for r in range(len(cu) - 1):
            slot = int(state_indices[r])
            for h in range(q.shape[1]):
                s = new[slot, h].copy() if slot >= 0 else np.zeros((k.shape[2], v.shape[2]))
                for t in range(cu[r], cu[r + 1]):
                    prev = s
                    s = gamma[t, h] * s + np.outer(k[t, h], v[t, h]) if update is None else update(s, gamma[t, h],
                                                                                                  k[t, h], v[t, h])
                    out[t, h] = q[t, h] @ (prev if read_before else s)
                if slot >= 0 and store:
                    new[slot, h] = s
        return out, new
    return ret


RETENTION_MUTANTS = {
    "gate_after_write": _retention_variant(update=lambda s, g, k, v: g * (s + np.outer(k, v))),
    "read_before_write": _retention_variant(read_before=True),
    "gamma_ignored": _retention_variant(update=lambda s, g, k, v: s + np.outer(k, v)),
    "state_not_stored": _retention_variant(store=False),
}


def _fails_some(checks, fn):
    failures = 0
    for check in checks:
        try:
            with np.errstate(all="ignore"):
                check(fn)
        except (AssertionError, ValueError, IndexError):
            failures += 1
    return failures


@pytest.mark.parametrize("name", sorted(ATTN_MUTANTS))
def test_attention_mutant_is_caught(name):
    assert _fails_some(pins.ATTN_CHECKS, ATTN_MUTANTS[name]) > 0


@pytest.mark.parametrize("name", sorted(PROJ_MUTANTS))
def test_projection_mutant_is_caught(name):
    assert _fails_some(pins.PROJ_CHECKS, PROJ_MUTANTS[name]) > 0


@pytest.mark.parametrize("name", sorted(APPEND_MUTANTS))
def test_append_mutant_is_caught(name):
    assert _fails_some(pins.APPEND_CHECKS, APPEND_MUTANTS[name]) > 0


@pytest.mark.parametrize("name", sorted(GATHER_MUTANTS))
def test_gather_mutant_is_caught(name):
    assert _fails_some(pins.GATHER_CHECKS, GATHER_MUTANTS[name]) > 0


def test_unmutated_copies_pass():
    """The mutant scaffolding itself is faithful when nothing is planted."""
    assert _fails_some(pins.ATTN_CHECKS, _attn_variant()) == 0
    assert _fails_some(pins.PROJ_CHECKS, _proj_variant()) == 0
    assert _fails_some(pins.GATHER_CHECKS, oracle.gather_last) == 0


@pytest.mark.parametrize("name", sorted(VARLEN_MUTANTS))
def test_varlen_mutant_is_caught(name):
    assert _fails_some(pins.VARLEN_CHECKS, VARLEN_MUTANTS[name]) > 0


@pytest.mark.parametrize("name", sorted(METADATA_MUTANTS))
def test_metadata_mutant_is_caught(name):
    assert _fails_some(pins.METADATA_CHECKS, METADATA_MUTANTS[name]) > 0


def test_unmutated_varlen_copies_pass():
    assert _fails_some(pins.VARLEN_CHECKS, _varlen_variant()) == 0
    assert _fails_some(pins.METADATA_CHECKS, _metadata_variant()) == 0


@pytest.mark.parametrize("name", sorted(FP8_DECODE_MUTANTS))
def test_e4m3_decode_mutant_is_caught(name):
    assert _fails_some(pins.FP8_DECODE_CHECKS, FP8_DECODE_MUTANTS[name]) > 0


@pytest.mark.parametrize("name", sorted(FP8_ENCODE_MUTANTS))
def test_e4m3_encode_mutant_is_caught(name):
    assert _fails_some(pins.FP8_ENCODE_CHECKS, FP8_ENCODE_MUTANTS[name]) > 0


@pytest.mark.parametrize("name", sorted(QUANT_MUTANTS))
def test_quantize_mutant_is_caught(name):
    assert _fails_some(pins.QUANT_CHECKS, QUANT_MUTANTS[name]) > 0


def test_unmutated_fp8_copies_pass():
    assert _fails_some(pins.FP8_DECODE_CHECKS, _decode_variant()) == 0
    assert _fails_some(pins.FP8_ENCODE_CHECKS, _encode_variant()) == 0
    assert _fails_some(pins.QUANT_CHECKS, _quant_variant()) == 0


@pytest.mark.parametrize("name", sorted(RETENTION_MUTANTS))
def test_retention_mutant_is_caught(name):
    assert _fails_some(pins.RETENTION_CHECKS, RETENTION_MUTANTS[name]) > 0


def test_unmutated_retention_copy_passes():
    assert _fails_some(pins.RETENTION_CHECKS, _retention_variant()) == 0


@pytest.mark.parametrize("name", sorted(APPEND_FP8_MUTANTS))
def test_append_fp8_mutant_is_caught(name):
    assert _fails_some(pins.APPEND_FP8_CHECKS, APPEND_FP8_MUTANTS[name]) > 0


def test_unmutated_append_fp8_copy_passes():
    assert _fails_some(pins.APPEND_FP8_CHECKS, _append_fp8_variant(lambda k: yo.quantize_rows(k.astype(np.float32)))) == 0


def _helper_mutants():
    def logical_block_offset_swapped(k_cache, v_cache, table_row, n):
        bs = k_cache.shape[2]
        if n == 0:
            return yo.logical_kv(k_cache, v_cache, table_row, 0)
        keys = [np.asarray(k_cache[table_row[j % bs], :, j // bs], float) for j in range(n)]
        values = [np.asarray(v_cache[table_row[j % bs], :, j // bs], float) for j in range(n)]
        return np.stack(keys), np.stack(values)

    def attn_one_scale_dropped(q, keys, values, scale):
        s = np.asarray(keys) @ np.asarray(q)
        w = np.exp(s - s.max())
        return (w @ values) / w.sum()

    def rms_sum(x, w, eps):
        x = np.asarray(x, float)
        return x / np.sqrt((x * x).sum(axis=1, keepdims=True) + eps) * w

    def positions_first(n, ql):
        return list(range(ql))

    return {"logical_kv": logical_block_offset_swapped, "attention_one_query": attn_one_scale_dropped, "rms_norm": rms_sum,
            "query_positions": positions_first}


@pytest.mark.parametrize("name", sorted(_helper_mutants()))
def test_helper_mutant_is_caught(name):
    assert _fails_some([pins.HELPER_CHECKS[name]], _helper_mutants()[name]) > 0
