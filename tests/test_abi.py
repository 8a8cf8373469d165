"""The C ABI library without a GPU: it loads, exports every call that
include/yoco.h declares, and rejects bad scalar arguments before launching
anything (these calls return before any HIP call is made)."""

import ctypes
import os
import re

import pytest

from yoco_shared_kv_gather_amd import binding as yb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "yoco.h")
FAKE = 4096          # a non-null, 16-byte aligned address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(yoco_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("yoco_gather_last", "yoco_kv_append", "yoco_cross_attn"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(yb.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(yb.SIGNATURES)


def test_version_and_status_strings():
    lib = yb.lib()
    assert lib.yoco_abi_version() == yb.ABI_VERSION
    for code, text in [(0, "ok"), (1, "invalid argument"), (2, "unsupported shape"),
                       (3, "workspace too small"), (4, "HIP runtime error")]:
        assert yb.status_string(code) == text


def _attn(**kw):
    args = dict(dtype=1, q=FAKE, num_seqs=2, num_q_heads=8, k=FAKE, v=FAKE, num_blocks=10, num_kv_heads=2,
                block_size=16, head_dim=128, table=FAKE, max_blocks=4, seq_lens=FAKE, max_seq_len=64, scale=0.1,
                part=0, flags=0, out=FAKE, ws=FAKE, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return yb.lib().yoco_cross_attn(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), yb.YOCO_ERR_UNSUPPORTED),
    (dict(num_q_heads=6, num_kv_heads=4), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(num_q_heads=48, num_kv_heads=2), yb.YOCO_ERR_UNSUPPORTED),
    (dict(block_size=12), yb.YOCO_ERR_UNSUPPORTED),
    (dict(part=100), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(dtype=7), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(flags=4), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(q=None), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(q=FAKE + 4), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(num_seqs=-1), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(max_seq_len=100000, part=64, ws_bytes=16), yb.YOCO_ERR_WORKSPACE_TOO_SMALL),
    (dict(ws_bytes=yb.CROSS_ATTN_QUEUE_BYTES - 16), yb.YOCO_ERR_WORKSPACE_TOO_SMALL),
    (dict(ws=None), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(scale=float("nan")), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(block_size=4, part=4096), yb.YOCO_ERR_UNSUPPORTED),
])
def test_cross_attn_rejects_before_launch(kw, status):
    assert _attn(**kw) == status
    assert yb.last_error_message()


def test_cross_attn_empty_batch_is_a_noop():
    assert _attn(num_seqs=0) == yb.YOCO_OK


def test_workspace_and_partition_sizes():
    # one partition needs only the work-queue counters
    assert yb.cross_attn_workspace_size(4, 8, 2, 128, 64, 16, 64) == yb.CROSS_ATTN_QUEUE_BYTES
    p = yb.cross_attn_partition_tokens(1, 8, 128, 524288, 32, 0)
    assert p % 64 == 0 and -(-524288 // p) <= 256
    assert yb.cross_attn_partition_tokens(1, 8, 128, 524288, 1, 0) <= 511      # slice of <= 511 blocks
    np_ = -(-1000 // 64)
    size = yb.cross_attn_workspace_size(3, 8, 2, 128, 1000, 16, 64)
    acc = 3 * 8 * np_ * 128 * 4
    assert size == yb.CROSS_ATTN_QUEUE_BYTES + -(-acc // 256) * 256 + 3 * 8 * np_ * 2 * 4
    assert yb.kv_append_workspace_size(yb.DTYPE_BF16, 3072, 8, 128) == 2 * 1024 * 3072 * 2
    assert yb.kv_append_workspace_size(yb.DTYPE_F32, 256, 1, 64) == 0


SPLIT_SHAPES = [
    # (num_seqs, num_kv_heads, head_dim, max_seq_len, block_size)
    (32, 8, 128, 32768, 16),       # decode32x32k
    (1, 8, 128, 524288, 32),       # long512k
    (48, 8, 128, 32768, 16),       # mixed48
    (64, 2, 256, 8192, 16),        # decode64
    (4, 2, 128, 1000, 16),
    (2, 1, 64, 5000, 1),
    (3000, 8, 128, 5000, 16),      # one workgroup per item: no pieces
]


def _split_parts(m, P, Ps, T):
    big = (m - T) // P if m > T else 0
    rest = m - big * P
    return [P] * big + ([Ps] * (rest // Ps) + ([rest % Ps] if rest % Ps else []) if m > 0 else [0])


def test_kernel_choice():
    """Which attention kernel a call runs: the matrix cores for an FP8 cache,
    for several query rows per request, and for bf16 at head_dim 256 while
    its partitions hold at least 512 tokens; the vector ALUs otherwise, when
    forced, below block_size 16 or above 2048 requests."""
    bf, f8, f32 = yb.DTYPE_BF16, yb.DTYPE_FP8_E4M3, yb.DTYPE_F32
    k = yb.cross_attn_kernel
    d64 = (64, 2, 256, 8192, 16)                       # decode64's sizes
    assert k(*d64, dtype=bf) == "matrix"
    assert yb.cross_attn_partition_split(*d64, dtype=bf)[0] >= 512
    for w in (512, 1024, 2048, 4096):
        short = yb.cross_attn_partition_split(*d64, dtype=bf, window=w)[0] < 512
        assert short == (w <= 2048)
        assert k(*d64, dtype=bf, window=w) == ("vector" if short else "matrix")
        assert k(*d64, dtype=bf, window=w, max_query_len=4) == "matrix"
        assert k(*d64, dtype=f8, window=w) == "matrix"
    assert k(*d64, dtype=bf, partition_tokens=256) == "vector"
    assert k(*d64, dtype=bf, partition_tokens=512) == "matrix"
    assert k(32, 8, 128, 32768, 16, dtype=bf) == "vector"
    assert k(32, 8, 128, 32768, 16, dtype=bf, max_query_len=4) == "matrix"
    assert k(32, 8, 128, 32768, 16, dtype=f8) == "matrix"
    assert k(32, 8, 128, 32768, 16, dtype=f32, max_query_len=4) == "vector"
    assert k(32, 8, 128, 32768, 16, dtype=f8, flags=yb.FLAG_VECTOR_KERNEL) == "vector"
    assert k(32, 8, 128, 32768, 8, dtype=f8) == "vector"
    assert k(4096, 8, 128, 32768, 16, dtype=f8) == "vector"
    assert k(32, 8, 128, 32768, 0, dtype=f8) is None
    assert k(32, 8, 128, -1, 16, dtype=f8) is None


@pytest.mark.parametrize("shape", SPLIT_SHAPES)
@pytest.mark.parametrize("dtype", [yb.DTYPE_F32, yb.DTYPE_BF16, yb.DTYPE_FP8_E4M3])
def test_partition_split_tiles_every_range(shape, dtype):
    """The split the library reports: full partitions of P tokens, then pieces
    of Ps (the last one shorter) covering at least min(m, T) tokens; together
    they tile every key range of m <= max_seq_len tokens, and the reported
    count is the most any such range gets (attained, so the workspace holds no
    idle slots beyond it).  Pieces on the persistent schedule of either kernel
    (the matrix-core kernel, which runs an FP8 cache, several rows and bf16 at
    head_dim 256 with long enough partitions when block_size >= 16, with at
    least ~2048 items instead of ~1024 over an FP8 cache)."""
    R, hkv, d, max_len, bs = shape
    P, Ps, T, most = yb.cross_attn_partition_split(R, hkv, d, max_len, bs, 0, dtype)
    matrix = yb.cross_attn_kernel(R, hkv, d, max_len, bs, 0, dtype) == "matrix"
    if not (matrix and dtype == yb.DTYPE_FP8_E4M3):       # the bf16 matrix plan is the vector kernel's
        assert P == yb.cross_attn_partition_tokens(R, hkv, d, max_len, bs, 0)
    assert P % 64 == 0 and Ps % 64 == 0 and 64 <= Ps <= P and 0 <= T <= max_len
    piece = max(P // 4 // 64 * 64, 256)
    if R > 2048 or piece >= P:
        assert (Ps, T) == (P, 0)
    else:
        assert Ps == piece and T > 0
    lens = set(range(0, min(max_len, 3 * P) + 1)) | set(range(max(0, max_len - 3 * P), max_len + 1))
    lens |= {T + k * P + e for k in range(0, max_len // P + 1) for e in (-1, 0, 1)}
    seen = 0
    for m in sorted(x for x in lens if 0 <= x <= max_len):
        parts = _split_parts(m, P, Ps, T)
        big = (m - T) // P if m > T else 0
        if m == 0:
            assert parts == [0]
        else:
            assert sum(parts) == m and min(parts) > 0
            assert parts[:big] == [P] * big and all(x <= Ps for x in parts[big:])
            assert m - big * P >= min(m, T)              # the pieces hold the last T tokens at least
        seen = max(seen, len(parts))
    assert seen == most
    # an explicit partition size is taken as is
    assert yb.cross_attn_partition_split(R, hkv, d, max_len, bs, 128, dtype)[:3] == (128, 128, 0)


@pytest.mark.parametrize("shape", SPLIT_SHAPES)
def test_workspace_holds_either_kernels_partitions(shape):
    """The workspace helpers do not take the cache type: they size for the
    largest of the plans of an fp32 cache (vector ALUs), a bf16 cache (either
    kernel, one plan) and an FP8 cache (matrix cores, twice the item floor)."""
    R, hkv, d, max_len, bs = shape
    most = max(yb.cross_attn_partition_split(R, hkv, d, max_len, bs, 0, dt)[3]
               for dt in (yb.DTYPE_F32, yb.DTYPE_BF16, yb.DTYPE_FP8_E4M3))
    ws = yb.cross_attn_workspace_size(R, 8 * hkv, hkv, d, max_len, bs, 0)
    acc = R * 8 * hkv * most * d * 4
    assert most == 1 and ws == yb.CROSS_ATTN_QUEUE_BYTES or \
        ws == yb.CROSS_ATTN_QUEUE_BYTES + -(-acc // 256) * 256 + R * 8 * hkv * most * 2 * 4


def _append(**kw):
    args = dict(dtype=1, x=FAKE, T=4, hidden=256, w=FAKE, eps=1e-6, wk=FAKE, wv=FAKE, slots=FAKE, k=FAKE, v=FAKE,
                nb=8, hkv=2, bs=16, d=128, ws=FAKE, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return yb.lib().yoco_kv_append(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=100), yb.YOCO_ERR_UNSUPPORTED),
    (dict(d=80), yb.YOCO_ERR_UNSUPPORTED),
    (dict(bs=3), yb.YOCO_ERR_UNSUPPORTED),
    (dict(eps=-1.0), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(ws_bytes=100), yb.YOCO_ERR_WORKSPACE_TOO_SMALL),
    (dict(x=None), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(wk=FAKE + 2), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(dtype=0, hidden=32768), yb.YOCO_ERR_UNSUPPORTED),
])
def test_kv_append_rejects_before_launch(kw, status):
    assert _append(**kw) == status


def test_kv_append_no_tokens_is_a_noop():
    assert _append(T=0) == yb.YOCO_OK


@pytest.mark.parametrize("args,status", [
    ((FAKE, 10, 24, FAKE, 2, FAKE, None, None), yb.YOCO_ERR_INVALID_ARGUMENT),   # row_bytes not /16
    ((FAKE, 10, 32, None, 2, FAKE, None, None), yb.YOCO_ERR_INVALID_ARGUMENT),   # null cu_seqlens
    ((FAKE + 8, 10, 32, FAKE, 2, FAKE, None, None), yb.YOCO_ERR_INVALID_ARGUMENT),
    ((FAKE, -1, 32, FAKE, 2, FAKE, None, None), yb.YOCO_ERR_INVALID_ARGUMENT),
    ((FAKE, 10, 32, FAKE, 0, FAKE, None, None), yb.YOCO_OK),                    # no requests
])
def test_gather_last_rejects_before_launch(args, status):
    assert yb.lib().yoco_gather_last(*args) == status


def _varlen(**kw):
    args = dict(dtype=1, q=FAKE, num_rows=6, qsl=FAKE, num_seqs=2, max_qlen=4, num_q_heads=8, k=FAKE, v=FAKE,
                k_scale=None, v_scale=None, num_blocks=10, num_kv_heads=2, block_size=16, head_dim=128, table=FAKE,
                max_blocks=4, seq_lens=FAKE, max_seq_len=64, window=0, scale=0.1, part=0, flags=0, out=FAKE,
                ws=FAKE, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return yb.lib().yoco_cross_attn_varlen(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(qsl=None), yb.YOCO_ERR_INVALID_ARGUMENT),                 # one row per request needs num_rows == num_seqs
    (dict(qsl=None, num_rows=2, max_qlen=2), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(window=-1), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(max_qlen=-1), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(k_scale=FAKE), yb.YOCO_ERR_INVALID_ARGUMENT),              # scales only for an 8-bit cache
    (dict(num_seqs=2049), yb.YOCO_ERR_UNSUPPORTED),
    (dict(head_dim=96), yb.YOCO_ERR_UNSUPPORTED),
    (dict(max_seq_len=100000, part=64, ws_bytes=4096), yb.YOCO_ERR_WORKSPACE_TOO_SMALL),
    (dict(out=None), yb.YOCO_ERR_INVALID_ARGUMENT),
])
def test_cross_attn_varlen_rejects_before_launch(kw, status):
    assert _varlen(**kw) == status
    assert yb.last_error_message()


def test_cross_attn_varlen_nothing_to_do():
    assert _varlen(num_rows=0) == yb.YOCO_OK
    assert _varlen(max_qlen=0) == yb.YOCO_OK


def test_varlen_workspace_follows_the_window():
    # a window caps the range the partitions split: window + max_query_len - 1 tokens
    full = yb.cross_attn_varlen_workspace_size(8, 2, 8, 2, 128, 100000, 4, 0, 16, 64)
    win = yb.cross_attn_varlen_workspace_size(8, 2, 8, 2, 128, 100000, 4, 637, 16, 64)
    np_full, np_win = -(-100000 // 64), -(-640 // 64)
    assert full == yb.CROSS_ATTN_QUEUE_BYTES + -(-8 * 8 * np_full * 128 * 4 // 256) * 256 + 8 * 8 * np_full * 8
    assert win == yb.CROSS_ATTN_QUEUE_BYTES + -(-8 * 8 * np_win * 128 * 4 // 256) * 256 + 8 * 8 * np_win * 8


@pytest.mark.parametrize("args,status", [
    ((FAKE, 10, 24, FAKE, 2, FAKE, 2, FAKE, FAKE, None, None), yb.YOCO_ERR_INVALID_ARGUMENT),   # row_bytes
    ((FAKE, 10, 32, None, 2, FAKE, 2, FAKE, FAKE, None, None), yb.YOCO_ERR_INVALID_ARGUMENT),   # indices
    ((FAKE, 10, 32, FAKE, 2, None, 2, FAKE, FAKE, None, None), yb.YOCO_ERR_INVALID_ARGUMENT),   # offsets
    ((FAKE, 10, 32, FAKE, 2, FAKE, 2, FAKE, None, None, None), yb.YOCO_ERR_INVALID_ARGUMENT),   # out offsets
    ((FAKE, 10, 32, FAKE, 2, FAKE, 8193, FAKE, FAKE, None, None), yb.YOCO_ERR_UNSUPPORTED),
    ((FAKE, 10, 32, FAKE, -2, FAKE, 2, FAKE, FAKE, None, None), yb.YOCO_ERR_INVALID_ARGUMENT),
])
def test_gather_logits_rejects_before_launch(args, status):
    assert yb.lib().yoco_gather_logits(*args) == status


def _retention(**kw):
    args = dict(dtype=1, q=FAKE, k=FAKE, v=FAKE, gamma=FAKE, num_tokens=40, num_heads=4, head_dim=128, cu=FAKE,
                num_reqs=2, max_seqlen=0, state=FAKE, num_slots=4, slots=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 30,
                stream=None)
    args.update(kw)
    return yb.lib().yoco_gated_retention(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=0), yb.YOCO_ERR_UNSUPPORTED),                       # fp32 q/k/v: no kernel
    (dict(dtype=2), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(head_dim=96), yb.YOCO_ERR_UNSUPPORTED),
    (dict(head_dim=256), yb.YOCO_ERR_UNSUPPORTED),
    (dict(num_tokens=-1), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(num_slots=-1), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(cu=None), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(slots=None), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(state=None), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(gamma=None), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(out=None), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(q=FAKE + 8), yb.YOCO_ERR_INVALID_ARGUMENT),               # 16-byte alignment
    (dict(out=FAKE + 2), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(state=FAKE + 4), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(max_seqlen=-1), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(ws=None), yb.YOCO_ERR_WORKSPACE_TOO_SMALL),               # max_seqlen 0: segmented, needs a workspace
    (dict(ws_bytes=1024), yb.YOCO_ERR_WORKSPACE_TOO_SMALL),
])
def test_gated_retention_rejects_before_launch(kw, status):
    assert _retention(**kw) == status
    assert yb.last_error_message()


def test_gated_retention_nothing_to_do():
    assert _retention(num_reqs=0) == yb.YOCO_OK
    assert _retention(num_heads=0) == yb.YOCO_OK
    assert _retention(num_tokens=0) == yb.YOCO_OK


def test_gated_retention_workspace_follows_the_schedule():
    # decode (max_seqlen 1) and one run per request (<= 2048 rows) need none;
    # segments of 2048 rows need a state and a gate per (segment, head)
    assert yb.gated_retention_workspace_size(5000, 8, 4, 128, 1) == 0
    assert yb.gated_retention_workspace_size(5000, 8, 4, 128, 2048) == 0
    segs = (8 + 5000 // 2048) * 4
    rup = lambda x: -(-x // 256) * 256
    assert yb.gated_retention_workspace_size(5000, 8, 4, 128, 0) == rup(segs * 128 * 128 * 4) + rup(segs * 4)
    assert yb.gated_retention_workspace_size(5000, 8, 4, 128, 2049) == rup(segs * 128 * 128 * 4) + rup(segs * 4)
    # more requests than a segmented launch schedules: one run per request
    assert yb.gated_retention_workspace_size(5000, 4096, 4, 64, 0) == 0
    assert yb.gated_retention_workspace_size(-1, 8, 4, 128, 0) == -1


def test_fp8_append_workspace_follows_the_path():
    # the tiled GEMM (bf16, more than 64 tokens) quantizes in its epilogue:
    # only the folded weights; the few-token and fp32 paths add fp32 rows
    fold = yb.kv_append_workspace_size(yb.DTYPE_BF16, 3072, 8, 128)
    rup = -(-fold // 256) * 256
    rows = lambda t: t * 2 * 8 * 128 * 4
    assert yb.kv_append_fp8_workspace_size(yb.DTYPE_BF16, 81000, 3072, 8, 128) == rup
    assert yb.kv_append_fp8_workspace_size(yb.DTYPE_BF16, 64, 3072, 8, 128) == rup + rows(64)
    assert yb.kv_append_fp8_workspace_size(yb.DTYPE_BF16, 65, 3072, 8, 128) == rup
    assert yb.kv_append_fp8_workspace_size(yb.DTYPE_F32, 100, 256, 1, 64) == 100 * 2 * 64 * 4
    assert yb.kv_append_fp8_workspace_size(yb.DTYPE_BF16, -1, 3072, 8, 128) == -1


def _append_fp8(**kw):
    args = dict(dtype=1, x=FAKE, T=100, hidden=256, w=FAKE, eps=1e-6, wk=FAKE, wv=FAKE, slots=FAKE, k=FAKE, v=FAKE,
                ks=FAKE, vs=FAKE, nb=8, hkv=2, bs=16, d=128, ws=FAKE, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return yb.lib().yoco_kv_append_fp8(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(k=FAKE + 4), yb.YOCO_ERR_INVALID_ARGUMENT),                # caches 16-byte aligned
    (dict(vs=FAKE + 2), yb.YOCO_ERR_INVALID_ARGUMENT),               # scales 4-byte aligned
    (dict(ks=None), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(ws_bytes=16), yb.YOCO_ERR_WORKSPACE_TOO_SMALL),
    (dict(d=96), yb.YOCO_ERR_UNSUPPORTED),
    (dict(dtype=7), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(T=-1), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(T=0, ws=None, ws_bytes=1 << 20), yb.YOCO_OK),              # nothing to do
])
def test_append_fp8_rejects(kw, status):
    assert _append_fp8(**kw) == status


def _scatter(**kw):
    args = dict(src=yb.DTYPE_F32, k_rows=FAKE, v_rows=FAKE, T=5, slots=FAKE, cache=yb.DTYPE_FP8_E4M3, k=FAKE,
                v=FAKE, ks=FAKE, vs=FAKE, nb=8, hkv=2, bs=16, d=128, stream=None)
    args.update(kw)
    return yb.lib().yoco_kv_scatter(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(src=yb.DTYPE_FP8_E4M3), yb.YOCO_ERR_INVALID_ARGUMENT),     # rows are fp32 or bf16
    (dict(cache=yb.DTYPE_BF16), yb.YOCO_ERR_INVALID_ARGUMENT),       # copy only into the same dtype
    (dict(ks=None), yb.YOCO_ERR_INVALID_ARGUMENT),                   # an FP8 cache needs scales
    (dict(cache=yb.DTYPE_F32), yb.YOCO_ERR_INVALID_ARGUMENT),        # a copy takes none
    (dict(k_rows=FAKE + 8), yb.YOCO_ERR_INVALID_ARGUMENT),           # 16-byte alignment
    (dict(d=80), yb.YOCO_ERR_UNSUPPORTED),
    (dict(bs=24), yb.YOCO_ERR_UNSUPPORTED),
    (dict(nb=0), yb.YOCO_ERR_INVALID_ARGUMENT),
    (dict(T=0), yb.YOCO_OK),
])
def test_scatter_rejects(kw, status):
    assert _scatter(**kw) == status
