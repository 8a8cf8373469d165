"""ctypes binding of libyoco.so (the C ABI in include/yoco.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  Torch tensors supply device memory and the current
HIP stream.  If the library is missing or cannot load, every call raises; there
is no fallback path.
"""

from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional, Tuple

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# YOCO_LIBRARY names another build of the same library (the host-ASan copy
# the CPU tests load); by default the one built next to this file.
LIB_PATH = os.environ.get("YOCO_LIBRARY") or os.path.join(PKG_DIR, "libyoco.so")

ABI_VERSION = 7
YOCO_OK = 0
YOCO_ERR_INVALID_ARGUMENT = 1
YOCO_ERR_UNSUPPORTED = 2
YOCO_ERR_WORKSPACE_TOO_SMALL = 3
YOCO_ERR_HIP = 4
DTYPE_F32 = 0
DTYPE_BF16 = 1
DTYPE_FP8_E4M3 = 2
CROSS_ATTN_QUEUE_BYTES = 2048
FLAG_REVERSE_ORDER = 1
FLAG_VECTOR_KERNEL = 2

_c = ctypes
_vp = _c.c_void_p
_i32 = _c.c_int32
_i64 = _c.c_int64
_u32 = _c.c_uint32
_f32 = _c.c_float

# name -> (restype, argtypes); mirrors include/yoco.h
SIGNATURES = {
    "yoco_abi_version": (_i32, []),
    "yoco_status_string": (_c.c_char_p, [_i32]),
    "yoco_last_error_message": (_c.c_char_p, []),
    "yoco_gather_last": (_i32, [_vp, _i64, _i64, _vp, _i32, _vp, _vp, _vp]),
    "yoco_kv_append_workspace_size": (_i64, [_i32, _i32, _i32, _i32]),
    "yoco_kv_append": (_i32, [_i32, _vp, _i32, _i32, _vp, _f32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                              _vp, _i64, _vp]),
    "yoco_cross_attn_partition_tokens": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "yoco_cross_attn_partition_split": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _u32, _vp]),
    "yoco_cross_attn_kernel": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _u32]),
    "yoco_cross_attn_workspace_size": (_i64, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "yoco_cross_attn": (_i32, [_i32, _vp, _i32, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _i32, _vp, _i32, _f32,
                               _i32, _u32, _vp, _vp, _i64, _vp]),
    "yoco_cross_attn_noalloc": (_i32, [_i32, _vp, _i32, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _i32, _vp, _i32,
                                       _f32, _i32, _u32, _vp, _vp]),
    "yoco_gather_logits": (_i32, [_vp, _i64, _i64, _vp, _i32, _vp, _i32, _vp, _vp, _vp, _vp]),
    "yoco_kv_scatter": (_i32, [_i32, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp]),
    "yoco_kv_append_fp8_workspace_size": (_i64, [_i32, _i32, _i32, _i32, _i32]),
    "yoco_kv_append_fp8": (_i32, [_i32, _vp, _i32, _i32, _vp, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                  _i32, _vp, _i64, _vp]),
    "yoco_cross_attn_varlen_workspace_size": (_i64, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "yoco_cross_attn_varlen": (_i32, [_i32, _vp, _i32, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                      _i32, _vp, _i32, _vp, _i32, _i32, _f32, _i32, _u32, _vp, _vp, _i64, _vp]),
    "yoco_set_validation": (None, [_i32]),
    "yoco_validation_enabled": (_i32, []),
    "yoco_validate_offsets": (_i32, [_vp, _i32, _i64]),
    "yoco_validate_slots": (_i32, [_vp, _i32, _i32, _i32]),
    "yoco_validate_block_table": (_i32, [_vp, _i32, _i32, _vp, _i32, _i32, _i32, _vp, _i32, _i32]),
    "yoco_validate_logits_indices": (_i32, [_vp, _i32, _vp, _i32, _i64]),
    "yoco_validate_state_indices": (_i32, [_vp, _i32, _i32]),
    "yoco_gated_retention_workspace_size": (_i64, [_i32, _i32, _i32, _i32, _i32]),
    "yoco_gated_retention": (_i32, [_i32, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _i32, _i32, _vp, _i32, _vp, _vp,
                                    _vp, _i64, _vp]),
}

_lock = threading.Lock()
_lib = None


class YocoError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libyoco.so once and declare its signatures; raises if it cannot."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(f"{LIB_PATH} is missing: build it with python -m yoco_shared_kv_gather_amd.build")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            version = handle.yoco_abi_version()
            if version != ABI_VERSION:
                raise ImportError(f"libyoco ABI version {version}, binding expects {ABI_VERSION}")
            _lib = handle
    return _lib


def _check(status: int):
    if status != YOCO_OK:
        msg = lib().yoco_last_error_message().decode()
        raise YocoError(status, msg or lib().yoco_status_string(status).decode())


def _torch():
    import torch
    return torch


def _stream_handle(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _i32_dev(t, name):
    torch = _torch()
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    return _dev(t, name)


# ---- yoco_gather_last -----------------------------------------------------------

def gather_last(hidden, cu_seqlens, out=None, out_index=None, stream=None):
    """out[r] = hidden[cu_seqlens[r+1]-1] (bitwise); returns (out, out_index)."""
    torch = _torch()
    num_reqs = cu_seqlens.numel() - 1
    row_shape = tuple(hidden.shape[1:])
    row_bytes = hidden[0].numel() * hidden.element_size() if hidden.shape[0] > 0 else \
        math.prod(row_shape) * hidden.element_size()
    if out is None:
        out = torch.empty((num_reqs,) + row_shape, dtype=hidden.dtype, device=hidden.device)
    if out_index is None:
        out_index = torch.empty(num_reqs, dtype=torch.int32, device=hidden.device)
    _check(lib().yoco_gather_last(_dev(hidden, "hidden"), hidden.shape[0], row_bytes,
                                  _i32_dev(cu_seqlens, "cu_seqlens"), num_reqs, _dev(out, "out"),
                                  _i32_dev(out_index, "out_index"), _stream_handle(stream)))
    return out, out_index


# ---- yoco_kv_append ---------------------------------------------------------------

def kv_append_workspace_size(dtype_code: int, hidden: int, num_kv_heads: int, head_dim: int) -> int:
    return int(lib().yoco_kv_append_workspace_size(dtype_code, hidden, num_kv_heads, head_dim))


def kv_append(x, rms_weight, eps, w_k, w_v, slot_mapping, k_cache, v_cache, workspace=None, stream=None):
    """RMSNorm + shared K/V projection of every row of x into its cache slot."""
    torch = _torch()
    code = _dtype_code(x)
    num_blocks, num_kv_heads, block_size, head_dim = k_cache.shape
    hidden = x.shape[1]
    need = kv_append_workspace_size(code, hidden, num_kv_heads, head_dim)
    if need < 0:
        raise YocoError(YOCO_ERR_INVALID_ARGUMENT, "bad kv_append shape")
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().yoco_kv_append(code, _dev(x, "x"), x.shape[0], hidden, _dev(rms_weight, "rms_weight"), float(eps),
                                _dev(w_k, "w_k"), _dev(w_v, "w_v"), _i32_dev(slot_mapping, "slot_mapping"),
                                _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), num_blocks, num_kv_heads,
                                block_size, head_dim, ws_ptr, ws_bytes, _stream_handle(stream)))


def _cache_code(k_cache, q_or_rows) -> int:
    """Cache dtype code: uint8 storage is an FP8 E4M3 cache, else the cache
    has the dtype of the queries (or rows)."""
    torch = _torch()
    if k_cache.dtype == torch.uint8:
        return DTYPE_FP8_E4M3
    code = _dtype_code(k_cache)
    if code != _dtype_code(q_or_rows):
        raise TypeError("cache and queries (rows) must share a dtype unless the cache is FP8 (uint8)")
    return code


def kv_scatter(k_rows, v_rows, slot_mapping, k_cache, v_cache, k_scale=None, v_scale=None, stream=None):
    """Write K/V rows [T][Hkv][D] into their slots; into an FP8 (uint8) cache
    they are quantized with one scale per (token, KV head)."""
    src = _dtype_code(k_rows)
    cache = _cache_code(k_cache, k_rows)
    num_blocks, num_kv_heads, block_size, head_dim = k_cache.shape
    _check(lib().yoco_kv_scatter(src, _dev(k_rows, "k_rows"), _dev(v_rows, "v_rows"), k_rows.shape[0],
                                 _i32_dev(slot_mapping, "slot_mapping"), cache, _dev(k_cache, "k_cache"),
                                 _dev(v_cache, "v_cache"), _dev(k_scale, "k_scale") if k_scale is not None else None,
                                 _dev(v_scale, "v_scale") if v_scale is not None else None, num_blocks, num_kv_heads,
                                 block_size, head_dim, _stream_handle(stream)))


def kv_append_fp8_workspace_size(dtype_code: int, num_tokens: int, hidden: int, num_kv_heads: int,
                                 head_dim: int) -> int:
    return int(lib().yoco_kv_append_fp8_workspace_size(dtype_code, num_tokens, hidden, num_kv_heads, head_dim))


def kv_append_fp8(x, rms_weight, eps, w_k, w_v, slot_mapping, k_cache, v_cache, k_scale, v_scale, workspace=None,
                  stream=None):
    """RMSNorm + shared K/V projection of every row of x, quantized into an
    FP8 (uint8) cache with per-(token, KV head) scales."""
    torch = _torch()
    code = _dtype_code(x)
    num_blocks, num_kv_heads, block_size, head_dim = k_cache.shape
    hidden = x.shape[1]
    need = kv_append_fp8_workspace_size(code, x.shape[0], hidden, num_kv_heads, head_dim)
    if need < 0:
        raise YocoError(YOCO_ERR_INVALID_ARGUMENT, "bad kv_append_fp8 shape")
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _check(lib().yoco_kv_append_fp8(code, _dev(x, "x"), x.shape[0], hidden, _dev(rms_weight, "rms_weight"),
                                    float(eps), _dev(w_k, "w_k"), _dev(w_v, "w_v"),
                                    _i32_dev(slot_mapping, "slot_mapping"), _dev(k_cache, "k_cache"),
                                    _dev(v_cache, "v_cache"), _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale"),
                                    num_blocks, num_kv_heads, block_size, head_dim, _dev(workspace, "workspace"),
                                    workspace.numel(), _stream_handle(stream)))


# ---- yoco_cross_attn -----------------------------------------------------------------

def cross_attn_partition_tokens(num_seqs, num_kv_heads, head_dim, max_seq_len, block_size,
                                partition_tokens=0) -> int:
    return int(lib().yoco_cross_attn_partition_tokens(num_seqs, num_kv_heads, head_dim, max_seq_len, block_size,
                                                       partition_tokens))


def cross_attn_partition_split(num_seqs, num_kv_heads, head_dim, max_seq_len, block_size, partition_tokens=0,
                               dtype=DTYPE_BF16, max_query_len=1, window=0, flags=0):
    """(P, Ps, T, most partitions per key range) of the split of every context
    into partitions that the attention call with these arguments makes, or
    None for invalid arguments."""
    split = (ctypes.c_int32 * 3)()
    most = int(lib().yoco_cross_attn_partition_split(dtype, num_seqs, max_query_len, num_kv_heads, head_dim,
                                                     max_seq_len, window, block_size, partition_tokens, flags,
                                                     split))
    return None if most < 0 else (int(split[0]), int(split[1]), int(split[2]), most)


def cross_attn_kernel(num_seqs, num_kv_heads, head_dim, max_seq_len, block_size, partition_tokens=0,
                      dtype=DTYPE_BF16, max_query_len=1, window=0, flags=0):
    """The attention kernel the call with these arguments runs: "matrix"
    (matrix cores) or "vector" (vector ALUs), or None for invalid arguments."""
    kind = int(lib().yoco_cross_attn_kernel(dtype, num_seqs, max_query_len, num_kv_heads, head_dim, max_seq_len,
                                            window, block_size, partition_tokens, flags))
    return None if kind < 0 else ("matrix" if kind == 1 else "vector")


def cross_attn_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, block_size,
                              partition_tokens=0) -> int:
    return int(lib().yoco_cross_attn_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                                     block_size, partition_tokens))


def cross_attn(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, scale=None, partition_tokens=0, flags=0,
               out=None, workspace=None, stream=None):
    """One cross layer: out[r][h] = softmax(scale q.K^T) V over request r's context.

    A workspace passed in must start with CROSS_ATTN_QUEUE_BYTES zero bytes
    before its first use (every call leaves them zero); allocate it with
    torch.zeros.  Calls that may run concurrently need separate workspaces."""
    torch = _torch()
    code = _dtype_code(q)
    num_seqs, num_q_heads, head_dim = q.shape
    num_blocks, num_kv_heads, block_size, _ = k_cache.shape
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    if out is None:
        out = torch.empty((num_seqs, num_q_heads, head_dim), dtype=torch.float32, device=q.device)
    need = cross_attn_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, block_size,
                                     partition_tokens)
    if need < 0:
        raise YocoError(YOCO_ERR_INVALID_ARGUMENT, "bad cross_attn shape")
    if workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().yoco_cross_attn(code, _dev(q, "q"), num_seqs, num_q_heads, _dev(k_cache, "k_cache"),
                                 _dev(v_cache, "v_cache"), num_blocks, num_kv_heads, block_size, head_dim,
                                 _i32_dev(block_table, "block_table"), block_table.shape[1],
                                 _i32_dev(seq_lens, "seq_lens"), int(max_seq_len), float(scale),
                                 int(partition_tokens), int(flags), _dev(out, "out"), ws_ptr, ws_bytes,
                                 _stream_handle(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024


def cross_attn_noalloc(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, out, scale=None, partition_tokens=0,
                       flags=0, stream=None):
    """yoco_cross_attn with the library's static scratch as workspace (no
    allocation by the library; `out` is the caller's).  Calls that overlap
    on one GPU race."""
    num_seqs, num_q_heads, head_dim = q.shape
    num_blocks, num_kv_heads, block_size, _ = k_cache.shape
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    code = _dtype_code(k_cache)
    _check(lib().yoco_cross_attn_noalloc(code, _dev(q, "q"), num_seqs, num_q_heads, _dev(k_cache, "k_cache"),
                                         _dev(v_cache, "v_cache"), num_blocks, num_kv_heads, block_size, head_dim,
                                         _i32_dev(block_table, "block_table"), block_table.shape[1],
                                         _i32_dev(seq_lens, "seq_lens"), int(max_seq_len), float(scale),
                                         int(partition_tokens), int(flags), _dev(out, "out"), _stream_handle(stream)))
    return out


# ---- yoco_gather_logits --------------------------------------------------------------

def gather_logits(hidden, logits_indices, query_start_loc, out=None, out_query_start_loc=None, out_max_query_len=None,
                  stream=None):
    """Rows at the logits positions and the cross-decoder's query_start_loc,
    rebuilt on the device.  Returns (rows, query_start_loc, max_query_len),
    the last two as int32 device tensors ([R+1] and [1])."""
    torch = _torch()
    num_idx = logits_indices.numel()
    num_reqs = query_start_loc.numel() - 1
    row_shape = tuple(hidden.shape[1:])
    row_bytes = math.prod(row_shape) * hidden.element_size()
    if out is None:
        out = torch.empty((num_idx,) + row_shape, dtype=hidden.dtype, device=hidden.device)
    if out_query_start_loc is None:
        out_query_start_loc = torch.empty(num_reqs + 1, dtype=torch.int32, device=hidden.device)
    if out_max_query_len is None:
        out_max_query_len = torch.empty(1, dtype=torch.int32, device=hidden.device)
    _check(lib().yoco_gather_logits(_dev(hidden, "hidden"), hidden.shape[0], row_bytes,
                                    _i32_dev(logits_indices, "logits_indices"), num_idx,
                                    _i32_dev(query_start_loc, "query_start_loc"), num_reqs, _dev(out, "out"),
                                    _i32_dev(out_query_start_loc, "out_query_start_loc"),
                                    _i32_dev(out_max_query_len, "out_max_query_len"), _stream_handle(stream)))
    return out, out_query_start_loc, out_max_query_len


# ---- yoco_cross_attn_varlen ------------------------------------------------------------

def cross_attn_varlen_workspace_size(num_rows, num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                     max_query_len, window, block_size, partition_tokens=0) -> int:
    return int(lib().yoco_cross_attn_varlen_workspace_size(num_rows, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                            max_seq_len, max_query_len, window, block_size,
                                                            partition_tokens))


def cross_attn_varlen(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, query_start_loc=None, max_query_len=1,
                      window=0, scale=None, partition_tokens=0, flags=0, out=None, workspace=None, stream=None,
                      k_scale=None, v_scale=None):
    """One cross layer with several query rows per request (query_start_loc,
    rows aligned to the end of each context, causal) and an optional sliding
    window.  q and out are [num_rows][Hq][D].  An FP8 cache is uint8 storage
    with k_scale / v_scale [num_blocks][Hkv][block_size] (q in bf16)."""
    torch = _torch()
    code = _cache_code(k_cache, q)
    if code == DTYPE_FP8_E4M3 and q.dtype != torch.bfloat16:
        raise TypeError("queries must be bfloat16 with an FP8 cache")
    num_rows, num_q_heads, head_dim = q.shape
    num_blocks, num_kv_heads, block_size, _ = k_cache.shape
    num_seqs = seq_lens.numel()
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    if out is None:
        out = torch.empty((num_rows, num_q_heads, head_dim), dtype=torch.float32, device=q.device)
    need = cross_attn_varlen_workspace_size(num_rows, num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                            max_query_len, window, block_size, partition_tokens)
    if need < 0:
        raise YocoError(YOCO_ERR_INVALID_ARGUMENT, "bad cross_attn_varlen shape")
    if workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    qsl_ptr = _i32_dev(query_start_loc, "query_start_loc") if query_start_loc is not None else None
    _check(lib().yoco_cross_attn_varlen(code, _dev(q, "q"), num_rows, qsl_ptr, num_seqs, int(max_query_len),
                                        num_q_heads, _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                        _dev(k_scale, "k_scale") if k_scale is not None else None,
                                        _dev(v_scale, "v_scale") if v_scale is not None else None,
                                        num_blocks, num_kv_heads, block_size, head_dim,
                                        _i32_dev(block_table, "block_table"), block_table.shape[1],
                                        _i32_dev(seq_lens, "seq_lens"), int(max_seq_len), int(window), float(scale),
                                        int(partition_tokens), int(flags), _dev(out, "out"), _dev(workspace, "workspace"),
                                        workspace.numel() * workspace.element_size(), _stream_handle(stream)))
    return out


# ---- yoco_gated_retention -------------------------------------------------------

def gated_retention_workspace_size(num_tokens, num_reqs, num_heads, head_dim, max_seqlen=0) -> int:
    return int(lib().yoco_gated_retention_workspace_size(num_tokens, num_reqs, num_heads, head_dim, max_seqlen))


def gated_retention(q, k, v, gamma, cu_seqlens, state, state_indices, max_seqlen=0, out=None, workspace=None,
                    stream=None):
    """Self-decoder gated retention over each request's rows:
    S_t = gamma_t S_{t-1} + k_t^T v_t, o_t = q_t S_t per head, from and back
    to the request's state slot.  q, k, v: bf16 [T][H][D]; gamma: fp32 [T][H];
    state: fp32 [slots][H][D][D] (updated in place); max_seqlen: a bound on
    any request's rows (0 = unknown), which only picks the schedule.  Returns
    out fp32 [T][H][D] (rows of no request are left as allocated)."""
    torch = _torch()
    num_tokens, num_heads, head_dim = q.shape
    if out is None:
        out = torch.empty((num_tokens, num_heads, head_dim), dtype=torch.float32, device=q.device)
    if gamma.dtype != torch.float32 or state.dtype != torch.float32 or out.dtype != torch.float32:
        raise TypeError("gamma, state and out must be float32")
    if k.shape != q.shape or v.shape != q.shape or tuple(gamma.shape) != (num_tokens, num_heads):
        raise ValueError("q, k, v must share [T][H][D] and gamma must be [T][H]")
    if state.dim() != 4 or tuple(state.shape[1:]) != (num_heads, head_dim, head_dim):
        raise ValueError("state must be [slots][H][D][D]")
    num_reqs = cu_seqlens.shape[0] - 1
    if state_indices.numel() != num_reqs:
        raise ValueError("state_indices needs one slot per request")
    need = gated_retention_workspace_size(num_tokens, num_reqs, num_heads, head_dim, max_seqlen)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    num_slots = state.shape[0]
    _check(lib().yoco_gated_retention(_dtype_code(q), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(gamma, "gamma"),
                                      num_tokens, num_heads, head_dim, _i32_dev(cu_seqlens, "cu_seqlens"), num_reqs,
                                      max_seqlen, _dev(state, "state") if num_slots > 0 else None, num_slots,
                                      _i32_dev(state_indices, "state_indices"), _dev(out, "out"),
                                      _dev(workspace, "workspace") if workspace is not None else None,
                                      workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                      _stream_handle(stream)))
    return out


def status_string(status: int) -> str:
    return lib().yoco_status_string(status).decode()


def last_error_message() -> str:
    return lib().yoco_last_error_message().decode()


def library_path() -> str:
    return LIB_PATH


def describe_launch(num_seqs, num_kv_heads, head_dim, max_seq_len, block_size, partition_tokens=0,
                    dtype=DTYPE_BF16, max_query_len=1, window=0, flags=0) -> Tuple[int, int]:
    """(full partition tokens, most partitions per key range) that the attention call will use."""
    split = cross_attn_partition_split(num_seqs, num_kv_heads, head_dim, max_seq_len, block_size, partition_tokens,
                                       dtype, max_query_len, window, flags)
    if split is None:
        raise ValueError("invalid sizes for a cross-attention launch")
    return split[0], split[3]
