"""Host-side precondition checks (no GPU): the exported yoco_validate_*
functions on host arrays, and the switch that makes every call run them."""

import ctypes
import os
import subprocess
import sys

import numpy as np
import pytest

from yoco_shared_kv_gather_amd import binding as yb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _p(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _msg():
    return yb.lib().yoco_last_error_message().decode()


def offsets(arr, num_reqs, num_rows):
    a, p = _p(arr)
    return yb.lib().yoco_validate_offsets(p, num_reqs, num_rows)


def test_offsets():
    assert offsets([0, 1, 3], 2, 3) == yb.YOCO_OK
    assert offsets([0, 1, 1, 3], 3, 5) == yb.YOCO_OK                   # an empty request
    assert offsets([0], 0, 0) == yb.YOCO_OK
    assert offsets([0, 2, 1], 2, 3) == yb.YOCO_ERR_INVALID_ARGUMENT
    assert "decrease" in _msg()
    assert offsets([0, 1, 4], 2, 3) == yb.YOCO_ERR_INVALID_ARGUMENT    # past the rows
    assert offsets([-1, 1, 2], 2, 3) == yb.YOCO_ERR_INVALID_ARGUMENT


def slots(arr, num_blocks, bs):
    a, p = _p(arr)
    return yb.lib().yoco_validate_slots(p, len(a), num_blocks, bs)


def test_slots():
    assert slots([10, -1, 17, 3, -1], 5, 4) == yb.YOCO_OK             # padding may repeat -1
    assert slots([10, 17, 10], 5, 4) == yb.YOCO_ERR_INVALID_ARGUMENT
    assert "share slot 10" in _msg()
    assert slots([20], 5, 4) == yb.YOCO_ERR_INVALID_ARGUMENT            # slot 20 = block 5 of 5
    assert slots([], 5, 4) == yb.YOCO_OK


def table(tab, lens, max_len, nblocks, bs, qsl=None, rows=0, window=0):
    t, tp = _p(tab)
    s, sp = _p(lens)
    if qsl is None:
        return yb.lib().yoco_validate_block_table(tp, len(s), t.shape[1], sp, max_len, nblocks, bs, None, rows, window)
    q, qp = _p(qsl)
    return yb.lib().yoco_validate_block_table(tp, len(s), t.shape[1], sp, max_len, nblocks, bs, qp, rows, window)


def test_block_table():
    """The pages' Replay figure (pages 0,2,1,4 with 3 and 5 free) passes;
    a used entry outside the pool, a context longer than its table row or
    than max_seq_len, or a negative length fails; entries past the context,
    or before a window's first visible block, are not read and not checked."""
    replay = [[0, 2, 1, 4]]
    assert table(replay, [15], 16, 6, 4) == yb.YOCO_OK
    assert table([[0, 2, 1, 9]], [15], 16, 6, 4) == yb.YOCO_ERR_INVALID_ARGUMENT
    assert "logical block 3 maps to page 9" in _msg()
    assert table([[0, 2, -1, 4]], [8], 16, 6, 4) == yb.YOCO_OK            # block 2 lies past 8 tokens
    assert table(replay, [17], 20, 6, 4) == yb.YOCO_ERR_INVALID_ARGUMENT  # does not fit a row of 16
    assert table(replay, [15], 12, 6, 4) == yb.YOCO_ERR_INVALID_ARGUMENT  # beyond max_seq_len
    assert table(replay, [-1], 16, 6, 4) == yb.YOCO_ERR_INVALID_ARGUMENT
    # a window of 3 with one query at position 14 reads positions 12..14: block 3 only
    assert table([[-7, -7, -7, 4]], [15], 16, 6, 4, window=3) == yb.YOCO_OK
    assert table([[-7, -7, -7, 4]], [15], 16, 6, 4, window=4) == yb.YOCO_ERR_INVALID_ARGUMENT
    # two query rows widen the range by one position
    assert table([[-7, -7, -7, 4]], [15], 16, 6, 4, qsl=[0, 2], rows=2, window=3) == yb.YOCO_ERR_INVALID_ARGUMENT
    assert table([[-7, -7, 5, 4]], [15], 16, 6, 4, qsl=[0, 2], rows=2, window=3) == yb.YOCO_OK
    assert table(replay, [15], 16, 6, 4, qsl=[0, 3], rows=2) == yb.YOCO_ERR_INVALID_ARGUMENT   # offsets past rows


def test_logits_indices():
    """The vLLM page's example passes; indices out of order or outside the
    batch fail."""
    qsl, qp = _p([0, 15, 20, 28])
    for idx, ok in [([14, 18, 19, 27], True), ([14, 19, 18, 27], False), ([14, 18, 28], False), ([], True)]:
        a, p = _p(idx)
        st = yb.lib().yoco_validate_logits_indices(p, len(a), qp, 3, 28)
        assert (st == yb.YOCO_OK) == ok, idx


def test_state_indices():
    a, p = _p([3, -1, 0, -1, 2])
    assert yb.lib().yoco_validate_state_indices(p, 5, 4) == yb.YOCO_OK
    a, p = _p([3, 1, 3])
    assert yb.lib().yoco_validate_state_indices(p, 3, 4) == yb.YOCO_ERR_INVALID_ARGUMENT
    a, p = _p([4])
    assert yb.lib().yoco_validate_state_indices(p, 1, 4) == yb.YOCO_ERR_INVALID_ARGUMENT


def test_switch_and_environment():
    """yoco_set_validation flips the switch; a fresh process reads
    YOCO_VALIDATE from its environment."""
    lib = yb.lib()
    before = lib.yoco_validation_enabled()
    lib.yoco_set_validation(1)
    assert lib.yoco_validation_enabled() == 1
    lib.yoco_set_validation(0)
    assert lib.yoco_validation_enabled() == 0
    lib.yoco_set_validation(before)
    code = "from yoco_shared_kv_gather_amd import binding as yb; print(yb.lib().yoco_validation_enabled())"
    for value, want in [("1", "1"), ("0", "0"), (None, "0")]:
        env = dict(os.environ)
        env.pop("YOCO_VALIDATE", None)
        if value is not None:
            env["YOCO_VALIDATE"] = value
        out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                             timeout=120)
        assert out.stdout.strip() == want, out.stderr
