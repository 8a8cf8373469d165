"""The float64 oracle against closed forms, invariants, library routines and
the pages' worked examples (CPU only)."""

import pytest

import oracle
from tests import oracle_pins as pins


@pytest.mark.parametrize("check", pins.ATTN_CHECKS, ids=lambda c: c.__name__)
def test_attention_pins(check):
    check(oracle.cross_attention)


@pytest.mark.parametrize("check", pins.PROJ_CHECKS, ids=lambda c: c.__name__)
def test_projection_pins(check):
    check(oracle.kv_project)


@pytest.mark.parametrize("check", pins.APPEND_CHECKS, ids=lambda c: c.__name__)
def test_append_pins(check):
    check(oracle.kv_append)


@pytest.mark.parametrize("check", pins.GATHER_CHECKS, ids=lambda c: c.__name__)
def test_gather_pins(check):
    check(oracle.gather_last)


@pytest.mark.parametrize("check", pins.VARLEN_CHECKS, ids=lambda c: c.__name__)
def test_varlen_pins(check):
    check(oracle.cross_attention_varlen)


@pytest.mark.parametrize("check", pins.METADATA_CHECKS, ids=lambda c: c.__name__)
def test_metadata_pins(check):
    check(oracle.cross_metadata)


@pytest.mark.parametrize("check", pins.GATHER_ROWS_CHECKS, ids=lambda c: c.__name__)
def test_gather_rows_pins(check):
    check(oracle.gather_rows)


@pytest.mark.parametrize("check", pins.FP8_DECODE_CHECKS, ids=lambda c: c.__name__)
def test_e4m3_decode_pins(check):
    check(oracle.e4m3_decode)


@pytest.mark.parametrize("check", pins.FP8_ENCODE_CHECKS, ids=lambda c: c.__name__)
def test_e4m3_encode_pins(check):
    check(oracle.e4m3_encode)


@pytest.mark.parametrize("check", pins.QUANT_CHECKS, ids=lambda c: c.__name__)
def test_quantize_pins(check):
    check(oracle.quantize_rows)


@pytest.mark.parametrize("check", pins.SCATTER_CHECKS, ids=lambda c: c.__name__)
def test_scatter_pins(check):
    check(oracle.kv_scatter)


@pytest.mark.parametrize("check", pins.APPEND_FP8_CHECKS, ids=lambda c: c.__name__)
def test_append_fp8_pins(check):
    check(oracle.kv_append_fp8)


@pytest.mark.parametrize("name", sorted(pins.HELPER_CHECKS))
def test_helper_pins(name):
    pins.HELPER_CHECKS[name](getattr(oracle, name))


def test_every_exported_function_has_a_pin():
    """Every function the oracle exports is run by at least one pin above (or
    by the dequantize closed form below)."""
    from oracle import yoco_oracle
    pinned = {"cross_attention", "kv_project", "kv_append", "gather_last", "cross_attention_varlen",
              "cross_metadata", "gather_rows", "e4m3_decode", "e4m3_encode", "quantize_rows", "kv_scatter",
              "kv_append_fp8", "gated_retention", "dequantize_cache"} | set(pins.HELPER_CHECKS)
    assert set(yoco_oracle.__all__) == pinned


def test_dequantize_cache_is_code_times_scale():
    """Closed form: code 0x38 (1.0) with scale 2.5 is 2.5; 0xC0 (-2.0) with
    scale 2.5 is -5.0; scale 0 gives 0."""
    import numpy as np
    codes = np.array([[[[0x38, 0xC0]], [[0x7E, 0x01]]]], dtype=np.uint8)     # [1][2][1][2]
    scales = np.array([[[2.5], [0.0]]], dtype=np.float32)
    out = oracle.dequantize_cache(codes, scales)
    assert out.tolist() == [[[[2.5, -5.0]], [[0.0, 0.0]]]]


@pytest.mark.parametrize("check", pins.RETENTION_CHECKS, ids=lambda c: c.__name__)
def test_retention_pins(check):
    check(oracle.gated_retention)
