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
