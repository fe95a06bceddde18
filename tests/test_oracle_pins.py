"""The CPU oracle against its pins (library routines, format facts, brute
force, exact sums and invariants); see tests/pins.py for what each pin is."""
import numpy as np
import pytest

import oracle
from tests import pins


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(orc, check):
    check(orc)


def test_encode_band_exhaustive(orc):
    """All 185M positive fp32 patterns in the rounding band vs torch."""
    pins.check_encode_band(orc)


@pytest.mark.slow
def test_encode_all_fp32_patterns(orc):
    """Every one of the 2^32 fp32 patterns (NaNs: NaN code) vs torch."""
    for hi in range(256):
        bits = np.arange(hi << 24, (hi + 1) << 24, dtype=np.uint64).astype(np.uint32)
        y = pins.f32_from_bits(bits)
        a = orc.e4m3_encode(y)
        nan = np.isnan(y)
        assert np.all((a[nan] & 0x7F) == 0x7F)
        assert np.array_equal(a[~nan], pins.torch_encode_sat(y[~nan]))


def test_metrics():
    """The parity metrics on hand-made cases."""
    g = np.array([0x3F80, 0x3F81, 0x8000, 0x0000, 0xBF80], np.uint16)
    o = np.array([0x3F80, 0x3F80, 0x0000, 0x8000, 0xBF82], np.uint16)
    assert list(oracle.bf16_ulp_distance(g, o)) == [0, 1, 0, 0, 2]
    assert list(oracle.bf16_ulp_distance([0x0001], [0x8001])) == [2]
    assert oracle.rel_frobenius(o, o) == 0.0
