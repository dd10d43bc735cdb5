"""Pins for the FP8 (E4M3) oracle: values fixed by the encoding's definition,
ties, saturation, a brute-force nearest search, and planted mutants."""

import math

import numpy as np
import pytest

from oracle import fp8


def test_decode_values_fixed_by_the_definition():
    # bias 7, 3 mantissa bits, subnormals below 2^-6, 0x7F/0xFF NaN
    d = fp8.decode_e4m3
    assert d(0x38) == 1.0 and d(0x40) == 2.0 and d(0x30) == 0.5
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x08) == 2.0 ** -6          # smallest normal
    assert d(0x01) == 2.0 ** -9          # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert d(0x39) == 1.125 and d(0x3F) == 1.875
    assert d(0x00) == 0.0 and math.copysign(1.0, d(0x80)) == -1.0
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))
    # 254 finite codes, distinct except +-0
    finite = d(np.arange(256))
    finite = finite[~np.isnan(finite)]
    assert finite.size == 254 and np.unique(finite).size == 253


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(fp8.encode_e4m3(fp8.decode_e4m3(codes)), codes)


def test_ties_go_to_the_even_code():
    e = fp8.encode_e4m3
    assert e(1.0625) == 0x38             # 1.0 (0x38) | 1.125 (0x39): even is 0x38
    assert e(1.1875) == 0x3A             # 1.125 (0x39) | 1.25 (0x3A)
    assert e(1.5 * 2.0 ** -9) == 0x02    # subnormal tie 0x01 | 0x02
    assert e(0.5 * 2.0 ** -9) == 0x00    # tie between 0 and the smallest subnormal
    assert e(-0.5 * 2.0 ** -9) == 0x80
    assert e(0.75 * 2.0 ** -9) == 0x01   # not a tie: nearer 2^-9
    assert e(416.0) == 0x7D              # exactly representable
    assert e(432.0) == 0x7E              # 416 (0x7D) | 448 (0x7E) tie: even is 0x7E
    assert e(1.0625 + 1e-9) == 0x39      # just above the tie


def test_saturation_and_signs():
    e = fp8.encode_e4m3
    for x in (448.0, 449.0, 464.0, 1e6, float("inf")):
        assert e(x) == 0x7E and e(-x) == 0xFE
    assert e(-0.0) == 0x80 and e(0.0) == 0x00
    assert e(float("nan")) == 0x7F


def test_encode_is_the_nearest_value_brute_force():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000) * 40, rng.standard_normal(5000) * 0.01,
                        rng.uniform(-500, 500, 5000)])
    codes = fp8.encode_e4m3(x)
    got = fp8.decode_e4m3(codes)
    table = fp8.decode_e4m3(np.arange(256))
    table = table[~np.isnan(table)]
    target = np.clip(x, -448, 448)
    best = np.min(np.abs(table[None, :] - target[:, None]), axis=1)
    assert np.array_equal(np.abs(got - target), best)
    # monotone in the input
    order = np.argsort(x)
    assert np.all(np.diff(got[order]) >= 0)


def test_quantize_divides_in_float32_then_encodes():
    x = np.array([1.0, -3.5, 0.1, 300.0], dtype=np.float32)
    s = np.float32(0.0123)
    q = fp8.quantize(x, s)
    assert np.array_equal(q, fp8.encode_e4m3((x / s).astype(np.float32)))
    assert fp8.quantize(np.float32(1000.0), 1.0) == 0x7E
    np.testing.assert_allclose(fp8.dequantize(q, s), np.float64(s) * fp8.decode_e4m3(q))
    # 1.3 / 0.5 = 2.6 lies in [2, 4), where codes are 0.25 apart: the stored
    # value is within half a step (0.125) of 2.6, i.e. 0.0625 after scaling
    v = fp8.dequantize(fp8.quantize(np.float32(1.3), 0.5), 0.5)
    assert abs(v - 1.3) <= 0.0625 and v == 0.5 * 2.5


def _mutant(name):
    """Wrong encoders a plausible slip would produce (built on the real one,
    bound now, before the test patches it in)."""
    table = fp8.decode_e4m3(np.arange(0x7F))
    orig = fp8.encode_e4m3
    if name == "bias8":
        return lambda x: orig(np.asarray(x, dtype=np.float64) * 2.0)
    if name == "truncate":
        def enc(x):
            x = np.asarray(x, dtype=np.float64)
            mag = np.minimum(np.abs(x), 448.0)
            c = np.searchsorted(table, mag, side="right") - 1
            c = np.where(np.signbit(x), c | 0x80, c)
            return c.astype(np.uint8)
        return enc
    if name == "ties_up":
        def enc(x):
            x = np.asarray(x, dtype=np.float64)
            mag = np.minimum(np.abs(x), 448.0)
            hi = np.minimum(np.searchsorted(table, mag, side="left"), 0x7E)
            lo = np.maximum(hi - 1, 0)
            pick_lo = (mag - table[lo]) < (table[hi] - mag)
            c = np.where(pick_lo & (hi > 0), lo, hi)
            c = np.where(np.signbit(x), c | 0x80, c)
            return c.astype(np.uint8)
        return enc
    if name == "no_saturation":
        def enc(x):
            x = np.asarray(x, dtype=np.float64)
            c = orig(x)
            return np.where(np.abs(x) > 464.0, np.uint8(0x7F) | (c & 0x80), c).astype(np.uint8)
        return enc
    raise KeyError(name)


@pytest.mark.parametrize("name", ["bias8", "truncate", "ties_up", "no_saturation"])
def test_planted_mutants_fail_a_pin(name, monkeypatch):
    monkeypatch.setattr(fp8, "encode_e4m3", _mutant(name))
    pins = [test_every_finite_code_round_trips, test_ties_go_to_the_even_code,
            test_saturation_and_signs, test_encode_is_the_nearest_value_brute_force]
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"mutant {name} passed every pin"
