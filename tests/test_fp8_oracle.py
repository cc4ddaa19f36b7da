"""Pins for the FP8 (e4m3) oracle: values of the OCP e4m3 format (closed
forms), the encoder's rounding and saturation, the relative error bound of a
round trip, and planted mistakes in a copy of the oracle's source."""
import types

import numpy as np
import pytest

from oracle import fp8

SRC = fp8.__file__

KNOWN = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5, 0x38: 1.0,
         0x3C: 1.5, 0x40: 2.0, 0x48: 4.0, 0x78: 256.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}


def pin_known_values(mod):
    for code, val in KNOWN.items():
        assert mod.e4m3_value(code) == val, hex(code)
    assert np.isnan(mod.e4m3_value(0x7F)) and np.isnan(mod.e4m3_value(0xFF))
    v = mod.decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)                        # 0x00..0x7e increasing
    assert np.array_equal(mod.decode(np.arange(0x80, 0xFF, dtype=np.uint8)), -v)


def pin_round_trip(mod):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = mod.decode(codes)
    assert np.array_equal(mod.encode(vals), codes)
    assert all(mod.encode_scalar(float(x)) == int(c) for x, c in zip(vals, codes))


def pin_ties_and_saturation(mod):
    v = mod.decode(np.arange(0x7F, dtype=np.uint8))
    mid = (v[:-1] + v[1:]) / 2
    got = mod.encode(mid)
    lo = np.arange(0x7E)
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8))
    eps = np.maximum(np.abs(mid) * 1e-9, 1e-30)
    assert np.array_equal(mod.encode(mid - eps), lo.astype(np.uint8))
    assert np.array_equal(mod.encode(mid + eps), (lo + 1).astype(np.uint8))
    big = np.array([448.0, 449.0, 463.99, 464.0, 480.0, 1e30, np.inf])
    assert np.all(mod.encode(big) == 0x7E) and np.all(mod.encode(-big) == 0xFE)
    assert mod.encode(np.array([np.nan]))[0] == 0x7F and mod.encode(np.array([-np.nan]))[0] == 0xFF
    assert mod.encode(np.array([-0.0]))[0] == 0x80 and mod.encode(np.array([0.0]))[0] == 0x00
    assert mod.encode(np.array([2.0 ** -10]))[0] == 0x00        # half of the smallest step: even 0
    assert mod.encode(np.array([3 * 2.0 ** -10]))[0] == 0x02    # 1.5 steps: even 2


def pin_error_bound(mod):
    rng = np.random.default_rng(5)
    scale = np.array([0.02, 1.0, 3.5], dtype=np.float32)
    x = rng.normal(0, 2, size=(4000, 3, 8)).astype(np.float32)
    q = mod.quantize(x, scale)
    deq = mod.decode(q) * scale[None, :, None]
    rel = np.abs(x.astype(np.float64) / scale[None, :, None])
    normal = (rel >= 2.0 ** -6) & (rel < 448)
    err = np.abs(deq - x) / scale[None, :, None]
    # nearest rounding: at most half the local step, 2^-4 of the magnitude for
    # normals and 2^-10 absolute (in scale units) for subnormals
    assert np.all(err[normal] <= rel[normal] * 2.0 ** -4 * (1 + 1e-6))
    assert np.all(err[~normal & (rel < 448)] <= 2.0 ** -10 * (1 + 1e-6))


def pin_scalar_equals_vector(mod):
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.normal(0, 60, 3000), rng.normal(0, 0.005, 3000)])
    assert np.array_equal(np.array([mod.encode_scalar(t) for t in x], dtype=np.uint8), mod.encode(x))


def pin_power_of_two_scale(mod):
    rng = np.random.default_rng(2)
    x = rng.normal(0, 1, size=(50, 2, 16)).astype(np.float32)
    s = np.array([0.25, 8.0], dtype=np.float32)
    assert np.array_equal(mod.quantize(x, s), mod.encode(x / s[None, :, None].astype(np.float64)))


def pin_exact_division_away_from_ties(mod):
    """Any scale: the float32 steps the quantizer takes, fl32(x * fl32(1/s)),
    stay within 2^-23 (relative) of the exact quotient x/s (two roundings of
    at most 2^-24 each), so the code must be the nearest-e4m3 code of x/s
    itself whenever x/s lies farther than 2^-21 (relative) from every point
    where the nearest code changes (the midpoints between adjacent values,
    and the saturation bound). Near such points the two may differ by one
    code; they are a small minority of the samples."""
    rng = np.random.default_rng(11)
    v = mod.decode(np.arange(0x7F, dtype=np.uint8))
    mids = (v[:-1] + v[1:]) / 2
    s = np.array([0.0173, 0.3, 1.7, 3.14159, 47.0, 1e-3], dtype=np.float32)
    x = np.concatenate([rng.normal(0, 1, (3000, len(s), 4)), rng.normal(0, 30, (3000, len(s), 4))]).astype(np.float32)
    got = mod.quantize(x, s)
    q = x.astype(np.float64) / s.astype(np.float64)[None, :, None]        # exact to 2^-53
    exact = mod.encode(q)
    a = np.abs(q)
    near = np.min(np.abs(a[..., None] - mids), axis=-1) <= a * 2.0 ** -21
    assert np.array_equal(got[~near], exact[~near])
    assert near.mean() < 1e-3
    # where they may differ, they differ by at most one code of the same sign
    dv = np.abs(mod.decode(got[near]) - mod.decode(exact[near]))
    step = np.abs(mod.decode(exact[near])) * 2.0 ** -2 + 2.0 ** -9
    assert np.all(dv <= step)


PINS = [pin_known_values, pin_round_trip, pin_ties_and_saturation, pin_error_bound,
        pin_scalar_equals_vector, pin_power_of_two_scale, pin_exact_division_away_from_ties]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pins_hold(pin):
    pin(fp8)


MUTANTS = {
    "exponent bias 8": ("* 2.0 ** (e - 7)", "* 2.0 ** (e - 8)"),
    "subnormal scale 2^-7": ("return sign * (m / 8.0) * 2.0 ** -6", "return sign * (m / 8.0) * 2.0 ** -7"),
    "ties to the odd code": ("((d_hi == d_lo) & (hi % 2 == 0))", "((d_hi == d_lo) & (hi % 2 == 1))"),
    "no saturation": ("code = np.where(a >= MAX_E4M3, 0x7E, code)", "code = np.where(a >= 480, 0x7F, code)"),
    "scale multiplied": ("inv = (np.float32(1.0) / np.asarray(scale, dtype=np.float32))",
                         "inv = (np.float32(1.0) * np.asarray(scale, dtype=np.float32))"),
    "sign dropped": ("code = np.where(np.isnan(v), 0x7F, code) | sign", "code = np.where(np.isnan(v), 0x7F, code)"),
    "reciprocal in half precision": ("inv = (np.float32(1.0) / np.asarray(scale, dtype=np.float32)).astype(np.float32)",
                                     "inv = (np.float32(1.0) / np.asarray(scale, dtype=np.float32)).astype(np.float16)"
                                     ".astype(np.float32)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert old in src
    mod = types.ModuleType("fp8_mutant")
    src = src.replace(old, new).replace("from .paged_attention import paged_attn_decode",
                                        "paged_attn_decode = None")
    exec(compile(src, "fp8_mutant", "exec"), mod.__dict__)
    failures = 0
    for pin in PINS:
        try:
            pin(mod)
        except Exception:
            failures += 1
    assert failures > 0, f"no pin caught mutant '{name}'"
