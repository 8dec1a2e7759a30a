"""Pins of the oracle's nearest-even bf16 rounding (used by its combine)."""
import json
import os
import struct

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", bits << 16))[0]


def test_every_finite_bf16_value_is_a_fixed_point():
    for bits in range(1 << 16):
        exp = (bits >> 7) & 0xFF
        if exp == 0xFF and (bits & 0x7F):
            assert oracle.bf16_round(float("nan")) == 0x7FC0
            continue
        assert oracle.bf16_round(_bf16_value(bits)) == bits, hex(bits)


def test_midpoints_round_to_even_and_off_midpoints_to_nearest():
    # consecutive positive bf16 values a < b (patterns p, p+1): the midpoint is
    # exact in double; it goes to the even pattern, a nudge either way decides.
    for p in list(range(0, 0x7F7F, 37)) + [0x7F7E, 0x3F80, 0x007F, 0x0080]:
        a, b = _bf16_value(p), _bf16_value(p + 1)
        m = (a + b) / 2
        even = p if p % 2 == 0 else p + 1
        assert oracle.bf16_round(m) == even
        assert oracle.bf16_round(-m) == even | 0x8000
        eps = (b - a) * 2.0 ** -20
        assert oracle.bf16_round(m - eps) == p
        assert oracle.bf16_round(m + eps) == p + 1


def test_agrees_with_torch_cast_on_random_fp32():
    import torch
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, size=60_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_round(float(v)) for v in f], dtype=np.uint16)
    np.testing.assert_array_equal(got, ref)


def test_golden_rounding_cases():
    g = json.load(open(GOLDEN))["bf16_rounding"]
    for name, v, hexbits in g["cases"]:
        assert oracle.bf16_round(v) == int(hexbits, 16), name


def test_infinities_and_nan():
    assert oracle.bf16_round(float("inf")) == 0x7F80
    assert oracle.bf16_round(float("-inf")) == 0xFF80
    assert oracle.bf16_round(1e300) == 0x7F80
    assert oracle.bf16_round(-1e300) == 0xFF80
    assert oracle.bf16_round(float("nan")) == 0x7FC0
    assert oracle.bf16_round(1e-300) == 0x0000
    assert oracle.bf16_round(-1e-300) == 0x8000
