"""Pins of the oracle's bf16 widening and correctly rounded output casts."""
import os

import numpy as np
import pytest
import torch

from oracle.numerics import bf16_to_f64, f64_to_bf16_bits, cast_out
from workloads import f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bf16_rne_cases.txt")


def _cases():
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        x, bits, *_ = line.split()
        out.append((float.fromhex(x), int(bits, 16)))
    return out


@pytest.mark.parametrize("x,bits", _cases())
def test_rne_golden_cases(x, bits):
    got = int(f64_to_bf16_bits(np.array([x]))[0])
    assert got == bits, f"{x!r}: got {got:#06x}, want {bits:#06x}"


def test_rne_matches_torch_on_float32_values():
    # Library special case: for values representable in float32, a single
    # round to bf16 is torch's float32 -> bfloat16 conversion.
    rng = np.random.default_rng(1)
    u = rng.integers(0, 2**32, size=400_000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = f64_to_bf16_bits(f.astype(np.float64))
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first {f[bad[0]]!r}"


def test_widening_roundtrips_every_bf16_pattern():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):        # the NaN patterns are widened too
        v = bf16_to_f64(b)
    finite = np.isfinite(v)
    assert np.array_equal(f64_to_bf16_bits(v[finite]), b[finite])
    # widening is exact: the float64 value equals the float32 with those upper bits
    f32 = (b.astype(np.uint32) << 16).view(np.float32)[finite]
    assert np.array_equal(v[finite], f32.astype(np.float64))


def test_cast_out_f32_is_ieee_nearest():
    x = np.array([1.0 + 2.0**-24, 1.0 + 3 * 2.0**-24, 1.0 + 2.0**-24 + 2.0**-50])
    y = cast_out(x, "f32")
    assert y[0] == np.float32(1.0)
    assert y[1] == np.float32(1.0 + 2.0**-22)
    assert y[2] == np.float32(1.0 + 2.0**-23)


def test_generator_quantisation_matches_torch():
    # the input generator's float32 -> bf16 rounding is torch's conversion
    rng = np.random.default_rng(2)
    f = (rng.standard_normal(200_000) * 10.0 ** rng.uniform(-30, 30, 200_000)).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(f), ref)
