"""The fp8 inputs the tests hand to the oracle: torch's e4m3 decoding against
the format's definition.

The fp8 parity tests give the oracle the fp8 tensors' values through torch's
float8_e4m3fn -> float64 conversion.  That conversion is pinned here, code by
code, to the OCP 8-bit float definition (sign, 4 exponent bits with bias 7,
3 significand bits, subnormals at exponent field 0, no infinities, NaN only
for S.1111.111), and the rounding of a few values to their nearest codes.
"""
import math

import pytest
import torch

pytestmark = pytest.mark.skipif(not hasattr(torch, "float8_e4m3fn"), reason="torch without float8 types")


def _e4m3(code: int) -> float:
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return math.nan
    x = math.ldexp(m / 8.0, -6) if e == 0 else math.ldexp(1.0 + m / 8.0, e - 7)
    return -x if s else x


def test_every_code_decodes_as_defined():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    vals = codes.view(torch.float8_e4m3fn).to(torch.float64).tolist()
    for c, v in enumerate(vals):
        ref = _e4m3(c)
        if math.isnan(ref):
            assert math.isnan(v), c
        else:
            assert v == ref, (c, v, ref)
    assert max(v for v in vals if not math.isnan(v)) == 448.0
    assert min(abs(v) for v in vals if v != 0 and not math.isnan(v)) == 2.0 ** -9


def test_rounding_to_nearest_code():
    x = torch.tensor([1.0, 1.0625, 1.07, 1.1875, 3.3, -0.01, 2.0 ** -10, 300.0], dtype=torch.float64)
    got = x.to(torch.float8_e4m3fn).to(torch.float64).tolist()
    # 1.0625 lies halfway between 1 and 1.125 and goes to the even significand.
    assert got == [1.0, 1.0, 1.125, 1.25, 3.25, -0.009765625, 0.0, 288.0]
