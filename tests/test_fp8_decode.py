"""The oracle's reading of fp8 inputs, pinned to the format's definition.

fp8 inputs reach the oracle through torch's upcast (``oracle.as_f64``). OCP
e4m3 (the 8-bit floating-point format of the Open Compute Project's OFP8
specification) has 1 sign bit, 4 exponent bits with bias 7 and 3 mantissa bits;
exponent 0 holds the subnormals m/8 * 2^-6; the codes with every exponent and
mantissa bit set (0x7f, 0xff) are NaN, and there are no infinities, so the
largest finite value is 1.75 * 2^8 = 448. All 256 codes are checked.
"""
import math

import torch

import oracle


def e4m3_by_definition(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def test_every_e4m3_code_decodes_by_definition():
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
    got = oracle.as_f64(codes)
    for c in range(256):
        want = e4m3_by_definition(c)
        if math.isnan(want):
            assert math.isnan(got[c]), hex(c)
        else:
            assert got[c] == want and math.copysign(1, got[c]) == math.copysign(1, want), hex(c)
    assert got[0x7e] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9


def test_every_finite_e4m3_value_is_a_bf16_value():
    # the kernels turn fp8 inputs into bf16 operands; this is lossless only
    # because 3 mantissa bits and exponents 2^-9 .. 2^8 fit bf16's 7 and 8 bits
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
    v = codes.double()
    fin = ~torch.isnan(v)
    assert torch.equal(v[fin].to(torch.bfloat16).double(), v[fin])
