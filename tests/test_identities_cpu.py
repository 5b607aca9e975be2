"""Arithmetic identities the HIP kernels rely on, checked in IEEE arithmetic on the CPU.

- The max pass of NVFP4 rotate+quantize folds the butterfly's last stage into the
  maximum: max(|fl(a + b)|, |fl(a - b)|) == fl(|a| + |b|) in float32 (round to nearest
  is monotonic and symmetric in sign).
- The large-tile NVFP4 GEMM converts each E4M3 scale to fp16 (every finite E4M3FN value,
  subnormals included, is an fp16 number, so the hardware FP8 -> fp16 convert is exact) and
  multiplies the fp16 E2M1 value by it in one fp16 multiply, which is exact for every code
  pair: e2m1 * d has at most 6 significant bits and lies in [2^-10, 2688].

E4M3 and E2M1 values are written out here from the formats' definitions (OCP E4M3FN:
bias 7, 3 mantissa bits, subnormals k * 2^-9; E2M1: {0, 0.5, 1, 1.5, 2, 3, 4, 6}).
"""
from __future__ import annotations

import numpy as np

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def e4m3_value(code: int) -> float:
    e, m = (code >> 3) & 15, code & 7
    mag = m * 2.0**-9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
    return -mag if code & 0x80 else mag


def test_folded_last_butterfly_stage_float32():
    rng = np.random.default_rng(12)
    n = 1 << 21
    # magnitudes from subnormal to near overflow, mixed signs, plus exact cancellations
    a = (rng.standard_normal(n) * np.exp2(rng.integers(-140, 120, n))).astype(np.float32)
    b = (rng.standard_normal(n) * np.exp2(rng.integers(-140, 120, n))).astype(np.float32)
    b[: n // 8] = -a[: n // 8]
    b[n // 8: n // 4] = a[n // 8: n // 4]
    b[n // 4: n // 4 + 1000] = np.float32(0.0)
    a[n // 4 + 1000: n // 4 + 2000] = np.float32(-0.0)
    with np.errstate(over="ignore"):
        lhs = np.maximum(np.abs(a + b), np.abs(a - b))
        rhs = np.abs(a) + np.abs(b)
    assert lhs.dtype == np.float32 and rhs.dtype == np.float32
    assert np.array_equal(lhs, rhs)


def test_every_e4m3_value_is_an_fp16_number():
    for code in range(256):
        if code & 0x7F == 0x7F:  # NaN
            continue
        d = e4m3_value(code)
        assert float(np.float16(d)) == d, code


def test_fp16_dequant_product_is_exact():
    for code in range(0x7F):
        dh = np.float16(e4m3_value(code))
        for i, x in enumerate(E2M1):
            for sgn in (1.0, -1.0):
                xs = np.float16(sgn * x)  # the convert's output, exact
                prod = xs * dh  # one fp16 multiply, round to nearest even
                assert prod.dtype == np.float16
                assert float(prod) == sgn * x * e4m3_value(code), (code, i, sgn)
                assert prod != 0 or x == 0.0 or code == 0
