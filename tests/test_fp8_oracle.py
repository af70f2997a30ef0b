"""The oracle's E4M3 codes against facts outside it (CPU only).

Pins: the 256 code values equal torch's float8_e4m3fn reading of the same
bytes (a library implementation of the OCP format), NaN positions included;
closed-form values (1.0 = 0x38, 448 = 0x7e, 2^-9 = 0x01, 2^-6 = 0x08);
in-range encoding equals torch's round-to-nearest-even cast, ties included;
saturation at 448 and NaN handling follow the stated reading; quantisation
divides in fp32 before rounding (a case where dividing in fp64 would round
to a different code).
"""
import math

import numpy as np
import pytest
import torch

from oracle import fp8


def test_code_values_match_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    ours = fp8.decode(np.arange(256))
    nan_r, nan_o = np.isnan(ref), np.isnan(ours)
    assert np.array_equal(nan_r, nan_o) and int(nan_o.sum()) == 2
    assert np.array_equal(ref[~nan_r], ours[~nan_o])


def test_closed_form_values():
    assert fp8.value(0x38) == 1.0
    assert fp8.value(0x7E) == 448.0 and fp8.value(0xFE) == -448.0
    assert fp8.value(0x01) == 2.0 ** -9
    assert fp8.value(0x08) == 2.0 ** -6
    assert fp8.value(0x00) == 0.0 and math.copysign(1.0, fp8.value(0x80)) < 0
    assert math.isnan(fp8.value(0x7F)) and math.isnan(fp8.value(0xFF))


def test_encoding_matches_torch_rne_in_range():
    rng = np.random.default_rng(8)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0,
        rng.uniform(-447.9, 447.9, 5000),
        rng.uniform(-2.0 ** -5, 2.0 ** -5, 5000),  # subnormals and the normal boundary
        # exact midpoints between neighbouring codes (ties)
        (fp8.decode(np.arange(0, 0x7D)) + fp8.decode(np.arange(1, 0x7E))) / 2.0,
    ]).astype(np.float32)
    ours = fp8.encode(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first {x[bad[:5]]}: {ours[bad[:5]]} vs {ref[bad[:5]]}"


def test_ties_go_to_even_mantissa():
    assert fp8.encode_one(1.0625) == 0x38      # between 1.0 (m=0) and 1.125 (m=1)
    assert fp8.encode_one(1.1875) == 0x3A      # between 1.125 (m=1) and 1.25 (m=2)
    assert fp8.encode_one(2.0 ** -10) == 0x00  # half the smallest subnormal
    assert fp8.encode_one(3 * 2.0 ** -10) == 0x02


@pytest.mark.parametrize("y,code", [(448.0, 0x7E), (463.9, 0x7E), (464.0, 0x7E), (1e30, 0x7E), (math.inf, 0x7E),
                                    (-500.0, 0xFE), (-math.inf, 0xFE), (0.0, 0x00), (-0.0, 0x80)])
def test_saturation_and_zero(y, code):
    assert fp8.encode_one(y) == code


def test_nan_stays_nan():
    assert fp8.encode_one(math.nan) == 0x7F
    assert fp8.encode_one(-math.nan) == 0xFF


def test_quantize_divides_in_fp32():
    # x / s in fp64 is just below the midpoint 1.0625 between the codes of
    # 1.0 and 1.125; the fp32 quotient rounds up onto the midpoint, which
    # then ties to even (1.0).  Find such a pair by search and check the
    # oracle takes the fp32 quotient.
    rng = np.random.default_rng(9)
    found = 0
    for _ in range(200000):
        s = np.float32(rng.uniform(0.5, 2.0))
        x = np.float32(1.0625 * float(s))
        q32 = np.float32(x) / np.float32(s)
        q64 = float(x) / float(s)
        if fp8.encode_one(float(q32)) != fp8.encode_one(q64):
            assert fp8.quantize(x, s) == fp8.encode_one(float(q32))
            found += 1
            if found >= 3:
                break
    assert found >= 1
