"""Pins for oracle.fp8 against the OCP E4M3 definition and torch's float8_e4m3fn."""
import math
import os

import numpy as np
import torch

from oracle import fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ocp_e4m3_landmarks.txt")


def test_landmarks():
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = line.split()
        got = fp8.decode(np.uint8(int(code, 16)))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val)
            if val == "-0.0":
                assert math.copysign(1, got) < 0


def test_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.decode(codes)
    same = (ref == got) | (np.isnan(ref) & np.isnan(got))
    assert same.all()


def test_round_trip_and_monotone():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(fp8.encode_rne_sat(fp8.decode(codes)), codes)
    pos = fp8.decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)


def test_ties_to_even_and_saturation():
    # midpoint of 1.0 (0x38) and 1.125 (0x39) -> even code 0x38
    assert fp8.encode_rne_sat(1.0625) == 0x38
    # midpoint of 1.125 (0x39) and 1.25 (0x3A) -> 0x3A
    assert fp8.encode_rne_sat(1.1875) == 0x3A
    # midpoint of the two smallest subnormals 2^-9 (0x01) and 2^-8 (0x02): 1.5*2^-9 -> 0x02
    assert fp8.encode_rne_sat(1.5 * 2.0 ** -9) == 0x02
    # half the smallest subnormal -> 0 (even)
    assert fp8.encode_rne_sat(2.0 ** -10) == 0x00
    assert fp8.encode_rne_sat(-2.0 ** -10) == 0x80
    assert fp8.encode_rne_sat(500.0) == 0x7E
    assert fp8.encode_rne_sat(-1e30) == 0xFE
    assert fp8.encode_rne_sat(float("nan")) == 0x7F


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000) * 50,
                        rng.standard_normal(50000) * 0.01,
                        (fp8.decode(np.arange(0x7E, dtype=np.uint8))[1:] +
                         fp8.decode(np.arange(0x7E, dtype=np.uint8))[:-1]) / 2])   # all midpoints
    x = x.astype(np.float32).astype(np.float64)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = fp8.encode_rne_sat(x)
    # torch keeps the sign of values that round to zero as well
    assert np.array_equal(ref, got)


def test_quantiser_scale_rule():
    x = np.array([0.5, -3.0, 2.0], dtype=np.float32)
    s = fp8.page_scale(x)
    assert s == np.float32(np.float32(3.0) / np.float32(448.0))
    codes = fp8.quantise(x, s)
    # the amax element maps to +-448 exactly or within one ulp of the grid
    assert abs(fp8.decode(codes[1])) == 448.0
    assert fp8.page_scale(np.zeros(4, np.float32)) == np.float32(1.0)
    back = fp8.decode(codes) * float(s)
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -4 + 1e-12)
