"""Pins for the oracle's FP8 E4M3 codec (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import fp8, sage

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")


def test_all_codes_round_trip():
    codes = np.arange(256, dtype=np.uint8)
    vals = fp8.decode(codes)
    finite = ~np.isnan(vals)
    assert finite.sum() == 254                       # only S.1111.111 is NaN
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF])
    back = fp8.encode_sat(vals[finite].astype(np.float32))
    assert np.array_equal(back, codes[finite])


def test_landmark_values():
    assert fp8.decode(0x7E) == 448.0                  # largest finite
    assert fp8.decode(0x01) == 2.0 ** -9              # smallest subnormal
    assert fp8.decode(0x08) == 2.0 ** -6              # smallest normal
    assert fp8.decode(0x38) == 1.0
    assert fp8.decode(0x80) == 0.0 and np.signbit(fp8.decode(0x80))


@pytest.mark.parametrize("x,code", [
    (1.0625, 0x38),        # tie between 1.0 (even) and 1.125 -> 1.0
    (1.1875, 0x3A),        # tie between 1.125 (odd) and 1.25 (even) -> 1.25
    (2.0 ** -10, 0x00),    # tie between 0 and 2^-9 -> 0
    (3 * 2.0 ** -10, 0x02),  # tie between 2^-9 (odd) and 2^-8 (even) -> 2^-8
    (432.0, 0x7E),         # tie between 416 (odd) and 448 (even)
    (449.0, 0x7E), (464.0, 0x7E), (1e6, 0x7E), (np.inf, 0x7E),   # saturation
    (-500.0, 0xFE), (-0.0, 0x80), (-2.0 ** -11, 0x80),
])
def test_rne_ties_and_saturation(x, code):
    assert int(fp8.encode_sat(np.array([x]))[0]) == code


def test_nearest_by_brute_force():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(4000) * np.exp2(rng.uniform(-12, 9, 4000))).astype(np.float32)
    got = fp8.decode(fp8.encode_sat(x))
    table = fp8.DECODE_TABLE[np.isfinite(fp8.DECODE_TABLE)]
    for xi, gi in zip(x.astype(np.float64), got):
        if abs(xi) >= 448:
            assert abs(gi) == 448 and np.sign(gi) == np.sign(xi)
            continue
        dist = np.abs(table - xi)
        best = dist.min()
        assert abs(gi - xi) == best                   # a nearest value is chosen


def test_agrees_with_torch_in_range():
    rng = np.random.default_rng(2)
    vals = fp8.DECODE_TABLE[:0x7F]
    mids = 0.5 * (vals[:-1] + vals[1:])
    x = np.concatenate([
        mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9), -mids,
        rng.uniform(-463.9, 463.9, 20000), rng.standard_normal(20000) * 0.01,
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.encode_sat(x), ref)


def test_dynamic_range_matches_pages():
    """The pages state the per-channel range after scaling to V_r is V_r * 2^9."""
    g = json.load(open(GOLDEN))["fp8_dynamic_range"]
    for vr, rng_ in ((g["v_range_sa2"], g["range_sa2"]), (g["v_range_sa2pp"], g["range_sa2pp"])):
        assert vr / fp8.decode(0x01) == rng_
        # a V entry of amax / range is scaled onto the smallest subnormal; well below it -> 0
        v = np.array([[1.0], [1.0 / rng_], [0.4 / rng_]], dtype=np.float16)
        codes, delta, amax = sage.quantize_v(v, vr)
        assert fp8.decode(codes[1, 0]) == pytest.approx(2.0 ** -9, rel=2e-3)
        assert codes[2, 0] == 0


def test_static_ranges_are_e4m3_max():
    g = json.load(open(GOLDEN))["sa2_static_ranges"]
    assert g["p_range"] == sage.DEFAULT.p_range == fp8.E4M3_MAX
    assert g["v_range"] == sage.DEFAULT.v_range == fp8.E4M3_MAX
