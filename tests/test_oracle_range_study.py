"""Pins for the (P_r, V_r) narrowing study (oracle only; runs on the CPU)."""
import json
import os

import numpy as np

from oracle import fp8, range_study as rs, sage as osage
from workloads import custom, make_inputs

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))


def test_bound_matches_pages():
    """The pages' bound P_r V_r <= 2047/2 is 2 x 32 x P_r V_r <= 65504; their three pairs meet
    it and SageAttention2's 448/448 does not."""
    pr = GOLDEN["pv_range_pairs"]
    assert pr["bound"] == 65504 / 64 == 2047 / 2
    for p_r, v_r in pr["pairs"]:
        assert p_r * v_r <= pr["bound"] and rs.fp16_bound_holds(p_r, v_r)
    sa2 = GOLDEN["sa2_static_ranges"]
    assert not rs.fp16_bound_holds(sa2["p_range"], sa2["v_range"])


def test_worst_case_block_finite_only_within_bound():
    """All 64 products at P_r V_r: the fp16 accumulator reaches 64 P_r V_r, finite for the pages'
    pairs (64 x 1008 = 64512 <= 65504) and inf for 448/448."""
    for p_r, v_r in GOLDEN["pv_range_pairs"]["pairs"]:
        pt = np.full((2, 64), p_r)
        vq = np.full((64, 3), v_r)
        assert np.all(fp8.decode(fp8.encode_sat(np.array([p_r, v_r], np.float32))) == [p_r, v_r])
        np.testing.assert_array_equal(rs.pv_local_fp16(pt, vq), 64 * p_r * v_r)
    out = rs.pv_local_fp16(np.full((1, 64), 448.0), np.full((64, 1), 448.0))
    assert np.isinf(out).all()


def test_accumulator_rounding_hand_example():
    """Hand-computed: group 1 sums exactly to 2049.9375 (256*8 + 31/16), one fp16 rounding gives
    2050 (rounding after every product would stay at 2048); group 2 adds 1 on the same fp16
    accumulator: 2051 is a tie between 2050 and 2052, round-half-even gives 2052 (a separate
    accumulator per group would give 2051)."""
    pt = np.zeros((1, 64))
    vq = np.zeros((64, 1))
    pt[0, 0], vq[0, 0] = 256.0, 8.0
    pt[0, 1:32], vq[1:32, 0] = 1.0, 0.0625
    pt[0, 32], vq[32, 0] = 1.0, 1.0
    assert float((pt @ vq)[0, 0]) == 2050.9375
    assert float(rs.pv_local_fp16(pt, vq)[0, 0]) == 2052.0


def test_accumulator_exact_without_rounding():
    """Small integer products: no fp16 rounding happens, so the model equals the exact product."""
    rng = np.random.default_rng(0)
    pt = rng.integers(0, 5, (8, 128)).astype(np.float64)
    vq = rng.integers(-3, 4, (128, 16)).astype(np.float64)
    np.testing.assert_array_equal(rs.pv_local_fp16(pt, vq), pt @ vq)


def test_v_underflow_grows_as_v_range_narrows():
    """The FP8 range of a channel spans V_r 2^9 below its max: halving V_r can only move more
    nonzero entries below it (and to code 0)."""
    q, k, v = rs.study_inputs("v_wide")
    q, k, v = q[:, :1, :256], k[:, :1, :256], v[:, :1, :256]
    prev = (-1.0, -1.0)
    for v_r in (448.0, 9.0, 4.5, 2.25):
        pro = osage.prologue(q, k, v, False, 8, osage.Geometry(v_range=v_r))
        below, flushed = rs.v_underflow(pro)
        assert below >= prev[0] and flushed >= prev[1] and flushed <= below
        prev = (below, flushed)
    assert prev[0] > 0


def test_study_rows():
    """Small run: the fp16 accumulator overflows with 448/448 and stays finite and accurate with
    the pages' pairs; the fp32-buffer SageAttention2 row is the accuracy reference."""
    w = custom(1, 1, 1, 256, 64, False, 8)
    q, k, v = make_inputs(w, seed=2)
    rows = rs.run(q, k, v, rs.STUDY_PAIRS)
    by = {(r["p_range"], r["v_range"], r["accum"]): r for r in rows}
    assert not by[(448.0, 448.0, "fp16")]["finite"]
    assert by[(448.0, 448.0, "fp32")]["cos"] > 0.999
    for p_r, v_r in GOLDEN["pv_range_pairs"]["pairs"]:
        r = by[(p_r, v_r, "fp16")]
        assert r["finite"] and r["bound_holds"] and r["cos"] > 0.998
