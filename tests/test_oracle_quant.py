"""Pins for the oracle's exact means, smoothing and grouped quantization (CPU only)."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import sage


def _random_fp16(rng, n, d):
    bits = rng.integers(0, 0x7C00, size=(n, d), dtype=np.uint16)        # finite, non-negative
    bits |= (rng.integers(0, 2, size=(n, d), dtype=np.uint16) << 15)    # random sign
    x = bits.view(np.float16)
    x[0, 0] = np.float16(65504.0)
    x[1, 0] = np.float16(-65504.0)
    x[2, 1] = np.float16(2.0 ** -24)                                   # smallest subnormal
    return x


def test_fixed_point_sum_is_exact_rational_sum():
    rng = np.random.default_rng(3)
    x = _random_fp16(rng, 37, 5)
    s = sage.fixed_point_colsum(x)
    for c in range(x.shape[1]):
        exact = sum(Fraction(float(v)) for v in x[:, c])
        assert Fraction(int(s[c]), 2 ** 24) == exact


def test_mean_is_order_free_and_within_one_ulp():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((300, 16)) * 3).astype(np.float16)
    m = sage.exact_mean(x)
    perm = rng.permutation(300)
    assert np.array_equal(m, sage.exact_mean(x[perm]))
    for c in range(16):
        exact = sum(Fraction(float(v)) for v in x[:, c]) / 300
        ulp = np.spacing(np.abs(m[c]))
        assert abs(Fraction(float(m[c])) - exact) <= Fraction(float(ulp))


def test_dequant_error_bound_and_code_range():
    rng = np.random.default_rng(5)
    gamma = (rng.standard_normal((256, 64)) * np.exp(rng.standard_normal((1, 64)))).astype(np.float32)
    gamma[17, 3] = 300.0                                                # outlier
    for R in (127, 7):
        gid = sage.group_ids(256, 128, 8, 4)
        codes, delta, amax = sage.quantize_groups(gamma, gid, R)
        assert codes.dtype == np.int8 and np.abs(codes.astype(int)).max() <= R
        err = np.abs(gamma.astype(np.float64) - codes.astype(np.float64) * delta[:, None].astype(np.float64))
        assert np.all(err <= delta[:, None].astype(np.float64) / 2 * (1 + 2.0 ** -20))
        for g in np.unique(gid):
            rows = gid == g
            assert np.abs(codes[rows].astype(int)).max() == R            # the group max maps to +-R
            assert amax[rows][0] == np.abs(gamma[rows]).max()


def test_zero_group_has_zero_scale_and_codes():
    gamma = np.zeros((8, 4), np.float32)
    gamma[4:] = 1.5
    codes, delta, _ = sage.quantize_groups(gamma, np.array([0] * 4 + [1] * 4), 127)
    assert np.all(codes[:4] == 0) and np.all(delta[:4] == 0)
    assert np.all(codes[4:] == 127) and np.all(delta[4:] == np.float32(1.5) / np.float32(127))


def _textbook(x, R):
    """Per-row symmetric quantization written from its definition in fp64."""
    amax = np.abs(x).max(axis=1, keepdims=True).astype(np.float64)
    y = x.astype(np.float64) * R / amax
    return np.rint(y), y


@pytest.mark.parametrize("R", [127, 7])
def test_per_token_special_case_is_textbook_per_row(R):
    rng = np.random.default_rng(6)
    x = rng.standard_normal((64, 32)).astype(np.float32)
    codes, delta, _ = sage.quantize_groups(x, sage.group_ids(64, 1, 1, 1), R)
    ref, y = _textbook(x, R)
    near_tie = np.abs(np.abs(y - np.floor(y)) - 0.5) < 1e-5
    assert np.all((codes == ref) | near_tie)
    assert np.allclose(delta, np.abs(x).max(axis=1) / R, rtol=1e-7)


@pytest.mark.parametrize("R", [127, 7])
def test_per_block_special_case_is_textbook_per_block(R):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((96, 16)).astype(np.float32)
    codes, _, _ = sage.quantize_groups(x, sage.group_ids(96, 32, 1, 1), R)
    for b in range(3):
        blk = x[32 * b:32 * (b + 1)]
        ref, y = _textbook(blk.reshape(1, -1), R)
        near_tie = np.abs(np.abs(y - np.floor(y)) - 0.5) < 1e-5
        assert np.all((codes[32 * b:32 * (b + 1)].reshape(1, -1) == ref) | near_tie)


def test_default_groups_follow_lane_layout():
    """K: keys 8a+4h+r of one 128-key block share a scale per h; Q: one scale per row."""
    g = sage.DEFAULT
    kid = sage.group_ids(300, g.k_slice, g.k_period, g.k_run)
    for j in range(300):
        same = {jj for jj in range(300) if kid[jj] == kid[j]}
        expect = {jj for jj in range(300) if jj // 128 == j // 128 and (jj % 8) // 4 == (j % 8) // 4}
        assert same == expect
    qid = sage.group_ids(300, g.q_slice, g.q_period, g.q_run)
    assert len(np.unique(qid)) == 300


def test_smoothing_removes_channel_mean():
    rng = np.random.default_rng(8)
    k = (rng.standard_normal((512, 32)) + 40 * rng.standard_normal((1, 32))).astype(np.float16)
    mu = sage.exact_mean(k)
    gam = sage.smooth(k, mu)
    assert np.abs(gam.astype(np.float64).mean(axis=0)).max() < 1e-4
    assert np.abs(gam).max() < np.abs(k.astype(np.float32)).max()


def test_integer_scores_are_exact():
    rng = np.random.default_rng(9)
    q = np.asarray(rng.choice([-127, 127], size=(1, 1, 64, 128)), np.int8)
    k = np.asarray(rng.integers(-127, 128, size=(1, 1, 64, 128)), np.int8)
    q[0, 0, 0] = 127
    k[0, 0, 0] = 127                                          # largest possible dot product
    pro = sage.Prologue.__new__(sage.Prologue)
    pro.H = pro.Hkv = 1
    pro.q_codes, pro.k_codes = q, k
    s = sage.scores_int(pro, 0, 0, slice(0, 64), slice(0, 64))
    brute = np.zeros((64, 64), np.int64)
    for i in range(64):
        for j in range(64):
            brute[i, j] = sum(int(a) * int(b) for a, b in zip(q[0, 0, i], k[0, 0, j]))
    assert np.array_equal(s, brute)
    assert s[0, 0] == 127 * 127 * 128


# ------------------------------------------------------------------------------------------
# bf16 inputs: exact means over a 2^-133 .. 2^128 range
# ------------------------------------------------------------------------------------------
def _bf16_columns(seed):
    """bf16 columns that stress an exact sum: random bit patterns (all finite exponents),
    huge values that cancel exactly around a subnormal residue, and mixed magnitudes."""
    from workloads import to_bf16
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 1 << 16, size=(64, 6), dtype=np.uint32)
    bits = np.where(((bits >> 7) & 0xFF) == 0xFF, bits & 0x807F, bits)       # no inf / nan
    x = (bits << 16).view(np.float32).copy()
    x[:, 1] = 0.0
    x[0:20, 1] = to_bf16(np.float32(3.0e38) * rng.uniform(0.5, 1.0, 20).astype(np.float32))
    x[20:40, 1] = -x[0:20, 1]                                                  # cancels exactly
    x[40, 1] = (np.array([3], np.uint32) << 16).view(np.float32)[0]            # a subnormal
    x[:, 2] = to_bf16(rng.standard_normal(64).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 64).astype(np.float32))
    return x


def test_bf16_exact_mean_is_rounded_rational_sum():
    from fractions import Fraction
    for seed in range(5):
        x = _bf16_columns(seed)
        assert sage.is_bf16(x)
        got = sage.exact_mean(x)
        for c in range(x.shape[1]):
            exact = sum(Fraction(float(v)) for v in x[:, c])            # exact rational sum
            ref = np.float32(np.float64(float(exact)) / np.float64(x.shape[0]))
            assert got[c] == ref, (seed, c, got[c], ref)


def test_bf16_exact_mean_order_free_and_matches_fp16_rule():
    x = _bf16_columns(7)
    perm = np.random.default_rng(8).permutation(x.shape[0])
    assert np.array_equal(sage.exact_mean(x), sage.exact_mean(x[perm]))
    # values exact in both formats (8 significant bits, 2^-8 .. 2^7) give the fp16 rule's result
    rng = np.random.default_rng(9)
    y = (rng.integers(-255, 256, size=(300, 16)) * 2.0 ** rng.integers(-8, 0, size=(300, 16))).astype(np.float32)
    assert sage.is_bf16(y)
    assert np.array_equal(sage.exact_mean(y), sage.exact_mean(y.astype(np.float16)))
