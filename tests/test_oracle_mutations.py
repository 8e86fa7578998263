"""Planted mistakes: each mutation of the oracle must be caught by at least one pin.

Every mutation is applied to the oracle on the CPU (monkeypatch), the pins below are run,
and the test passes only if some pin fails.  This shows that the pins constrain the parts
of the oracle they claim to pin: a dropped or sign-flipped Delta_S, a wrong GQA head map,
an off-by-one causal mask, a wrong softmax scale, a lost V scale, a wrong K group shape, a
missed rescale of the running row sum, a mean divided by n + 1, codes truncated instead of
rounded, an FP8 codec that saturates at 240, and smoothing skipped while its bias is kept.
"""
import math

import numpy as np
import pytest

from oracle import fp8, sage
import test_oracle_attention as A
import test_oracle_fp8 as F
import test_oracle_quant as Qt


def _pins():
    yield lambda: A.test_unquantized_reduces_to_exact_attention(False, 4, 2)
    yield lambda: A.test_unquantized_reduces_to_exact_attention(True, 4, 2)
    yield lambda: A.test_unquantized_ragged_close_to_exact()
    yield lambda: A.test_weights_normalised(True)
    yield lambda: A.test_brute_force_tiny(True, 7)
    yield lambda: A.test_k_shift_invariance_exact_and_bitwise()
    yield lambda: Qt.test_default_groups_follow_lane_layout()
    yield lambda: Qt.test_mean_is_order_free_and_within_one_ulp()
    yield lambda: Qt.test_dequant_error_bound_and_code_range()
    yield lambda: F.test_rne_ties_and_saturation(432.0, 0x7E)
    yield lambda: F.test_nearest_by_brute_force()


def _caught():
    for pin in _pins():
        try:
            pin()
        except AssertionError:
            return True
    return False


def test_unmutated_oracle_passes_every_pin():
    assert not _caught()


def _wrap(mp, name, fn):
    orig = getattr(sage, name)
    mp.setattr(sage, name, lambda *a, **kw: fn(orig, *a, **kw))


MUTATIONS = {
    "delta_s_sign": lambda mp: _wrap(mp, "delta_s", lambda f, *a: -f(*a)),
    "delta_s_dropped": lambda mp: _wrap(mp, "delta_s", lambda f, *a: 0 * f(*a)),
    "gqa_map_modulo": lambda mp: mp.setattr(sage.Prologue, "kv_head", lambda self, h: h % self.Hkv),
    "causal_masks_diagonal": lambda mp: _wrap(
        mp, "logits", lambda f, pro, b, h, qb: _mask_diag(f(pro, b, h, qb), pro, qb)),
    "softmax_scale_1_over_d": lambda mp: _wrap(
        mp, "logits", lambda f, pro, b, h, qb: f(pro, b, h, qb) / math.sqrt(pro.d)),
    "v_scale_doubled": lambda mp: _wrap(
        mp, "quantize_v", lambda f, *a: (lambda r: (r[0], r[1] * 2, r[2]))(f(*a))),
    "k_group_too_wide": lambda mp: _wrap(
        mp, "group_ids", lambda f, n, s, p, r: f(n, s, p, r * 2)),
    "row_sum_not_rescaled": lambda mp: mp.setattr(np, "exp", _exp_one_for_alpha),
    "mean_divides_by_n_plus_1": lambda mp: _wrap(
        mp, "exact_mean", lambda f, x: (f(x) * np.float32(x.shape[0] / (x.shape[0] + 1))).astype(np.float32)),
    "codes_truncated": lambda mp: mp.setattr(np, "rint", np.trunc),
    "fp8_saturates_at_240": lambda mp: _wrap_fp8(mp, lambda f, x: f(np.clip(np.asarray(x), -240.0, 240.0))),
    "smoothing_skipped": lambda mp: _wrap(mp, "smooth", lambda f, x, mu: f(x, 0 * np.asarray(mu))),
}


def _wrap_fp8(mp, fn):
    orig = fp8.encode_sat
    mp.setattr(fp8, "encode_sat", lambda *a, **kw: fn(orig, *a, **kw))


def _mask_diag(z, pro, qb):
    if pro.causal:
        r0 = qb * pro.geom.bq
        z = z.copy()
        for t in range(z.shape[0]):
            if r0 + t > 0:
                z[t, r0 + t] = -np.inf
    return z


_real_exp = np.exp


def _exp_one_for_alpha(x, *a, **kw):
    """exp that returns 1 for 1-D arguments: inside attend_block those are the running-max
    corrections alpha, so the row sum and accumulator are never rescaled."""
    r = _real_exp(x, *a, **kw)
    if np.ndim(x) == 1:
        return np.ones_like(r)
    return r


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    MUTATIONS[name](monkeypatch)
    assert _caught(), f"planted mistake {name!r} passed every pin"
