"""Pins for two readings the pages leave open, CPU only.

Row sum.  The pages do not say whether the softmax normaliser l sums the quantized weights
P~_q / P_r (the weights that multiply V) or the unquantized probabilities p.  The oracle takes
the first; the second is kept behind prologue(row_sum="unquantized").  Held against exact fp64
attention on stand-ins for the four workload shapes, the chosen reading must be at least as
accurate: strictly lower RMSE where the P~V quantization dominates the error (INT8 QK), and
within 1e-4 (relative) where the INT4-range QK quantization dominates it.

Static range of P~.  P~ = E4M3sat(RN32(p * P_r)) with delta_P = 1 / P_r (a static range,
valid because p <= 1).  Only the block holding a row's running maximum reaches its largest p
(in (1/2, 1] with the power-of-two maximum below), and entries with p * P_r at or below 2^-10
are coded as zero; p_quant_stats counts them.  Pinned here against scalar loops and the E4M3
grid.

Running maximum.  The pages do not say which maximum the online softmax subtracts; any m at or
above the row maximum gives the same unquantized softmax and keeps p <= 1.  The oracle takes
the plain maximum; the maximum rounded up so that e^m is a power of two (block_top) is kept
behind prologue(max_ref="pow2").  Against exact fp64 attention on the same four stand-ins and
three seeds, the chosen reading must be at least as accurate: strictly lower RMSE where the
P~V quantization dominates the error (INT8 QK) -- there the plain maximum codes the block's
largest weight exactly as P_r -- and within 2e-3 (relative) under INT4-range QK, where the
two differ by noise of that size either way.
"""
import math

import numpy as np
import pytest

from oracle import fp8, sage
from workloads import custom, make_inputs

# stand-ins for the tiny, bench, llm and dit shapes at sizes the oracle finishes in seconds
SAMPLES = {
    "tiny": (custom(1, 2, 2, 256, 64, False, 8), False, 8, True),
    "bench": (custom(1, 2, 2, 1024, 128, False, 8, q_bias_std=1.0), False, 8, True),
    "llm": (custom(1, 2, 2, 1024, 128, True, 4, q_bias_std=1.0, outlier_frac=0.01, outlier_scale=10.0),
            True, 4, False),
    "dit": (custom(1, 2, 2, 1250, 64, False, 8, text_tokens=226, text_std=2.0), False, 8, True),
}


def _err(o, e):
    rmse = math.sqrt(((o - e) ** 2).mean())
    cos = (o * e).sum() / math.sqrt((o * o).sum() * (e * e).sum())
    return rmse, float(np.abs(o - e).max()), cos


@pytest.mark.parametrize("name", list(SAMPLES))
def test_row_sum_reading_no_less_accurate(name):
    w, causal, bits, pv_dominated = SAMPLES[name]
    q, k, v = make_inputs(w, seed=0)
    e = sage.exact_attention(q, k, v, causal)
    rw, mw, cw = _err(sage.sage_attention(q, k, v, causal, bits, row_sum="weights"), e)
    ru, mu, cu = _err(sage.sage_attention(q, k, v, causal, bits, row_sum="unquantized"), e)
    print(f"{name}: RMSE {rw:.6g} (weights) vs {ru:.6g} (unquantized p); max-abs {mw:.4g} vs {mu:.4g}; "
          f"cos {cw:.7f} vs {cu:.7f}")
    assert rw <= ru * (1 + 1e-4)
    assert cw >= cu - 1e-6
    if pv_dominated:
        assert rw < ru


@pytest.mark.parametrize("name", list(SAMPLES))
def test_running_max_reading_no_less_accurate(name):
    w, causal, bits, pv_dominated = SAMPLES[name]
    for seed in range(3):
        q, k, v = make_inputs(w, seed=seed)
        e = sage.exact_attention(q, k, v, causal)
        rx, _, cx = _err(sage.sage_attention(q, k, v, causal, bits, max_ref="exact"), e)
        rp, _, cp = _err(sage.sage_attention(q, k, v, causal, bits, max_ref="pow2"), e)
        print(f"{name} seed {seed}: RMSE {rx:.6g} (plain maximum) vs {rp:.6g} (power of two); "
              f"cos {cx:.7f} vs {cp:.7f}")
        assert rx <= rp * (1 + 2e-3)
        if pv_dominated:
            assert rx < rp and cx > cp


def test_running_max_readings_agree_without_pv_quantization():
    """With P V unquantized nothing is rounded at the maximum's scale: both readings give the same
    output up to fp64 rounding."""
    q, k, v = make_inputs(custom(1, 2, 1, 300, 64, True, 8, q_bias_std=1.0), seed=3)
    a = sage.sage_attention(q, k, v, True, 8, quant_pv=False, max_ref="exact")
    b = sage.sage_attention(q, k, v, True, 8, quant_pv=False, max_ref="pow2")
    assert np.abs(a - b).max() <= 1e-12 * np.abs(a).max()


def test_row_sum_readings_agree_without_pv_quantization():
    """With P V unquantized the weights are p itself: both readings give the same output."""
    q, k, v = make_inputs(custom(1, 2, 1, 300, 64, True, 8, q_bias_std=1.0), seed=3)
    a = sage.sage_attention(q, k, v, True, 8, quant_pv=False, row_sum="weights")
    b = sage.sage_attention(q, k, v, True, 8, quant_pv=False, row_sum="unquantized")
    assert np.array_equal(a, b)


def test_row_sum_switch_rejects_unknown_reading():
    q, k, v = make_inputs(custom(1, 1, 1, 8, 16), seed=0)
    with pytest.raises(ValueError):
        sage.prologue(q, k, v, row_sum="l1")
    with pytest.raises(ValueError):
        sage.prologue(q, k, v, max_ref="mean")


def _scalar_counts(pro, b, h, qb):
    """p_quant_stats by scalar loops over (row, key), written from the definitions."""
    g = pro.geom
    z = sage.logits(pro, b, h, qb)
    zero = sub = zero_blk = n = rb = below = 0
    smallest_normal = 2.0 ** -6
    for r in range(z.shape[0]):
        m = -math.inf
        for kb in range(pro.nkb):
            keys = range(kb * g.bk, min(pro.N, (kb + 1) * g.bk))
            vals = [z[r, j] for j in keys]
            m = max([m] + vals)
            ps = [math.exp(x - m) if x > -math.inf else None for x in vals]
            live = [p for p in ps if p is not None]
            if not live:
                continue
            rb += 1
            bmax = max(live)
            below += bmax < 1.0
            for p in live:
                n += 1
                code = float(fp8.round_sat(np.array([np.float32(p * g.p_range)]))[0])
                zero += p > 0 and code == 0
                sub += 0 < code < smallest_normal
                code_blk = float(fp8.round_sat(np.array([np.float32(p * (g.p_range / bmax))]))[0])
                zero_blk += p > 0 and code_blk == 0
    return dict(n=n, zero_static=zero, subnormal_static=sub, zero_block_scale=zero_blk, rows_blocks=rb,
                rows_blocks_below_one=below)


@pytest.mark.parametrize("causal", [False, True])
def test_p_quant_stats_match_scalar_loops(causal):
    # wide logits (q scaled x6) so that some p fall below the E4M3 range
    w = custom(1, 1, 1, 70, 16, causal, 8, q_bias_std=1.0)
    q, k, v = make_inputs(w, seed=5)
    q = (q.astype(np.float32) * 6).astype(np.float16)
    g = sage.Geometry(bq=16, bk=16, k_slice=16)
    pro = sage.prologue(q, k, v, causal, 8, g)
    tot = {}
    for qb in range(pro.nqb):
        got = sage.p_quant_stats(pro, 0, 0, qb)
        assert got == _scalar_counts(pro, 0, 0, qb)
        for key, val in got.items():
            tot[key] = tot.get(key, 0) + val
    assert tot["zero_static"] > 0 and tot["subnormal_static"] > 0      # the cases are exercised
    assert tot["zero_block_scale"] <= tot["zero_static"]
    assert 0 < tot["rows_blocks_below_one"] < tot["rows_blocks"]


@pytest.mark.parametrize("max_ref", ["exact", "pow2"])
def test_static_range_reaches_p_range_only_in_the_running_max_block(max_ref):
    """Plain maximum: in the block that raises (or first sets) a row's running maximum the largest
    p is 1 and its P~ is exactly P_r = 448; in every other block every p is below 1 (P~ may still
    round up to 448 from p > 432/448, the E4M3 midpoint below 448), so the static scale 1/P_r
    never saturates.  Power-of-two maximum: the largest p of the block that sets it lies in
    (1/2, 1], so its P~ in [224, 448]; every p stays <= 1 and P~ <= 448."""
    w = custom(1, 1, 1, 512, 32, False, 8, q_bias_std=1.0)
    q, k, v = make_inputs(w, seed=9)
    pro = sage.prologue(q, k, v, False, 8, max_ref=max_ref)
    g = pro.geom
    z = sage.logits(pro, 0, 0, 0)
    m = np.full(z.shape[0], -np.inf)
    others = 0
    for kb in range(pro.nkb):
        zb = z[:, kb * g.bk:(kb + 1) * g.bk]
        top = sage.block_top(zb, max_ref)
        m_new = np.maximum(m, top)
        p = np.exp(zb - m_new[:, None])
        pt = fp8.round_sat((p * g.p_range).astype(np.float32)).max(axis=1)
        holds = top == m_new
        if max_ref == "exact":
            assert np.all(p.max(axis=1)[holds] == 1.0) and np.all(pt[holds] == 448.0)
            assert np.all(p.max(axis=1)[~holds] < 1.0)
        else:
            pm = p.max(axis=1)[holds]
            assert np.all(pm > 0.5) and np.all(pm <= 1.0) and np.all(pt[holds] >= 224.0)
            assert np.all(p.max(axis=1) <= 1.0)
        assert np.all(pt <= 448.0)
        others += int(np.count_nonzero(~holds))
        m = m_new
    assert others > 0


def test_flushed_mass_matches_scalar_loops():
    w = custom(1, 1, 1, 70, 16, True, 8, q_bias_std=1.0)
    q, k, v = make_inputs(w, seed=5)
    q = (q.astype(np.float32) * 6).astype(np.float16)
    g = sage.Geometry(bq=16, bk=16, k_slice=16)
    pro = sage.prologue(q, k, v, True, 8, g)
    seen = 0.0
    for qb in range(pro.nqb):
        got = sage.p_flushed_mass(pro, 0, 0, qb)
        z = sage.logits(pro, 0, 0, qb)
        for r in range(z.shape[0]):
            top = max(z[r])
            tot = sum(math.exp(x - top) for x in z[r] if x > -math.inf)
            fl, m = 0.0, -math.inf
            for kb in range(pro.nkb):
                keys = range(kb * g.bk, min(pro.N, (kb + 1) * g.bk))
                m = max([m] + [z[r, j] for j in keys])
                for j in keys:
                    if z[r, j] == -math.inf:
                        continue
                    p = math.exp(z[r, j] - m)
                    if p > 0 and float(fp8.round_sat(np.array([np.float32(p * g.p_range)]))[0]) == 0:
                        fl += math.exp(z[r, j] - top)
            assert got[r] == pytest.approx(fl / tot, rel=1e-9, abs=1e-300)
        seen += got.sum()
    assert seen > 0
