"""Pins for the oracle's attention steps (Delta_S, logits, online softmax, FP8 PV), CPU only.

With quantization switched off the method must reduce to textbook softmax attention, since
smoothing only adds row constants to the logits; this pins the sign and scale of Delta_S, the
online softmax, the causal mask and the GQA head mapping.  Other pins: invariance of the
output under adding a constant row to K, normalisation of the quantized weights, and a
brute-force re-computation on tiny inputs.
"""
import math

import numpy as np
import pytest

from oracle import fp8, sage
from workloads import custom, make_inputs


def _grid_inputs(B, H, Hkv, N, d, seed, step=2.0 ** -6, lim=4.0):
    """fp16 inputs on a coarse grid: with N a power of two every mean and every smoothed
    value is exact in fp32, so smoothing introduces no rounding at all."""
    rng = np.random.default_rng(seed)
    def draw(h):
        x = np.clip(rng.standard_normal((B, h, N, d)), -lim / 1.01, lim / 1.01)
        return (np.round(x / step) * step).astype(np.float16)
    return draw(H), draw(Hkv), draw(Hkv)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv", [(2, 2), (4, 2)])
def test_unquantized_reduces_to_exact_attention(causal, H, Hkv):
    q, k, v = _grid_inputs(1, H, Hkv, 256, 32, seed=10)
    k = (k.astype(np.float32) + np.float32(2.0)).astype(np.float16)    # a large K mean
    o = sage.sage_attention(q, k, v, causal, 8, quant_qk=False, quant_pv=False)
    e = sage.exact_attention(q, k, v, causal)
    assert np.abs(o - e).max() < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_exact_attention_matches_torch_sdpa(causal):
    """The fp64 reference itself, against PyTorch's scaled_dot_product_attention on the CPU in
    float64 (an independent implementation; GQA by repeating each kv head H / Hkv times)."""
    torch = pytest.importorskip("torch")
    q, k, v = make_inputs(custom(2, 4, 2, 77, 32, q_bias_std=1.0), seed=21)
    e = sage.exact_attention(q, k, v, causal)
    tq, tk, tv = (torch.from_numpy(x.astype(np.float64)) for x in (q, k, v))
    tk, tv = tk.repeat_interleave(2, dim=1), tv.repeat_interleave(2, dim=1)
    t = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal).numpy()
    assert np.abs(e - t).max() < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_exact_attention_rows_is_a_row_slice(causal):
    q, k, v = make_inputs(custom(1, 1, 1, 300, 32, q_bias_std=1.0), seed=22)
    e = sage.exact_attention(q, k, v, causal)[0, 0]
    rows = np.array([0, 1, 127, 128, 200, 299])
    assert np.abs(sage.exact_attention_rows(q[0, 0], k[0, 0], v[0, 0], rows, causal) - e[rows]).max() < 1e-13


def test_unquantized_ragged_close_to_exact():
    q, k, v = make_inputs(custom(2, 2, 1, 301, 64, q_bias_std=1.0), seed=11)
    for causal in (False, True):
        o = sage.sage_attention(q, k, v, causal, 8, quant_qk=False, quant_pv=False)
        e = sage.exact_attention(q, k, v, causal)
        assert np.abs(o - e).max() < 1e-5


def test_q_smoothing_alone_is_exact():
    """Smoothing Q with the bias term added back changes nothing (quantization off)."""
    q, k, v = _grid_inputs(1, 2, 2, 256, 32, seed=12)
    q = (q.astype(np.float32) + np.float32(1.5)).astype(np.float16)
    a = sage.sage_attention(q, k, v, False, 8, quant_qk=False, quant_pv=False, smooth_q=True)
    b = sage.sage_attention(q, k, v, False, 8, quant_qk=False, quant_pv=False, smooth_q=False)
    assert np.abs(a - b).max() < 1e-12


def test_k_shift_invariance_exact_and_bitwise():
    q, k, v = _grid_inputs(1, 2, 2, 256, 64, seed=13, lim=3.9)
    rng = np.random.default_rng(14)
    c = (np.round(np.clip(rng.standard_normal((1, 2, 1, 64)), -3.9, 3.9) / 2.0 ** -6) * 2.0 ** -6)
    k2 = (k.astype(np.float64) + c).astype(np.float16)
    assert np.array_equal(k2.astype(np.float64), k.astype(np.float64) + c)   # shift is exact
    e1, e2 = sage.exact_attention(q, k, v), sage.exact_attention(q, k2, v)
    assert np.abs(e1 - e2).max() < 1e-12
    for bits in (8, 4):
        p1, p2 = sage.prologue(q, k, v, False, bits), sage.prologue(q, k2, v, False, bits)
        assert np.array_equal(p1.gamma_k, p2.gamma_k)
        assert np.array_equal(p1.k_codes, p2.k_codes) and np.array_equal(p1.k_delta, p2.k_delta)
        o1 = sage.sage_attention(q, k, v, False, bits)
        o2 = sage.sage_attention(q, k2, v, False, bits)
        assert np.array_equal(o1, o2)


@pytest.mark.parametrize("causal", [False, True])
def test_weights_normalised(causal):
    """With V = 1 the output is the sum of the attention weights: 1 for fp32 P, and 1 for the
    quantized P~ too, since l sums the very weights that multiply V (V = 1 is exact in FP8)."""
    q, k, _ = make_inputs(custom(1, 2, 2, 300, 64, q_bias_std=1.0), seed=15)
    v = np.ones_like(k)
    o = sage.sage_attention(q, k, v, causal, 8, quant_pv=False)
    assert np.abs(o - 1).max() < 1e-12
    oq = sage.sage_attention(q, k, v, causal, 8)
    one = 448.0 * float(np.float32(1.0) / np.float32(448.0))     # V_q * delta_V for V = 1
    assert np.abs(oq - one).max() < 1e-12


def test_online_softmax_state():
    """l * e^m of the online pass equals the two-pass sum of e^z (P V unquantized, so the
    weights are p itself); m is the row maximum, or (default reading) the smallest m >= it with
    e^m a power of two."""
    q, k, v = make_inputs(custom(1, 1, 1, 384, 64), seed=16)
    for max_ref in ("exact", "pow2"):
        pro = sage.prologue(q, k, v, False, 8, quant_pv=False, max_ref=max_ref)
        _, m, l = sage.attend_block(pro, 0, 0, 1, return_state=True)
        z = sage.logits(pro, 0, 0, 1)
        top = z.max(axis=1)
        assert np.allclose(l * np.exp(m - top), np.exp(z - top[:, None]).sum(axis=1), rtol=1e-12)
        if max_ref == "exact":
            assert np.array_equal(m, top)
        else:
            e = m / math.log(2.0)                       # an integer, at most one above log2(e) max z
            assert np.allclose(e, np.rint(e), rtol=0, atol=1e-9)
            assert np.all(m >= top) and np.all(m - top < math.log(2.0))


def test_quantized_accuracy_is_near_exact():
    q, k, v = make_inputs("tiny")
    o = sage.sage_attention(q, k, v, False, 8)
    e = sage.exact_attention(q, k, v)
    cos = (o * e).sum() / math.sqrt((o * o).sum() * (e * e).sum())
    assert cos > 0.999
    o4 = sage.sage_attention(q, k, v, False, 4)
    cos4 = (o4 * e).sum() / math.sqrt((o4 * o4).sum() * (e * e).sum())
    assert 0.95 < cos4 < cos


# ----------------------------------------------------------------------------------------
# brute force on tiny inputs: scalar loops, written independently of the vectorised oracle
# ----------------------------------------------------------------------------------------
def _brute(q, k, v, causal, R, bq, bk, kslice, kperiod, krun, p_range, v_range):
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    f32 = np.float32
    out = np.zeros((B, H, N, d))
    for b in range(B):
        for h in range(H):
            hk = h // (H // Hkv)
            K = k[b, hk]
            muk = [f32(sum(float(K[j, c]) for j in range(N)) / N) for c in range(d)]
            gk = [[f32(f32(K[j, c]) - muk[c]) for c in range(d)] for j in range(N)]
            kg = {}
            for j in range(N):
                kg.setdefault((j // kslice, (j % kperiod) // krun), []).append(j)
            kcode = [[0] * d for _ in range(N)]
            kdel = [f32(0)] * N
            for members in kg.values():
                amax = max(abs(gk[j][c]) for j in members for c in range(d))
                dl = f32(amax / f32(R))
                inv = f32(f32(R) / amax) if amax > 0 else f32(0)
                for j in members:
                    kdel[j] = dl
                    for c in range(d):
                        kcode[j][c] = int(max(-R, min(R, np.rint(f32(gk[j][c] * inv)))))
            V = v[b, hk]
            vam = [max(abs(f32(V[j, c])) for j in range(N)) for c in range(d)]
            vdl = [f32(a / f32(v_range)) for a in vam]
            vinv = [f32(f32(v_range) / a) if a > 0 else f32(0) for a in vam]
            vq = [[float(fp8.round_sat(np.array([f32(f32(V[j, c]) * vinv[c])]))[0]) for c in range(d)] for j in range(N)]
            Q = q[b, h]
            for qb in range(-(-N // bq)):
                rows = list(range(qb * bq, min(N, (qb + 1) * bq)))
                muq = [f32(sum(float(Q[i, c]) for i in rows) / len(rows)) for c in range(d)]
                gq = {i: [f32(f32(Q[i, c]) - muq[c]) for c in range(d)] for i in rows}
                ds = [sum(float(muq[c]) * float(gk[j][c]) for c in range(d)) for j in range(N)]
                for i in rows:
                    amax = max(abs(x) for x in gq[i])
                    qd = f32(amax / f32(R))
                    qinv = f32(f32(R) / amax) if amax > 0 else f32(0)
                    qc = [int(max(-R, min(R, np.rint(f32(x * qinv))))) for x in gq[i]]
                    z = []
                    for j in range(N):
                        s = sum(qc[c] * kcode[j][c] for c in range(d))
                        zz = (s * float(qd) * float(kdel[j]) + ds[j]) / math.sqrt(d)
                        z.append(-math.inf if (causal and j > i) else zz)
                    m, l, acc = -math.inf, 0.0, [0.0] * d
                    for kb in range(-(-N // bk)):
                        blk = range(kb * bk, min(N, (kb + 1) * bk))
                        mn = max([m] + [z[j] for j in blk])
                        al = math.exp(m - mn) if m > -math.inf else 0.0
                        ps = {j: (math.exp(z[j] - mn) if z[j] > -math.inf else 0.0) for j in blk}
                        pt = {j: float(fp8.round_sat(np.array([f32(ps[j] * p_range)]))[0]) for j in blk}
                        l = l * al + sum(pt.values()) / p_range     # the weights that multiply V
                        for c in range(d):
                            acc[c] = acc[c] * al + sum(pt[j] * vq[j][c] for j in blk)
                        m = mn
                    for c in range(d):
                        out[b, h, i, c] = acc[c] * float(vdl[c]) / (p_range * l)
    return out


@pytest.mark.parametrize("causal,R", [(False, 127), (True, 7)])
def test_brute_force_tiny(causal, R):
    q, k, v = make_inputs(custom(1, 2, 1, 21, 8, q_bias_std=1.0), seed=17)
    g = sage.Geometry(bq=8, bk=8, q_slice=1, q_period=1, q_run=1, k_slice=8, k_period=8, k_run=4)
    o = sage.sage_attention(q, k, v, causal, 8 if R == 127 else 4, g)
    ref = _brute(q, k, v, causal, R, 8, 8, 8, 8, 4, 448.0, 448.0)
    assert np.abs(o - ref).max() < 1e-9 * max(1.0, np.abs(ref).max())


def _attend_perturbed(pro, b, h, qb, eps):
    """The online softmax and FP8 P~V of one Q block with every p scaled by (1 + eps) before its
    FP8 rounding (l keeps the exact p): a stand-in for any faithful computation of the logits."""
    g = pro.geom
    hk = pro.kv_head(h)
    z = sage.logits(pro, b, h, qb)
    vq = fp8.decode(pro.v_codes[b, hk])
    m = np.full(z.shape[0], -np.inf)
    l = np.zeros(z.shape[0])
    acc = np.zeros((z.shape[0], pro.d))
    for kb in range(pro.nkb):
        zb = z[:, kb * g.bk:min(pro.N, (kb + 1) * g.bk)]
        m_new = np.maximum(m, sage.block_top(zb, pro.max_ref))
        alpha = np.where(np.isfinite(m), np.exp(m - m_new), 0.0)
        p = np.exp(zb - m_new[:, None])
        pt = fp8.round_sat((p * (1.0 + eps) * g.p_range).astype(np.float32))
        l = l * alpha + pt.sum(axis=1) / g.p_range
        acc = acc * alpha[:, None] + pt @ vq[kb * g.bk:min(pro.N, (kb + 1) * g.bk)]
        m = m_new
    return acc * pro.v_delta[b, hk].astype(np.float64)[None, :] / (g.p_range * l[:, None])


def test_fp8_midpoint_slack_bounds_flipped_decisions():
    """Perturbing every p by 2^-15 (relative) flips the P~ codes that sit within that distance of
    an E4M3 midpoint; the output must move by no more than fp8_midpoint_slack (rel 2^-14) allows,
    and some codes must actually flip (the bound is exercised)."""
    q, k, v = make_inputs(custom(1, 2, 1, 300, 64, True, 8, q_bias_std=1.0), seed=31)
    pro = sage.prologue(q, k, v, True, 8)
    moved = 0
    for h in range(2):
        for qb in range(pro.nqb):
            base = sage.attend_block(pro, 0, h, qb)
            slack = sage.fp8_midpoint_slack(pro, 0, h, qb, rel=2.0 ** -14)
            assert np.all(slack >= 0)
            for eps in (2.0 ** -15, -2.0 ** -15):
                d = np.abs(_attend_perturbed(pro, 0, h, qb, eps) - base)
                assert np.all(d <= slack + 1e-12)
                moved += int(np.count_nonzero(d > 1e-12))
    assert moved > 0


def _attend_shifted(pro, b, h, qb, flip, up):
    """The online softmax and FP8 P~V of one Q block under the power-of-two running maximum,
    where the rows flip[r] take, in every block, the integer maximum one higher (up) or one lower
    than the oracle's: the alternative that a computation of the logits in fp32 can reach where
    a maximum sits on an integer."""
    g = pro.geom
    hk = pro.kv_head(h)
    z = sage.logits(pro, b, h, qb)
    vq = fp8.decode(pro.v_codes[b, hk])
    rows = z.shape[0]
    m = np.full(rows, -np.inf)
    l = np.zeros(rows)
    acc = np.zeros((rows, pro.d))
    off = np.zeros(rows)
    for kb in range(pro.nkb):
        zb = z[:, kb * g.bk:min(pro.N, (kb + 1) * g.bk)]
        m_true = np.maximum(m, sage.block_top(zb, "pow2"))
        off = np.where(flip, (1.0 if up else -1.0) * math.log(2.0), 0.0)
        m_new = m_true + off
        alpha = np.where(np.isfinite(m), np.exp(m - m_new), 0.0)
        p = np.exp(zb - m_new[:, None])
        pt = fp8.round_sat((p * g.p_range).astype(np.float32))
        l = l * alpha + pt.sum(axis=1) / g.p_range
        acc = acc * alpha[:, None] + pt @ vq[kb * g.bk:min(pro.N, (kb + 1) * g.bk)]
        m = m_new
    return acc * pro.v_delta[b, hk].astype(np.float64)[None, :] / (g.p_range * l[:, None])


def test_fp8_slack_bounds_a_shifted_integer_maximum():
    """With a tolerance wide enough that the integer-maximum decision counts as ambiguous in every
    row (int_rel 1/2) and the midpoint tolerance switched off (rel 2^-60), a run whose rows all
    take the integer maximum one higher from the start must stay within fp8_midpoint_slack: such a
    shift scales every p by 1/2 and only the E4M3 subnormal range rounds differently.  (One lower
    is an alternative only where the maximum sits on an integer, so p still stays <= 1; that is
    the same scaling the other way.)  Wide logits put entries in the subnormal range."""
    q, k, v = make_inputs(custom(1, 1, 1, 384, 64, False, 8, q_bias_std=1.0), seed=41)
    q = (q.astype(np.float32) * 4).astype(np.float16)
    pro = sage.prologue(q, k, v, False, 8, max_ref="pow2")
    moved = 0
    for qb in range(pro.nqb):
        base = sage.attend_block(pro, 0, 0, qb)
        slack = sage.fp8_midpoint_slack(pro, 0, 0, qb, rel=2.0 ** -60, int_rel=0.5)
        flip = np.ones(base.shape[0], bool)
        d = np.abs(_attend_shifted(pro, 0, 0, qb, flip, True) - base)
        assert np.all(d <= slack + 1e-12)
        moved += int(np.count_nonzero(d > 1e-12))
    assert moved > 0
