"""(P_r, V_r) narrowing study for FP8 P~V with a half-precision accumulator -- oracle only.

TEST INFRASTRUCTURE ONLY: like the rest of oracle/, this module is imported by tests and by
nothing on the product path.  It runs entirely on the CPU (numpy, fp64 unless stated).

Sources (pages):
  * pith.science verdict on arXiv 2505.21136 (SageAttention2++), keys "core_discovery" and
    "key_machinery": the P~V product uses the FP8 matrix instruction that accumulates in fp16;
    one instruction sums 32 products, so |32 p v| must stay within 65504, and with the result of
    a second instruction added in fp16 before the fp32 buffer ("delayed FP32 buffering") the
    ranges must satisfy P_r * V_r <= 2047 / 2.  delta_P = max(P~) / P_r, delta_V = max|V| / V_r.
  * zhaifeiyue.github.io commentary on arXiv 2505.21136: the three options
    (P_r, V_r) = (224, 4.5), (112, 9), (448, 2.25).
  * the same verdict, key "skeptic_critique" (load_bearing_attack, concrete_test): narrowing V_r
    shrinks each channel's FP8 dynamic range to V_r * 2^9, so entries below amax / (V_r 2^9) lose
    all precision; the test counts such entries and checks accuracy.

gfx950 has no FP8 matrix instruction that accumulates in fp16, so this is a numerical study of
the method in the oracle, not a GPU path.

Readings (the pages are silent on these):
  * fp16 accumulator model: the 32 products of one instruction are summed exactly and added to
    the fp16 accumulator with one round-to-nearest-even (overflow gives inf); two instructions
    share the accumulator, which is then added to the fp64 buffer (fp32 on the GPU).
  * V entries "below the FP8 range" are those with |v| V_r / amax_c < 2^-9 (the smallest E4M3
    subnormal); "flushed" ones have code 0 although v != 0.
"""
from __future__ import annotations

import numpy as np

from . import fp8
from . import sage

F64 = np.float64
GROUP = 32          # products summed by one FP8 matrix instruction (k = 32)
PAIR = 2            # instructions that share the fp16 accumulator before the fp32 buffer


def fp16_bound_holds(p_range: float, v_range: float) -> bool:
    """Worst-case accumulator magnitude 2 * 32 * P_r * V_r within fp16's 65504 (core_discovery)."""
    return PAIR * GROUP * p_range * v_range <= 65504.0


def pv_local_fp16(pt: np.ndarray, vq: np.ndarray, group: int = GROUP, pair: int = PAIR) -> np.ndarray:
    """Block-local P~V [rows, d] through the fp16 accumulator model (module readings).

    pt: P~ values (decoded FP8), [rows, keys]; vq: V values (decoded FP8), [keys, d].
    Products of FP8 values and sums of 32 of them are exact in fp64 (at most 49 bits).
    """
    rows, n = pt.shape
    out = np.zeros((rows, vq.shape[1]), F64)
    with np.errstate(over="ignore", invalid="ignore"):
        for g0 in range(0, n, group * pair):
            acc = np.zeros((rows, vq.shape[1]), np.float16)
            for g in range(g0, min(n, g0 + group * pair), group):
                part = pt[:, g:g + group].astype(F64) @ vq[g:g + group].astype(F64)
                acc = (acc.astype(F64) + part).astype(np.float16)
            out += acc.astype(F64)
    return out


def attend_block_fp16acc(pro: sage.Prologue, b: int, h: int, qb: int) -> np.ndarray:
    """Output rows of Q block qb with the block-local P~V through the fp16 accumulator model;
    everything else as in sage.attend_block (same online softmax, same FP8 P~ and V)."""
    g = pro.geom
    hk = pro.kv_head(h)
    z = sage.logits(pro, b, h, qb)
    rows = z.shape[0]
    vq = fp8.decode(pro.v_codes[b, hk])
    p_r = F64(g.p_range)
    m = np.full(rows, -np.inf)
    l = np.zeros(rows)
    acc = np.zeros((rows, pro.d))
    np_err = np.seterr(invalid="ignore", over="ignore")   # an overflowed block carries inf to O
    for kb in range(pro.nkb):
        c0, c1 = kb * g.bk, min(pro.N, (kb + 1) * g.bk)
        zb = z[:, c0:c1]
        m_new = np.maximum(m, sage.block_top(zb, pro.max_ref))
        finite = np.isfinite(m_new)
        alpha = np.where(np.isfinite(m), np.exp(m - np.where(finite, m_new, 0.0)), 0.0)
        p = np.where(finite[:, None], np.exp(zb - np.where(finite, m_new, 0.0)[:, None]), 0.0)
        pt = fp8.round_sat((p * p_r).astype(np.float32))
        l = l * alpha + pt.sum(axis=1) / p_r         # the weights that multiply V, as attend_block
        acc = acc * alpha[:, None] + pv_local_fp16(pt, vq[c0:c1])
        m = m_new
    np.seterr(**np_err)
    return acc * pro.v_delta[b, hk].astype(F64)[None, :] / (p_r * l[:, None])


def v_underflow(pro: sage.Prologue) -> tuple[float, float]:
    """Fractions of nonzero V entries below the FP8 range and flushed to code 0 (module readings)."""
    v = pro.v16.astype(F64)
    amax = pro.v_amax.astype(F64)[:, :, None, :]
    nz = v != 0
    scaled = np.abs(v) * pro.geom.v_range / np.where(amax > 0, amax, 1.0)
    below = nz & (scaled < 2.0 ** -9)
    flushed = nz & (fp8.decode(pro.v_codes) == 0)
    total = max(int(nz.sum()), 1)
    return float(below.sum()) / total, float(flushed.sum()) / total


def accuracy(o: np.ndarray, ref: np.ndarray) -> dict:
    """CosSim, relative L1 and RMSE of o against ref (both fp64), the pages' accuracy measures."""
    o = o.astype(F64).ravel()
    ref = ref.astype(F64).ravel()
    finite = bool(np.all(np.isfinite(o)))
    if not finite:
        return {"cos": float("nan"), "rel_l1": float("inf"), "rmse": float("inf"), "finite": False}
    cos = float(o @ ref / np.sqrt((o @ o) * (ref @ ref)))
    return {"cos": cos, "rel_l1": float(np.abs(o - ref).sum() / np.abs(ref).sum()),
            "rmse": float(np.sqrt(np.mean((o - ref) ** 2))), "finite": True}


def run(q, k, v, pairs, causal: bool = False, qk_bits: int = 8) -> list[dict]:
    """One row per (P_r, V_r, accumulator): accuracy against exact attention and V underflow."""
    ref = sage.exact_attention(q, k, v, causal)
    B, H = q.shape[:2]
    rows = []
    for p_r, v_r, accum in pairs:
        geom = sage.Geometry(p_range=float(p_r), v_range=float(v_r))
        pro = sage.prologue(q, k, v, causal, qk_bits, geom)
        out = np.zeros(ref.shape)
        for b in range(B):
            for h in range(H):
                for qb in range(pro.nqb):
                    r0, r1 = qb * geom.bq, min(pro.N, (qb + 1) * geom.bq)
                    if accum == "fp16":
                        out[b, h, r0:r1] = attend_block_fp16acc(pro, b, h, qb)
                    else:
                        out[b, h, r0:r1] = sage.attend_block(pro, b, h, qb)
        below, flushed = v_underflow(pro)
        rows.append({"p_range": float(p_r), "v_range": float(v_r), "accum": accum,
                     "bound_holds": fp16_bound_holds(p_r, v_r), "v_below_range": below,
                     "v_flushed": flushed, **accuracy(out, ref)})
    return rows


STUDY_PAIRS = [(448.0, 448.0, "fp32"), (448.0, 448.0, "fp16"), (224.0, 4.5, "fp16"),
               (112.0, 9.0, "fp16"), (448.0, 2.25, "fp16")]


def study_inputs(kind: str, seed: int = 0):
    """Synthetic inputs for the study: B1 H2 N1024 d64.  'plain': N(0,1) Q/K/V with a K channel
    bias; 'v_wide': as plain, but each V channel also holds a few entries 64x larger, which
    widens its dynamic range the way the skeptic's test targets."""
    from workloads import custom, make_inputs
    w = custom(1, 2, 2, 1024, 64, False, 8)
    q, k, v = make_inputs(w, seed=seed)
    if kind == "v_wide":
        rng = np.random.default_rng(seed + 100)
        v = v.astype(F64)
        idx = rng.integers(0, v.shape[2], size=(v.shape[0], v.shape[1], 4, v.shape[3]))
        for b in range(v.shape[0]):
            for h in range(v.shape[1]):
                for c in range(v.shape[3]):
                    v[b, h, idx[b, h, :, c], c] *= 64.0
        v = v.astype(np.float16)
    return q, k, v


if __name__ == "__main__":    # python -m oracle.range_study  (prints the table quoted in the docs)
    for kind in ("plain", "v_wide"):
        print(f"inputs: {kind} (B1 H2 N1024 d64, seed 0)")
        print("| P_r | V_r | accumulator | P_r*V_r <= 2047/2 | V below FP8 range | V flushed | CosSim | rel. L1 | RMSE |")
        print("|---|---|---|---|---|---|---|---|---|")
        for r in run(*study_inputs(kind), STUDY_PAIRS):
            print(f"| {r['p_range']:g} | {r['v_range']:g} | {r['accum']} | {r['bound_holds']} | "
                  f"{100 * r['v_below_range']:.3f} % | {100 * r['v_flushed']:.3f} % | {r['cos']:.6f} | "
                  f"{r['rel_l1']:.5f} | {r['rmse']:.3g} |")
        print()
