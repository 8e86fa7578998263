"""SageAttention2 quantized attention forward: plain, slow CPU oracle.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's CPU
baseline may import this module.  It shares no code with the GPU path and imports nothing
from it; the GPU path never calls it.

Pages cited (titles as they appear on the pages):
  [SA2]   "SageAttention2: Efficient Attention with Thorough Outlier Smoothing and Per-thread
          INT4 Quantization" (mlsanity.com paper page for arXiv 2411.10958), section
          "Abstract (arXiv)".
  [SA2c]  zhaifeiyue.github.io commentary on arXiv 2411.10958 (SageAttention2): the analysis
          paragraphs on the paper's Sec. 3.4 (FP22 accumulator, two-level accumulation), on
          per-thread quantization bound to the NVIDIA mma layout, and on smoothing.
  [SA2pp] pith.science verdict on arXiv 2505.21136 (SageAttention2++), JSON keys
          "key_machinery" (delta_P = max(P~)/P_r, per-channel delta_V = max|V|/V_r),
          "core_discovery" (P_r, V_r ranges) and "supporting_citations" (online softmax,
          FlashAttention tiling).

What is computed, per (batch b, query head h); kv(h) = h div (H / Hkv):

  O1  exact means.  Every fp16 value is an integer multiple of 2**-24, so x * 2**24 is an
      exact int64 and the column sums are exact and order-free.  mean = RN32(RN64(sum) /
      (n * 2**24)).  mu_K over all N keys; mu_Q over the valid rows of each Q block of bq rows.
  O2  smoothing [SA2 abstract: smooth Q; title: outlier smoothing; SA2c: smoothing of K]:
      gamma_K = RN32(K - mu_K), gamma_Q = RN32(Q - mu_Q[block]).
  O3  K groups and codes [SA2 abstract: thread-level granularity; SA2c: the grouping follows
      the matrix-instruction layout]: one scale per group; codes = clamp(rint(RN32(gamma *
      RN32(R / amax))), -R, R), delta = RN32(amax / R); R = 127 (8-bit) or 7 (4-bit range).
  O4  Q groups and codes: same rule with the Q grouping.
  O5  Delta_S[qb, j] = sum_c mu_Q[qb, c] * gamma_K[j, c]  (fp64): Q smoothing moves the
      mean of the block's queries out of the quantized product; this term adds it back.
  O6  S_int = codes_Q . codes_K^T, exact integer.
  O7  logits z = (S_int * delta_Q(i) * delta_K(j) + Delta_S[qb(i), j]) / sqrt(d); -inf above
      the diagonal when causal (top-left aligned).
  O8  V: per-channel amax over all N keys; delta_V = RN32(amax / V_r);
      V_q = E4M3sat(RN32(V * RN32(V_r / amax))) [SA2pp key_machinery].
  O9  online softmax over KV blocks of bk keys (FlashAttention tiling with the online
      normalizer [SA2pp supporting_citations]): m' = max(m, blockmax z) (reading: see
      block_top); alpha = e^(m - m');
      p = e^(z - m'); P~_q = E4M3sat(RN32(p * P_r)) with the static range delta_P = 1 / P_r,
      valid because p <= 1 everywhere (reading: [SA2pp key_machinery] describes a per-block
      scale max(P~) / P_r instead, which equals 1 / P_r only in the block holding the running
      maximum; p_quant_stats measures the difference); l = l * alpha + sum P~_q / P_r (the
      weights that multiply V; see attend_block); two-level accumulation [SA2 abstract; SA2c
      on Sec. 3.4]: local = sum_j P~_q * V_q over the block (exact), acc = acc * alpha + local.
  O10 O = acc * delta_V[c] / (P_r * l).

Readings where the pages are silent are listed with each function.

Parity unpinned: the default quantization-group geometry (Geometry's defaults: one scale per
query row, one per (KV block, lane half) of keys) beyond its special cases (per token, per
block), which are pinned against textbook quantization.  The pages fix only "thread-level
granularity" on NVIDIA's layout; which gfx950 lanes share a scale is a contract with the GPU
library (its configuration call exports the same numbers), not something a pin can derive.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import fp8

F32 = np.float32
F64 = np.float64


# --------------------------------------------------------------------------------------
# geometry
# --------------------------------------------------------------------------------------
@dataclass(frozen=True)
class Geometry:
    """Block sizes and quantization-group shapes.

    A quantization group of rows (queries or keys) is the set of rows that share
    (row div slice, (row mod period) div run); a group spans all d channels.
    The defaults are the ones of the gfx950 kernel (one scale per MFMA lane):
      * Q: per query row (slice 1) -- in S^T = K Q^T on the 32x32 integer MFMA every lane
        column is one query;
      * K: (KV block, (j mod 8) div 4) -- the 16 keys a lane accumulates per 32-key tile
        are j = 8a + 4*(lane div 32) + r, so each lane sees one half of the block's keys.
    """

    bq: int = 128            # Q block: Q-smoothing block and workgroup tile
    bk: int = 128            # KV block: online-softmax block and K quantization slice
    q_slice: int = 1
    q_period: int = 1
    q_run: int = 1
    k_slice: int = 128
    k_period: int = 8
    k_run: int = 4
    p_range: float = 448.0   # P_r
    v_range: float = 448.0   # V_r


DEFAULT = Geometry()


def qk_range(qk_bits: int) -> int:
    """R: 127 for INT8 codes, 7 for INT4-range codes carried in int8 lanes [SA2 abstract]."""
    if qk_bits == 8:
        return 127
    if qk_bits == 4:
        return 7
    raise ValueError("qk_bits must be 4 or 8")


def group_ids(n: int, slice_: int, period: int, run: int) -> np.ndarray:
    """Group id of rows 0..n-1: rows with equal (i div slice, (i mod period) div run)."""
    i = np.arange(n, dtype=np.int64)
    return (i // slice_) * period + (i % period) // run


# --------------------------------------------------------------------------------------
# O1 / O2: exact means and smoothing
# --------------------------------------------------------------------------------------
def fixed_point_colsum(x16: np.ndarray) -> np.ndarray:
    """Exact column sums of an fp16 [n, d] array, in units of 2**-24, as int64."""
    x16 = np.asarray(x16)
    assert x16.dtype == np.float16
    xi = (x16.astype(F64) * 2.0 ** 24).astype(np.int64)   # exact: |x * 2**24| < 2**40
    return xi.sum(axis=0, dtype=np.int64)


def is_bf16(x: np.ndarray) -> bool:
    """bf16 inputs are passed as float32 arrays whose values are all bf16 numbers (numpy has no
    bf16 type): the low 16 bits of every element are zero."""
    x = np.asarray(x)
    return x.dtype == F32 and not np.any(x.view(np.uint32) & 0xFFFF)


def exact_mean(x: np.ndarray) -> np.ndarray:
    """O1: RN32(RN64(RN64(exact column sum) / n)) of an fp16 or bf16 [n, d] array.

    Reading: the pages fix neither the order nor the precision of the mean; this rule makes
    the result independent of summation order, so a parallel reduction can match it bit
    for bit.  fp16: the exact sum is an int64 count of 2**-24 units.  bf16 spans 2**-133 ..
    2**128, beyond any int64 fixed point: math.fsum returns the correctly rounded fp64 value of
    the exact sum directly.
    """
    n = x.shape[0]
    if x.dtype == np.float16:
        s = fixed_point_colsum(x)
        return (s.astype(F64) / F64(n * 2.0 ** 24)).astype(F32)
    assert is_bf16(x), "inputs must be fp16 or bf16 values (float32 arrays)"
    s = np.array([math.fsum(x[:, c].astype(F64)) for c in range(x.shape[1])], F64)
    return (s / F64(n)).astype(F32)


def smooth(x16: np.ndarray, mu: np.ndarray) -> np.ndarray:
    """O2: gamma = RN32(fp32(x) - mu)."""
    return (x16.astype(F32) - np.asarray(mu, dtype=F32)).astype(F32)


# --------------------------------------------------------------------------------------
# O3 / O4: grouped symmetric quantization
# --------------------------------------------------------------------------------------
def quantize_groups(gamma: np.ndarray, gid: np.ndarray, R: int):
    """Symmetric per-group quantization of gamma [n, d] (fp32) to integer codes in [-R, R].

    Returns (codes int8 [n, d], delta_row fp32 [n], amax_row fp32 [n]) where delta_row[i]
    is the scale of row i's group.

    Readings (pages silent): delta = RN32(amax / R); codes use the fp32 reciprocal
    RN32(R / amax), then an fp32 product, then round-half-even, clamped to +-R.
    A group whose amax is 0 gets delta = 0 and all-zero codes.
    """
    gamma = np.asarray(gamma, dtype=F32)
    n = gamma.shape[0]
    uniq, inv_idx = np.unique(gid, return_inverse=True)
    row_amax = np.abs(gamma).max(axis=1) if gamma.shape[1] else np.zeros(n, F32)
    gmax = np.zeros(len(uniq), dtype=F32)
    np.maximum.at(gmax, inv_idx, row_amax.astype(F32))
    delta_g = (gmax / F32(R)).astype(F32)
    with np.errstate(divide="ignore"):
        inv_g = np.where(gmax > 0, F32(R) / np.where(gmax > 0, gmax, F32(1)), F32(0)).astype(F32)
    inv_row = inv_g[inv_idx]
    prod = (gamma * inv_row[:, None]).astype(F32)
    codes = np.clip(np.rint(prod), -R, R).astype(np.int8)
    return codes, delta_g[inv_idx].astype(F32), gmax[inv_idx].astype(F32)


# --------------------------------------------------------------------------------------
# O8: V per-channel FP8
# --------------------------------------------------------------------------------------
def quantize_v(v16: np.ndarray, v_range: float):
    """O8: per-channel FP8 E4M3 quantization of V [n, d] (fp16).

    Returns (codes uint8 [n, d], delta_v fp32 [d], amax fp32 [d]).
    """
    vf = v16.astype(F32)
    amax = np.abs(vf).max(axis=0) if vf.shape[0] else np.zeros(vf.shape[1], F32)
    delta = (amax / F32(v_range)).astype(F32)
    with np.errstate(divide="ignore"):
        inv = np.where(amax > 0, F32(v_range) / np.where(amax > 0, amax, F32(1)), F32(0)).astype(F32)
    prod = (vf * inv[None, :]).astype(F32)
    codes = fp8.encode_sat(prod)
    return codes, delta, amax.astype(F32)


# --------------------------------------------------------------------------------------
# prologue: everything that does not depend on the (query block, key block) pair
# --------------------------------------------------------------------------------------
@dataclass
class Prologue:
    B: int
    H: int
    Hkv: int
    N: int
    d: int
    causal: bool
    qk_bits: int
    geom: Geometry
    quant_qk: bool
    quant_pv: bool
    smooth_q: bool
    smooth_k: bool
    row_sum: str               # "weights" (default) or "unquantized": see attend_block
    max_ref: str               # "exact" (default) or "pow2": see block_top
    # per (b, kv head)
    mu_k: np.ndarray = field(repr=False)       # f32 [B, Hkv, d]
    gamma_k: np.ndarray = field(repr=False)    # f32 [B, Hkv, N, d]
    k_codes: np.ndarray = field(repr=False)    # i8  [B, Hkv, N, d]
    k_delta: np.ndarray = field(repr=False)    # f32 [B, Hkv, N]  (scale of each key's group)
    v_codes: np.ndarray = field(repr=False)    # u8  [B, Hkv, N, d]
    v_delta: np.ndarray = field(repr=False)    # f32 [B, Hkv, d]
    v_amax: np.ndarray = field(repr=False)     # f32 [B, Hkv, d]
    v16: np.ndarray = field(repr=False)        # original V (for the unquantized-PV mode)
    # per (b, q head)
    mu_q: np.ndarray = field(repr=False)       # f32 [B, H, nqb, d]
    gamma_q: np.ndarray = field(repr=False)    # f32 [B, H, N, d]
    q_codes: np.ndarray = field(repr=False)    # i8  [B, H, N, d]
    q_delta: np.ndarray = field(repr=False)    # f32 [B, H, N]

    @property
    def nqb(self) -> int:
        return -(-self.N // self.geom.bq)

    @property
    def nkb(self) -> int:
        return -(-self.N // self.geom.bk)

    def kv_head(self, h: int) -> int:
        return h // (self.H // self.Hkv)


def prologue(q, k, v, causal: bool = False, qk_bits: int = 8, geom: Geometry = DEFAULT, *,
             quant_qk: bool = True, quant_pv: bool = True, smooth_q: bool = True,
             smooth_k: bool = True, row_sum: str = "weights", max_ref: str = "exact") -> Prologue:
    """Steps O1-O4 and O8 on fp16 inputs q [B,H,N,d], k/v [B,Hkv,N,d] (numpy float16), or on
    bf16 inputs (float32 arrays of bf16 values, see is_bf16).

    The switches turn parts of the method off; they exist so that tests can reduce the
    oracle to textbook attention (all off) and check each part against it.  row_sum selects
    the reading of the softmax row sum (see attend_block); only tests comparing the two
    readings change it; max_ref likewise selects the running maximum's reading (see block_top).
    """
    if row_sum not in ("weights", "unquantized"):
        raise ValueError("row_sum must be 'weights' or 'unquantized'")
    if max_ref not in ("pow2", "exact"):
        raise ValueError("max_ref must be 'pow2' or 'exact'")
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    assert q.dtype == k.dtype == v.dtype
    assert q.dtype == np.float16 or (is_bf16(q) and is_bf16(k) and is_bf16(v)), "fp16 or bf16 inputs"
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, N, d) and v.shape == (B, Hkv, N, d) and H % Hkv == 0
    R = qk_range(qk_bits)
    g = geom
    nqb = -(-N // g.bq)

    mu_k = np.zeros((B, Hkv, d), F32)
    gamma_k = np.zeros((B, Hkv, N, d), F32)
    k_codes = np.zeros((B, Hkv, N, d), np.int8)
    k_delta = np.zeros((B, Hkv, N), F32)
    v_codes = np.zeros((B, Hkv, N, d), np.uint8)
    v_delta = np.zeros((B, Hkv, d), F32)
    v_amax = np.zeros((B, Hkv, d), F32)
    kgid = group_ids(N, g.k_slice, g.k_period, g.k_run)
    for b in range(B):
        for hk in range(Hkv):
            if smooth_k:
                mu_k[b, hk] = exact_mean(k[b, hk])
            gamma_k[b, hk] = smooth(k[b, hk], mu_k[b, hk])
            k_codes[b, hk], k_delta[b, hk], _ = quantize_groups(gamma_k[b, hk], kgid, R)
            v_codes[b, hk], v_delta[b, hk], v_amax[b, hk] = quantize_v(v[b, hk], g.v_range)

    mu_q = np.zeros((B, H, nqb, d), F32)
    gamma_q = np.zeros((B, H, N, d), F32)
    q_codes = np.zeros((B, H, N, d), np.int8)
    q_delta = np.zeros((B, H, N), F32)
    qgid = group_ids(N, g.q_slice, g.q_period, g.q_run)
    for b in range(B):
        for h in range(H):
            for qb in range(nqb):
                r0, r1 = qb * g.bq, min(N, (qb + 1) * g.bq)
                if smooth_q:
                    mu_q[b, h, qb] = exact_mean(q[b, h, r0:r1])
                gamma_q[b, h, r0:r1] = smooth(q[b, h, r0:r1], mu_q[b, h, qb])
            q_codes[b, h], q_delta[b, h], _ = quantize_groups(gamma_q[b, h], qgid, R)

    return Prologue(B, H, Hkv, N, d, bool(causal), qk_bits, g, quant_qk, quant_pv, smooth_q,
                    smooth_k, row_sum, max_ref, mu_k, gamma_k, k_codes, k_delta, v_codes, v_delta, v_amax, v,
                    mu_q, gamma_q, q_codes, q_delta)


# --------------------------------------------------------------------------------------
# O5 / O6 / O7
# --------------------------------------------------------------------------------------
def delta_s(pro: Prologue, b: int, h: int, qb: int) -> np.ndarray:
    """O5: Delta_S[qb, :] = mu_Q[qb] . gamma_K^T over all N keys, fp64 [N]."""
    hk = pro.kv_head(h)
    return pro.gamma_k[b, hk].astype(F64) @ pro.mu_q[b, h, qb].astype(F64)


def scores_int(pro: Prologue, b: int, h: int, rows: slice, keys: slice) -> np.ndarray:
    """O6: exact integer S_int[rows, keys] = codes_Q . codes_K^T (int64).

    The fp64 product is exact: every partial sum is an integer below 127*127*d < 2**53.
    """
    hk = pro.kv_head(h)
    qc = pro.q_codes[b, h, rows].astype(F64)
    kc = pro.k_codes[b, hk, keys].astype(F64)
    return (qc @ kc.T).astype(np.int64)


def logits(pro: Prologue, b: int, h: int, qb: int) -> np.ndarray:
    """O7: fp64 logits of the rows of Q block qb against all N keys (masked with -inf)."""
    g = pro.geom
    hk = pro.kv_head(h)
    r0, r1 = qb * g.bq, min(pro.N, (qb + 1) * g.bq)
    if pro.quant_qk:
        s = scores_int(pro, b, h, slice(r0, r1), slice(0, pro.N)).astype(F64)
        s = s * pro.q_delta[b, h, r0:r1].astype(F64)[:, None] * pro.k_delta[b, hk].astype(F64)[None, :]
    else:
        s = pro.gamma_q[b, h, r0:r1].astype(F64) @ pro.gamma_k[b, hk].astype(F64).T
    z = (s + delta_s(pro, b, h, qb)[None, :]) / math.sqrt(pro.d)
    if pro.causal:
        i = np.arange(r0, r1)[:, None]
        j = np.arange(pro.N)[None, :]
        z = np.where(j > i, -np.inf, z)
    return z


# --------------------------------------------------------------------------------------
# O9 / O10
# --------------------------------------------------------------------------------------
LOG2E = 1.4426950408889634
LN2 = 0.6931471805599453


def block_top(zb: np.ndarray, max_ref: str) -> np.ndarray:
    """O9: what a KV block contributes to the running maximum that the softmax subtracts: fp64
    [rows] from the block's logits zb [rows, keys] (natural units, -inf where masked).

    Reading (the pages name an online softmax with a running maximum [SA2pp supporting_citations]
    and a static P~ range that needs p <= 1, but not which maximum): "exact", the default, is the
    plain row maximum, so the largest weight of the block that sets it is p = 1 and its P~ is
    exactly P_r.  "pow2" rounds it up to ln2 * ceil(log2(e) * max z), so that e^(z - m) =
    2^(log2(e) z - k) with an integer k: the same unquantized softmax (any m at or above the row
    maximum gives it, with every p <= 1), but the quantized weights P~ = E4M3(p * P_r) of that
    block then scale by 2^(exact - pow2) in (1/2, 1] and its largest one is rounded too.  It is
    kept for the test that holds both against exact attention (a GPU form of it would need no
    per-element subtraction of the maximum).  The running maximum is the largest block top seen
    so far (a ceiling of a maximum is the maximum of the ceilings).
    """
    top = zb.max(axis=1)
    if max_ref == "exact":
        return top
    fin = np.isfinite(top)
    return np.where(fin, np.ceil(np.where(fin, top, 0.0) * LOG2E) * LN2, top)


def attend_block(pro: Prologue, b: int, h: int, qb: int, return_state: bool = False):
    """O9-O10 for the rows of Q block qb: output fp64 [rows, d].

    Reading (pages silent on the row sum): l accumulates the weights that multiply V -- the
    quantized P~_q / P_r in the FP8 mode, p itself when P V is not quantized -- so the output
    is a weighted mean whose weights sum to exactly 1.  The other plain reading, l summing the
    unquantized p as a FlashAttention-style normaliser, is kept as pro.row_sum ==
    "unquantized" so that tests can hold the two against exact attention.  Blocks are visited
    in ascending key order.
    """
    g = pro.geom
    hk = pro.kv_head(h)
    z = logits(pro, b, h, qb)
    rows = z.shape[0]
    d = pro.d
    if pro.quant_pv:
        vq = fp8.decode(pro.v_codes[b, hk])            # exact fp64 values of the codes
        p_r = F64(g.p_range)
        vscale = pro.v_delta[b, hk].astype(F64)
    else:
        vq = pro.v16[b, hk].astype(F64)
        p_r = F64(1.0)
        vscale = np.ones(d, F64)
    m = np.full(rows, -np.inf)
    l = np.zeros(rows)
    acc = np.zeros((rows, d))
    for kb in range(pro.nkb):
        c0, c1 = kb * g.bk, min(pro.N, (kb + 1) * g.bk)
        zb = z[:, c0:c1]
        m_new = np.maximum(m, block_top(zb, pro.max_ref))
        finite = np.isfinite(m_new)
        alpha = np.where(np.isfinite(m), np.exp(m - np.where(finite, m_new, 0.0)), 0.0)
        p = np.where(finite[:, None], np.exp(zb - np.where(finite, m_new, 0.0)[:, None]), 0.0)
        if pro.quant_pv:
            pt = fp8.round_sat((p * p_r).astype(F32))     # P~_q = E4M3sat(RN32(p * P_r))
        else:
            pt = p
        if pro.row_sum == "weights":
            l = l * alpha + pt.sum(axis=1) / p_r           # the weights that multiply V
        else:
            l = l * alpha + p.sum(axis=1)                  # the unquantized probabilities
        local = pt @ vq[c0:c1]                             # block-local accumulation
        acc = acc * alpha[:, None] + local                 # global accumulation
        m = m_new
    out = acc * vscale[None, :] / (p_r * l[:, None])
    if return_state:
        return out, m, l
    return out


def fp8_midpoint_slack(pro: Prologue, b: int, h: int, qb: int, rel: float = 2.0 ** -14,
                       int_rel: float | None = None) -> np.ndarray:
    """How far O of Q block qb may move when P~ decisions that sit on an E4M3 rounding midpoint go
    the other way: fp64 [rows, d].

    Reading: a P~ element whose p * P_r lies within `rel` (relative) of the midpoint between two
    E4M3 values has two correct codes -- a computation of the logits in fp32 (any faithful one,
    as on the GPU) may land on either side.  Both results are outputs of the method, so a parity
    check accepts either.  O = N / L with N = sum P~ V_q delta_V and L = sum P~ (in P~ units);
    codes moving by gaps g_j give O' - O = sum g_j (v_j - O) / (L + sum g_j), so
    |O' - O| <= sum g_j (|V_q[j] delta_V| + |O|) / (L - sum g_j); later rescalings scale the g_j
    of an earlier block by factors <= 1.  Zero where no decision is ambiguous (almost everywhere).

    With the power-of-two running maximum (block_top), the integer k = ceil(log2(e) max z) is a
    decision too: where a block's log2-unit maximum lies within `rel` of an integer that the
    running maximum would take, k may come out one higher or lower.  That scales every later p
    of the row by exactly 2 or 1/2, which E4M3 rounding commutes with except in its subnormal
    range; acc and l scale alike, so O moves only through entries with p * P_r < 2^-5, each by
    at most one subnormal step at the smaller scale (2^-8 in P~ units).  Those entries get that
    gap from the ambiguous block on.  int_rel (default: rel) is that decision's tolerance.
    """
    if int_rel is None:
        int_rel = rel
    g = pro.geom
    hk = pro.kv_head(h)
    z = logits(pro, b, h, qb)
    rows = z.shape[0]
    vals = np.unique(fp8.decode(np.arange(256, dtype=np.uint8)))
    vals = vals[np.isfinite(vals) & (vals >= 0)]
    mids = (vals[1:] + vals[:-1]) / 2.0
    gaps = vals[1:] - vals[:-1]
    vmag = np.abs(fp8.decode(pro.v_codes[b, hk])) * pro.v_delta[b, hk].astype(F64)[None, :]
    p_r = F64(g.p_range)
    m = np.full(rows, -np.inf)
    gv = np.zeros((rows, pro.d))                       # sum g_j |V_q[j] delta_V|
    gs = np.zeros(rows)                                # sum g_j
    shifted = np.zeros(rows, bool)                     # rows whose integer maximum was ambiguous
    for kb in range(pro.nkb):
        c0, c1 = kb * g.bk, min(pro.N, (kb + 1) * g.bk)
        zb = z[:, c0:c1]
        if pro.max_ref == "pow2":
            t = zb.max(axis=1) * LOG2E                 # block maximum in log2 units
            tf = np.isfinite(t)
            n = np.rint(np.where(tf, t, 0.0))
            k_run = np.where(np.isfinite(m), np.rint(np.where(np.isfinite(m), m, 0.0) * LOG2E), -np.inf)
            near = tf & (np.abs(t - n) <= int_rel * np.maximum(1.0, np.abs(t))) & (n >= k_run)
            shifted |= near
        m_new = np.maximum(m, block_top(zb, pro.max_ref))
        finite = np.isfinite(m_new)
        p = np.where(finite[:, None], np.exp(zb - np.where(finite, m_new, 0.0)[:, None]), 0.0)
        x = p * p_r
        i = np.clip(np.searchsorted(mids, x), 0, len(mids) - 1)
        gap = np.zeros(x.shape)
        for j in (i - 1, i):                            # the two closest midpoints
            jj = np.clip(j, 0, len(mids) - 1)
            hit = np.abs(x - mids[jj]) <= rel * np.maximum(x, mids[jj])
            gap = np.where(hit, np.maximum(gap, gaps[jj]), gap)
        sub = shifted[:, None] & (p > 0) & (x < 2.0 ** -5)
        gap = np.where(sub, np.maximum(gap, 2.0 ** -8), gap)
        gv += gap @ vmag[c0:c1]
        gs += gap.sum(axis=1)
        m = m_new
    out, _, l = attend_block(pro, b, h, qb, return_state=True)
    big_l = p_r * l                                    # L in P~ units
    denom = np.where(big_l - gs > 0, big_l - gs, np.inf)
    return (gv + gs[:, None] * np.abs(out)) / denom[:, None]


def p_quant_stats(pro: Prologue, b: int, h: int, qb: int) -> dict:
    """How the static range treats the probabilities of Q block qb (FP8 mode).

    Static range: P~ = E4M3sat(RN32(p * P_r)) with the fixed scale delta_P = 1 / P_r, because
    0 < p <= 1 everywhere (p = e^(z - m) with m the running maximum of block_top).  Only a block
    that holds its row's running maximum has max p = 1 (max p in (1/2, 1] when the maximum is
    rounded to a power of two); in later blocks max p is smaller, and an entry with
    p * P_r below half the smallest E4M3 subnormal (2^-10) is coded as zero.  The per-block
    form of the scale, delta_P = max(P~) / P_r, would code each block's entries relative to
    the block's own maximum instead; `zero_block_scale` counts the zeros that form would give
    on the same p (for comparison only: the method here uses the static range).

    Returns counts over the unmasked (row, key) entries: n, zero_static (p > 0 but P~ = 0),
    subnormal_static (0 < P~ < 2^-6, the E4M3 subnormal range), zero_block_scale, and the
    number of (row, block) pairs whose block maximum p is below 1 (rows_blocks_below_one) out
    of rows_blocks.
    """
    g = pro.geom
    z = logits(pro, b, h, qb)
    rows = z.shape[0]
    m = np.full(rows, -np.inf)
    out = dict(n=0, zero_static=0, subnormal_static=0, zero_block_scale=0, rows_blocks=0,
               rows_blocks_below_one=0)
    for kb in range(pro.nkb):
        c0, c1 = kb * g.bk, min(pro.N, (kb + 1) * g.bk)
        zb = z[:, c0:c1]
        m_new = np.maximum(m, block_top(zb, pro.max_ref))
        live = np.isfinite(zb)
        p = np.where(live, np.exp(zb - np.where(np.isfinite(m_new), m_new, 0.0)[:, None]), 0.0)
        pt = fp8.round_sat((p * g.p_range).astype(F32))
        bmax = p.max(axis=1)
        has = live.any(axis=1)
        scale = np.where(bmax > 0, g.p_range / np.where(bmax > 0, bmax, 1.0), 0.0)
        pt_blk = fp8.round_sat((p * scale[:, None]).astype(F32))
        out["n"] += int(live.sum())
        out["zero_static"] += int(np.count_nonzero(live & (p > 0) & (pt == 0)))
        out["subnormal_static"] += int(np.count_nonzero(live & (pt > 0) & (pt < 2.0 ** -6)))
        out["zero_block_scale"] += int(np.count_nonzero(live & (p > 0) & (pt_blk == 0)))
        out["rows_blocks"] += int(has.sum())
        out["rows_blocks_below_one"] += int(np.count_nonzero(has & (bmax < 1.0)))
        m = m_new
    return out


def p_flushed_mass(pro: Prologue, b: int, h: int, qb: int) -> np.ndarray:
    """Per row of Q block qb: the share of its exact softmax weight e^(z - max z) / sum that
    falls on entries the static range codes as zero (p * P_r at or below 2^-10, p taken against
    the running maximum of its block, as in the online softmax).  fp64 [rows]."""
    g = pro.geom
    z = logits(pro, b, h, qb)
    top = z.max(axis=1)
    w = np.exp(z - top[:, None])
    total = w.sum(axis=1)
    m = np.full(z.shape[0], -np.inf)
    flushed = np.zeros(z.shape[0])
    for kb in range(pro.nkb):
        c0, c1 = kb * g.bk, min(pro.N, (kb + 1) * g.bk)
        zb = z[:, c0:c1]
        m = np.maximum(m, block_top(zb, pro.max_ref))
        live = np.isfinite(zb)
        p = np.where(live, np.exp(zb - m[:, None]), 0.0)
        pt = fp8.round_sat((p * g.p_range).astype(F32))
        flushed += np.where(live & (p > 0) & (pt == 0), w[:, c0:c1], 0.0).sum(axis=1)
    return flushed / total


def sage_attention(q, k, v, causal: bool = False, qk_bits: int = 8, geom: Geometry = DEFAULT,
                   **switches) -> np.ndarray:
    """Whole forward pass: fp64 O [B, H, N, d] (the GPU rounds it to fp16)."""
    pro = prologue(q, k, v, causal, qk_bits, geom, **switches)
    out = np.zeros((pro.B, pro.H, pro.N, pro.d))
    for b in range(pro.B):
        for h in range(pro.H):
            for qb in range(pro.nqb):
                r0, r1 = qb * geom.bq, min(pro.N, (qb + 1) * geom.bq)
                out[b, h, r0:r1] = attend_block(pro, b, h, qb)
    return out


def sage_attention_varlen(q, k, v, cu_seqlens, causal: bool = False, qk_bits: int = 8,
                          geom: Geometry = DEFAULT, **switches) -> np.ndarray:
    """Variable-length batch (the blog page's precision-control tip on varlen inputs): q [T, H, d],
    k/v [T, Hkv, d] hold the sequences back to back, sequence s being rows cu[s] .. cu[s+1]-1.

    Reading (the page names the feature, not its arithmetic): each sequence is one batch entry
    of its own -- its keys alone are attended, smoothed (mu_K over its tokens, mu_Q per 128-row
    block from its first row) and grouped -- so the result is the fixed-length forward pass on
    each slice.  Returns fp64 [T, H, d].
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    cu = [int(x) for x in cu_seqlens]
    out = np.zeros(q.shape)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        qs, ks, vs = (np.ascontiguousarray(x[a:b].transpose(1, 0, 2))[None] for x in (q, k, v))
        out[a:b] = sage_attention(qs, ks, vs, causal, qk_bits, geom, **switches)[0].transpose(1, 0, 2)
    return out


# --------------------------------------------------------------------------------------
# accuracy reference
# --------------------------------------------------------------------------------------
def exact_attention(q, k, v, causal: bool = False) -> np.ndarray:
    """softmax(Q K^T / sqrt(d)) V in fp64 (two-pass softmax), GQA by h div (H / Hkv)."""
    q = np.asarray(q).astype(F64)
    k = np.asarray(k).astype(F64)
    v = np.asarray(v).astype(F64)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    out = np.zeros((B, H, N, d))
    for b in range(B):
        for h in range(H):
            hk = h // (H // Hkv)
            s = q[b, h] @ k[b, hk].T / math.sqrt(d)
            if causal:
                s = np.where(np.arange(N)[None, :] > np.arange(N)[:, None], -np.inf, s)
            s = s - s.max(axis=1, keepdims=True)
            e = np.exp(s)
            out[b, h] = (e / e.sum(axis=1, keepdims=True)) @ v[b, hk]
    return out


def exact_attention_rows(q, k, v, rows, causal: bool = False) -> np.ndarray:
    """softmax(Q K^T / sqrt(d)) V in fp64 for the query rows `rows` of one head: q [N, d], k/v
    [N, d]; query i sees keys j <= i when causal.  Returns [len(rows), d]."""
    rows = np.asarray(rows)
    q = np.asarray(q).astype(F64)[rows]
    k = np.asarray(k).astype(F64)
    v = np.asarray(v).astype(F64)
    s = q @ k.T / math.sqrt(q.shape[1])
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] > rows[:, None], -np.inf, s)
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return (e / e.sum(axis=1, keepdims=True)) @ v
