"""Seeded synthetic inputs for the quantized attention forward.

This module only draws random tensors: it holds none of the method's arithmetic, and both
the CPU oracle's tests and the GPU path's tests/benchmark take their inputs from here.

The shapes and value structure stand in for the workloads the pages describe (the real
models' activations are not available): LLM prefill with long causal context and outlier
channels in Q/K, video-DiT attention with a short text prefix and a long video sequence,
and a kernel sweep at N = 8K, d = 128.  Recipe (all configs):

  rng = numpy.random.default_rng(seed)        (PCG64)
  draw order: q, k, v base ~ N(0, 1) (float32, BHND); then row scaling (text prefix);
  then the per-(head, channel) K bias; then the per-(head, channel) Q bias; then the
  outlier (head, channel) mask; finally cast to fp16 with round-to-nearest-even.
  Biases have shape [1, heads, 1, d]: shared by batch and tokens.  V gets no bias.

Variable-length batches (make_varlen_inputs) pack sequences back to back, [T, heads, d]; the
same draw order applies, but every sequence gets its own K and Q biases (different prompts
have different channel offsets, which is what per-sequence smoothing has to absorb).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Hkv: int
    N: int
    d: int
    causal: bool
    qk_bits: int
    k_bias_std: float = 4.0
    q_bias_std: float = 0.0
    text_tokens: int = 0          # leading rows drawn with std text_std instead of 1
    text_std: float = 1.0
    outlier_frac: float = 0.0     # fraction of (head, channel) pairs of Q and K scaled
    outlier_scale: float = 1.0

    @property
    def ops(self) -> float:
        """Numerator of the effective-TOPS metric: 4*B*H*N^2*d, halved when causal."""
        o = 4.0 * self.B * self.H * self.N * self.N * self.d
        return o / 2 if self.causal else o


WORKLOADS = {
    # small parity case: non-causal MHA, K outlier channels, INT8 QK + FP8 PV
    "tiny": Workload("tiny", 1, 2, 2, 256, 64, False, 8),
    # kernel sweep point: N = 8K, d = 128, K and Q channel biases
    "bench": Workload("bench", 1, 16, 16, 8192, 128, False, 8, q_bias_std=1.0),
    # LLM prefill: causal, 1% of (head, channel) pairs of Q and K scaled x10, INT4-range QK
    "llm": Workload("llm", 1, 32, 32, 16384, 128, True, 4, q_bias_std=1.0,
                    outlier_frac=0.01, outlier_scale=10.0),
    # video DiT: 226 text tokens (std 2) then 17550 video tokens (std 1), d = 64
    "dit": Workload("dit", 2, 30, 30, 17776, 64, False, 8, text_tokens=226, text_std=2.0),
    # long-context causal GQA: 32 query heads over 8 kv heads, N = 96K
    "gqa": Workload("gqa", 1, 32, 8, 98304, 128, True, 8),
}


def to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returned as float32 holding
    bf16 values (numpy has no bf16 type; torch converts them to torch.bfloat16 exactly)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def custom(B, H, Hkv, N, d, causal=False, qk_bits=8, **kw) -> Workload:
    return Workload("custom", B, H, Hkv, N, d, causal, qk_bits, **kw)


def make_inputs(w: Workload | str, seed: int = 0, dtype: str = "fp16"):
    """q [B,H,N,d], k/v [B,Hkv,N,d] as numpy float16 (dtype "fp16"), or as float32 arrays of
    bf16 values (dtype "bf16", see to_bf16), drawn by the recipe above."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((w.B, w.H, w.N, w.d), dtype=np.float32)
    k = rng.standard_normal((w.B, w.Hkv, w.N, w.d), dtype=np.float32)
    v = rng.standard_normal((w.B, w.Hkv, w.N, w.d), dtype=np.float32)
    if w.text_tokens:
        t = min(w.text_tokens, w.N)
        for x in (q, k, v):
            x[:, :, :t, :] *= np.float32(w.text_std)
    if w.k_bias_std:
        k += (w.k_bias_std * rng.standard_normal((1, w.Hkv, 1, w.d))).astype(np.float32)
    if w.q_bias_std:
        q += (w.q_bias_std * rng.standard_normal((1, w.H, 1, w.d))).astype(np.float32)
    if w.outlier_frac:
        n_pairs = int(round(w.outlier_frac * w.H * w.d))
        pick = rng.choice(w.H * w.d, n_pairs, replace=False)
        for p in pick:
            h, c = divmod(int(p), w.d)
            q[:, h, :, c] *= np.float32(w.outlier_scale)
            k[:, h * w.Hkv // w.H, :, c] *= np.float32(w.outlier_scale)
    if dtype == "bf16":
        return to_bf16(q), to_bf16(k), to_bf16(v)
    return q.astype(np.float16), k.astype(np.float16), v.astype(np.float16)


@dataclass(frozen=True)
class VarlenWorkload:
    name: str
    lens: tuple
    H: int
    Hkv: int
    d: int
    causal: bool
    qk_bits: int
    k_bias_std: float = 4.0
    q_bias_std: float = 0.0

    @property
    def B(self) -> int:
        return len(self.lens)

    @property
    def T(self) -> int:
        return int(sum(self.lens))

    @property
    def N(self) -> int:
        return int(max(self.lens))

    @property
    def cu_seqlens(self) -> list:
        return [0] + [int(x) for x in np.cumsum(self.lens)]

    @property
    def ops(self) -> float:
        """Numerator of the effective-TOPS metric summed over sequences: 4*H*n^2*d each,
        halved when causal."""
        o = sum(4.0 * self.H * n * n * self.d for n in self.lens)
        return o / 2 if self.causal else o


def varlen_lengths(n_seq: int, lo: int, hi: int, seed: int) -> tuple:
    """n_seq lengths drawn log-uniformly from [lo, hi] (rounded to integers)."""
    rng = np.random.default_rng(seed)
    return tuple(int(round(x)) for x in np.exp(rng.uniform(np.log(lo), np.log(hi), n_seq)))


VARLEN_WORKLOADS = {
    # a prefill batch of 16 prompts of mixed length (256 .. 16K tokens, log-uniform), causal GQA
    "varlen": VarlenWorkload("varlen", varlen_lengths(16, 256, 16384, seed=7), 32, 8, 128, True, 8,
                             q_bias_std=1.0),
}


def make_varlen_inputs(w: VarlenWorkload, seed: int = 0):
    """q [T,H,d], k/v [T,Hkv,d] as numpy float16 (recipe above, biases per sequence)."""
    rng = np.random.default_rng(seed)
    T = w.T
    q = rng.standard_normal((T, w.H, w.d), dtype=np.float32)
    k = rng.standard_normal((T, w.Hkv, w.d), dtype=np.float32)
    v = rng.standard_normal((T, w.Hkv, w.d), dtype=np.float32)
    cu = w.cu_seqlens
    if w.k_bias_std:
        kb = (w.k_bias_std * rng.standard_normal((w.B, w.Hkv, w.d))).astype(np.float32)
        for s in range(w.B):
            k[cu[s]:cu[s + 1]] += kb[s]
    if w.q_bias_std:
        qb = (w.q_bias_std * rng.standard_normal((w.B, w.H, w.d))).astype(np.float32)
        for s in range(w.B):
            q[cu[s]:cu[s + 1]] += qb[s]
    return q.astype(np.float16), k.astype(np.float16), v.astype(np.float16)
