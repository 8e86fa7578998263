"""GPU parity on seeded random problems, against the oracle, through the C ABI.

The same bars as test_gpu_parity.py (whose checks these tests call), on problems drawn from a
fixed seed: varlen batches (1-5 sequences of 1-699 tokens), bf16 inputs and the NHD layout, over
batch, GQA group size, ragged length, head dim, causal, INT8/INT4-range QK, FP8/fp16 P V and the
channel-bias strengths of the input recipe.  (Fixed-length fp16 problems drawn the same way are
test_gpu_parity.py's random cases.)

SAGE_RANDOM_SWEEP=<seed> adds a wider sweep drawn from that seed: 100 fixed-length problems with
every prologue tensor, output element and int32 score tile checked, 25 varlen, 25 bf16 and 15 NHD
problems (a few minutes).
"""
import os

import numpy as np
import pytest
import torch

import test_gpu_parity as P
from workloads import custom

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    import quantized_attention_smooth_amd as p
    return p


def _problem(rng):
    B, Hkv, G = int(rng.integers(1, 4)), int(rng.integers(1, 4)), int(rng.choice([1, 2, 3, 4]))
    if rng.random() < 0.7:
        N = int(rng.integers(1, 900))
    else:
        N = int(rng.choice([1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 257, 384, 512]))
    d, causal = int(rng.choice([64, 128])), bool(rng.integers(0, 2))
    bits, pv = int(rng.choice([4, 8])), int(rng.choice([8, 16]))
    kb, qb = float(rng.choice([0.0, 1.0, 4.0, 10.0])), float(rng.choice([0.0, 1.0, 3.0]))
    w = custom(B, Hkv * G, Hkv, N, d, causal, bits, k_bias_std=kb, q_bias_std=qb)
    name = f"B{B}-H{Hkv * G}-Hkv{Hkv}-N{N}-d{d}-{'c' if causal else 'f'}-int{bits}-pv{pv}-kb{kb:g}-qb{qb:g}"
    return name, w, pv


def _varlen(rng):
    lens = [int(rng.integers(1, 700)) for _ in range(int(rng.integers(1, 6)))]
    Hkv, G = int(rng.integers(1, 3)), int(rng.choice([1, 2, 4]))
    d, causal = int(rng.choice([64, 128])), bool(rng.integers(0, 2))
    bits, pv = int(rng.choice([4, 8])), int(rng.choice([8, 16]))
    name = f"varlen-{'-'.join(map(str, lens))}-H{Hkv * G}-Hkv{Hkv}-d{d}-{'c' if causal else 'f'}-int{bits}-pv{pv}"
    return name, lens, Hkv * G, Hkv, d, causal, bits, pv


def _draw(seed, nfull, nvar, nbf, nnhd):
    rng = np.random.default_rng(seed)
    full = [_problem(rng) + (int(rng.integers(0, 1 << 30)),) for _ in range(nfull)]
    var = [_varlen(rng) for _ in range(nvar)]
    bf = [_problem(rng) for _ in range(nbf)]
    nhd = [_problem(rng) for _ in range(nnhd)]
    return full, var, bf, nhd


_, VARLEN, BF16, NHD = _draw(31337, 0, 8, 8, 6)
_sweep = os.environ.get("SAGE_RANDOM_SWEEP")
if _sweep:
    S_FULL, S_VARLEN, S_BF16, S_NHD = _draw(int(_sweep), 100, 25, 25, 15)
    VARLEN, BF16, NHD = VARLEN + S_VARLEN, BF16 + S_BF16, NHD + S_NHD

    @pytest.mark.parametrize("name,w,pv,seed", S_FULL, ids=[c[0] for c in S_FULL])
    def test_sweep_full_parity(sa, name, w, pv, seed):
        P._say(f"[case {name}] seed {seed}")
        q, k, v = P.make_inputs(w, seed=seed)
        P._full_parity(sa, name, q, k, v, w.causal, w.qk_bits, pv)


@pytest.mark.parametrize("name,lens,H,Hkv,d,causal,bits,pv", VARLEN, ids=[c[0] for c in VARLEN])
def test_random_varlen_parity(sa, name, lens, H, Hkv, d, causal, bits, pv):
    P.test_varlen_parity(sa, name, lens, H, Hkv, d, causal, bits, pv)


@pytest.mark.parametrize("name,w,pv", BF16, ids=[c[0] for c in BF16])
def test_random_bf16_parity(sa, name, w, pv):
    P.test_bf16_parity(sa, "bf16-" + name, w, pv)


@pytest.mark.parametrize("name,w,pv", NHD, ids=[c[0] for c in NHD])
def test_random_nhd_matches_hnd(sa, name, w, pv):
    P._say(f"[case nhd-{name}]")
    P.test_nhd_layout_matches_hnd(sa, w, pv)
    torch.cuda.synchronize()
