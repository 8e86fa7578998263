"""Pins for the oracle's variable-length batches (sage.sage_attention_varlen), CPU only.

A varlen batch packs sequences back to back; each is attended, smoothed and quantized on its
own.  Pinned against: textbook softmax attention over all packed tokens with a block-diagonal
(and, when causal, per-sequence lower-triangular) mask, written out here; invariance under a
constant shift of one sequence's keys, which holds bit for bit only if every sequence has its
own K mean and K groups; and the fixed-length path where the two must coincide.
"""
import math

import numpy as np
import pytest

from oracle import sage

LENS = [1, 127, 128, 129, 300]


def _packed(lens, H, Hkv, d, seed, step=None, lim=None):
    rng = np.random.default_rng(seed)
    T = sum(lens)
    def draw(h):
        x = rng.standard_normal((T, h, d))
        if step is not None:
            x = np.round(np.clip(x, -lim / 1.01, lim / 1.01) / step) * step
        return x.astype(np.float16)
    q, k, v = draw(H), draw(Hkv), draw(Hkv)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(int)
    return q, k, v, cu


def _masked_exact(q, k, v, cu, causal):
    """softmax over all T packed keys with the keys of other sequences (and, when causal, later
    keys of the same sequence) masked out; fp64."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    T, H, d = q.shape
    G = H // k.shape[1]
    seg = np.repeat(np.arange(len(cu) - 1), np.diff(cu))
    pos = np.arange(T) - cu[seg]
    allowed = seg[:, None] == seg[None, :]
    if causal:
        allowed &= pos[None, :] <= pos[:, None]
    out = np.zeros((T, H, d))
    for h in range(H):
        s = q[:, h] @ k[:, h // G].T / math.sqrt(d)
        s = np.where(allowed, s, -np.inf)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h] = e / e.sum(axis=1, keepdims=True) @ v[:, h // G]
    return out


@pytest.mark.parametrize("causal", [False, True])
def test_unquantized_varlen_is_block_diagonal_attention(causal):
    q, k, v, cu = _packed(LENS, 4, 2, 32, seed=20)
    o = sage.sage_attention_varlen(q, k, v, cu, causal, 8, quant_qk=False, quant_pv=False)
    e = _masked_exact(q, k, v, cu, causal)
    assert np.abs(o - e).max() < 1e-5


def test_varlen_single_sequence_equals_fixed_length():
    q, k, v, cu = _packed([300], 2, 1, 64, seed=21)
    o = sage.sage_attention_varlen(q, k, v, cu, True, 8)
    f = sage.sage_attention(*(np.ascontiguousarray(x.transpose(1, 0, 2))[None] for x in (q, k, v)), True, 8)
    assert np.array_equal(o, f[0].transpose(1, 0, 2))


def test_varlen_equal_lengths_equal_batch():
    lens = [256, 256, 256]
    q, k, v, cu = _packed(lens, 2, 2, 64, seed=22)
    o = sage.sage_attention_varlen(q, k, v, cu, False, 4)
    bq, bk, bv = (np.ascontiguousarray(x.reshape(3, 256, x.shape[1], 64).transpose(0, 2, 1, 3)) for x in (q, k, v))
    f = sage.sage_attention(bq, bk, bv, False, 4)
    assert np.array_equal(o, f.transpose(0, 2, 1, 3).reshape(o.shape))


@pytest.mark.parametrize("bits", [8, 4])
def test_shifting_one_sequences_keys_changes_nothing(bits):
    """Sequences of 128 and 256 keys on a 2^-6 grid: the per-sequence K mean absorbs an exact
    constant shift of sequence 0's keys, so every output is bit-identical.  A batch-wide mean
    (or K groups spanning sequences) would move sequence 1's smoothed keys and codes."""
    lens = [128, 256]
    q, k, v, cu = _packed(lens, 2, 2, 64, seed=23, step=2.0 ** -6, lim=3.9)
    rng = np.random.default_rng(24)
    c = np.round(np.clip(rng.standard_normal((1, 2, 64)), -3.9, 3.9) / 2.0 ** -6) * 2.0 ** -6
    k2 = k.astype(np.float64)
    k2[:128] += c
    k2 = k2.astype(np.float16)
    assert np.array_equal(k2[:128].astype(np.float64), k[:128].astype(np.float64) + c)   # exact shift
    o1 = sage.sage_attention_varlen(q, k, v, cu, True, bits)
    o2 = sage.sage_attention_varlen(q, k2, v, cu, True, bits)
    assert np.array_equal(o1, o2)
    # the same shift seen through one 384-token sequence does change the result
    whole = [0, 384]
    assert not np.array_equal(sage.sage_attention_varlen(q, k, v, whole, True, bits),
                              sage.sage_attention_varlen(q, k2, v, whole, True, bits))
