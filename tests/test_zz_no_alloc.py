"""GPU check of the allocation-free entry point (sage_attn_fwd_noalloc) through the C ABI: its
output equals that of sage_attn_fwd_ex with a caller-allocated workspace, bit for bit (the same
kernels on the same inputs), for two calls in a row, the second on a smaller problem, so that
what the first call left in the shared device array cannot leak into the second."""
import ctypes
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import quantized_attention_smooth_amd as m
    return m


CASES = [  # (B, H, Hkv, N, d, causal, qk_bits, pv_bits, layout, dtype) -- second smaller than first
    (2, 8, 2, 1000, 128, True, 8, 8, "HND", torch.float16),
    (1, 2, 1, 300, 64, False, 4, 16, "NHD", torch.bfloat16),
]


def test_noalloc_matches_workspace_entry_point(sa):
    lib = sa._lib
    dev = torch.device("cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    gen = torch.Generator().manual_seed(5)
    for (B, H, Hkv, N, d, causal, qk, pv, layout, dt) in CASES:
        _say(f"[noalloc] B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal} qk{qk} pv{pv} {layout} {dt}")
        qs = (B, H, N, d) if layout == "HND" else (B, N, H, d)
        ks = (B, Hkv, N, d) if layout == "HND" else (B, N, Hkv, d)
        q = torch.randn(qs, generator=gen).to(dt).to(dev)
        k = (torch.randn(ks, generator=gen) + 3.0).to(dt).to(dev)
        v = torch.randn(ks, generator=gen).to(dt).to(dev)
        pb = sa.Problem(B, H, Hkv, N, d, causal, qk, pv, layout, dtype=dt)
        o_ref = torch.empty_like(q)
        o_na = torch.full_like(q, float("nan"))
        ws = sa.alloc_workspace(sa.problem_ws_bytes(pb), dev)
        ptr = lambda t: ctypes.c_void_p(t.data_ptr())
        assert lib.sage_attn_fwd_ex(pb.ref, ptr(q), ptr(k), ptr(v), ptr(o_ref), ptr(ws), ws.numel(), stream) == 0
        assert lib.sage_attn_fwd_noalloc(pb.ref, ptr(q), ptr(k), ptr(v), ptr(o_na), stream) == 0, \
            lib.sage_last_error()
        torch.cuda.synchronize()
        a, b = o_ref.float().cpu().numpy(), o_na.float().cpu().numpy()
        assert np.isfinite(a).all()
        assert np.array_equal(a, b), float(np.abs(a - b).max())
