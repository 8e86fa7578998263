"""C ABI checks that need no GPU: the library loads, exports every symbol the header
declares, reports its configuration, sizes workspaces, and rejects bad arguments before
making any HIP call (the host has no GPU, so only calls that fail validation are made)."""
import ctypes
import os
import re

import pytest

from oracle import sage as oracle_sage

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sage_attn.h")


def _build_module():
    """quantized_attention_smooth_amd/build.py, loaded by path so that building never needs the
    package (whose import loads the library) to import first."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_sage_build", os.path.join(ROOT, "quantized_attention_smooth_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def pkg():
    b = _build_module()
    if not os.path.exists(b.LIB):
        b.build()
    import quantized_attention_smooth_amd as p
    return p


def _declared():
    text = open(HEADER).read()
    return set(re.findall(r"^(?:int|const char\*)\s+(sage_\w+)\s*\(", text, flags=re.M))


def test_exports_every_declared_symbol(pkg):
    declared = _declared()
    assert declared == set(pkg.EXPORTS)
    lib = ctypes.CDLL(pkg.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_config_matches_oracle_geometry(pkg):
    cfg = pkg.get_config()
    g = oracle_sage.DEFAULT
    assert cfg["version"] == 1 and cfg["fp8_format"] == 1
    for f in ("bq", "bk", "q_slice", "q_period", "q_run", "k_slice", "k_period", "k_run"):
        assert cfg[f] == getattr(g, f), f
    assert cfg["p_range"] == g.p_range and cfg["v_range"] == g.v_range


def test_workspace_bytes(pkg):
    n1 = pkg.workspace_bytes(1, 2, 2, 256, 64, False, 8)
    assert n1 > 0 and n1 % 256 == 0
    # fp16 V (pv_bits = 16) takes one more byte per V element than its FP8 codes
    assert pkg.workspace_bytes(1, 2, 2, 256, 64, False, 8, 16) >= n1 + 2 * 256 * 64
    # codes (K, V, Q) + Delta_S dominate: 3 * 256*64*2 + 2*2*256*4 bytes at least
    assert n1 >= 3 * 256 * 64 * 2 + 2 * 2 * 256 * 4
    assert pkg.workspace_bytes(1, 2, 2, 257, 64, False, 8) > n1           # one more 128-row block
    # every launch is a 1-D grid: batch x heads beyond 65535 is a valid problem
    assert pkg.workspace_bytes(1100, 64, 8, 3, 64, True, 8) > 0
    # causal stores only the Delta_S triangle: about half of the non-causal 9.7 GB
    causal, full = pkg.workspace_bytes(1, 32, 8, 98304, 128, True, 8), pkg.workspace_bytes(1, 32, 8, 98304, 128, False, 8)
    assert 4.5 * 2 ** 30 < causal < 6 * 2 ** 30 < 9 * 2 ** 30 < full


@pytest.mark.parametrize("args,status", [
    ((0, 2, 2, 256, 64, 0, 8, 8), -1),    # B < 1
    ((1, 3, 2, 256, 64, 0, 8, 8), -1),    # H % Hkv
    ((1, 2, 2, 0, 64, 0, 8, 8), -1),      # N < 1
    ((1, 2, 2, 256, 64, 2, 8, 8), -1),    # causal not 0/1
    ((1, 2, 2, 256, 96, 0, 8, 8), -2),    # d
    ((1, 2, 2, 256, 64, 0, 6, 8), -2),    # qk_bits
    ((1, 2, 2, 256, 64, 0, 8, 4), -2),    # pv_bits
    ((1, 2, 2, 256, 64, 0, 8, 32), -2),   # pv_bits
    ((1, 2, 2, (1 << 23) + 1, 64, 0, 8, 8), -2),   # N beyond the exact-sum bound
    ((1, 32768, 32768, 1 << 23, 64, 0, 8, 8), -1),  # statistics + Q launch beyond 2^31 - 1 workgroups
])
def test_validation_errors(pkg, args, status):
    lib = pkg._lib
    n = ctypes.c_size_t(0)
    assert lib.sage_attn_workspace_bytes(*args, ctypes.byref(n)) == status
    fake = ctypes.c_void_p(0x1000)          # never dereferenced: validation fails first
    assert lib.sage_attn_fwd(fake, fake, fake, fake, *args, ctypes.c_void_p(0x10000), 1 << 40, None) == status


def test_null_and_workspace_errors(pkg):
    lib = pkg._lib
    fake = ctypes.c_void_p(0x1000)
    dims = (1, 2, 2, 256, 64, 0, 8, 8)
    need = pkg.workspace_bytes(*dims)
    ws = ctypes.c_void_p(0x100000)
    assert lib.sage_attn_fwd(None, fake, fake, fake, *dims, ws, need, None) == -1
    assert lib.sage_attn_fwd(fake, fake, fake, None, *dims, ws, need, None) == -1
    assert lib.sage_attn_fwd(fake, fake, fake, fake, *dims, None, need, None) == -3
    assert lib.sage_attn_fwd(fake, fake, fake, fake, *dims, ws, need - 1, None) == -3
    assert lib.sage_attn_fwd(fake, fake, fake, fake, *dims, ctypes.c_void_p(0x100010), need, None) == -3
    assert lib.sage_qk_tile_debug(fake, fake, fake, *dims, ws, need, None, 0, 0, 2, 0, fake) == -1   # qb
    assert lib.sage_qk_tile_debug(fake, fake, fake, *dims, ws, need, None, 1, 0, 0, 0, fake) == -1   # b
    assert lib.sage_qk_tile_debug(fake, fake, fake, *dims, ws, need, None, 0, 0, 0, 0, None) == -1
    assert lib.sage_quant_debug(fake, None, fake, *dims, ws, need, None, *([None] * 9)) == -1
    # no V codes or scales exist when V stays fp16
    dims16 = dims[:-1] + (16,)
    need16 = pkg.workspace_bytes(*dims16)
    for i in (3, 4):
        outs = [None] * 9
        outs[i] = fake
        assert lib.sage_quant_debug(fake, fake, fake, *dims16, ws, need16, None, *outs) == -1
    assert lib.sage_get_config(None) == -1


def test_status_strings(pkg):
    lib = pkg._lib
    for s in (0, -1, -2, -3, -4, 7):
        assert len(lib.sage_status_string(s)) > 0
    assert lib.sage_last_error() == b""


def test_python_wrapper_rejects_unsupported(pkg):
    import torch
    q = torch.zeros(1, 2, 16, 64, dtype=torch.float16)
    with pytest.raises(NotImplementedError):
        pkg.sageattn(q, q, q, attn_mask=torch.zeros(16, 16))
    with pytest.raises(ValueError):
        pkg.sageattn(q, q, q)                     # CPU tensors
    with pytest.raises(ValueError):
        pkg.sageattn(q.float(), q, q)


def test_module_front_end_modes_and_checks(pkg):
    """SageAttention maps the quant_mode names onto (qk_bits, pv_bits) and checks its arguments
    (host side only: nothing here touches a GPU)."""
    import torch
    assert pkg.QUANT_MODES == {"qk_int8_pv_fp8": (8, 8), "qk_int8_pv_fp16": (8, 16),
                               "qk_int4_pv_fp8": (4, 8), "qk_int4_pv_fp16": (4, 16)}
    a = pkg.SageAttention(head_dim=128, is_causal=True, quant_mode="qk_int8_pv_fp16")
    assert (a.qk_bits, a.pv_bits, a.is_causal) == (8, 16, True)
    for bad in (dict(head_dim=96), dict(head_dim=64, quant_mode="qk_fp8_pv_fp8"),
                dict(head_dim=64, tensor_layout="BSHD")):
        with pytest.raises(ValueError):
            pkg.SageAttention(**bad)
    q = torch.zeros(1, 2, 16, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        a(q, q, q)                                # head_dim mismatch
    with pytest.raises(ValueError):
        pkg.SageAttention(head_dim=64)(q, q, q)   # CPU tensors


def test_problem_descriptor_validation(pkg):
    lib = pkg._lib
    n = ctypes.c_size_t(0)
    ok = pkg.Problem(2, 4, 2, 300, 64, True, 8, 8, "NHD")
    assert lib.sage_attn_workspace_bytes_ex(ok.ref, ctypes.byref(n)) == 0
    assert n.value == pkg.workspace_bytes(2, 4, 2, 300, 64, True, 8)     # layout does not change the workspace
    bad = pkg.Problem(2, 4, 2, 300, 64, True, 8, 8, "NHD")
    bad.c.layout = 2
    assert lib.sage_attn_workspace_bytes_ex(bad.ref, ctypes.byref(n)) == -1
    bad.c.layout, bad.c.dtype = 0, 7
    assert lib.sage_attn_workspace_bytes_ex(bad.ref, ctypes.byref(n)) == -1
    assert lib.sage_attn_workspace_bytes_ex(None, ctypes.byref(n)) == -1
    for cu, status in (([0, 5, 9], 0), ([1, 5, 9], -1), ([0, 5, 5], -1), ([0, 5, 3], -1),
                       ([0, 1, (1 << 23) + 2], -2)):
        p = pkg.Problem(2, 4, 2, 0, 64, True, 8, 8, "HND", cu_seqlens=cu)
        assert lib.sage_attn_workspace_bytes_ex(p.ref, ctypes.byref(n)) == status, cu
    fake = ctypes.c_void_p(0x1000)
    p = pkg.Problem(2, 4, 2, 0, 64, True, 8, 8, "HND", cu_seqlens=[0, 5, 9])
    assert lib.sage_attn_fwd_ex(p.ref, fake, fake, None, fake, ctypes.c_void_p(0x100000), 1 << 30, None) == -1
    assert lib.sage_attn_fwd_ex(p.ref, fake, fake, fake, fake, None, 1 << 30, None) == -3


def test_varlen_workspace_is_per_sequence(pkg):
    """A varlen batch needs the fixed-length sections of each sequence plus its table: one
    sequence of n tokens takes at least the workspace of the fixed-length problem of length n."""
    n = ctypes.c_size_t(0)
    p = pkg.Problem(1, 4, 2, 0, 128, True, 8, 8, "HND", cu_seqlens=[0, 1000])
    assert pkg._lib.sage_attn_workspace_bytes_ex(p.ref, ctypes.byref(n)) == 0
    assert n.value >= pkg.workspace_bytes(1, 4, 2, 1000, 128, True, 8)
    p2 = pkg.Problem(2, 4, 2, 0, 128, True, 8, 8, "HND", cu_seqlens=[0, 1000, 1100])
    m = ctypes.c_size_t(0)
    assert pkg._lib.sage_attn_workspace_bytes_ex(p2.ref, ctypes.byref(m)) == 0
    assert m.value > n.value


def test_bf16_workspace_holds_the_limb_sums(pkg):
    """bf16 inputs keep each exact K column sum in 12 int64 limbs instead of one."""
    import torch
    n16, nbf = ctypes.c_size_t(0), ctypes.c_size_t(0)
    p16 = pkg.Problem(1, 2, 2, 256, 64, False, 8, 8, "HND", dtype=torch.float16)
    pbf = pkg.Problem(1, 2, 2, 256, 64, False, 8, 8, "HND", dtype=torch.bfloat16)
    assert pkg._lib.sage_attn_workspace_bytes_ex(p16.ref, ctypes.byref(n16)) == 0
    assert pkg._lib.sage_attn_workspace_bytes_ex(pbf.ref, ctypes.byref(nbf)) == 0
    assert nbf.value - n16.value >= 11 * 8 * 2 * 64


def _hip_device_count() -> int:
    """GPUs the HIP runtime sees (0 when none, or when the runtime cannot be loaded)."""
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return 0
    n = ctypes.c_int(0)
    return n.value if hip.hipGetDeviceCount(ctypes.byref(n)) == 0 else 0


def test_valid_call_without_a_device_reports_hip_error(pkg):
    """A call that passes validation reaches its first launch; with no GPU that launch fails and
    the library returns SAGE_ERR_HIP with the runtime's message for this very launch.  Runs only
    on a host without a GPU: the pointers are fake and must never reach a kernel."""
    if _hip_device_count() > 0:
        pytest.skip("a GPU is present: this check needs a host without one")
    lib = pkg._lib
    fake, ws = ctypes.c_void_p(0x10000000), ctypes.c_void_p(0x20000000)
    dims = (1, 2, 2, 256, 64, 0, 8, 8)
    assert lib.sage_attn_fwd(fake, fake, fake, fake, *dims, ws, pkg.workspace_bytes(*dims), None) == -4
    msg = lib.sage_last_error().decode()
    assert msg.startswith("prologue launch:") and len(msg) > len("prologue launch: ")
    p = pkg.Problem(2, 4, 2, 0, 64, True, 8, 8, "HND", cu_seqlens=[0, 5, 9])
    n = ctypes.c_size_t(0)
    assert lib.sage_attn_workspace_bytes_ex(p.ref, ctypes.byref(n)) == 0
    assert lib.sage_attn_fwd_ex(p.ref, fake, fake, fake, fake, ws, n.value, None) == -4
    assert lib.sage_last_error().decode().startswith("sequence table launch:")
    assert lib.sage_attn_attend(fake, *dims, ws, pkg.workspace_bytes(*dims), None) == -4
    assert lib.sage_last_error().decode().startswith("attention launch:")


def test_host_code_under_address_and_undefined_behavior_sanitizers(tmp_path):
    """The library's host code (csrc/api.hip: validation, workspace carve-up, varlen table) built
    with AddressSanitizer and UndefinedBehaviorSanitizer on the host side (the device side of
    that file is only the allocation-free entry point's array) and driven by
    tests/abi_host_check.cpp with stand-in launchers that fill every workspace section and the
    output in host memory (sections tagged, so overlaps show too)."""
    import shutil
    import subprocess
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
    if not hipcc:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "abi_host_check")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    cmd = [hipcc, "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", *san,
           os.path.join(ROOT, "quantized_attention_smooth_amd", "csrc", "api.hip"),
           os.path.join(ROOT, "tests", "abi_host_check.cpp"), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert b.returncode == 0, b.stdout + b.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


def test_noalloc_entry_point_checks(pkg):
    """The allocation-free entry point: fixed-length problems only, and problems whose workspace
    exceeds its 128 MiB array are refused with SAGE_ERR_WORKSPACE before any HIP call."""
    lib = pkg._lib
    fake = ctypes.c_void_p(0x10000000)
    big = pkg.Problem(1, 32, 8, 98304, 128, True, 8, 8, "HND")            # about 5.5 GB of workspace
    assert lib.sage_attn_fwd_noalloc(big.ref, fake, fake, fake, fake, None) == -3
    msg = lib.sage_last_error().decode()
    assert "134217728" in msg and "allocation-free" in msg
    var = pkg.Problem(2, 4, 2, 0, 64, True, 8, 8, "HND", cu_seqlens=[0, 5, 9])
    assert lib.sage_attn_fwd_noalloc(var.ref, fake, fake, fake, fake, None) == -1
    ok = pkg.Problem(1, 2, 2, 256, 64, False, 8, 8, "HND")
    assert lib.sage_attn_fwd_noalloc(ok.ref, None, fake, fake, fake, None) == -1
    assert lib.sage_attn_fwd_noalloc(None, fake, fake, fake, fake, None) == -1
    bad = pkg.Problem(1, 2, 2, 256, 96, False, 8, 8, "HND")
    assert lib.sage_attn_fwd_noalloc(bad.ref, fake, fake, fake, fake, None) == -2
    # the benchmark's shape fits
    n = ctypes.c_size_t(0)
    bench = pkg.Problem(1, 16, 16, 8192, 128, False, 8, 8, "HND")
    assert lib.sage_attn_workspace_bytes_ex(bench.ref, ctypes.byref(n)) == 0 and n.value <= 128 << 20
    if _hip_device_count() == 0:            # no GPU: a valid call fails at the device lookup
        assert lib.sage_attn_fwd_noalloc(ok.ref, fake, fake, fake, fake, None) == -4
        assert len(lib.sage_last_error()) > 0


def test_package_fails_loudly_without_its_library(tmp_path):
    """A copy of the package without libsage_mi355x.so must refuse to import (ImportError naming
    the missing library): there is no CPU or PyTorch fallback for the attention path."""
    import shutil
    import subprocess
    import sys
    dst = tmp_path / "quantized_attention_smooth_amd"
    dst.mkdir()
    for f in ("__init__.py", "build.py", "counters.py"):
        shutil.copy(os.path.join(ROOT, "quantized_attention_smooth_amd", f), dst / f)
    code = ("import sys; sys.path.insert(0, sys.argv[1])\n"
            "try:\n"
            "    import quantized_attention_smooth_amd\n"
            "except ImportError as e:\n"
            "    print('ImportError:', e); sys.exit(3)\n"
            "sys.exit(0)\n")
    r = subprocess.run([sys.executable, "-c", code, str(tmp_path)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 3, r.stdout + r.stderr
    assert "libsage_mi355x.so" in r.stdout and "not built" in r.stdout
