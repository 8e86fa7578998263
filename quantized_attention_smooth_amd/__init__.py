"""MI355X (gfx950) SageAttention2 quantized attention forward.

A thin Python binding over the C ABI in include/sage_attn.h (libsage_mi355x.so, built by
quantized_attention_smooth_amd/build.py).  Every step of the computation runs in the library's
HIP kernels; this module only checks arguments, allocates the output and the workspace with
torch, and passes raw device pointers and the current stream.  There is no fallback: if the
library is missing or fails to load, importing this package raises ImportError.

    from quantized_attention_smooth_amd import sageattn
    o = sageattn(q, k, v, is_causal=True, qk_bits=8, pv_bits=8)   # like F.scaled_dot_product_attention
    o = sageattn(q, k, v, tensor_layout="NHD")                     # q [B, N, H, d]
    o = sageattn_varlen(q, k, v, cu_seqlens, is_causal=True)       # packed q [T, H, d]
    attn = SageAttention(head_dim=128, is_causal=True, quant_mode="qk_int8_pv_fp16")
    o = attn(q, k, v)                                              # module-style, reuses its workspace
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["sageattn", "sageattn_varlen", "SageAttention", "QUANT_MODES", "fwd", "prologue", "attend", "workspace_bytes", "get_config",
           "quant_debug", "qk_tile_debug", "Problem", "LIB_PATH", "SageError", "mfma_rate_probe", "MFMA_PROBE_KINDS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsage_mi355x.so")

SAGE_OK = 0
SAGE_ERR_INVALID_ARG = -1
SAGE_ERR_UNSUPPORTED = -2
SAGE_ERR_WORKSPACE = -3
SAGE_ERR_HIP = -4

#: every symbol include/sage_attn.h declares
EXPORTS = ("sage_get_config", "sage_attn_workspace_bytes", "sage_attn_fwd", "sage_attn_prologue",
           "sage_attn_attend", "sage_quant_debug", "sage_qk_tile_debug", "sage_status_string",
           "sage_last_error", "sage_attn_workspace_bytes_ex", "sage_attn_fwd_ex", "sage_attn_prologue_ex",
           "sage_attn_attend_ex", "sage_quant_debug_ex", "sage_mfma_rate_probe",
           "sage_attn_fwd_noalloc")

LAYOUTS = {"HND": 0, "NHD": 1}
#: quant_mode names of the blog page's precision-control section (INT8 QK with FP8 or fp16 PV),
#: plus their INT4-range QK counterparts, as (qk_bits, pv_bits)
QUANT_MODES = {"qk_int8_pv_fp8": (8, 8), "qk_int8_pv_fp16": (8, 16),
               "qk_int4_pv_fp8": (4, 8), "qk_int4_pv_fp16": (4, 16)}
DTYPES = {torch.float16: 0, torch.bfloat16: 1}


class SageConfig(ctypes.Structure):
    _fields_ = [("version", ctypes.c_int), ("bq", ctypes.c_int), ("bk", ctypes.c_int),
                ("q_slice", ctypes.c_int), ("q_period", ctypes.c_int), ("q_run", ctypes.c_int),
                ("k_slice", ctypes.c_int), ("k_period", ctypes.c_int), ("k_run", ctypes.c_int),
                ("p_range", ctypes.c_float), ("v_range", ctypes.c_float), ("fp8_format", ctypes.c_int)]


class SageProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("Hkv", ctypes.c_int), ("N", ctypes.c_int),
                ("d", ctypes.c_int), ("causal", ctypes.c_int), ("qk_bits", ctypes.c_int), ("pv_bits", ctypes.c_int),
                ("layout", ctypes.c_int), ("dtype", ctypes.c_int), ("cu_seqlens", ctypes.POINTER(ctypes.c_int))]


class Problem:
    """sage_problem_t plus the host cu_seqlens array it points to (kept alive here)."""

    def __init__(self, B, H, Hkv, N, d, causal=False, qk_bits=8, pv_bits=8, layout="HND", dtype=torch.float16,
                 cu_seqlens=None):
        self._cu = None
        cu_ptr = None
        if cu_seqlens is not None:
            vals = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
            self._cu = (ctypes.c_int * len(vals))(*vals)
            cu_ptr = ctypes.cast(self._cu, ctypes.POINTER(ctypes.c_int))
            if len(vals) != B + 1:
                raise ValueError(f"cu_seqlens needs B + 1 = {B + 1} entries, got {len(vals)}")
        if layout not in LAYOUTS:
            raise ValueError(f"tensor_layout must be one of {sorted(LAYOUTS)}")
        if dtype not in DTYPES:
            raise ValueError("dtype must be torch.float16 or torch.bfloat16")
        self.c = SageProblem(B, H, Hkv, N, d, int(causal), qk_bits, pv_bits, LAYOUTS[layout], DTYPES[dtype], cu_ptr)

    @property
    def ref(self):
        return ctypes.byref(self.c)


class SageError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python quantized_attention_smooth_amd/build.py`")
    try:
        lib = ctypes.CDLL(LIB_PATH)
    except OSError as e:
        raise ImportError(f"cannot load {LIB_PATH}: {e}") from e
    P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.sage_get_config.argtypes = [ctypes.POINTER(SageConfig)]
    lib.sage_attn_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I, ctypes.POINTER(S)]
    lib.sage_attn_fwd.argtypes = [P, P, P, P, I, I, I, I, I, I, I, I, P, S, P]
    lib.sage_attn_prologue.argtypes = [P, P, P, I, I, I, I, I, I, I, I, P, S, P]
    lib.sage_attn_attend.argtypes = [P, I, I, I, I, I, I, I, I, P, S, P]
    lib.sage_quant_debug.argtypes = [P, P, P, I, I, I, I, I, I, I, I, P, S, P] + [P] * 9
    lib.sage_qk_tile_debug.argtypes = [P, P, P, I, I, I, I, I, I, I, I, P, S, P, I, I, I, I, P]
    PP = ctypes.POINTER(SageProblem)
    lib.sage_attn_workspace_bytes_ex.argtypes = [PP, ctypes.POINTER(S)]
    lib.sage_attn_fwd_ex.argtypes = [PP, P, P, P, P, P, S, P]
    lib.sage_attn_prologue_ex.argtypes = [PP, P, P, P, P, S, P]
    lib.sage_attn_attend_ex.argtypes = [PP, P, P, S, P]
    lib.sage_quant_debug_ex.argtypes = [PP, P, P, P, P, S, P] + [P] * 9
    lib.sage_mfma_rate_probe.argtypes = [I, I, P, S, ctypes.POINTER(ctypes.c_double), P]
    lib.sage_attn_fwd_noalloc.argtypes = [PP, P, P, P, P, P]
    lib.sage_status_string.argtypes = [I]
    lib.sage_status_string.restype = ctypes.c_char_p
    lib.sage_last_error.argtypes = []
    lib.sage_last_error.restype = ctypes.c_char_p
    for name in ("sage_get_config", "sage_attn_workspace_bytes", "sage_attn_fwd", "sage_attn_prologue",
                 "sage_attn_attend", "sage_quant_debug", "sage_qk_tile_debug", "sage_attn_workspace_bytes_ex",
                 "sage_attn_fwd_ex", "sage_attn_prologue_ex", "sage_attn_attend_ex", "sage_quant_debug_ex",
                 "sage_mfma_rate_probe", "sage_attn_fwd_noalloc"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


_lib = _load()


def _check(status: int) -> None:
    if status == SAGE_OK:
        return
    text = _lib.sage_status_string(status).decode()
    if status == SAGE_ERR_HIP:
        raise SageError(status, f"{text}: {_lib.sage_last_error().decode()}")
    if status == SAGE_ERR_UNSUPPORTED:
        raise NotImplementedError(text)
    raise ValueError(text)


def get_config() -> dict:
    cfg = SageConfig()
    _check(_lib.sage_get_config(ctypes.byref(cfg)))
    return {name: getattr(cfg, name) for name, _ in SageConfig._fields_}


def workspace_bytes(B: int, H: int, Hkv: int, N: int, d: int, causal: bool, qk_bits: int,
                    pv_bits: int = 8) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.sage_attn_workspace_bytes(B, H, Hkv, N, d, int(causal), qk_bits, pv_bits, ctypes.byref(n)))
    return n.value


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _on(device):
    """Make the tensors' GPU current for a library call: its kernels launch on torch's current
    stream of that GPU, and torch's default stream is the null stream, which HIP resolves
    against the current device."""
    return torch.cuda.device(device)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _shapes(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, heads, N, d]")
    if q.dtype != torch.float16 or k.dtype != torch.float16 or v.dtype != torch.float16:
        raise ValueError("q, k, v must be float16")
    if not (q.is_cuda and k.is_cuda and v.is_cuda) or not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same GPU")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous (layout [B, heads, N, d])")
    B, H, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    return B, H, k.shape[1], N, d


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    """A uint8 device tensor whose data pointer is 256-byte aligned."""
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + nbytes]


def fwd(q, k, v, o, workspace, is_causal: bool = False, qk_bits: int = 8, pv_bits: int = 8) -> None:
    """sage_attn_fwd on caller-provided tensors (o and workspace are written)."""
    B, H, Hkv, N, d = _shapes(q, k, v)
    if o.shape != q.shape or o.dtype != torch.float16 or not o.is_contiguous() or o.device != q.device:
        raise ValueError("o must be a contiguous float16 tensor shaped like q on q's device")
    with _on(q.device):
        _check(_lib.sage_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, Hkv, N, d, int(is_causal), qk_bits,
                                  pv_bits, _ptr(workspace), workspace.numel(), _stream(q.device)))


def prologue(q, k, v, workspace, is_causal: bool = False, qk_bits: int = 8, pv_bits: int = 8) -> None:
    """sage_attn_prologue: fill `workspace` with the quantized/smoothed operands."""
    B, H, Hkv, N, d = _shapes(q, k, v)
    with _on(q.device):
        _check(_lib.sage_attn_prologue(_ptr(q), _ptr(k), _ptr(v), B, H, Hkv, N, d, int(is_causal), qk_bits,
                                       pv_bits, _ptr(workspace), workspace.numel(), _stream(q.device)))


def attend(o, workspace, shape, Hkv: int, is_causal: bool = False, qk_bits: int = 8, pv_bits: int = 8) -> None:
    """sage_attn_attend: the fused attention kernel on a workspace filled by prologue().

    shape = (B, H, N, d) of q/o."""
    B, H, N, d = shape
    if tuple(o.shape) != (B, H, N, d) or o.dtype != torch.float16 or not o.is_contiguous() or not o.is_cuda:
        raise ValueError("o must be a contiguous float16 CUDA tensor of shape (B, H, N, d)")
    with _on(o.device):
        _check(_lib.sage_attn_attend(_ptr(o), B, H, Hkv, N, d, int(is_causal), qk_bits, pv_bits, _ptr(workspace),
                                     workspace.numel(), _stream(o.device)))


def problem_ws_bytes(pb: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.sage_attn_workspace_bytes_ex(pb.ref, ctypes.byref(n)))
    return n.value


def _check_qkv(q, k, v, ndim: int):
    if q.dim() != ndim or k.dim() != ndim or v.dim() != ndim:
        raise ValueError(f"q, k, v must be {ndim}-D")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in DTYPES:
        raise ValueError("q, k, v must share one dtype, float16 or bfloat16")
    if not (q.is_cuda and k.is_cuda and v.is_cuda) or not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same GPU")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if k.shape != v.shape:
        raise ValueError(f"k shape {tuple(k.shape)} differs from v shape {tuple(v.shape)}")


def fwd_ex(pb: Problem, q, k, v, o, workspace) -> None:
    """sage_attn_fwd_ex on caller-provided tensors (o and workspace are written)."""
    with _on(q.device):
        _check(_lib.sage_attn_fwd_ex(pb.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(workspace), workspace.numel(),
                                     _stream(q.device)))


def prologue_ex(pb: Problem, q, k, v, workspace) -> None:
    with _on(q.device):
        _check(_lib.sage_attn_prologue_ex(pb.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(workspace), workspace.numel(),
                                          _stream(q.device)))


def attend_ex(pb: Problem, o, workspace) -> None:
    with _on(o.device):
        _check(_lib.sage_attn_attend_ex(pb.ref, _ptr(o), _ptr(workspace), workspace.numel(), _stream(o.device)))


def sageattn(q, k, v, attn_mask=None, dropout_p: float = 0.0, is_causal: bool = False, scale=None,
             qk_bits: int = 8, pv_bits: int = 8, tensor_layout: str = "HND", workspace=None):
    """Quantized drop-in for F.scaled_dot_product_attention(q, k, v, is_causal=...).

    tensor_layout "HND": q [B, H, N, d], k/v [B, Hkv, N, d]; "NHD": q [B, N, H, d],
    k/v [B, N, Hkv, d].  fp16 or bf16 (all three alike), contiguous; d in {64, 128}; qk_bits 8
    (INT8 codes) or 4 (INT4-range codes); pv_bits 8 (FP8 P~ and V, the fast mode) or 16 (16-bit
    P and V, the high-fidelity mode).  Grouped-query attention maps head h to kv head
    h // (H // Hkv).  Returns o shaped, laid out and typed like q.
    """
    if attn_mask is not None or dropout_p != 0.0 or scale is not None:
        raise NotImplementedError("attn_mask, dropout and custom scale are not supported")
    pb = _dense_problem(q, k, v, is_causal, qk_bits, pv_bits, tensor_layout)
    nbytes = problem_ws_bytes(pb)
    if workspace is None or workspace.numel() < nbytes:
        workspace = alloc_workspace(nbytes, q.device)
    o = torch.empty_like(q)
    fwd_ex(pb, q, k, v, o, workspace)
    return o


def _dense_problem(q, k, v, is_causal, qk_bits, pv_bits, tensor_layout) -> Problem:
    """The problem descriptor of a fixed-length batch, after checking the tensors."""
    if tensor_layout == "HND" and q.dtype == torch.float16:
        B, H, Hkv, N, d = _shapes(q, k, v)
    else:
        _check_qkv(q, k, v, 4)
        if tensor_layout == "HND":
            (B, H, N, d), Hkv = q.shape, k.shape[1]
            ok = k.shape[0] == B and k.shape[2] == N and k.shape[3] == d
        elif tensor_layout == "NHD":
            (B, N, H, d), Hkv = q.shape, k.shape[2]
            ok = k.shape[0] == B and k.shape[1] == N and k.shape[3] == d
        else:
            raise ValueError(f"tensor_layout must be one of {sorted(LAYOUTS)}")
        if not ok:
            raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    return Problem(B, H, Hkv, N, d, is_causal, qk_bits, pv_bits, tensor_layout, q.dtype)


class SageAttention:
    """Module-style front end (the blog page's core-API call: an attention object built from
    head_dim, is_causal and quant_mode that replaces a model's attention function).

    quant_mode: one of QUANT_MODES -- "qk_int8_pv_fp8" (fast), "qk_int8_pv_fp16" (high
    fidelity: V and P stay 16-bit), or the INT4-range QK forms.  Calling it on q, k, v (laid out
    as tensor_layout, fp16 or bf16) returns o; the workspace is kept and reused while it is
    large enough, so repeated calls of one shape allocate only the output.  Calls share that
    workspace: calls of one object that may overlap (on different streams) race."""

    def __init__(self, head_dim: int, is_causal: bool = False, quant_mode: str = "qk_int8_pv_fp8",
                 tensor_layout: str = "HND"):
        if head_dim not in (64, 128):
            raise ValueError(f"head_dim must be 64 or 128, got {head_dim}")
        if quant_mode not in QUANT_MODES:
            raise ValueError(f"quant_mode must be one of {sorted(QUANT_MODES)}, got {quant_mode!r}")
        if tensor_layout not in LAYOUTS:
            raise ValueError(f"tensor_layout must be one of {sorted(LAYOUTS)}")
        self.head_dim, self.is_causal, self.quant_mode, self.tensor_layout = head_dim, bool(is_causal), quant_mode, tensor_layout
        self.qk_bits, self.pv_bits = QUANT_MODES[quant_mode]
        self._workspace = None

    def __call__(self, q, k, v):
        if q.shape[-1] != self.head_dim:
            raise ValueError(f"head dim {q.shape[-1]} differs from this module's head_dim {self.head_dim}")
        pb = _dense_problem(q, k, v, self.is_causal, self.qk_bits, self.pv_bits, self.tensor_layout)
        nbytes = problem_ws_bytes(pb)
        ws = self._workspace
        if ws is None or ws.numel() < nbytes or ws.device != q.device:
            ws = self._workspace = alloc_workspace(nbytes, q.device)
        o = torch.empty_like(q)
        fwd_ex(pb, q, k, v, o, ws)
        return o

    def __repr__(self):
        return (f"SageAttention(head_dim={self.head_dim}, is_causal={self.is_causal}, "
                f"quant_mode={self.quant_mode!r}, tensor_layout={self.tensor_layout!r})")


def sageattn_varlen(q, k, v, cu_seqlens, is_causal: bool = False, qk_bits: int = 8, pv_bits: int = 8,
                    workspace=None):
    """Variable-length batch: q [T, H, d], k/v [T, Hkv, d] hold the sequences back to back;
    sequence s is tokens cu_seqlens[s] .. cu_seqlens[s + 1] - 1 (cu_seqlens: a host list or CPU
    tensor of B + 1 increasing ints from 0 to T).  Each sequence is attended, smoothed and
    quantized on its own.  fp16 or bf16.  Returns o [T, H, d]."""
    _check_qkv(q, k, v, 3)
    T, H, d = q.shape
    Hkv = k.shape[1]
    if k.shape[0] != T or k.shape[2] != d:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    if hasattr(cu_seqlens, "is_cuda") and cu_seqlens.is_cuda:
        raise ValueError("cu_seqlens must be on the host (a list or a CPU tensor)")
    cu = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
    if len(cu) < 2 or cu[-1] != T:
        raise ValueError(f"cu_seqlens must end at the token count {T}")
    pb = Problem(len(cu) - 1, H, Hkv, 0, d, is_causal, qk_bits, pv_bits, "HND", q.dtype, cu)
    nbytes = problem_ws_bytes(pb)
    if workspace is None or workspace.numel() < nbytes:
        workspace = alloc_workspace(nbytes, q.device)
    o = torch.empty_like(q)
    fwd_ex(pb, q, k, v, o, workspace)
    return o


def quant_debug(q, k, v, is_causal: bool = False, qk_bits: int = 8, pv_bits: int = 8) -> dict:
    """Prologue outputs in plain layouts (see sage_quant_debug in include/sage_attn.h); q, k, v
    [B, heads, N, d] fp16 or bf16.  With pv_bits = 16 there are no V codes or scales and those
    entries are None."""
    _check_qkv(q, k, v, 4)
    (B, H, N, d), Hkv = q.shape, k.shape[1]
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    nqb = -(-N // get_config()["bq"])
    dev = q.device
    out = {
        "mu_k": torch.empty(B, Hkv, d, dtype=torch.float32, device=dev),
        "k_codes": torch.empty(B, Hkv, N, d, dtype=torch.int8, device=dev),
        "k_scales": torch.empty(B, Hkv, N, dtype=torch.float32, device=dev),
        "v_codes": torch.empty(B, Hkv, N, d, dtype=torch.uint8, device=dev),
        "v_scales": torch.empty(B, Hkv, d, dtype=torch.float32, device=dev),
        "mu_q": torch.empty(B, H, nqb, d, dtype=torch.float32, device=dev),
        "q_codes": torch.empty(B, H, N, d, dtype=torch.int8, device=dev),
        "q_scales": torch.empty(B, H, N, dtype=torch.float32, device=dev),
        "delta_s": torch.empty(B, H, nqb, N, dtype=torch.float32, device=dev),
    }
    if pv_bits == 16:
        out["v_codes"] = out["v_scales"] = None
    pb = Problem(B, H, Hkv, N, d, is_causal, qk_bits, pv_bits, "HND", q.dtype)
    ws = alloc_workspace(problem_ws_bytes(pb), dev)
    names = ("mu_k", "k_codes", "k_scales", "v_codes", "v_scales", "mu_q", "q_codes", "q_scales", "delta_s")
    with _on(dev):
        _check(_lib.sage_quant_debug_ex(pb.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(ws), ws.numel(), _stream(dev),
                                        *[_ptr(out[n]) for n in names]))
    return out


def qk_tile_debug(q, k, v, b: int, h: int, qb: int, kb: int, is_causal: bool = False, qk_bits: int = 8,
                  pv_bits: int = 8):
    """Raw int32 S tile [bq, bk] of the attention kernel's integer MFMA path."""
    B, H, Hkv, N, d = _shapes(q, k, v)
    cfg = get_config()
    tile = torch.empty(cfg["bq"], cfg["bk"], dtype=torch.int32, device=q.device)
    ws = alloc_workspace(workspace_bytes(B, H, Hkv, N, d, is_causal, qk_bits, pv_bits), q.device)
    with _on(q.device):
        _check(_lib.sage_qk_tile_debug(_ptr(q), _ptr(k), _ptr(v), B, H, Hkv, N, d, int(is_causal), qk_bits, pv_bits,
                                       _ptr(ws), ws.numel(), _stream(q.device), b, h, qb, kb, _ptr(tile)))
    return tile


#: matrix instructions the rate probe can run (sage_mfma_rate_probe's kind)
MFMA_PROBE_KINDS = {"int8": 0, "fp8": 1, "fp6": 2, "fp16": 3}


def mfma_rate_probe(kind: str, iters: int, sink) -> float:
    """Enqueue the library's matrix-unit rate probe on the current stream of sink's device (a
    device tensor of at least 512 KiB, overwritten) and return the ops the launch performs; the
    caller times it (a measurement utility, not part of the method)."""
    ops = ctypes.c_double(0.0)
    with _on(sink.device):
        _check(_lib.sage_mfma_rate_probe(MFMA_PROBE_KINDS[kind], int(iters), _ptr(sink), sink.numel() * sink.element_size(),
                                         ctypes.byref(ops), _stream(sink.device)))
    return ops.value
