#!/usr/bin/env python3
"""Benchmark of the SageAttention2 quantized attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload bench|llm|dit|gqa|tiny|varlen] [--pv-bits 8|16]

A step is one whole forward pass (quantize/smooth prologue + fused attention kernel) over the
workload's seeded synthetic inputs, which are resident in HBM before the timed region.  The
K timed steps are bracketed by torch.cuda.synchronize(); per-kernel times come from HIP
events recorded on the stream the kernels are launched on (torch's current stream, which the
binding passes to the library).

Prints one JSON line: effective attention TOPS = 4*B*H*N^2*d / t (halved when causal), the
roofline of the dominant kernel (the fused attention kernel, MFMA bound) and the CPU oracle's
rate on a bounded sample of the same workload.  The breakdown gives the prologue and attention
times of the timed steps, and the prologue once more with the caches (L2 and the 256 MB MALL)
emptied before each call, since back-to-back steps can find their inputs still cached.
QK^T and PV each carry half of the kernel's
ops, on different matrix instructions, so its peak is the harmonic mix of the two dense peaks:
INT8 5.0 P (QK^T, 8-bit codes), FP6 10.1 P (QK^T, INT4-range codes), FP8 5.0 P (P~V) and
fp16 2.5 P (PV in the fp16 mode).

Other modes:
  --calibrate-copy   run a plain device copy of known size (for scaling rocprofv3's
                     FETCH_SIZE / WRITE_SIZE counters to bytes)
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective attention TOPS (4·B·H·N²·d/t, ½ if causal) at N=8K–32K, d=64/128"
# MI355X dense matrix peaks, TOPS / TFLOP/s
PEAK_QK = {8: 5000.0, 4: 10100.0}      # INT8 codes on the int8 MFMA; INT4-range codes on FP6
PEAK_PV = {8: 5000.0, 16: 2500.0}      # FP8 P~ V; fp16 P V
PEAK_HBM_GBPS = 8000.0


def attn_peak(qk_bits: int, pv_bits: int) -> float:
    """Peak of a kernel that spends half its ops on QK^T and half on PV."""
    return 1.0 / (0.5 / PEAK_QK[qk_bits] + 0.5 / PEAK_PV[pv_bits])


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.txt")
ATTN_SRC = os.path.join(ROOT, "quantized_attention_smooth_amd", "csrc", "attention.hip")


def _describe(w, pv_bits: int) -> str:
    kind = "causal" if w.causal else "non-causal"
    heads = f"H{w.H}" if w.H == w.Hkv else f"H{w.H}/Hkv{w.Hkv}"
    size = f"{w.B} sequences of {min(w.lens)}-{w.N} tokens (T={w.T})" if hasattr(w, "lens") else f"B{w.B} N{w.N}"
    return (f"{w.name}: {size} {heads} d{w.d} {kind}, "
            f"{'INT8' if w.qk_bits == 8 else 'INT4-range'} QK + {'FP8' if pv_bits == 8 else 'fp16'} PV")


def _src_hash() -> str:
    return hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()


def _traffic(workload: str, pv_bits: int):
    """HBM bytes per attention-kernel launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    e = t.get("workloads", {}).get(workload if pv_bits == 8 else f"{workload}-pv16", {}).get("attn_fwd")
    if not e or t.get("attention_src_sha256") != _src_hash():
        return None
    return (e["fetch_kib"] * t["fetch_factor"] + e["write_kib"] * t["write_factor"]) * 1024.0


def cpu_baseline(w, q1, k1, v1, budget_s: float, pv_bits: int = 8, head_ops: float | None = None) -> dict:
    """The oracle as it stands, on one head of one sequence (q1, k1, v1: [1, 1, n, d]): its full
    prologue plus as many query blocks as fit the budget (spread over the sequence),
    extrapolated by block cost (causal block qb costs qb + 1 key blocks) to that head, then to
    the workload by the ratio of their ops (head_ops: the sampled head's share)."""
    import numpy as np
    from oracle import sage as osage
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - reporting only
        blas = 1
    t0 = time.perf_counter()
    pro = osage.prologue(q1, k1, v1, w.causal, w.qk_bits, quant_pv=pv_bits == 8)
    t_pro = time.perf_counter() - t0
    nqb = pro.nqb
    cost = [(qb + 1) if w.causal else pro.nkb for qb in range(nqb)]
    order = []
    step = max(1, nqb // 16)
    for s in range(step):
        order += list(range(nqb - 1 - s, -1, -step))
    done_cost, t_att = 0, 0.0
    nblk = 0
    for qb in order:
        t1 = time.perf_counter()
        osage.attend_block(pro, 0, 0, qb)
        t_att += time.perf_counter() - t1
        done_cost += cost[qb]
        nblk += 1
        if t_pro + t_att >= budget_s:
            break
    per_unit = t_att / done_cost
    t_head = t_pro + per_unit * sum(cost)
    t_total = t_head * w.ops / head_ops
    value = w.ops / t_total / 1e12
    cores = len(os.sched_getaffinity(0))
    return {
        "value": value, "unit": "TOPS", "cores": int(min(cores, blas)), "kind": "oracle",
        "sample": (f"numpy oracle on one head ({pro.N} tokens): full prologue ({t_pro:.1f} s) + {nblk} of {nqb} "
                   f"query blocks ({t_att:.1f} s), extrapolated by block cost to the head and by ops to the "
                   f"workload "
                   f"(est. {t_total:.0f} s for the workload); BLAS threads {blas} of {cores} host cores in the "
                   f"process's affinity set, elementwise 1 thread"),
        "_blocks": order[:nblk], "_pro": pro,
    }


def environment() -> dict:
    """Host, software and device facts for the record (read outside the timed region)."""
    import platform
    import subprocess

    import torch
    env = {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None), "python": platform.python_version()}
    try:
        env["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        env["rocm"] = None
    try:
        env["gpu"] = torch.cuda.get_device_name(0)
    except Exception:  # pragma: no cover - reporting only
        env["gpu"] = None
    cpu = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    env["cpu_model"] = cpu
    env["cpu_cores_affinity"] = len(os.sched_getaffinity(0))
    return env


def under_profiler() -> bool:
    """True inside a rocprofv3 run: its tool library is preloaded into every child process too,
    so no other program is started from here then."""
    return "ROCPROF_OUTPUT_PATH" in os.environ or "rocprofiler" in os.environ.get("LD_PRELOAD", "")


def smi_clocks() -> dict | None:
    """The GPU's current graphics clocks (MHz, one per XCD) as its management tool reports them
    (best effort: None when the tool is missing or fails, or under the profiler)."""
    import subprocess
    if under_profiler():
        return None
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "--json"], capture_output=True, text=True,
                           timeout=30)
        if r.returncode != 0:
            return None
        d = json.loads(r.stdout)
        d = d["gpu_data"][0] if isinstance(d, dict) and "gpu_data" in d else (d[0] if isinstance(d, list) else d)
        clk = d["clock"]
        vals = [v["clk"]["value"] for k, v in clk.items() if k.startswith("gfx") and isinstance(v, dict)]
        mx = [v["max_clk"]["value"] for k, v in clk.items() if k.startswith("gfx") and isinstance(v, dict)]
        return {"gfx_mhz": vals, "gfx_max_mhz": max(mx) if mx else None}
    except Exception:  # pragma: no cover - reporting only
        return None


def clocks_under_load(step, seconds: float = 4.0) -> dict | None:
    """Graphics clocks sampled while the step runs back to back (untimed): the management tool
    runs in a thread while this thread keeps the GPU busy."""
    import threading

    import torch
    if under_profiler():
        return None
    box = {}
    th = threading.Thread(target=lambda: box.setdefault("c", smi_clocks()))
    t0 = time.perf_counter()
    step()
    th.start()
    while th.is_alive() and time.perf_counter() - t0 < seconds + 30:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
    th.join()
    return box.get("c")


def measured_peaks(dev, qk_bits: int, pv_bits: int, iters: int = 6000, reps: int = 3) -> dict:
    """Sustained dense MFMA rates from the library's rate probe (register operands, two waves per
    SIMD), for the two instructions the attention kernel uses, and their harmonic mix."""
    import torch

    import quantized_attention_smooth_amd as sa
    sink = torch.empty(1 << 18, dtype=torch.float32, device=dev)
    kinds = {"qk": "int8" if qk_bits == 8 else "fp6", "pv": "fp8" if pv_bits == 8 else "fp16"}
    out = {}
    for role, kind in kinds.items():
        sa.mfma_rate_probe(kind, 100, sink)                 # warm-up
        best = 0.0
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            ops = sa.mfma_rate_probe(kind, iters, sink)
            e1.record()
            torch.cuda.synchronize()
            best = max(best, ops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        out[f"{role}_{kind}_TOPS"] = best
    out["mix_TOPS"] = 1.0 / (0.5 / out[f"qk_{kinds['qk']}_TOPS"] + 0.5 / out[f"pv_{kinds['pv']}_TOPS"])
    return out


def accuracy(o_gpu, q1, k1, v1, causal: bool, row_blocks, pro) -> dict:
    """O of the sampled query blocks of one head against exact fp64 attention and against the
    oracle: cosine similarity, RMSE, relative L1 (sum |o - e| / sum |e|) and the largest error,
    set beside the pages' figures."""
    import numpy as np
    from oracle import sage as osage
    rows = np.concatenate([np.arange(qb * 128, min(pro.N, qb * 128 + 128)) for qb in row_blocks])
    e = osage.exact_attention_rows(q1[0, 0], k1[0, 0], v1[0, 0], rows, causal)
    orc = np.concatenate([osage.attend_block(pro, 0, 0, qb) for qb in row_blocks])
    g = np.asarray(o_gpu, dtype=np.float64)[rows]

    def cmp(a, b):
        return {"cos": float((a * b).sum() / np.sqrt((a * a).sum() * (b * b).sum())),
                "rmse": float(np.sqrt(((a - b) ** 2).mean())),
                "rel_l1": float(np.abs(a - b).sum() / np.abs(b).sum()),
                "max_abs": float(np.abs(a - b).max())}
    return {"rows": int(rows.size), "gpu_vs_exact": cmp(g, e), "oracle_vs_exact": cmp(orc, e),
            "gpu_vs_oracle": {**cmp(g, orc), "max_abs_over_max_oracle": float(np.abs(g - orc).max() / np.abs(orc).max())},
            "pages": "CosSim 99.45 % average, 96.72 % worst layer, RMSE 0.0313 (SageAttention2 notes, per-thread "
                     "INT4, real model layers); CosSim 99.97 %, L1 0.01862 (SageAttention2++ verdict page, "
                     "CogvideoX layers)"}


def calibrate_copy(nbytes: int = 1 << 30, reps: int = 3) -> None:
    import torch
    x = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": nbytes, "reps": reps}), flush=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="bench")
    ap.add_argument("--pv-bits", type=int, default=8, choices=(8, 16),
                    help="8: FP8 P~ and V (fast mode); 16: fp16 P and V (high-fidelity mode)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--seq-len", type=int, default=None,
                    help="sequence length N in place of a fixed-length workload's own (the metric spans N = 8K-32K)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the quantized attention forward is a single-GPU kernel "
              f"here (heads shard across GPUs with no communication); --gpus {args.gpus} is not supported.",
              file=sys.stderr)
        return 2
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only (WORLD_SIZE > 1 given)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.calibrate_copy:
        calibrate_copy()
        return 0

    import quantized_attention_smooth_amd as sa
    from workloads import VARLEN_WORKLOADS, WORKLOADS, make_inputs, make_varlen_inputs

    pv = args.pv_bits
    varlen = args.workload in VARLEN_WORKLOADS
    if varlen and args.seq_len:
        print("--seq-len applies to fixed-length workloads only", file=sys.stderr)
        return 2
    if varlen:
        w = VARLEN_WORKLOADS[args.workload]
        q, k, v = make_varlen_inputs(w, seed=0)
        pb = sa.Problem(w.B, w.H, w.Hkv, 0, w.d, w.causal, w.qk_bits, pv, "HND", cu_seqlens=w.cu_seqlens)
    else:
        w = WORKLOADS[args.workload]
        if args.seq_len:
            w = dataclasses.replace(w, N=args.seq_len, name=f"{w.name}@N{args.seq_len}")
        q, k, v = make_inputs(w, seed=0)
        pb = sa.Problem(w.B, w.H, w.Hkv, w.N, w.d, w.causal, w.qk_bits, pv, "HND")
    dev = torch.device("cuda:0")
    qd = torch.from_numpy(q).to(dev)
    kd = torch.from_numpy(k).to(dev)
    vd = torch.from_numpy(v).to(dev)
    o = torch.empty_like(qd)
    ws = sa.alloc_workspace(sa.problem_ws_bytes(pb), dev)

    def step():
        sa.prologue_ex(pb, qd, kd, vd, ws)
        sa.attend_ex(pb, o, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if not torch.isfinite(o).all():
        print("non-finite output", file=sys.stderr)
        return 1

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record()
    for s in range(K):
        ev[s][0].record()
        sa.prologue_ex(pb, qd, kd, vd, ws)
        ev[s][1].record()
        sa.attend_ex(pb, o, ws)
        ev[s][2].record()
    e_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms_step = e_start.elapsed_time(e_end) / K
    pro_all = [e[0].elapsed_time(e[1]) for e in ev]
    att_all = [e[1].elapsed_time(e[2]) for e in ev]
    step_all = [e[0].elapsed_time(e[2]) for e in ev]
    pro_ms = float(np.mean(pro_all))
    att_ms = float(np.mean(att_all))

    # The prologue alone with the caches emptied first: back to back, the inputs the previous step
    # read can still sit in the 256 MB memory-side cache (MALL).  Writing a 512 MB buffer before
    # each call evicts them, so this time is the HBM-bound one.
    o_host = o.float().cpu().numpy()                                    # for the accuracy report
    flush = torch.empty(128 << 20, dtype=torch.float32, device=dev)
    cold = []
    for _ in range(min(K, 10)):
        flush.fill_(0.0)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        sa.prologue_ex(pb, qd, kd, vd, ws)
        c1.record()
        cold.append((c0, c1))
    torch.cuda.synchronize()
    pro_cold_ms = float(np.mean([c0.elapsed_time(c1) for c0, c1 in cold]))
    ops = w.ops
    value = ops / (ms_step * 1e-3) / 1e12
    achieved = ops / (att_ms * 1e-3) / 1e12
    lens = w.lens if varlen else [w.N] * w.B
    tokens = sum(lens)
    n_q, n_kv = tokens * w.H * w.d, tokens * w.Hkv * w.d
    ds_elems = 0                                                          # Delta_S rows, all heads
    for n in lens:
        nqb = -(-n // 128)
        ds_elems += w.H * (128 * nqb * (nqb + 1) // 2 if w.causal else nqb * nqb * 128)
    # read q, k, v once (fp16); write Q/K codes (1 byte), V as FP8 codes or fp16, Delta_S rows
    pro_bytes = 2 * (n_q + 2 * n_kv) + (n_q + n_kv) + n_kv * (pv // 8) + 4 * ds_elems
    # the practical HBM rate for that much traffic: a plain device copy moving the same bytes
    # (half read, half written), timed like the flushed prologue
    copy_src = torch.empty(pro_bytes // 2 // 4, dtype=torch.float32, device=dev)
    copy_dst = torch.empty_like(copy_src)
    copy_src.fill_(1.0)
    copies = []
    for _ in range(min(K, 10)):
        flush.fill_(0.0)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        copy_dst.copy_(copy_src)
        c1.record()
        copies.append((c0, c1))
    torch.cuda.synchronize()
    copy_cold_ms = float(np.mean([c0.elapsed_time(c1) for c0, c1 in copies]))
    del flush, copy_src, copy_dst
    traffic = _traffic(w.name if args.seq_len else args.workload, pv)
    peak = attn_peak(w.qk_bits, pv)
    meas = measured_peaks(dev, w.qk_bits, pv)
    qk_t = "int8" if w.qk_bits == 8 else "fp6 (INT4-range codes)"
    pv_t = "P~V fp8" if pv == 8 else "PV fp16"

    line = {
        "metric": METRIC, "value": value, "unit": "TOPS", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("i8" if w.qk_bits == 8 else "fp6e2m3") + ("+fp8e4m3" if pv == 8 else "+fp16"),
        "data": "synthetic",
        "config": {"workload": _describe(w, pv), "B": w.B, "H": w.H, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "causal": w.causal, "qk_bits": w.qk_bits, "pv_bits": pv, "seed": 0,
                   **({"cu_seqlens": w.cu_seqlens} if varlen else {})},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": traffic,
                     "traffic_source": ("HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE "
                                        "runs of this kernel source (profiles/traffic_counters.txt), not measured "
                                        "in this run; null when the source changed since"),
                     "measured_peak": meas["mix_TOPS"], "frac_of_measured_peak": achieved / meas["mix_TOPS"],
                     "measured_peaks": meas,
                     "kernel": f"attn_fwd (fused QK^T {qk_t} MFMA + softmax + {pv_t} MFMA)",
                     "per_unit": f"4*d = {4 * w.d} int8/fp8 ops per score element; "
                                 f"{ops / (4 * w.d):.4g} score elements per launch"},
        "breakdown": {"prologue_ms": pro_ms, "attention_ms": att_ms,
                      "step_ms_median": float(np.median(step_all)), "step_ms_min": float(np.min(step_all)),
                      "attention_ms_median": float(np.median(att_all)), "attention_ms_min": float(np.min(att_all)),
                      "prologue_ms_median": float(np.median(pro_all)), "prologue_ms_min": float(np.min(pro_all)),
                      "timing": ("K timed steps between two torch.cuda.synchronize() calls after W warm-up steps; "
                                 "ms_per_step = the span of all K by HIP events / K; per-kernel times are HIP events "
                                 "on the stream the kernels run on, mean / median / min over the K steps"),
                      "prologue_GBps_algorithmic": pro_bytes / (pro_ms * 1e-3) / 1e9,
                      "prologue_frac_hbm": pro_bytes / (pro_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                      "prologue_ms_caches_flushed": pro_cold_ms,
                      "prologue_GBps_algorithmic_caches_flushed": pro_bytes / (pro_cold_ms * 1e-3) / 1e9,
                      # K (and V when it is quantized) is read a second time for its codes
                      "prologue_GBps_two_reads_caches_flushed":
                          (pro_bytes + 2 * n_kv * (2 if pv == 8 else 1)) / (pro_cold_ms * 1e-3) / 1e9,
                      "copy_same_bytes_ms_caches_flushed": copy_cold_ms,
                      "prologue_vs_copy_caches_flushed": copy_cold_ms / pro_cold_ms,
                      "wall_s_timed": wall},
    }
    line["environment"] = environment()
    line["environment"]["gpu_clocks_under_load"] = clocks_under_load(step)
    line["environment"]["gpu_clocks_idle_after"] = smi_clocks()
    line["environment"]["gpu_clocks_note"] = (
        "clocks as amd-smi reports them (one per XCD) while steps run back to back and after; on the "
        "boxes measured so far it reported ~100 MHz in both cases, so these values do not track the "
        "kernels' clock.  The hardware counters do: GRBM_GUI_ACTIVE per XCD over the dispatch time gives "
        "1.8-2.0 GHz during the attention kernel (profiles/attn_fwd_counters.md).")
    if not args.no_cpu_baseline:
        if varlen:                      # one head of the longest sequence
            s = int(np.argmax(w.lens))
            a, b = w.cu_seqlens[s], w.cu_seqlens[s + 1]
            q1, k1, v1 = (np.ascontiguousarray(x[a:b, :1].transpose(1, 0, 2))[None] for x in (q, k, v))
            o1 = o_host[a:b, 0]
            n = b - a
        else:                           # head (0, 0)
            q1, k1, v1 = (np.ascontiguousarray(x[:1, :1]) for x in (q, k, v))
            o1 = o_host[0, 0]
            n = w.N
        head_ops = 4.0 * n * n * w.d / (2 if w.causal else 1)
        cb = cpu_baseline(w, q1, k1, v1, args.cpu_budget, pv, head_ops)
        blocks, pro = cb.pop("_blocks"), cb.pop("_pro")
        line["cpu_baseline"] = cb
        # accuracy of the first, middle and last sampled query blocks of that head
        pick = sorted({blocks[0], blocks[len(blocks) // 2], blocks[-1]})
        line["accuracy"] = {"head": "query head 0 of " + ("the longest sequence" if varlen else "sequence 0"),
                            "query_blocks": pick, **accuracy(o1, q1, k1, v1, w.causal, pick, pro)}
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
