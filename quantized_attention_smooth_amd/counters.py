"""Summaries of rocprofv3 runs of this library's kernels (measurement tooling).

    python -m quantized_attention_smooth_amd.counters DIR [DIR ...]        counter table
    python -m quantized_attention_smooth_amd.counters --trace DIR           kernel-trace table
    python -m quantized_attention_smooth_amd.counters --traffic CALIB_FETCH_DIR CALIB_WRITE_DIR \
        NAME=FETCH_DIR,WRITE_DIR [...]                                         HBM traffic (JSON)

Each DIR is the output directory of one `rocprofv3 --pmc ... -f csv -d DIR -o run -- python3
bench.py ...` pass (its run_counter_collection.csv).  Counter values are averaged per dispatch
of each kernel of the library; every pass of one workload is merged into one table, and the
derived figures below are printed when their counters are present:

  cycles      GRBM_GUI_ACTIVE / 8: the dispatch's length in GPU clocks (the counter is summed over
              the 8 XCDs); with the dispatch's duration from the trace timestamps, the clock
  MFMA busy   SQ_VALU_MFMA_BUSY_CYCLES / (cycles * 1024 SIMDs): the share of the SIMDs' cycles
              the matrix unit was busy (the counter sums its busy cycles over all SIMDs)
  VALU busy   SQ_ACTIVE_INST_VALU * 4 / (cycles * 1024): wave-cycles spent issuing vector
              instructions (reported in quad cycles, summed over waves) per SIMD cycle
  co-exec     SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES: share of matrix-busy cycles
              in which a vector instruction was issued as well
  waits       SQ_WAIT_INST_ANY, SQ_WAIT_INST_LDS, SQ_ACTIVE_INST_* as shares of SQ_WAVE_CYCLES
              (all in quad cycles)
  LDS bank conflict cycles per LDS instruction; TCC hit rate
  MFMA ops    SQ_INSTS_VALU_MFMA_MOPS_{I8,F8,F6F4} * 512 (the counters count 512-op units)
"""
from __future__ import annotations

import collections
import csv
import hashlib
import os
import sys

SIMDS = 1024          # 256 CUs x 4 SIMDs
XCDS = 8
SHORT = {"attn_fwd": "attn_fwd", "stats_and_q": "stats_and_q", "kv_quant": "kv_quant", "init_stats": "init_stats"}


def _kernel(name: str) -> str | None:
    for k, v in SHORT.items():
        if f"::{k}" in name or name.startswith(k):
            return v
    return None


def load(dirs):
    """{kernel: {counter: mean value per dispatch}} over every run_counter_collection.csv."""
    per = collections.defaultdict(lambda: collections.defaultdict(dict))   # kernel -> counter -> dispatch -> v
    dur = collections.defaultdict(dict)                                      # kernel -> dispatch -> ns
    for d in dirs:
        f = os.path.join(d, "run_counter_collection.csv")
        for r in csv.DictReader(open(f)):
            k = _kernel(r["Kernel_Name"])
            if k is None:
                continue
            per[k][r["Counter_Name"]][(d, r["Dispatch_Id"])] = float(r["Counter_Value"])
            dur[k][(d, r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    out = {}
    for k, cs in per.items():
        out[k] = {c: sum(v.values()) / len(v) for c, v in cs.items()}
        out[k]["_dispatches"] = max(len(v) for v in cs.values())
        out[k]["_duration_ns"] = sum(dur[k].values()) / len(dur[k])
    return out


def derived(c: dict) -> dict:
    g = c.get
    d = {}
    cyc = g("GRBM_GUI_ACTIVE") / XCDS if g("GRBM_GUI_ACTIVE") else None
    if cyc:
        d["dispatch cycles (per XCD)"] = cyc
        if g("_duration_ns"):
            d["clock during the dispatch, GHz"] = cyc / g("_duration_ns")
        if g("SQ_VALU_MFMA_BUSY_CYCLES") is not None:
            d["MFMA busy (of SIMD cycles)"] = g("SQ_VALU_MFMA_BUSY_CYCLES") / (cyc * SIMDS)
        if g("SQ_ACTIVE_INST_VALU") is not None:
            d["VALU issue (wave-cycles per SIMD cycle)"] = 4 * g("SQ_ACTIVE_INST_VALU") / (cyc * SIMDS)
        if g("SQ_ACTIVE_INST_VALU2") is not None:
            d["dual VALU issue (of SIMD cycles)"] = 4 * g("SQ_ACTIVE_INST_VALU2") / (cyc * SIMDS)
    if g("SQ_VALU_MFMA_COEXEC_CYCLES") is not None and g("SQ_VALU_MFMA_BUSY_CYCLES"):
        d["co-exec (of MFMA-busy cycles)"] = g("SQ_VALU_MFMA_COEXEC_CYCLES") / g("SQ_VALU_MFMA_BUSY_CYCLES")
    if g("SQ_WAVE_CYCLES"):
        for key in ("SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_LDS",
                    "SQ_ACTIVE_INST_VALU"):
            if g(key) is not None:
                d[f"{key} (of wave cycles)"] = g(key) / g("SQ_WAVE_CYCLES")
    if g("SQ_INSTS_LDS") and g("SQ_LDS_BANK_CONFLICT") is not None:
        d["LDS bank-conflict cycles per LDS instruction"] = g("SQ_LDS_BANK_CONFLICT") / g("SQ_INSTS_LDS")
    if g("TCC_HIT_sum") is not None and g("TCC_MISS_sum") is not None and g("TCC_HIT_sum") + g("TCC_MISS_sum") > 0:
        d["L2 hit rate"] = g("TCC_HIT_sum") / (g("TCC_HIT_sum") + g("TCC_MISS_sum"))
    if g("SQ_WAVES") and g("SQ_INSTS_VALU") is not None:
        d["VALU instructions per wave"] = g("SQ_INSTS_VALU") / g("SQ_WAVES")
        if g("SQ_INSTS_MFMA") is not None:
            d["MFMA instructions per wave"] = g("SQ_INSTS_MFMA") / g("SQ_WAVES")
        if g("SQ_INSTS_LDS") is not None:
            d["LDS instructions per wave"] = g("SQ_INSTS_LDS") / g("SQ_WAVES")
    for t in ("I8", "F8", "F6F4"):
        if g(f"SQ_INSTS_VALU_MFMA_MOPS_{t}") is not None:
            d[f"MFMA {t} ops"] = 512 * g(f"SQ_INSTS_VALU_MFMA_MOPS_{t}")
    return d


def table(dirs, kernels=("attn_fwd", "stats_and_q", "kv_quant")) -> str:
    data = load(dirs)
    lines = []
    for k in kernels:
        if k not in data:
            continue
        c = data[k]
        lines.append(f"### {k} ({int(c['_dispatches'])} dispatches averaged)\n")
        lines.append("| counter | per dispatch |")
        lines.append("|---|---|")
        lines.append(f"| (mean dispatch duration, us) | {c['_duration_ns'] / 1e3:.1f} |")
        for name in sorted(x for x in c if not x.startswith("_")):
            lines.append(f"| {name} | {c[name]:.6g} |")
        for name, v in derived(c).items():
            lines.append(f"| *{name}* | {v:.4g} |")
        lines.append("")
    return "\n".join(lines)


def trace_table(d: str) -> str:
    """The --kernel-trace --stats summary (run_kernel_stats.csv) as a markdown table, times in us."""
    rows = list(csv.DictReader(open(os.path.join(d, "run_kernel_stats.csv"))))
    out = ["| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("void ", "").replace("sage::(anonymous namespace)::", "").split("(")[0]
        if _kernel(name) is None and "mfma_probe" not in name:
            continue
        out.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                   f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |")
    return "\n".join(out)


def _counter_mean(d: str, counter: str, kernel: str | None) -> tuple[float, int]:
    vals = []
    for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
        if r["Counter_Name"] != counter:
            continue
        if kernel is None:
            if "copyBuffer" not in r["Kernel_Name"] and "elementwise" not in r["Kernel_Name"]:
                continue
        elif _kernel(r["Kernel_Name"]) != kernel:
            continue
        vals.append(float(r["Counter_Value"]))
    return (sum(vals) / len(vals) if vals else float("nan")), len(vals)


def traffic(calib_fetch: str, calib_write: str, runs: dict, copy_bytes: int = 1 << 30) -> dict:
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of every library kernel, scaled by what the same
    counters read for a plain device copy of copy_bytes (the copy's largest dispatch).  The
    SHA-256 of the attention and prologue sources in this tree are recorded with them: the
    figures describe those sources only."""
    def biggest(d, counter):
        vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv")))
                if r["Counter_Name"] == counter]
        return max(vals)
    fk, wk = biggest(calib_fetch, "FETCH_SIZE"), biggest(calib_write, "WRITE_SIZE")
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    sha = {k: hashlib.sha256(open(os.path.join(here, f"{k}.hip"), "rb").read()).hexdigest()
           for k in ("attention", "prologue")}
    out = {"attention_src_sha256": sha["attention"], "prologue_src_sha256": sha["prologue"],
           "fetch_factor": copy_bytes / 1024.0 / fk, "write_factor": copy_bytes / 1024.0 / wk,
           "calibration": {"copy_bytes": copy_bytes, "fetch_kib_read": fk, "write_kib_read": wk}, "workloads": {}}
    for name, (fd, wd) in runs.items():
        e = {}
        for k in SHORT.values():
            f, nf = _counter_mean(fd, "FETCH_SIZE", k)
            w, nw = _counter_mean(wd, "WRITE_SIZE", k)
            if nf and nw:
                e[k] = {"fetch_kib": f, "write_kib": w, "dispatches": [nf, nw],
                        "bytes": (f * out["fetch_factor"] + w * out["write_factor"]) * 1024.0}
        out["workloads"][name] = e
    return out


if __name__ == "__main__":
    import json
    if sys.argv[1] == "--trace":
        print(trace_table(sys.argv[2]))
    elif sys.argv[1] == "--traffic":
        runs = {}
        for spec in sys.argv[4:]:
            name, dirs = spec.split("=", 1)
            fd, wd = dirs.split(",")
            runs[name] = (fd, wd)
        print(json.dumps(traffic(sys.argv[2], sys.argv[3], runs), indent=1))
    else:
        print(table(sys.argv[1:]))
