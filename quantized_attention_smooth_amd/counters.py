"""Summaries of rocprofv3 counter runs of this library's kernels (measurement tooling).

    python -m quantized_attention_smooth_amd.counters DIR [DIR ...]

Each DIR is the output directory of one `rocprofv3 --pmc ... -f csv -d DIR -o run -- python3
bench.py ...` pass (its run_counter_collection.csv).  Counter values are averaged per dispatch
of each kernel of the library; every pass of one workload is merged into one table, and the
derived figures below are printed when their counters are present:

  MFMA busy   SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE * SIMDs): the share of the SIMDs'
              cycles the matrix unit was busy during the dispatch (GRBM_GUI_ACTIVE counts the
              cycles of the dispatch on one XCD, the busy cycles are summed over all SIMDs)
  VALU busy   SQ_ACTIVE_INST_VALU * 4 / (GRBM_GUI_ACTIVE * SIMDs) -- wave-cycles the SQ reports
              in quad cycles, one issuing wave per SIMD at a time
  waits       SQ_WAIT_INST_ANY, SQ_WAIT_INST_LDS (quad cycles) as shares of SQ_WAVE_CYCLES
  LDS bank conflict cycles per LDS instruction; TCC hit rate
  MFMA ops    SQ_INSTS_VALU_MFMA_MOPS_{I8,F8} * 512 (the counters count 512-op units)
"""
from __future__ import annotations

import collections
import csv
import os
import sys

SIMDS = 1024          # 256 CUs x 4 SIMDs
SHORT = {"attn_fwd": "attn_fwd", "stats_and_q": "stats_and_q", "kv_quant": "kv_quant", "delta_s": "delta_s",
         "init_stats": "init_stats"}


def _kernel(name: str) -> str | None:
    for k, v in SHORT.items():
        if f"::{k}" in name or name.startswith(k):
            return v
    return None


def load(dirs):
    """{kernel: {counter: mean value per dispatch}} over every run_counter_collection.csv."""
    per = collections.defaultdict(lambda: collections.defaultdict(dict))   # kernel -> counter -> dispatch -> v
    for d in dirs:
        f = os.path.join(d, "run_counter_collection.csv")
        for r in csv.DictReader(open(f)):
            k = _kernel(r["Kernel_Name"])
            if k is None:
                continue
            per[k][r["Counter_Name"]][(d, r["Dispatch_Id"])] = float(r["Counter_Value"])
    out = {}
    for k, cs in per.items():
        out[k] = {c: sum(v.values()) / len(v) for c, v in cs.items()}
        out[k]["_dispatches"] = max(len(v) for v in cs.values())
    return out


def derived(c: dict) -> dict:
    g = c.get
    d = {}
    if g("GRBM_GUI_ACTIVE"):
        cyc = g("GRBM_GUI_ACTIVE")
        if g("SQ_VALU_MFMA_BUSY_CYCLES") is not None:
            d["MFMA busy (of SIMD cycles)"] = g("SQ_VALU_MFMA_BUSY_CYCLES") / (cyc * SIMDS)
        if g("SQ_ACTIVE_INST_VALU") is not None:
            d["VALU issue busy (of SIMD cycles)"] = 4 * g("SQ_ACTIVE_INST_VALU") / (cyc * SIMDS)
    if g("SQ_WAVE_CYCLES"):
        for key in ("SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_LDS"):
            if g(key) is not None:
                d[f"{key} (of wave cycles)"] = 4 * g(key) / g("SQ_WAVE_CYCLES")
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
    for t in ("I8", "F8"):
        if g(f"SQ_INSTS_VALU_MFMA_MOPS_{t}") is not None:
            d[f"MFMA {t} ops"] = 512 * g(f"SQ_INSTS_VALU_MFMA_MOPS_{t}")
    return d


def table(dirs, kernels=("attn_fwd", "stats_and_q", "kv_quant", "delta_s")) -> str:
    data = load(dirs)
    lines = []
    for k in kernels:
        if k not in data:
            continue
        c = data[k]
        lines.append(f"### {k} ({int(c['_dispatches'])} dispatches averaged)\n")
        lines.append("| counter | per dispatch |")
        lines.append("|---|---|")
        for name in sorted(x for x in c if not x.startswith("_")):
            lines.append(f"| {name} | {c[name]:.6g} |")
        for name, v in derived(c).items():
            lines.append(f"| *{name}* | {v:.4g} |")
        lines.append("")
    return "\n".join(lines)


if __name__ == "__main__":
    print(table(sys.argv[1:]))
