"""How often the static P~ range codes a probability as zero, on the five workload shapes.

TEST INFRASTRUCTURE ONLY (oracle side): calls nothing but the oracle and the seeded input
generators.  Run `python -m oracle.p_range_stats` from the repository root.

For each workload (full size, seed 0) the oracle's prologue runs on single heads -- query head
0 and the last query head, with their kv heads, of the first sequence, plus the second
sequence for the two-sequence workload -- and p_quant_stats counts, over the first, middle and
last Q blocks of each sampled head, the unmasked (row, key) entries whose P~ = E4M3(p * P_r) is
zero although p > 0, those in the E4M3 subnormal range, what the per-block scale
max(P~) / P_r would have coded as zero instead, and the share of each row's exact softmax
weight that the zeroed entries carry (p_flushed_mass).
"""
from __future__ import annotations

import sys
import time

import numpy as np

from . import sage


def sampled_stats(name: str, seed: int = 0) -> dict:
    sys.path.insert(0, ".")
    from workloads import WORKLOADS, make_inputs
    w = WORKLOADS[name]
    q, k, v = make_inputs(w, seed=seed)
    tot: dict = {}
    batches = [0, 1] if w.B > 1 else [0]
    for b in batches:
        for h in (0, w.H - 1):
            hk = h // (w.H // w.Hkv)
            sl = lambda x, i: np.ascontiguousarray(x[b:b + 1, i:i + 1])
            pro = sage.prologue(sl(q, h), sl(k, hk), sl(v, hk), w.causal, w.qk_bits)
            for qb in sorted({0, pro.nqb // 2, pro.nqb - 1}):
                for key, val in sage.p_quant_stats(pro, 0, 0, qb).items():
                    tot[key] = tot.get(key, 0) + val
                fm = sage.p_flushed_mass(pro, 0, 0, qb)
                tot["mass_sum"] = tot.get("mass_sum", 0.0) + float(fm.sum())
                tot["mass_max"] = max(tot.get("mass_max", 0.0), float(fm.max()))
                tot["rows"] = tot.get("rows", 0) + fm.size
    return tot


def main() -> None:
    print("| workload | entries | P~ = 0 with p > 0 | P~ subnormal | zero under a per-block scale | "
          "(row, block) pairs with max p < 1 | softmax weight on zeroed entries, mean / max per row |")
    print("|---|---|---|---|---|---|---|")
    for name in ("tiny", "bench", "llm", "dit", "gqa"):
        t0 = time.perf_counter()
        s = sampled_stats(name)
        n = s["n"]
        print(f"| {name} | {n} | {s['zero_static']} ({100 * s['zero_static'] / n:.3f} %) | "
              f"{s['subnormal_static']} ({100 * s['subnormal_static'] / n:.3f} %) | "
              f"{s['zero_block_scale']} ({100 * s['zero_block_scale'] / n:.3f} %) | "
              f"{s['rows_blocks_below_one']} of {s['rows_blocks']} | "
              f"{s['mass_sum'] / s['rows']:.2e} / {s['mass_max']:.2e} |  ({time.perf_counter() - t0:.0f} s)",
              flush=True)


if __name__ == "__main__":
    main()
