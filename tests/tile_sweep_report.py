"""Deviation study on causal prefix slices of two workloads (report only).

The page "Is Flash Attention Stable?" explainer (aibr.jp, sections 3 and 4)
compares the output of the tiled method with an FP64 golden value while the
block sizes Br and Bc and the tile order vary, and sets it next to a
Baseline Attention computed in the conventional order (about ten times less
deviation at BF16 in its measurements).  This script runs that study here:
every (Br, Bc) in {16, 32, 64, 128}^2 at three precisions (bf16 inputs with
O rounded to bf16; bf16 inputs with O left in fp32; fp32), descending and
shuffled tile orders, fp16 I/O, and the materialised baseline (fa_fwd_baseline)
with S and A held in fp32 or in bf16, each against the FP64 oracle.  The
slices are rows 0..2047 of heads 0..3 of the 16K causal workload and rows
0..1023 of heads 0..3 of the GPT-2-sized causal workload; under the causal
mask each is a self-contained problem.  It prints one table per slice and
the FlashAttention / baseline deviation ratios.  Values are reported, not
asserted (the per-point bars are asserted by the GPU parity tests).

    python tests/tile_sweep_report.py [--json PATH]
"""
import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import io_aware_exact_03_amd as fa  # noqa: E402
from bench import deviation_study  # noqa: E402

SLICES = [("long_causal", 2048, 4), ("gpt2_causal", 1024, 4)]


def ratios(rows):
    """max and mean |dO| of the tiled kernel at the default tile over the
    baseline's, per precision and baseline intermediate type."""
    by = {(r[0], r[1], r[2], r[3]): r for r in rows}
    out = []
    for prec in ("bf16", "bf16_f32out", "f16", "f32"):
        fa_row = by.get((prec, "tuned", 128, 64)) or by.get((prec, "tiled", 128, 64)) or by.get((prec, "tiled", 128, 32))
        for inter in ("f32", "bf16"):
            base = by.get((prec, "baseline-inter-" + inter, 0, 0))
            if fa_row and base:
                out.append([prec, inter, fa_row[4] / base[4], fa_row[5] / base[5]])
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--json", default=None)
    args = ap.parse_args()
    result = {}
    for key, N, H in SLICES:
        study = deviation_study(torch, fa, key, N, H)
        study["ratios"] = ratios(study["rows"])
        result[key] = study
        print(f"\n{study['slice']}")
        print(f"{'precision':<12} {'kernel':<22} {'Br':>4} {'Bc':>4} {'max|dO|':>10} {'mean|dO|':>10} {'max|dLSE|':>10}")
        for r in study["rows"]:
            print(f"{r[0]:<12} {r[1]:<22} {r[2]:>4} {r[3]:>4} {r[4]:>10.3e} {r[5]:>10.3e} {r[6]:>10.3e}")
        print("tiled / baseline deviation (max, mean):")
        for p, inter, rmax, rmean in study["ratios"]:
            print(f"  {p:<12} baseline S,A in {inter:<5}: {rmax:7.3f} {rmean:7.3f}")
    if args.json:
        with open(args.json, "w") as f:
            json.dump(result, f, indent=1)


if __name__ == "__main__":
    main()
