"""Forward throughput over the sequence-length range N = 1K .. 16K.

The pages report the method's speed for sequence lengths from about one
thousand to sixteen thousand tokens (page "FlashAttention: Fast and
Memory-Efficient Exact Attention with IO-Awareness", ai-paper-library,
Results: GPT-2 at 1K, Long Range Arena at 1K-4K, Path-X at 16K).  This
report runs the bf16 forward on one fixed amount of work per point: H = 16
heads, B = 16384 / N sequences (so B*N = 16384 query rows per head), for
d in {64, 128}, with and without the causal mask; inputs i.i.d. N(0, 1)
rounded to bf16, seed 2000 + log2(N).

Per point: 10 warm-up launches, then 50 launches each bracketed by HIP
events on the launch stream; the median, 10th and 90th percentile launch
times, TFLOP/s at the median (FLOP = 4*d per visible pair) and its fraction
of the dense bf16 matrix-core peak.  64 seeded query rows per point are
checked against the FP64 oracle (max|dO| <= 2e-2, max|dLSE| <= 1e-3); the
script exits non-zero if any point misses that bar.

    python tests/n_sweep_report.py [--json PATH] [--quick]
"""
import argparse
import json
import math
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import io_aware_exact_03_amd as fa  # noqa: E402
import oracle  # noqa: E402
from workloads import random_qkv, allowed_pairs  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6
TOL_O, TOL_LSE = 2e-2, 1e-3


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--json", default=None)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--reps", type=int, default=50)
    ap.add_argument("--quick", action="store_true", help="N in {1K, 4K, 16K} only")
    args = ap.parse_args()
    ns = (1024, 4096, 16384) if args.quick else (1024, 2048, 4096, 8192, 16384)
    H = 16
    rows_out = []
    ok = True
    print("| d | causal | N | B | median us | p10 us | p90 us | TFLOP/s | % of peak | max abs dO | max abs dLSE |")
    print("|---|---|---|---|---|---|---|---|---|---|---|", flush=True)
    for d in (64, 128):
        for N in ns:
            B = 16384 // N
            seed = 2000 + int(math.log2(N))
            qf, kf, vf, _ = random_qkv(B, H, N, d, seed, "bf16")
            q, k, v = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in (qf, kf, vf))
            scale = float(np.float32(1.0 / math.sqrt(d)))
            out = torch.empty_like(q)
            lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
            for causal in (False, True):
                def call():
                    fa.fwd(q, k, v, causal=causal, scale=scale, out=out, lse=lse)
                for _ in range(args.warmup):
                    call()
                s = torch.cuda.current_stream()
                evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(args.reps)]
                for e0, e1 in evs:
                    e0.record(s)
                    call()
                    e1.record(s)
                torch.cuda.synchronize()
                us = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])
                med, p10, p90 = (float(np.percentile(us, p)) for p in (50, 10, 90))
                pairs = allowed_pairs(N, B, H, causal)
                tf = 4 * d * pairs / (med * 1e-6) / 1e12
                # parity on seeded sample rows
                rng = np.random.default_rng(seed)
                sample = np.sort(rng.choice(B * H * N, size=64, replace=False))
                o_ref, l_ref = oracle.attention_rows_f64(qf, kf, vf, sample, scale, causal)
                o_gpu = out.reshape(-1, d)[torch.from_numpy(sample).cuda()].double().cpu().numpy()
                l_gpu = lse.reshape(-1)[torch.from_numpy(sample).cuda()].double().cpu().numpy()
                d_o = float(np.abs(o_gpu - o_ref).max())
                d_l = float(np.abs(l_gpu - l_ref).max())
                good = d_o <= TOL_O and d_l <= TOL_LSE
                ok &= good
                r = dict(d=d, causal=causal, N=N, B=B, H=H, median_us=med, p10_us=p10, p90_us=p90,
                         tflops=tf, frac=tf / PEAK_BF16_TFLOPS, max_dO=d_o, max_dLSE=d_l, ok=good)
                rows_out.append(r)
                print(f"| {d} | {'yes' if causal else 'no'} | {N} | {B} | {med:.1f} | {p10:.1f} | {p90:.1f} | "
                      f"{tf:.1f} | {100 * tf / PEAK_BF16_TFLOPS:.1f} | {d_o:.2e} | {d_l:.2e}"
                      f"{'' if good else ' FAIL'} |", flush=True)
            del q, k, v, out, lse
    if args.json:
        with open(args.json, "w") as f:
            json.dump(rows_out, f, indent=1)
    sys.exit(0 if ok else 1)


if __name__ == "__main__":
    main()
