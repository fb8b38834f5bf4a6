"""Key-range split of the forward (fa_fwd_ws) on grids too small for the GPU.

A head-sharded problem leaves each GPU few heads (the 16K causal workload
on 8 GPUs is B1 H2 N16384 per GPU), and a long single sequence is one head.
With few query tiles the longest causal tile runs alone at the end.  The
split shares each query tile's key tiles over several workgroups and merges
the fp32 partial results by their log-sum-exp: the partial softmax
statistics that the method accumulates tile by tile (page "Ch.04 Attention
optimisation: FlashAttention and sparse attention", mdooai.com, "Key points
of the formulas"), here combined across workgroups instead of within one.

Per shape: unsplit and split runs alternate (A B A B ..., 5 rounds of 10
launches each, after warm-up) so that clock drift does not favour either;
reported: mean time per launch, TFLOP/s (4*d per visible pair), the
workspace size, and max|dO| between the two outputs.

    python tests/split_report.py [--json PATH]
"""
import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import io_aware_exact_03_amd as fa  # noqa: E402
from workloads import random_qkv  # noqa: E402

SHAPES = [(1, 2, 16384, 128, True), (1, 1, 32768, 128, True), (1, 2, 16384, 64, False),
          (1, 1, 65536, 128, True), (2, 2, 8192, 128, True), (1, 4, 16384, 128, True)]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--json", default=None)
    ap.add_argument("--rounds", type=int, default=5)
    ap.add_argument("--reps", type=int, default=10)
    args = ap.parse_args()
    rows = []
    print("| shape | unsplit us | unsplit TFLOP/s | split us | split TFLOP/s | speed-up | workspace MiB | max abs dO split vs unsplit |")
    print("|---|---|---|---|---|---|---|---|", flush=True)
    for B, H, N, d, causal in SHAPES:
        q, k, v, _ = random_qkv(B, H, N, d, 7, "bf16", 0.5)
        tq, tk, tv = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in (q, k, v))
        need = fa.fa_fwd_workspace_size(B, H, N, d, fa.DTYPE_BF16)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        o1, l1 = fa.fwd(tq, tk, tv, causal=causal)
        o2, l2 = fa.fwd(tq, tk, tv, causal=causal, workspace=ws)
        torch.cuda.synchronize()
        diff = float((o1.float() - o2.float()).abs().max())
        times = {None: [], "ws": []}
        for _ in range(3):
            fa.fwd(tq, tk, tv, causal=causal, out=o1, lse=l1)
            fa.fwd(tq, tk, tv, causal=causal, out=o2, lse=l2, workspace=ws)
        s = torch.cuda.current_stream()
        for _ in range(args.rounds):
            for key in (None, "ws"):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(s)
                for _ in range(args.reps):
                    if key is None:
                        fa.fwd(tq, tk, tv, causal=causal, out=o1, lse=l1)
                    else:
                        fa.fwd(tq, tk, tv, causal=causal, out=o2, lse=l2, workspace=ws)
                e1.record(s)
                torch.cuda.synchronize()
                times[key].append(e0.elapsed_time(e1) * 1e3 / args.reps)
        pairs = B * H * N * (N + 1) // 2 if causal else B * H * N * N
        tu, ts = float(np.mean(times[None])), float(np.mean(times["ws"]))
        r = dict(B=B, H=H, N=N, d=d, causal=causal, unsplit_us=tu, split_us=ts,
                 unsplit_tflops=4 * d * pairs / (tu * 1e-6) / 1e12, split_tflops=4 * d * pairs / (ts * 1e-6) / 1e12,
                 workspace_bytes=need, max_dO_split_vs_unsplit=diff)
        rows.append(r)
        print(f"| B{B} H{H} N{N} d{d} {'causal' if causal else 'dense'} | {tu:.1f} | {r['unsplit_tflops']:.1f} | "
              f"{ts:.1f} | {r['split_tflops']:.1f} | {tu / ts:.2f} | {need / 2**20:.0f} | {diff:.2e} |", flush=True)
        del tq, tk, tv, ws, o1, o2, l1, l2
    if args.json:
        with open(args.json, "w") as f:
            json.dump(rows, f, indent=1)


if __name__ == "__main__":
    main()
