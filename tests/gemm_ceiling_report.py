"""Reference ceiling: the sustained rate of a plain bf16 GEMM (torch.matmul,
served by the ROCm GEMM library) on this GPU, on N(0,1) inputs and on
all-zero inputs, over loops of a few seconds.

Context for the attention kernels' fraction of the bf16 matrix-core peak:
under the board's power limit the clock depends on the data in the matrix
cores, so a dense GEMM on random data does not reach the 2516.6 TFLOP/s
dense peak either.  Nothing here is part of the attention path.

    python tests/gemm_ceiling_report.py [--seconds S]
"""
import argparse
import time

import torch

PEAK_BF16_TFLOPS = 2516.6


def run(M, N, K, kind, seconds):
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    if kind == "randn":
        a = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
        b = torch.randn((K, N), generator=g, device=dev).to(torch.bfloat16)
    else:
        a = torch.zeros((M, K), device=dev, dtype=torch.bfloat16)
        b = torch.zeros((K, N), device=dev, dtype=torch.bfloat16)
    c = torch.empty((M, N), device=dev, dtype=torch.bfloat16)
    for _ in range(5):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    n = 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            torch.matmul(a, b, out=c)
        n += 10
        torch.cuda.synchronize()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    tf = 2 * M * N * K / (ms * 1e-3) / 1e12
    print(f"GEMM {M}x{N}x{K} {kind:6} {ms * 1e3:9.1f} us/call  {tf:7.1f} TFLOP/s  "
          f"{tf / PEAK_BF16_TFLOPS:.3f} of {PEAK_BF16_TFLOPS}", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--seconds", type=float, default=3.0)
    args = ap.parse_args()
    for shape in ((8192, 8192, 8192), (16384, 16384, 8192)):
        run(*shape, "randn", args.seconds)
        run(*shape, "zeros", args.seconds)


if __name__ == "__main__":
    main()
