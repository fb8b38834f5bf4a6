#!/usr/bin/env python3
"""Benchmark of the gfx950 exact-attention forward (one GPU).

One step = one forward pass (fa_fwd) over the whole workload with inputs
already resident in device memory.  Default workload: 16K-token causal
attention, B=1, H=16, N=16384, d=128, bf16 inputs 0.5*N(0,1).

Prints ONE JSON line:
  value       algorithmic TFLOP/s over the timed steps (wall clock, after a
              device synchronise on both sides); FLOP = 4*d per visible
              (query, key) pair, masked pairs and softmax not counted
  roofline    the attention kernel's average launch time from HIP events on
              the launch stream, against the dense bf16 matrix-core peak
              (plus the 10th/50th/90th percentile of single launches, from a
              separate pass after the timed region);
              traffic = measured HBM bytes per launch from the committed
              rocprofv3 counter summary if it was taken on the current
              kernel sources, else null; likewise sclk_ghz, the shader clock
              the kernel ran at in that counter run (GPU-busy cycles per
              XCD over the dispatch time), with the matrix-core peak at that
              clock (256 CUs x sclk x 4096 FLOP/clk) and the fraction of it
  cpu_baseline the FP64 oracle timed on the host cores on a bounded sample
              of query rows of the same workload, in the same unit; the
              GPU/oracle deviation on those rows is reported beside it
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Dense bf16 matrix-core peak of MI355X: 256 CUs x 2.4 GHz x 4096 FLOP/clk/CU.
PEAK_BF16_TFLOPS = 2516.6
BF16_FLOP_PER_CLK = 256 * 4096
PEAK_F32_MFMA_TFLOPS = 157.3
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["fa_common.h", "fa_internal.h", "fa_bf16_tiles.h", "fa_fwd_bf16.hip",
                  "fa_fwd_bf16_pipe.hip", "fa_fwd_f32.hip"]


def kernel_source_hash():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "io_aware_exact_03_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _profiled(workload, key):
    """A figure of the committed counter summary for this workload, or None
    when it is missing or was taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    entry = t.get(workload)
    if not entry or entry.get("source_sha256") != kernel_source_hash():
        return None
    return entry.get(key)


def measured_traffic(workload):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)."""
    return _profiled(workload, "bytes_per_launch")


def measured_sclk(workload):
    """Shader clock (GHz) of the counter run: GRBM_GUI_ACTIVE / 8 XCDs over
    the dispatch time."""
    return _profiled(workload, "sclk_ghz")


def sclk_fields(achieved, workload, dtype):
    """The matrix-core peak at the profiled shader clock, and the fraction
    of it reached (bf16 only; None when no valid counter run exists)."""
    ghz = measured_sclk(workload) if dtype == "bf16" else None
    if not ghz:
        return {"sclk_ghz": None, "peak_at_sclk": None, "frac_at_sclk": None}
    peak = BF16_FLOP_PER_CLK * ghz * 1e9 / 1e12
    return {"sclk_ghz": round(ghz, 3), "peak_at_sclk": round(peak, 1), "frac_at_sclk": round(achieved / peak, 4)}


def algorithmic_bytes(w, inp):
    """Q read once, the visible K/V rows read once, O and LSE written once."""
    import numpy as np
    elem = 2 if w.dtype == "bf16" else 4
    B, H, N, d = w.B, w.H, w.N, w.d
    q_o = 2 * B * H * N * d * elem + B * H * N * 4
    if inp["key_len"] is not None:
        kv_rows = int(np.minimum(inp["key_len"], N).sum()) * H
    else:
        kv_rows = B * H * N
    return q_o + 2 * kv_rows * d * elem


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, inp, o_gpu, lse_gpu, seconds, seed):
    """Oracle on batches of sampled query rows until `seconds` have passed."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(seed)
    B, H, N, d = w.B, w.H, w.N, w.d
    total_rows = B * H * N
    order = rng.permutation(total_rows)
    kl = inp["key_len"]
    bm = inp["block_mask"]
    nb = (N + 127) // 128

    def visible(rows):
        bh, i = rows // N, rows % N
        b = bh // H
        cnt = np.full(rows.shape, N, dtype=np.int64)
        if kl is not None:
            cnt = np.minimum(cnt, kl[b].astype(np.int64))
        if w.causal:
            cnt = np.minimum(cnt, i + 1)
        if bm is not None:
            m = bm.reshape(nb, nb)
            c = np.zeros(rows.shape, dtype=np.int64)
            for kb in range(nb):
                lo = kb * 128
                hi = np.minimum((kb + 1) * 128, cnt)
                c += m[i // 128, kb].astype(np.int64) * np.maximum(0, hi - lo)
            cnt = c
        return cnt

    done, flop, elapsed = 0, 0, 0.0
    max_do, max_dlse = 0.0, 0.0
    batch = 64
    t_start = time.perf_counter()
    while done < total_rows and elapsed < seconds:
        rows = np.sort(order[done:done + batch])
        t0 = time.perf_counter()
        o_ref, lse_ref = oracle.attention_rows_f64(inp["q"], inp["k"], inp["v"], rows,
                                                   float(inp["scale"]), w.causal, kl, bm, 128)
        elapsed += time.perf_counter() - t0
        flop += int(4 * d * visible(rows).sum())
        fin = np.isfinite(lse_ref)
        og = o_gpu.reshape(-1, d)[rows]
        lg = lse_gpu.reshape(-1)[rows]
        if fin.any():
            max_do = max(max_do, float(np.abs(og[fin] - o_ref[fin]).max()))
            max_dlse = max(max_dlse, float(np.abs(lg[fin] - lse_ref[fin]).max()))
        done += rows.size
        if time.perf_counter() - t_start > 4 * seconds:
            break
        batch = min(4096, batch * 2)
    tflops = flop / elapsed / 1e12 if elapsed > 0 else None
    return dict(value=tflops, unit="TFLOP/s", cores=oracle.threads(), cpu_model=cpu_model(), kind="oracle",
                sample=f"{done} query rows of {total_rows} (uniform without replacement, seed "
                       f"{seed}), FP64 C oracle, {elapsed:.1f} s, {flop / 1e9:.2f} GFLOP "
                       f"algorithmic"), max_do, max_dlse, done


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long_causal")
    ap.add_argument("--br", type=int, default=0, help="query rows per tile (0 = tuned)")
    ap.add_argument("--bc", type=int, default=0, help="key rows per tile (0 = tuned)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="oracle time budget for the CPU baseline (0 = skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy (3 times), the known-size "
                         "reference that scales the FETCH_SIZE/WRITE_SIZE counters")
    args = ap.parse_args()

    if args.copy_calibration:
        import torch
        n = 512 << 20
        x = torch.ones(n, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3}))
        return

    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (--gpus {args.gpus} requested); "
              "the attention path shards over (batch, head) pairs with no communication",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import io_aware_exact_03_amd as fa
    from workloads import WORKLOADS, make_inputs, allowed_pairs

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(3)
    w = WORKLOADS[args.workload]
    inp = make_inputs(w)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(inp[n]).to(tdt).to(dev) for n in ("q", "k", "v"))
    kl = torch.from_numpy(inp["key_len"]).to(dev) if inp["key_len"] is not None else None
    bm = torch.from_numpy(inp["block_mask"]).to(dev) if inp["block_mask"] is not None else None
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    scale = float(inp["scale"])
    br, bc = fa.fa_tile_shape(0 if w.dtype == "bf16" else 1, w.d, inp["block_mask"] is not None,
                              args.br, args.bc)

    def step():
        fa.fwd(q, k, v, causal=w.causal, key_len=kl, block_mask=bm, scale=scale,
               Br=args.br, Bc=args.bc, out=out, lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / args.steps
    kern_ms = ev0.elapsed_time(ev1) / args.steps

    # Per-launch spread, measured after the timed region in a pass of its own
    # (one HIP event pair around each launch, on the launch stream).
    stream = torch.cuda.current_stream()
    spread = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(min(args.steps, 50))]
    for e0, e1 in spread:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    launch_ms = sorted(e0.elapsed_time(e1) for e0, e1 in spread)

    def pct(p):
        if not launch_ms:
            return float("nan")
        return launch_ms[min(len(launch_ms) - 1, int(round(p / 100 * (len(launch_ms) - 1))))]

    pairs = allowed_pairs(w.N, w.B, w.H, w.causal, inp["key_len"], inp["block_mask"])
    flop = 4 * w.d * pairs
    value = flop / (wall_ms * 1e-3) / 1e12
    achieved = flop / (kern_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS

    o_host = out.double().cpu().numpy()
    lse_host = lse.double().cpu().numpy()
    cpu = None
    dev_o = dev_l = None
    if args.cpu_seconds > 0:
        cpu, dev_o, dev_l, _ = cpu_baseline(w, inp, o_host, lse_host, args.cpu_seconds, seed=w.seed)

    line = {
        "metric": "attention fwd TFLOP/s (bf16)" if w.dtype == "bf16" else "attention fwd TFLOP/s (fp32)",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.key, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "key_padding": w.key_len_range is not None,
                   "block_sparse": w.sparse_globals > 0, "tile_br_bc": [br, bc],
                   "visible_pairs": pairs, "algorithmic_flop": flop,
                   "frac_of_bf16_peak": round(value / peak, 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(w.key),
                     **sclk_fields(achieved, w.key, w.dtype),
                     "kernel_ms": round(kern_ms, 5),
                     "launch_ms_p10_p50_p90": [round(pct(10), 5), round(pct(50), 5), round(pct(90), 5)],
                     "algorithmic_bytes": algorithmic_bytes(w, inp)},
        "cpu_baseline": cpu,
        "max_abs_dO_sampled": dev_o,
        "max_abs_dLSE_sampled": dev_l,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
