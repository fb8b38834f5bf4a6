"""Backward-pass report: accuracy on the 16K causal workload's prefix slice
against the FP64 backward oracle (bf16 and fp16 I/O), and time / TFLOP/s of
the backward on the full bf16 workloads and, with fp16 I/O, on the 16K causal
and block-sparse workloads.

FLOP convention: 10*d per visible (query, key) pair -- five products of 2*d
(the recomputed scores, dP, dV, dK, dQ), the count a method that does not
store the probabilities cannot avoid.  The kernels here execute seven (the dQ
kernel recomputes the scores and dP), 14*d per pair.

    python tests/bwd_report.py [--json PATH]
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
import oracle  # noqa: E402
from workloads import WORKLOADS, ORDER, make_inputs, causal_prefix, allowed_pairs  # noqa: E402


def dev(x, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype).cuda()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--json", default=None)
    ap.add_argument("--reps", type=int, default=10)
    args = ap.parse_args()
    out = {}
    # accuracy on the causal prefix slice
    w = WORKLOADS["long_causal"]
    for fmt, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        inp = causal_prefix(w, N=2048, H=4, fmt=fmt)
        rng = np.random.default_rng(2024)
        dout = rng.standard_normal(inp["q"].shape).astype(np.float32)
        tq, tk, tv = dev(inp["q"], tdt), dev(inp["k"], tdt), dev(inp["v"], tdt)
        tdo = dev(dout, tdt)
        o, lse = fa.fwd(tq, tk, tv, causal=True)
        dq, dk, dv = fa.bwd(tq, tk, tv, o, tdo, lse, causal=True, workspace=None)
        torch.cuda.synchronize()
        ref = oracle.attention_bwd_f64(inp["q"], inp["k"], inp["v"], tdo.float().cpu().numpy(),
                                       float(inp["scale"]), True)
        acc = {}
        for name, g, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
            e = np.abs(g.double().cpu().numpy() - r)
            acc[name] = dict(max_abs_err=float(e.max()), mean_abs_err=float(e.mean()),
                             max_abs_ref=float(np.abs(r).max()))
        out[f"accuracy_long_causal_prefix_{fmt}"] = acc
        print(f"accuracy, {fmt} (B1 H4 N2048 d128 causal prefix of the 16K workload):")
        for k_, v_ in acc.items():
            print(f"  {k_}: max|err| {v_['max_abs_err']:.3e}  mean|err| {v_['mean_abs_err']:.3e}  "
                  f"max|ref| {v_['max_abs_ref']:.3e}", flush=True)
    # timing on the full bf16 workloads
    timing = {}
    runs = [(key, torch.bfloat16) for key in ORDER if WORKLOADS[key].dtype == "bf16"]
    runs += [("long_causal", torch.float16), ("block_sparse", torch.float16)]
    for key, tdt in runs:
        w = WORKLOADS[key]
        inp = make_inputs(w)
        tq, tk, tv = dev(inp["q"], tdt), dev(inp["k"], tdt), dev(inp["v"], tdt)
        tdo = dev(np.random.default_rng(1).standard_normal(inp["q"].shape).astype(np.float32), tdt)
        kl = torch.from_numpy(inp["key_len"]).cuda() if inp["key_len"] is not None else None
        bm = torch.from_numpy(inp["block_mask"]).cuda() if inp["block_mask"] is not None else None
        o, lse = fa.fwd(tq, tk, tv, causal=w.causal, key_len=kl, block_mask=bm)
        grads = [torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv)]
        delta = torch.empty_like(lse)

        def call():
            fa.bwd(tq, tk, tv, o, tdo, lse, causal=w.causal, key_len=kl, block_mask=bm,
                   dq=grads[0], dk=grads[1], dv=grads[2], delta=delta)
        for _ in range(3):
            call()
        s = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(args.reps):
            call()
        e1.record(s)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.reps
        pairs = allowed_pairs(w.N, w.B, w.H, w.causal, inp["key_len"], inp["block_mask"])
        tf = 10 * w.d * pairs / (ms * 1e-3) / 1e12
        tag = "bf16" if tdt == torch.bfloat16 else "f16"
        timing[f"{key}_{tag}"] = dict(ms=ms, tflops_10d=tf, tflops_executed_14d=tf * 1.4)
        print(f"  {key:14s} {tag:4s} bwd {ms * 1e3:9.1f} us   {tf:7.1f} TFLOP/s (10d/pair)", flush=True)
    out["timing"] = timing
    if args.json:
        with open(args.json, "w") as f:
            json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
