"""Grouped-query / multi-query attention: time and accuracy at full workload
shapes.

The page on FlashAttention-2 adoption (tcdigital.jp, section on the synergy
with MQA/GQA) says the method is combined with query heads that share
key/value heads.  This report runs the 16K causal shape (B1 H16 N16384 d128,
0.5*N(0,1)) and the block-sparse shape (B4 H16 N4096 d64, N(0,1), the
band + global 128x128 mask) with H_kv = 16 (multi-head), 4 (groups of four)
and 1 (multi-query).  Per point: forward and backward time per call (HIP
events on the launch stream, 10 timed calls after 3 warm-up calls), TFLOP/s
(forward 4*d, backward 10*d per visible pair), the backward also without
its split workspace, and max|dO| / max|dLSE| of the forward on 32 seeded
rows against the FP64 oracle.

    python tests/gqa_report.py [--json PATH]
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
from workloads import WORKLOADS, random_qkv, band_global_block_mask, allowed_pairs  # noqa: E402


def timed(call, reps):
    for _ in range(3):
        call()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        call()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--json", default=None)
    ap.add_argument("--reps", type=int, default=10)
    args = ap.parse_args()
    rows = []
    print("| shape | H_kv | fwd us | fwd TFLOP/s | bwd us | bwd TFLOP/s | bwd us, no workspace | workspace MiB "
          "| max abs dO | max abs dLSE |")
    print("|---|---|---|---|---|---|---|---|---|---|", flush=True)
    for key in ("long_causal", "block_sparse"):
        w = WORKLOADS[key]
        B, H, N, d = w.B, w.H, w.N, w.d
        bm = None
        for hkv in (16, 4, 1):
            rng = np.random.Generator(np.random.PCG64(3000 + hkv + d))
            q = random_qkv(B, H, N, d, 0, "bf16", w.amp, rng=rng)[0]
            _, k, v, rng = random_qkv(B, hkv, N, d, 0, "bf16", w.amp, rng=rng)
            if w.sparse_globals:
                nb = (N + 127) // 128
                bm = band_global_block_mask(nb, rng, w.sparse_globals)
            tq, tk, tv = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in (q, k, v))
            tdo = torch.from_numpy(rng.standard_normal(q.shape, dtype=np.float32)).to(torch.bfloat16).cuda()
            tbm = torch.from_numpy(bm).cuda() if bm is not None else None
            scale = float(np.float32(w.scale))
            o, lse = fa.fwd(tq, tk, tv, causal=w.causal, block_mask=tbm, scale=scale)
            grads = [torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv)]
            delta = torch.empty_like(lse)
            fwd_us = timed(lambda: fa.fwd(tq, tk, tv, causal=w.causal, block_mask=tbm, scale=scale,
                                          out=o, lse=lse), args.reps)
            need = fa.fa_bwd_workspace_size(B, H, hkv, N, d)
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
            bwd_us = timed(lambda: fa.bwd(tq, tk, tv, o, tdo, lse, causal=w.causal, block_mask=tbm,
                                          scale=scale, dq=grads[0], dk=grads[1], dv=grads[2],
                                          delta=delta, workspace=ws), args.reps)
            bwd_plain_us = timed(lambda: fa.bwd(tq, tk, tv, o, tdo, lse, causal=w.causal, block_mask=tbm,
                                                scale=scale, dq=grads[0], dk=grads[1], dv=grads[2],
                                                delta=delta, workspace=None), args.reps)
            pairs = allowed_pairs(N, B, H, w.causal, None, bm)
            sample = np.sort(rng.choice(B * H * N, size=32, replace=False))
            o_ref, l_ref = oracle.attention_rows_f64(q, k, v, sample, scale, w.causal, None, bm)
            idx = torch.from_numpy(sample).cuda()
            d_o = float(np.abs(o.reshape(-1, d)[idx].double().cpu().numpy() - o_ref).max())
            d_l = float(np.abs(lse.reshape(-1)[idx].double().cpu().numpy() - l_ref).max())
            r = dict(shape=key, H_kv=hkv, fwd_us=fwd_us, fwd_tflops=4 * d * pairs / (fwd_us * 1e-6) / 1e12,
                     bwd_us=bwd_us, bwd_tflops=10 * d * pairs / (bwd_us * 1e-6) / 1e12,
                     bwd_no_workspace_us=bwd_plain_us, workspace_bytes=need, max_dO=d_o, max_dLSE=d_l)
            rows.append(r)
            print(f"| {key} | {hkv} | {fwd_us:.1f} | {r['fwd_tflops']:.1f} | {bwd_us:.1f} | "
                  f"{r['bwd_tflops']:.1f} | {bwd_plain_us:.1f} | {need / 2**20:.0f} | {d_o:.2e} | {d_l:.2e} |",
                  flush=True)
            del tq, tk, tv, tdo, o, lse, grads, delta, ws
    if args.json:
        with open(args.json, "w") as f:
            json.dump(rows, f, indent=1)


if __name__ == "__main__":
    main()
