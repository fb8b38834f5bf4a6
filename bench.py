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
              kernel sources, else null
  power       board power, shader clock and energy per launch, sampled
              through the SMI library over a loop of back-to-back launches
              of at least 2 s after the timed region (this run, this GPU);
              roofline.diagnostic_clock (sclk_ghz, peak_at_sclk, frac_at_sclk)
              comes from it and is diagnostic only: roofline.frac against the
              2.4 GHz peak is the figure compared with the target
  cpu_baseline the FP64 oracle timed on the host cores on a bounded sample
              of query rows of the same workload, in the same unit; the
              GPU/oracle deviation on those rows is reported beside it
  tile_sweep  (16K causal workload only) the deviation study on rows
              0..2047 of heads 0..3: max|dO|, mean|dO| and max|dLSE| against
              the FP64 oracle for every (Br, Bc) in {16, 32, 64, 128}^2 at
              three precisions (bf16 O, bf16 inputs with O left in fp32, fp32),
              non-ascending key-tile orders, and the materialised baseline
  baseline_attention  time of the materialised baseline (S, then A, in
              device memory) on the same workload, and the tiled kernel's
              speed-up over it
  n_curve     TFLOP/s and fraction of the bf16 peak at N = 1K..16K (16 heads,
              B = 16384/N, d = 64 and 128, causal and not)
  backward    (bf16 workloads) the backward pass (fa_bwd) on the same
              workload and forward outputs with a seeded N(0,1) dO: median
              launch time and TFLOP/s at 10*d FLOP per visible pair
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
KERNEL_SOURCES = ["fa_common.h", "fa_internal.h", "fa_bf16_tiles.h", "fa_fwd_bf16_pipe.hip",
                  "fa_fwd_flat.hip", "fa_fwd_f32.hip", "fa_study_kernel.h", "fa_fwd_bf16.hip"]


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


def sclk_fields(achieved, power, dtype):
    """The matrix-core peak at the shader clock measured in this run (the
    power loop's median over the XCDs), and the fraction of it reached,
    nested under "diagnostic_clock" so that it is not read as the figure
    compared with the target (that is roofline.frac, against the published
    2.4 GHz peak).  None when no clock reading exists."""
    ghz = power.get("gfx_clock_ghz") if power and dtype == "bf16" else None
    if not ghz:
        return {"diagnostic_clock": None}
    peak = BF16_FLOP_PER_CLK * ghz * 1e9 / 1e12
    return {"diagnostic_clock": {"sclk_ghz": round(ghz, 3), "peak_at_sclk": round(peak, 1),
                                 "frac_at_sclk": round(achieved / peak, 4),
                                 "note": "diagnostic only; roofline.frac is the figure compared with the target"}}


def _smi_handle(torch):
    """SMI handle of the GPU torch calls cuda:0 (matched by PCI bus), or the
    only GPU the SMI library sees."""
    import amdsmi
    amdsmi.amdsmi_init()
    handles = amdsmi.amdsmi_get_processor_handles()
    if not handles:
        raise RuntimeError("SMI sees no GPU")
    props = torch.cuda.get_device_properties(0)
    bus = getattr(props, "pci_bus_id", None)
    for h in handles:
        try:
            bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)
            if bus is not None and int(bdf.split(":")[1], 16) == int(bus):
                return amdsmi, h
        except Exception:
            pass
    if len(handles) == 1:
        return amdsmi, handles[0]
    raise RuntimeError(f"cannot match cuda:0 (bus {bus}) among {len(handles)} SMI GPUs")


def power_loop(torch, step, seconds=2.0, period=0.02):
    """Back-to-back launches for at least `seconds` while a thread samples the
    SMI metrics every `period` s: board power, the shader clock of each XCD,
    the power limit, throttle status and the energy counter.  Returns a dict
    (or {"error": ...} when the SMI library is unavailable)."""
    import threading
    try:
        amdsmi, h = _smi_handle(torch)
    except Exception as e:  # no SMI access: reported, never fatal
        return {"error": f"{type(e).__name__}: {e}"}
    samples = []
    stop = threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                clks = sorted(c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and c > 0)
                samples.append(dict(t=time.perf_counter(), power=m.get("current_socket_power"),
                                    clk=clks[len(clks) // 2] if clks else m.get("current_gfxclk"),
                                    clk_min=clks[0] if clks else None,
                                    throttle=m.get("throttle_status"),
                                    hotspot=m.get("temperature_hotspot")))
            except Exception:
                pass
            stop.wait(period)

    def energy():
        e = amdsmi.amdsmi_get_energy_count(h)
        return e["energy_accumulator"] * e["counter_resolution"] * 1e-6  # joules

    try:
        limit = amdsmi.amdsmi_get_power_info(h).get("power_limit")
        # Some amdsmi releases report this field in microwatts, others in
        # watts; no board draws 100 kW, so a larger figure is microwatts.
        if isinstance(limit, (int, float)) and limit > 1e5:
            limit = limit / 1e6
    except Exception:
        limit = None

    # Residency accumulators of the firmware's limiters (package power,
    # thermal, PROCHOT) and, per XCD, the time the shader clock sat below
    # the host's limit and why: their increase over the loop says which
    # limiter held the clock down.
    acc_keys = ("accumulation_counter", "ppt_residency_acc", "socket_thm_residency_acc", "vr_thm_residency_acc",
                "hbm_thm_residency_acc", "prochot_residency_acc", "xcp_stats.gfx_busy_acc",
                "xcp_stats.gfx_below_host_limit_acc", "xcp_stats.gfx_below_host_limit_ppt_acc",
                "xcp_stats.gfx_below_host_limit_thm_acc", "xcp_stats.gfx_below_host_limit_total_acc",
                "xcp_stats.gfx_low_utilization_acc")

    def flat_numbers(x):
        if isinstance(x, (int, float)):
            return [x]
        if isinstance(x, (list, tuple)):
            return [y for z in x for y in flat_numbers(z)]
        return []

    def accumulators():
        try:
            m = amdsmi.amdsmi_get_gpu_metrics_info(h)
        except Exception:
            return {}
        return {k: sum(flat_numbers(m.get(k))) for k in acc_keys if flat_numbers(m.get(k))}
    torch.cuda.synchronize()
    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    time.sleep(3 * period)
    a0 = accumulators()
    e0 = energy()
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(20):
            step()
        n += 20
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            break
    t1 = time.perf_counter()
    e1 = energy()
    a1 = accumulators()
    stop.set()
    th.join()
    busy = [x for x in samples if t0 + 0.1 <= x["t"] <= t1]
    num = lambda key: [x[key] for x in busy if isinstance(x[key], (int, float))]
    mean = lambda v: sum(v) / len(v) if v else None
    pw, clk, cmin = num("power"), num("clk"), num("clk_min")
    joules = e1 - e0
    out = {
        "loop_s": round(t1 - t0, 3), "launches": n, "samples": len(busy),
        "board_power_w_avg": round(mean(pw), 1) if pw else None,
        "board_power_w_max": max(pw) if pw else None,
        "power_limit_w": limit,
        # median over samples of each sample's median XCD clock (single
        # readings of an XCD between dispatches can be far below the rest)
        "gfx_clock_ghz": round(sorted(clk)[len(clk) // 2] / 1000.0, 4) if clk else None,
        "gfx_clock_ghz_min_xcd": round(min(cmin) / 1000.0, 4) if cmin else None,
        "energy_j_per_launch": round(joules / n, 6) if n else None,
        "avg_power_from_energy_w": round(joules / (t1 - t0), 1),
        "throttle_status_seen": sorted({x["throttle"] for x in busy if x["throttle"] not in (None, "N/A")}),
        "hotspot_c_max": max(num("hotspot")) if num("hotspot") else None,
        "limiter_accumulator_deltas": {k.replace("xcp_stats.", "xcd_sum."): a1[k] - a0[k] for k in a1 if k in a0},
    }
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:
        pass
    return out


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
    ap.add_argument("--power-seconds", type=float, default=2.0,
                    help="length of the SMI power/clock loop after the timed region (0 = skip)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the tile sweep and the sequence-length curve")
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

    power = power_loop(torch, step, args.power_seconds) if args.power_seconds > 0 else None

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
                     **sclk_fields(achieved, power, w.dtype),
                     "kernel_ms": round(kern_ms, 5),
                     "launch_ms_p10_p50_p90": [round(pct(10), 5), round(pct(50), 5), round(pct(90), 5)],
                     "algorithmic_bytes": algorithmic_bytes(w, inp)},
        "cpu_baseline": cpu,
        "max_abs_dO_sampled": dev_o,
        "max_abs_dLSE_sampled": dev_l,
        "power": power,
    }
    if not args.no_extras:
        if w.key == "long_causal":
            line["tile_sweep"] = deviation_study(torch, fa, "long_causal", 2048, 4)
        if w.dtype == "bf16":
            line["baseline_attention"] = baseline_speed(torch, fa, w, inp, kern_ms)
        line["n_curve"] = n_curve(torch, fa)
        if w.dtype == "bf16":
            line["backward"] = backward_speed(torch, fa, w, q, k, v, out, lse, kl, bm, scale, pairs)
    print(json.dumps(line), flush=True)


TILES = [(a, b) for a in (16, 32, 64, 128) for b in (16, 32, 64, 128)]


def deviation_study(torch, fa, key, N, H, orders=True):
    """The deviation study on a causal prefix of workload `key` (rows
    0..N-1 of heads 0..H-1, a self-contained causal problem): output and LSE
    deviation from the FP64 oracle for
      * the tiled kernels at every (Br, Bc) in {16, 32, 64, 128}^2, with bf16
        inputs and O rounded to bf16 ("bf16"), bf16 inputs and O left in fp32
        ("bf16_f32out"), the running output rounded to bf16 after every key
        tile ("bf16_acc16"), and fp32 inputs and arithmetic ("f32", the
        unrounded float32 draw), plus the tuned default and fp16 I/O;
      * key tiles visited last-first and shuffled (bf16_f32out);
      * the materialised baseline with S and A held in fp32 or in bf16, O in
        bf16 or fp32, and the fp32 baseline.
    Each row: [precision, kernel, Br, Bc, max|dO|, mean|dO|, max|dLSE|]."""
    import numpy as np
    import oracle
    from workloads import WORKLOADS, causal_prefix
    w = WORKLOADS[key]
    dev = torch.device("cuda:0")
    refs, dev_in = {}, {}
    for fmt in ("bf16", "f32", "f16"):
        inp = causal_prefix(w, N=N, H=H, fmt=fmt)
        refs[fmt] = oracle.attention_f64(inp["q"], inp["k"], inp["v"], float(inp["scale"]), True)
        tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[fmt]
        dev_in[fmt] = [torch.from_numpy(inp[n]).to(tdt).to(dev) for n in ("q", "k", "v")]
    scale = float(np.float32(1.0 / math.sqrt(w.d)))
    rows = []

    def add(prec, kernel, br, bc, o, lse, ref_fmt):
        torch.cuda.synchronize()
        o_ref, lse_ref = refs[ref_fmt]
        do = np.abs(o.double().cpu().numpy() - o_ref)
        dl = np.abs(lse.double().cpu().numpy() - lse_ref)
        rows.append([prec, kernel, br, bc, float("%.4g" % do.max()), float("%.4g" % do.mean()),
                     float("%.4g" % dl.max())])

    q, k, v = dev_in["bf16"]
    o, lse = fa.fwd(q, k, v, causal=True, scale=scale)
    add("bf16", "tuned", 128, 64, o, lse, "bf16")
    o32 = torch.empty(q.shape, dtype=torch.float32, device=dev)
    for br, bc in TILES:
        o, lse = fa.fwd(q, k, v, causal=True, scale=scale, Br=br, Bc=bc)
        add("bf16", "tiled", br, bc, o, lse, "bf16")
        o, lse = fa.fwd(q, k, v, causal=True, scale=scale, Br=br, Bc=bc, out=o32)
        add("bf16_f32out", "tiled", br, bc, o, lse, "bf16")
        o, lse = fa.fwd(q, k, v, causal=True, scale=scale, Br=br, Bc=bc, acc16=True)
        add("bf16_acc16", "tiled", br, bc, o, lse, "bf16")
    if orders:
        for name, order in (("tiled-desc", fa.ORDER_DESCENDING), ("tiled-shuffled", fa.ORDER_SHUFFLED)):
            for br, bc in ((16, 16), (128, 64)):
                o, lse = fa.fwd(q, k, v, causal=True, scale=scale, Br=br, Bc=bc, out=o32, tile_order=order)
                add("bf16_f32out", name, br, bc, o, lse, "bf16")
    for inter in ("f32", "io"):
        o, lse = fa.baseline(q, k, v, causal=True, scale=scale, inter=inter)
        add("bf16", "baseline-inter-" + ("f32" if inter == "f32" else "bf16"), 0, 0, o, lse, "bf16")
        o, lse = fa.baseline(q, k, v, causal=True, scale=scale, inter=inter, out=o32)
        add("bf16_f32out", "baseline-inter-" + ("f32" if inter == "f32" else "bf16"), 0, 0, o, lse, "bf16")
    q, k, v = dev_in["f16"]
    o, lse = fa.fwd(q, k, v, causal=True, scale=scale)
    add("f16", "tuned", 128, 64, o, lse, "f16")
    o, lse = fa.baseline(q, k, v, causal=True, scale=scale, inter="f32")
    add("f16", "baseline-inter-f32", 0, 0, o, lse, "f16")
    q, k, v = dev_in["f32"]
    for br, bc in TILES:
        o, lse = fa.fwd(q, k, v, causal=True, scale=scale, Br=br, Bc=bc)
        add("f32", "tiled", br, bc, o, lse, "f32")
    o, lse = fa.baseline(q, k, v, causal=True, scale=scale, inter="f32")
    add("f32", "baseline-inter-f32", 0, 0, o, lse, "f32")
    return {"slice": f"{key}: rows 0..{N - 1} of heads 0..{H - 1} (causal prefix, B={w.B} d={w.d})",
            "columns": ["precision", "kernel", "Br", "Bc", "max_dO", "mean_dO", "max_dLSE"], "rows": rows}


def baseline_speed(torch, fa, w, inp, fa_ms, launches=3):
    """Time of the materialised baseline (S and A in fp32, then in bf16) on
    the full workload, next to the tiled kernel's: the speed-up of the
    IO-aware method over the standard evaluation order."""
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(inp[n]).to(torch.bfloat16).to(dev) for n in ("q", "k", "v"))
    kl = torch.from_numpy(inp["key_len"]).to(dev) if inp["key_len"] is not None else None
    bm = torch.from_numpy(inp["block_mask"]).to(dev) if inp["block_mask"] is not None else None
    out = {}
    for inter, code in (("f32", fa.DTYPE_F32), ("bf16", fa.DTYPE_BF16)):
        need = fa.fa_fwd_baseline_workspace_size(w.B, w.H, w.N, fa.DTYPE_BF16, code)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)

        def call():
            fa.baseline(q, k, v, causal=w.causal, key_len=kl, block_mask=bm, scale=float(inp["scale"]),
                        inter="f32" if inter == "f32" else "io", workspace=ws)
        call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(launches):
            call()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / launches
        out[f"inter_{inter}"] = {"ms": round(ms, 3), "workspace_gb": round(need / 1e9, 2),
                                 "tiled_speedup": round(ms / fa_ms, 2)}
        del ws
    return out


def backward_speed(torch, fa, w, q, k, v, o, lse, kl, bm, scale, pairs, launches=10):
    """Median launch time of fa_bwd on the workload (its forward's O and LSE,
    dO drawn N(0,1) on the GPU from a seeded generator), and its rate at
    10*d FLOP per visible pair (five products of 2*d)."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 7)
    dout = torch.randn(q.shape, generator=g, device=dev).to(q.dtype)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)

    def call():
        fa.bwd(q, k, v, o, dout, lse, causal=w.causal, key_len=kl, block_mask=bm, scale=scale,
               dq=dq, dk=dk, dv=dv, delta=delta)
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    st = torch.cuda.current_stream()
    for e0, e1 in ev:
        e0.record(st)
        call()
        e1.record(st)
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)[launches // 2]
    tf = 10 * w.d * pairs / (ms * 1e-3) / 1e12
    del dout, dq, dk, dv, delta
    return {"us": round(ms * 1e3, 1), "tflops_10d": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "launches": launches}


def n_curve(torch, fa, launches=20):
    """Median-of-launches TFLOP/s at N = 1K..16K, 16 heads, B = 16384/N,
    d = 64 and 128, causal and not; N(0,1) bf16 inputs drawn on the GPU from
    a seeded generator (seed 2000 + log2 N)."""
    dev = torch.device("cuda:0")
    out = []
    for d in (64, 128):
        for N in (1024, 2048, 4096, 8192, 16384):
            B, H = 16384 // N, 16
            g = torch.Generator(device=dev)
            g.manual_seed(2000 + int(math.log2(N)))
            q, k, v = (torch.randn((B, H, N, d), generator=g, device=dev).to(torch.bfloat16) for _ in range(3))
            o = torch.empty_like(q)
            lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
            for causal in (False, True):
                for _ in range(5):
                    fa.fwd(q, k, v, causal=causal, out=o, lse=lse)
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(launches)]
                st = torch.cuda.current_stream()
                for e0, e1 in ev:
                    e0.record(st)
                    fa.fwd(q, k, v, causal=causal, out=o, lse=lse)
                    e1.record(st)
                torch.cuda.synchronize()
                ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)[launches // 2]
                pairs = B * H * (N * (N + 1) // 2 if causal else N * N)
                tf = 4 * d * pairs / (ms * 1e-3) / 1e12
                out.append({"N": N, "B": B, "d": d, "causal": causal, "us": round(ms * 1e3, 2),
                            "tflops": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4)})
            del q, k, v, o, lse
    return out


if __name__ == "__main__":
    main()
