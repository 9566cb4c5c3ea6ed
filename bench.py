#!/usr/bin/env python3
"""Throughput of the routed MoE expert-FFN path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_fp8]

One step is one pass of the whole path over one batch of synthetic, seeded
inputs already resident in HBM (weights in the prepared layout, written once by
moe_prepare_weights before timing): routing plan (and top-k from logits where the
workload routes from logits), gate_up grouped GEMM with the fused clamped
SwiGLU and requantisation, down grouped GEMM, router-weighted combine — the
same kernels moe_forward launches, called through the C ABI's stage entry
points so that the two GEMM launches can carry HIP timing events (the timed
variants of the leg entry points) on the stream they run on.  K steps run back to back between two device synchronisations.

Prints one JSON line with tokens/s, the dominant kernel's roofline fraction
(from its live HIP-event duration) and the CPU oracle timed on a bounded sample
of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks
PEAK_HBM_GBS = 8000.0
# MX: the f8 x f4 MFMA runs at the FP8 rate; NVFP4 x BF16 decodes its weights to bf16 for the bf16 MFMA
PEAK_TFLOPS = {"fp8_block128": 5000.0, "bf16": 2500.0, "w4a8_mx": 5000.0, "nvfp4_w4a16": 2500.0}
DTYPE = {"fp8_block128": "fp8_e4m3", "bf16": "bf16", "w4a8_mx": "mxfp4xmxfp8", "nvfp4_w4a16": "nvfp4xbf16"}
COUNTERS = os.path.join(ROOT, "profiles", "gate_up_counters.json")
KERNEL_SOURCES = [os.path.join(ROOT, "mixture_experts_ffn_topk_amd", "csrc", f) for f in ("gemm.hip", "device.h", "prepare.hip")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def weight_bytes_per_expert(sh) -> tuple[int, int]:
    """Algorithmic bytes of one expert's (gate_up, down) weights + their scales."""
    H, I = sh.hidden, sh.inter
    if sh.fmt == "fp8_block128":
        return 2 * I * H + (2 * I // 128) * (H // 128) * 4, H * I + (H // 128) * (I // 128) * 4
    if sh.fmt == "bf16":
        return 2 * I * H * 2, H * I * 2
    if sh.fmt == "nvfp4_w4a16":  # E2M1 values, one E4M3 scale per 16, one fp32 global scale
        return 2 * I * H // 2 + 2 * I * (H // 16) + 4, H * I // 2 + H * (I // 16) + 4
    return 2 * I * H // 2 + 2 * I * (H // 32), H * I // 2 + H * (I // 32)


def act_bytes(sh) -> int:
    T, H = sh.tokens, sh.hidden
    if sh.fmt == "fp8_block128":
        return T * H + T * (H // 128) * 4
    if sh.fmt in ("bf16", "nvfp4_w4a16"):
        return T * H * 2
    return T * H + T * (H // 32)


def cpu_baseline(sh, inp, ids, w, budget_s: float) -> dict:
    """The CPU oracle (numpy fp64), timed on a bounded sample of the same workload:
    the experts in ascending order until the time budget is used, each over all of
    its routed rows, then scaled to the whole workload by the sampled share of pairs."""
    import numpy as np
    import oracle
    try:
        import threadpoolctl
        cores = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas")
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    geo = oracle.Geometry(sh.hidden, sh.inter, sh.experts, sh.topk, sh.fmt, sh.clamp)
    t0 = time.perf_counter()
    plan = oracle.build_plan(ids, sh.experts)
    xd = oracle.dequant_activations(geo, inp["x"], inp["x_sf"])
    start, src = plan["expert_start_indices"], plan["src_info"]
    done_rows, n_exp = 0, 0
    for e in range(sh.experts):
        r0, r1 = int(start[e]), int(start[e + 1])
        if r1 == r0:
            continue
        w13d, w2d = oracle.dequant_expert(geo, inp["w13"], inp["w13_sf"], inp["w2"], inp["w2_sf"], e,
                                          inp.get("w13_gs"), inp.get("w2_gs"))
        oracle.expert_rows(geo, xd[src[r0:r1] // sh.topk], w13d, w2d)
        done_rows += r1 - r0
        n_exp += 1
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    total = int(start[-1])
    tok_s = sh.tokens * (done_rows / total) / el
    return {"value": round(tok_s, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"fp64 numpy oracle over experts in id order until {budget_s:.0f}s: {n_exp} experts, "
                      f"{done_rows} of {total} routed rows ({el:.1f}s), scaled by the row share; "
                      f"BLAS threads={cores}, dequantisation single-threaded"}


def write_counters(workload: str, fetch_dir: str, write_dir: str, command: str) -> int:
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE,
    both with --copy-calibration) into profiles/gate_up_counters.json: the gate_up
    kernel's HBM bytes per launch, each counter scaled by what it reads for the
    plain 1 GiB elementwise copy of the same run."""
    import csv
    import glob

    def rows(d, counter):
        out = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter:
                    out.append((r["Kernel_Name"], float(r["Counter_Value"])))
        return out

    def gate_up(vals):
        v = [x for n, x in vals if "ffn_gemm_kernel" in n and ", true, " in n.split(">")[0]]
        return sum(v) / len(v)

    def copy_kb(vals, want_kb):
        v = [x for n, x in vals if "elementwise_kernel" in n and x > 0.25 * want_kb]
        return sum(v) / len(v)

    gib_kb = float(1 << 20)
    fetch, write = rows(fetch_dir, "FETCH_SIZE"), rows(write_dir, "WRITE_SIZE")
    f_kb, w_kb = gate_up(fetch), gate_up(write)
    f_factor, w_factor = gib_kb / copy_kb(fetch, gib_kb), gib_kb / copy_kb(write, gib_kb)
    traffic = (f_kb * f_factor + w_kb * w_factor) * 1024.0
    out = {"workload": workload, "kernel_source_sha": kernel_source_hash(), "kernel": "ffn_gemm_kernel gate_up",
           "fetch_kb_per_launch": f_kb, "write_kb_per_launch": w_kb, "fetch_copy_factor": f_factor,
           "write_copy_factor": w_factor, "traffic_bytes_per_launch": round(traffic), "command": command}
    with open(COUNTERS, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the first few dozen steps after start-up run several percent slower (measured: the
    # decode step 0.263 ms over steps 6-55, 0.246-0.248 ms from then on), so the
    # default warm-up reaches the steady state
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="decode_fp8")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of CPU oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--write-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/gate_up_counters.json from two rocprofv3 --pmc output folders and exit")
    ap.add_argument("--counters-command", default="", help="the command the --pmc runs used (recorded)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for HBM counter calibration under rocprofv3)")
    args = ap.parse_args()
    if args.write_counters:
        return write_counters(args.workload, args.write_counters[0], args.write_counters[1], args.counters_command)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode (the expert-parallel exchange is "
              "outside it); run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import moe_synth
    from mixture_experts_ffn_topk_amd import MoEFFN

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    sh = moe_synth.WORKLOADS[args.workload]
    log(f"workload {sh.name}: generating seeded inputs")
    inp = moe_synth.make_inputs(sh)
    T, k, E, H, I = sh.tokens, sh.topk, sh.experts, sh.hidden, sh.inter

    def dev(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).cuda()

    x, x_sf = dev(inp["x"]), dev(inp["x_sf"])
    weights = {"w13": dev(inp["w13"]), "w13_sf": dev(inp["w13_sf"]), "w2": dev(inp["w2"]), "w2_sf": dev(inp["w2_sf"]),
               "w13_gs": dev(inp.get("w13_gs")), "w2_gs": dev(inp.get("w2_gs"))}
    logits = dev(inp["logits"])
    if sh.routing == "precomputed":
        topk_idx, topk_w = dev(inp["topk_idx"]), dev(inp["topk_weights"])
    else:
        topk_idx = torch.empty((T, k), dtype=torch.int64, device="cuda")
        topk_w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe = MoEFFN(H, I, E, k, T, fmt=sh.fmt, route_mode=sh.routing, activation_clamp=sh.clamp)
    # one-time weight relayout (the pages' pre-permuted weights); outside the timed region
    canonical = weights
    weights = moe.prepare_weights(canonical)
    torch.cuda.synchronize()
    del canonical
    plan = moe.alloc_plan(T)
    ws = moe.alloc_workspace(T)
    h, hsf = moe.alloc_intermediate(T)
    y = torch.empty((T * k, H), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    # Per-kernel durations come from HIP events that the two GEMM legs' kernel
    # launches carry themselves (moe_ffn_gate_up_timed / moe_ffn_down_timed), in a
    # sample of the timed steps (every stride-th step): the events hold each
    # kernel's own start and end, with no marker commands between the kernels.
    # torch creates an event at its first record, done here, before the timing.
    stride = max(1, args.steps // 10)
    sampled = list(range(0, args.steps, stride))
    ev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(4)] for i in sampled}
    for e4 in ev.values():
        for e in e4:
            e.record(stream)

    def step(e=None):
        if sh.routing == "precomputed":
            moe.plan(T, plan, topk_idx=topk_idx, ws=ws, stream=stream)
        else:
            moe.plan(T, plan, routing_logits=logits, topk_idx_out=topk_idx, topk_weights_out=topk_w, ws=ws,
                     stream=stream)
        moe.ffn_gate_up(T, x, x_sf, weights, plan, h, hsf, stream=stream, events=None if e is None else e[:2])
        moe.ffn_down(T, h, hsf, weights, plan, y, stream=stream, events=None if e is None else e[2:])
        moe.combine(T, y, topk_w, plan, out, stream=stream)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    counts = plan["expert_counts"].cpu().numpy()
    active = int((counts > 0).sum())
    pairs = int(counts.sum())

    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev.get(i))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gate_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev.values()]))
    down_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev.values()]))

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1)
        for _ in range(3):
            torch.add(a, 0, out=b)  # a plain elementwise copy: reads and writes 1 GiB
        torch.cuda.synchronize()
        del a, b

    # ---------------------------------------------------------------- roofline of the dominant kernel (gate_up)
    wb_gu, wb_dn = weight_bytes_per_expert(sh)
    gu_bytes = active * wb_gu + act_bytes(sh)
    dn_bytes = active * wb_dn
    gu_flops = 4.0 * pairs * H * I
    dn_flops = 2.0 * pairs * H * I
    peak_f = PEAK_TFLOPS[sh.fmt]
    t_mem, t_mma = gu_bytes / (PEAK_HBM_GBS * 1e9), gu_flops / (peak_f * 1e12)
    bound = "hbm" if t_mem >= t_mma else "mfma"
    if bound == "hbm":
        achieved, peak, unit = gu_bytes / (gate_ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        achieved, peak, unit = gu_flops / (gate_ms * 1e-3) / 1e12, peak_f, "TFLOP/s"
    traffic = None
    if os.path.exists(COUNTERS):
        try:
            c = json.load(open(COUNTERS))
            if c.get("workload") == sh.name and c.get("kernel_source_sha") == kernel_source_hash():
                traffic = c["traffic_bytes_per_launch"]
        except Exception:
            traffic = None
    roofline = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic,
                "kernel": "ffn_gemm_kernel gate_up (FFN leg 1)",
                "algorithmic_bytes": gu_bytes, "algorithmic_flops": gu_flops, "avg_launch_ms": round(gate_ms, 4),
                "event_timed_steps": len(ev),
                "down_leg": {"avg_launch_ms": round(down_ms, 4),
                             "hbm_frac": round(dn_bytes / (down_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                             "mfma_frac": round(dn_flops / (down_ms * 1e-3) / 1e12 / peak_f, 4)}}

    ms_per_step = elapsed * 1e3 / args.steps
    tok_s = T * args.steps / elapsed
    total_bytes = active * (wb_gu + wb_dn) + act_bytes(sh) + T * H * 2 + T * k * 8
    result = {
        "metric": "MoE FFN tokens/s + achieved TFLOP/s & HBM GB/s vs MI355X peak",
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": DTYPE[sh.fmt], "data": "synthetic",
        "config": {"workload": sh.name, "tokens": T, "hidden": H, "intermediate": I, "experts": E, "topk": k,
                   "format": sh.fmt, "routing": sh.routing, "active_experts": active, "routed_pairs": pairs,
                   "parallelism": "single GPU"},
        "step_tflops": round((gu_flops + dn_flops) / (ms_per_step * 1e-3) / 1e12, 2),
        "step_hbm_gbs": round(total_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a bounded sample)")
        ids = inp["topk_idx"] if sh.routing == "precomputed" else topk_idx.cpu().numpy()
        w = inp["topk_weights"] if sh.routing == "precomputed" else topk_w.cpu().numpy()
        result["cpu_baseline"] = cpu_baseline(sh, inp, ids, w, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
