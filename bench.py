#!/usr/bin/env python3
"""Throughput of the routed MoE expert-FFN path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill_fp8_zipf]

One step is one pass of the whole path over one batch of synthetic, seeded
inputs already resident in HBM (weights in the prepared layout, written once by
moe_prepare_weights before timing): routing plan (and top-k from logits where the
workload routes from logits), gate_up grouped GEMM with the fused clamped
SwiGLU and requantisation, down grouped GEMM, router-weighted combine — the
same kernels moe_forward launches, called through the C ABI's stage entry
points so that the two GEMM launches can carry HIP timing events (the timed
variants of the leg entry points) on the stream they run on.

The timed workload (default: the prefill shape, T = 8192, the largest one-GPU
configuration) runs W warm-up steps, then exactly K steps back to back between
two device synchronisations: `value` is T * K / that wall time.  Then K more
steps with an event pair around each give the median and minimum step time.  A
weight-bound workload also reads a 512 MB scrub buffer before each of K further
steps, outside the step's events, so that no weight byte stays in the
memory-side cache between steps.

The weight-bound decode shape is measured beside it in the same run (the
`decode` object), right after the timed workload's steps: its own W
warm-up steps, K steps back to back, K steps with the scrub between them
(median and minimum), then 100 steps with per-step events (the start-up
transient, in means of 5) and K steps back to back once more (`settled`).

Prints one JSON line with tokens/s, the dominant kernel's roofline fraction
(from its live HIP-event duration), whole-step roofline fractions, and the CPU
oracle timed on a bounded sample of the same workload.
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
# NVFP4 x NVFP4 decodes both operands to bf16 (exactly) for the bf16 MFMA
PEAK_TFLOPS = {"fp8_block128": 5000.0, "bf16": 2500.0, "w4a8_mx": 5000.0, "nvfp4_w4a16": 2500.0, "nvfp4": 2500.0}
DTYPE = {"fp8_block128": "fp8_e4m3", "bf16": "bf16", "w4a8_mx": "mxfp4xmxfp8", "nvfp4_w4a16": "nvfp4xbf16",
         "nvfp4": "nvfp4xnvfp4"}
COUNTERS = os.path.join(ROOT, "profiles", "gate_up_counters.json")
KERNEL_SOURCES = [os.path.join(ROOT, "mixture_experts_ffn_topk_amd", "csrc", f) for f in ("gemm.hip", "gemm_common.h", "device.h", "launch.h", "prepare.hip")]


def _code_only(text: str) -> str:
    """C/C++ source with comments and whitespace runs removed: what the compiler sees
    of it, so that an edit of a comment does not count as a kernel change."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
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
    if sh.fmt == "nvfp4":  # as above, plus the intermediate's per-expert scale
        return 2 * I * H // 2 + 2 * I * (H // 16) + 8, H * I // 2 + H * (I // 16) + 4
    return 2 * I * H // 2 + 2 * I * (H // 32), H * I // 2 + H * (I // 32)


def act_bytes(sh) -> int:
    T, H = sh.tokens, sh.hidden
    if sh.fmt == "fp8_block128":
        return T * H + T * (H // 128) * 4
    if sh.fmt in ("bf16", "nvfp4_w4a16"):
        return T * H * 2
    if sh.fmt == "nvfp4":
        return T * H // 2 + T * (H // 16)
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
        oracle.expert_rows(geo, xd[src[r0:r1] // sh.topk], w13d, w2d,
                           None if "c_scales" not in inp else float(inp["c_scales"][e]))
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
    both with --copy-calibration) into the workload's entry of profiles/gate_up_counters.json:
    the gate_up kernel's HBM bytes per launch, each counter scaled by what it reads for the
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
    table = {}
    if os.path.exists(COUNTERS):
        try:
            table = json.load(open(COUNTERS)).get("workloads", {})
        except (ValueError, AttributeError):
            table = {}
    table[workload] = out
    with open(COUNTERS, "w") as fh:
        json.dump({"workloads": table}, fh, indent=1)
    print(json.dumps(out))
    return 0


def counter_summary(workload: str, out_md: str, dirs: list, command: str) -> int:
    """Summarise rocprofv3 --pmc runs of this script (one folder per pass) into a
    markdown table per kernel of the step: each counter's mean per launch, and the
    derived figures -- MFMA busy fraction and effective clock (SQ_VALU_MFMA_BUSY_CYCLES,
    GRBM_GUI_ACTIVE and the launches' own timestamps), issued MFMA work against the
    algorithmic flops, HBM bytes from FETCH_SIZE / WRITE_SIZE scaled by what they
    read for the plain 1 GiB copy (--copy-calibration), and the L2 hit rate."""
    import csv
    import glob

    import numpy as np

    import moe_synth
    sh = moe_synth.WORKLOADS[workload]
    inp = moe_synth.make_inputs(sh, with_weights=False)
    ids = np.asarray(inp["topk_idx"]).reshape(-1) if "topk_idx" in inp else None
    if ids is None:  # from-logits routing: the same top-k the kernel takes (ties to the lower index)
        ids = np.argsort(-inp["logits"], axis=1, kind="stable")[:, :sh.topk].reshape(-1)
    cnt = np.bincount(ids[(ids >= 0) & (ids < sh.experts)], minlength=sh.experts)
    active, pairs = int((cnt > 0).sum()), int(cnt.sum())
    wb_gu, wb_dn = weight_bytes_per_expert(sh)
    algo = {"gate_up": (4.0 * pairs * sh.hidden * sh.inter, active * wb_gu + act_bytes(sh)),
            "down": (2.0 * pairs * sh.hidden * sh.inter, active * wb_dn)}

    def kind(name):
        if "ffn_gemm_kernel" in name:
            return "gate_up" if ", true, " in name.split(">")[0] else "down"
        for k in ("combine", "plan_", "route_"):
            if k in name:
                return k.strip("_")
        if "elementwise_kernel" in name:
            return "copy"
        return None

    vals, durs, per_launch = {}, {}, {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                k = kind(r["Kernel_Name"])
                if k is None:
                    continue
                vals.setdefault((k, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
                dkey = (f, int(r["Dispatch_Id"]))
                durs.setdefault(k, {})[dkey] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                per_launch.setdefault(k, {}).setdefault(dkey, {})[r["Counter_Name"]] = float(r["Counter_Value"])
    gib_kb = float(1 << 20)

    def mean(k, c, pred=None):
        v = [x for x in vals.get((k, c), []) if pred is None or pred(x)]
        return sum(v) / len(v) if v else None

    f_copy = mean("copy", "FETCH_SIZE", lambda x: x > 0.25 * gib_kb)
    w_copy = mean("copy", "WRITE_SIZE", lambda x: x > 0.25 * gib_kb)
    f_fac = gib_kb / f_copy if f_copy else None
    w_fac = gib_kb / w_copy if w_copy else None
    lines = [f"# Counters: {workload} (T={sh.tokens}, hidden {sh.hidden}, intermediate {sh.inter}, {sh.experts} experts, "
             f"top-{sh.topk}, {sh.fmt})", "", "One rocprofv3 `--pmc` pass per counter group, each its own run (on one MI355X; `$REPO` is the repository "
             "root, `$OUT` an output folder):", "",
             "```", command, "```", "",
             f"Routing: {active} active experts, {pairs} routed pairs.  Copy calibration: FETCH_SIZE factor "
             f"{f_fac if f_fac is None else round(f_fac, 3)}, WRITE_SIZE factor {w_fac if w_fac is None else round(w_fac, 3)} "
             "(1 GiB read and written by a plain elementwise copy in the same process).", ""]
    counters = sorted({c for (_, c) in vals})
    for k in ("gate_up", "down", "combine", "plan"):
        if not any(kk == k for (kk, _) in vals):
            continue
        dur = float(np.mean(list(durs[k].values())))
        lines += [f"## {k}", "", f"Mean launch duration under the profiler: {dur:.1f} us "
                  f"({len(durs[k])} profiled launches over all passes).", "", "| counter | mean per launch |", "|---|---|"]
        for c in counters:
            m = mean(k, c)
            if m is not None:
                lines.append(f"| {c} | {m:,.0f} |")
        lines += ["", "| derived | value |", "|---|---|"]
        busy, grbm = mean(k, "SQ_VALU_MFMA_BUSY_CYCLES"), mean(k, "GRBM_GUI_ACTIVE")
        if busy is not None and grbm is not None and dur > 50.0:  # (a few-us kernel's GRBM count is mostly overhead)
            per_xcd = grbm / 8.0
            lines.append(f"| MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / (GRBM_GUI_ACTIVE / 8 XCDs)) | "
                         f"{busy / 1024.0 / per_xcd:.3f} |")
            lines.append(f"| effective clock (GRBM_GUI_ACTIVE / 8 / launch duration) | {per_xcd / dur / 1e3:.2f} GHz |")
        mops = mean(k, "SQ_INSTS_VALU_MFMA_MOPS_F8") or mean(k, "SQ_INSTS_VALU_MFMA_MOPS_BF16") or \
            mean(k, "SQ_INSTS_VALU_MFMA_MOPS_F6F4")
        if mops is not None and k in algo:
            lines.append(f"| issued MFMA flops (MOPS x 512) / algorithmic flops | {mops * 512 / algo[k][0]:.3f} |")
        fetch, write = mean(k, "FETCH_SIZE"), mean(k, "WRITE_SIZE")
        if fetch is not None and f_fac:
            lines.append(f"| HBM fetch (FETCH_SIZE x {f_fac:.3f}) | {fetch * f_fac * 1024 / 1e6:,.1f} MB |")
        if write is not None and w_fac:
            lines.append(f"| HBM write (WRITE_SIZE x {w_fac:.3f}) | {write * w_fac * 1024 / 1e6:,.1f} MB |")
        if fetch is not None and write is not None and f_fac and w_fac and k in algo:
            t = (fetch * f_fac + write * w_fac) * 1024
            lines.append(f"| traffic / algorithmic bytes ({algo[k][1] / 1e6:,.1f} MB) | {t / algo[k][1]:.2f} |")
        hit, miss = mean(k, "TCC_HIT_sum"), mean(k, "TCC_MISS_sum")
        if hit is not None and miss is not None and hit + miss > 0:
            lines.append(f"| L2 hit rate (TCC_HIT / (TCC_HIT + TCC_MISS)) | {hit / (hit + miss):.3f} |")
        lines.append("")
        seq = [(key, c) for key, c in sorted(per_launch.get(k, {}).items())
               if "GRBM_GUI_ACTIVE" in c and "SQ_VALU_MFMA_BUSY_CYCLES" in c]
        if seq and busy and dur > 50.0:
            lines += ["Launches of the counter pass in dispatch order (duration, effective clock, MFMA busy):", ""]
            lines.append("; ".join(f"{durs[k][key]:.0f} us, {c['GRBM_GUI_ACTIVE'] / 8 / durs[k][key] / 1e3:.2f} GHz, "
                                   f"{c['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024 / (c['GRBM_GUI_ACTIVE'] / 8):.3f}"
                                   for key, c in seq) + ".")
            lines.append("")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))
    return 0


class Leg:
    """The step's kernels on one workload: inputs resident in HBM, weights in the
    prepared layout (written once, untimed), caller-owned plan, intermediate and y."""

    def __init__(self, name: str, fuse_combine: bool = False, fuse_plan: bool = False):
        import numpy as np
        import torch

        import moe_synth
        from mixture_experts_ffn_topk_amd import MoEFFN

        sh = moe_synth.WORKLOADS[name]
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

        self.sh, self.inp = sh, inp
        self.fuse = fuse_combine
        self.fuse_plan = fuse_plan  # the plan built in the gate_up launch (moe_plan_ffn_gate_up)
        self.x, self.x_sf = dev(inp["x"]), dev(inp["x_sf"])
        canonical = {"w13": dev(inp["w13"]), "w13_sf": dev(inp["w13_sf"]), "w2": dev(inp["w2"]),
                     "w2_sf": dev(inp["w2_sf"]), "w13_gs": dev(inp.get("w13_gs")), "w2_gs": dev(inp.get("w2_gs")),
                     "c_input_scales": dev(inp.get("c_scales"))}
        self.logits = dev(inp["logits"])
        if sh.routing == "precomputed":
            self.topk_idx, self.topk_w = dev(inp["topk_idx"]), dev(inp["topk_weights"])
        else:
            self.topk_idx = torch.empty((T, k), dtype=torch.int64, device="cuda")
            self.topk_w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        self.moe = MoEFFN(H, I, E, k, T, fmt=sh.fmt, route_mode=sh.routing, activation_clamp=sh.clamp,
                          fuse_combine=fuse_combine)
        # one-time weight relayout (the pages' pre-permuted weights); outside every timed region
        self.weights = self.moe.prepare_weights(canonical)
        torch.cuda.synchronize()
        del canonical
        self.plan = self.moe.alloc_plan(T)
        self.ws = self.moe.alloc_workspace(T)
        self.h, self.hsf = self.moe.alloc_intermediate(T)
        self.y = torch.empty((T * k, H), dtype=torch.bfloat16, device="cuda")
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        self.stream = torch.cuda.current_stream()
        self._calls = None

    def checked_step(self):
        """One step through the binding's methods, which check every tensor argument."""
        m, T, s = self.moe, self.sh.tokens, self.stream
        if self.sh.routing == "precomputed":
            m.plan(T, self.plan, topk_idx=self.topk_idx, ws=self.ws, stream=s)
        else:
            m.plan(T, self.plan, routing_logits=self.logits, topk_idx_out=self.topk_idx, topk_weights_out=self.topk_w,
                   ws=self.ws, stream=s)
        m.ffn_gate_up(T, self.x, self.x_sf, self.weights, self.plan, self.h, self.hsf, stream=s)
        if self.fuse_plan:  # the same plan and h again, from the one-launch form
            if self.sh.routing == "precomputed":
                m.plan_ffn_gate_up(T, self.x, self.x_sf, self.weights, self.plan, self.h, self.hsf,
                                   topk_idx=self.topk_idx, ws=self.ws, stream=s)
            else:
                m.plan_ffn_gate_up(T, self.x, self.x_sf, self.weights, self.plan, self.h, self.hsf,
                                   routing_logits=self.logits, topk_idx_out=self.topk_idx,
                                   topk_weights_out=self.topk_w, ws=self.ws, stream=s)
        if self.fuse:
            m.ffn_down_combine(T, self.h, self.hsf, self.weights, self.plan, self.topk_w, self.y, self.out, stream=s)
        else:
            m.ffn_down(T, self.h, self.hsf, self.weights, self.plan, self.y, stream=s)
            m.combine(T, self.y, self.topk_w, self.plan, self.out, stream=s)

    def _build_calls(self):
        """The C ABI calls of one step with their arguments marshalled once (the same
        buffers every step, already checked by checked_step), so that issuing a step
        costs the host a few microseconds and the GPU never waits for it."""
        import ctypes
        m, T, sh = self.moe, self.sh.tokens, self.sh
        lib, h, s = m.lib, m._h, self.stream.cuda_stream
        self._ws_s, self._ps = m._weights_struct(self.weights), m._plan_struct(self.plan)
        W, P = ctypes.byref(self._ws_s), ctypes.byref(self._ps)
        nb = self.ws.numel() * self.ws.element_size()
        hsf = None if self.hsf is None else self.hsf.data_ptr()
        x_sf = None if self.x_sf is None else self.x_sf.data_ptr()
        if sh.routing == "precomputed":
            plan = (h, T, self.topk_idx.data_ptr(), None, None, None, P, self.ws.data_ptr(), nb, s)
        else:
            plan = (h, T, None, self.logits.data_ptr(), self.topk_idx.data_ptr(), self.topk_w.data_ptr(), P,
                    self.ws.data_ptr(), nb, s)
        gu = (h, T, self.x.data_ptr(), x_sf, W, P, self.h.data_ptr(), hsf, s)
        # moe_plan_ffn_gate_up: the routing arguments of moe_plan, then those of the gate_up leg
        pgu = plan[:6] + (self.x.data_ptr(), x_sf, W, P, self.h.data_ptr(), hsf, self.ws.data_ptr(), nb, s)
        if self.fuse:
            dn = (h, T, self.h.data_ptr(), hsf, W, P, self.topk_w.data_ptr(), self.y.data_ptr(), None, None,
                  self.out.data_ptr(), s)
        else:
            dn = (h, T, self.h.data_ptr(), hsf, W, P, self.y.data_ptr(), s)
        comb = (h, T, self.y.data_ptr(), self.topk_w.data_ptr(), P, self.out.data_ptr(), s)
        self._calls = (lib, plan, gu, dn, comb, pgu)

    def step(self, legs=None):
        """One pass of the whole path.  legs: optional hipEvent_t handles (gate_up
        start/stop, down start/stop) that the two GEMM launches carry themselves."""
        if self._calls is None:
            self._build_calls()
        lib, plan, gu, dn, comb, pgu = self._calls
        if legs is None:
            st = lib.moe_plan_ffn_gate_up(*pgu) if self.fuse_plan else lib.moe_plan(*plan) | lib.moe_ffn_gate_up(*gu)
            st |= lib.moe_ffn_down_combine(*dn) if self.fuse else lib.moe_ffn_down(*dn)
        else:
            if self.fuse_plan:
                st = lib.moe_plan_ffn_gate_up_timed(*pgu, legs[0], legs[1])
            else:
                st = lib.moe_plan(*plan) | lib.moe_ffn_gate_up_timed(*gu, legs[0], legs[1])
            st |= lib.moe_ffn_down_combine_timed(*dn, legs[2], legs[3]) if self.fuse else \
                lib.moe_ffn_down_timed(*dn, legs[2], legs[3])
        if not self.fuse:
            st |= lib.moe_combine(*comb)
        if st != 0:
            raise RuntimeError(f"a step's C ABI call failed (status bits {st})")

    def release(self):
        """Drop the leg's device buffers (the host inputs stay)."""
        for name in ("x", "x_sf", "logits", "topk_idx", "topk_w", "moe", "weights", "plan", "ws", "h", "hsf", "y",
                     "out", "_calls", "_ws_s", "_ps"):
            if hasattr(self, name):
                setattr(self, name, None)

    def counts(self):
        c = self.plan["expert_counts"].cpu().numpy()
        return int((c > 0).sum()), int(c.sum())

    def algorithmic(self):
        """(gate_up bytes, down bytes, whole-step bytes, gate_up flops, down flops) of one step."""
        sh = self.sh
        active, pairs = self.counts()
        wb_gu, wb_dn = weight_bytes_per_expert(sh)
        gu_bytes = active * wb_gu + act_bytes(sh)
        dn_bytes = active * wb_dn
        step_bytes = active * (wb_gu + wb_dn) + act_bytes(sh) + sh.tokens * sh.hidden * 2 + sh.tokens * sh.topk * 8
        return gu_bytes, dn_bytes, step_bytes, 4.0 * pairs * sh.hidden * sh.inter, 2.0 * pairs * sh.hidden * sh.inter


def _events(n):
    """n timing events, each recorded once so that torch creates its HIP event."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in ev:
        e.record()
    return ev


def warm_up(leg: Leg, steps: int):
    """`steps` untimed steps back to back, each between two events: the mean step
    time of the first and of the last five, which shows the start-up ramp (the
    kernels themselves run slower over the first ~20 steps after start-up)."""
    import torch
    marks = [_events(2) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in marks:
        a.record(leg.stream)
        leg.step()
        b.record(leg.stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in marks]
    if len(per) < 10:
        return None
    return {"steps": len(per), "first_5_ms": round(sum(per[:5]) / 5, 4), "last_5_ms": round(sum(per[-5:]) / 5, 4)}


def timed_steps(leg: Leg, steps: int, step_markers: bool, scrub=None):
    """`steps` steps between two device synchronisations.  The two GEMM launches of
    every (steps/10)-th step carry timing events.  step_markers: an event pair around
    every step (median and minimum step time).  scrub: (buffer, 0-d output) -- the
    buffer is read (summed) before each step, outside the step's events, so that no
    weight byte is still cached from the previous step (a read, so that no dirty
    lines are left for the step to write back).  Returns (elapsed s, per-step ms list or None, gate_up ms, down ms)."""
    import numpy as np
    import torch
    from mixture_experts_ffn_topk_amd import _event_handles
    stride = max(1, steps // 10)
    legs = {i: _events(4) for i in range(0, steps, stride)}
    handles = {i: _event_handles(e[:2]) + _event_handles(e[2:]) for i, e in legs.items()}
    marks = [_events(2) for _ in range(steps)] if step_markers else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if scrub is not None:
            torch.sum(scrub[0], 0, out=scrub[1])  # reads every byte of the buffer, writes 4
        if marks:
            marks[i][0].record(leg.stream)
        leg.step(handles.get(i))
        if marks:
            marks[i][1].record(leg.stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in marks] if marks else None
    gu = float(np.mean([e[0].elapsed_time(e[1]) for e in legs.values()]))
    dn = float(np.mean([e[2].elapsed_time(e[3]) for e in legs.values()]))
    return elapsed, per, gu, dn


def roofline(leg: Leg, gate_ms: float, down_ms: float) -> dict:
    """The dominant kernel (the gate_up GEMM) against its binding roof; the down leg beside it."""
    sh = leg.sh
    gu_bytes, dn_bytes, _, gu_flops, dn_flops = leg.algorithmic()
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
            c = json.load(open(COUNTERS)).get("workloads", {}).get(sh.name, {})
            if c.get("kernel_source_sha") == kernel_source_hash():
                traffic = c["traffic_bytes_per_launch"]
        except Exception:
            traffic = None
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic,
            "kernel": "ffn_gemm_kernel gate_up (FFN leg 1)",
            "algorithmic_bytes": gu_bytes, "algorithmic_flops": gu_flops, "avg_launch_ms": round(gate_ms, 4),
            "down_leg": {"avg_launch_ms": round(down_ms, 4),
                         "hbm_frac": round(dn_bytes / (down_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         "mfma_frac": round(dn_flops / (down_ms * 1e-3) / 1e12 / peak_f, 4)}}


def step_fracs(leg: Leg, ms: float) -> dict:
    """Whole-step roofline fractions at a step time of `ms`."""
    _, _, step_bytes, gu_flops, dn_flops = leg.algorithmic()
    return {"step_hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "step_mfma_frac": round((gu_flops + dn_flops) / (ms * 1e-3) / 1e12 / PEAK_TFLOPS[leg.sh.fmt], 4)}


def dense_reference(workload: str, reps: int) -> int:
    """Context for the MFMA-bound legs: the vendor library's dense GEMM (hipBLASLt
    through torch.matmul for bf16, torch._scaled_mm with one scale per tensor for
    FP8) at each leg's flop count -- M = routed pairs, no gather, no SwiGLU, no
    block scales -- timed on the GPU.  Prints one JSON line."""
    import torch
    import moe_synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    sh = moe_synth.WORKLOADS[workload]
    if sh.fmt not in ("bf16", "fp8_block128"):
        print(f"no dense vendor GEMM for {sh.fmt}", file=sys.stderr)
        return 2
    M = sh.tokens * sh.topk
    peak = PEAK_TFLOPS[sh.fmt] * 1e12
    legs = {"gate_up": (M, 2 * sh.inter, sh.hidden), "down": (M, sh.hidden, sh.inter)}
    g = torch.Generator(device="cuda").manual_seed(0)
    res = {}
    for name, (m, n, kk) in legs.items():
        if sh.fmt == "bf16":
            a = torch.randn((m, kk), generator=g, device="cuda").to(torch.bfloat16)
            b = torch.randn((kk, n), generator=g, device="cuda").to(torch.bfloat16)
            fn, lib = (lambda: torch.matmul(a, b)), "torch.matmul bf16"
        else:
            a = (0.5 * torch.randn((m, kk), generator=g, device="cuda")).to(torch.float8_e4m3fn)
            bt = (0.5 * torch.randn((n, kk), generator=g, device="cuda")).to(torch.float8_e4m3fn)
            one = torch.ones((), device="cuda")
            fn = lambda: torch._scaled_mm(a, bt.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
            lib = "torch._scaled_mm e4m3 per-tensor scales"
        for _ in range(10):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        fl = 2.0 * m * n * kk
        res[name] = {"m_n_k": [m, n, kk], "ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 1),
                     "frac_of_peak": round(fl / (ms * 1e-3) / peak, 4), "library": lib}
        del a
    print(json.dumps({"dense_reference": workload, "legs": res}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first: the first ~20 steps after start-up run slower (warmup_curve)")
    ap.add_argument("--workload", default="prefill_fp8_zipf",
                    help="the timed workload (default: the largest one-GPU configuration, the prefill shape)")
    ap.add_argument("--decode-workload", default="decode_fp8",
                    help="the weight-bound workload measured beside it (with a cache scrub); 'none' to skip")
    ap.add_argument("--scrub-mb", type=int, default=512, help="cache scrub between the weight-bound steps (MB)")
    ap.add_argument("--fuse-combine", type=int, default=0, choices=(0, 1),
                    help="1: the combine runs in the down GEMM's epilogue (moe_ffn_down_combine)")
    ap.add_argument("--fuse-plan", type=int, default=1, choices=(0, 1),
                    help="1: the routing plan is built inside the gate_up launch where that applies "
                         "(moe_plan_ffn_gate_up; otherwise that call launches the plan kernel itself)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of CPU oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--write-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/gate_up_counters.json from two rocprofv3 --pmc output folders and exit")
    ap.add_argument("--counters-command", default="", help="the command the --pmc runs used (recorded)")
    ap.add_argument("--counter-summary", nargs="+", metavar=("OUT_MD", "DIR"),
                    help="summarise rocprofv3 --pmc folders (one per pass) of --workload into OUT_MD and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for HBM counter calibration under rocprofv3)")
    ap.add_argument("--dense-reference", action="store_true",
                    help="time the vendor dense GEMM at each leg's flop count for --workload (bf16, FP8), "
                         "print one JSON line and exit")
    args = ap.parse_args()
    if args.dense_reference:
        return dense_reference(args.workload, args.steps)
    if args.write_counters:
        return write_counters(args.workload, args.write_counters[0], args.write_counters[1], args.counters_command)
    if args.counter_summary:
        return counter_summary(args.workload, args.counter_summary[0], args.counter_summary[1:], args.counters_command)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode (the expert-parallel exchange is "
              "outside it); run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2

    leg = Leg(args.workload, args.fuse_combine, args.fuse_plan)
    # the weight-bound leg is set up now (inputs, prepared weights), so that it runs
    # right after the timed workload's steps, with no idle gap between them
    with_decode = args.decode_workload != "none" and args.decode_workload != args.workload
    dec = Leg(args.decode_workload, args.fuse_combine, args.fuse_plan) if with_decode else None
    sh = leg.sh
    T, k, E, H, I = sh.tokens, sh.topk, sh.experts, sh.hidden, sh.inter
    scrub = ((torch.zeros(args.scrub_mb << 18, dtype=torch.float32, device="cuda"),
              torch.zeros((), dtype=torch.float32, device="cuda")) if args.scrub_mb > 0 else None)

    log(f"warmup {args.warmup} steps")
    leg.checked_step()  # (at least one step, through the checked binding; the plan's counts then exist)
    curve = warm_up(leg, args.warmup - 1)
    active, pairs = leg.counts()
    weight_bound = roofline(leg, 1.0, 1.0)["bound"] == "hbm"

    # The timed region: exactly `steps` steps back to back (the GEMM launches of every
    # (steps/10)-th step carry their timing events).  Then as many steps with an event
    # pair around each, for the median and minimum step time.  A weight-bound workload
    # then runs as many again with the scrub buffer rewritten before each step
    # (outside the step's events): its median and minimum without memory-side cache reuse.
    log(f"timing {args.steps} steps")
    elapsed, _, gate_ms, down_ms = timed_steps(leg, args.steps, False)
    _, per, _, _ = timed_steps(leg, args.steps, True)
    scrubbed = None
    if weight_bound and scrub is not None:
        _, per_s, gu_s, dn_s = timed_steps(leg, args.steps, True, scrub)
        med = float(np.median(per_s))
        scrubbed = {"scrub_mb": args.scrub_mb, "step_ms_median": round(med, 4),
                    "step_ms_min": round(float(np.min(per_s)), 4),
                    "step_hbm_frac_median": step_fracs(leg, med)["step_hbm_frac"],
                    "gate_up_avg_launch_ms": round(gu_s, 4), "down_avg_launch_ms": round(dn_s, 4)}

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1)
        for _ in range(3):
            torch.add(a, 0, out=b)  # a plain elementwise copy: reads and writes 1 GiB
        torch.cuda.synchronize()
        del a, b

    ms_per_step = elapsed * 1e3 / args.steps
    tok_s = T * args.steps / elapsed
    _, _, step_bytes, gu_flops, dn_flops = leg.algorithmic()
    result = {
        "metric": "MoE FFN tokens/s + achieved TFLOP/s & HBM GB/s vs MI355X peak",
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": DTYPE[sh.fmt], "data": "synthetic",
        "config": {"workload": sh.name, "tokens": T, "hidden": H, "intermediate": I, "experts": E, "topk": k,
                   "format": sh.fmt, "routing": sh.routing, "active_experts": active, "routed_pairs": pairs,
                   "parallelism": "single GPU"},
        "step_ms_median": round(float(np.median(per)), 4), "step_ms_min": round(float(np.min(per)), 4),
        "step_tflops": round((gu_flops + dn_flops) / (ms_per_step * 1e-3) / 1e12, 2),
        "step_hbm_gbs": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        **step_fracs(leg, ms_per_step),
        "scrubbed": scrubbed, "fused_combine": bool(args.fuse_combine),
        "plan_in_gate_up": bool(args.fuse_plan) and leg.moe.plan_in_gate_up(T),
        "warmup_curve": curve,
        "roofline": roofline(leg, gate_ms, down_ms),
    }


    # The weight-bound decode shape beside it: its own warm-up, then the same number of
    # steps back to back, then as many with the cache scrub between steps.  Then the
    # same steps once more after 100 further steps: a sustained weight-streaming load
    # runs its kernels up to ~12 % slower from ~4 to ~15 ms after it starts (a transient
    # of the part's power management, not of the work: the kernel durations rise and
    # fall back with identical work), which W = 5 warm-up steps leave inside the timed
    # steps; `startup_ms_per_5_steps` shows it step by step.
    if with_decode:
        dec.checked_step()
        dcurve = warm_up(dec, args.warmup - 1)
        el, _, gu, dn = timed_steps(dec, args.steps, False)
        _, per_s, gu_s, dn_s = timed_steps(dec, args.steps, True, scrub)
        _, per_settle, _, _ = timed_steps(dec, 100, True)
        el2, _, gu2, dn2 = timed_steps(dec, args.steps, False)
        ms_b2b, ms_settled = el * 1e3 / args.steps, el2 * 1e3 / args.steps
        med = float(np.median(per_s))
        result["decode"] = {
            "workload": dec.sh.name, "tokens": dec.sh.tokens, "ms_per_step": round(ms_b2b, 4),
            "plan_in_gate_up": bool(args.fuse_plan) and dec.moe.plan_in_gate_up(dec.sh.tokens),
            "tokens_per_s": round(dec.sh.tokens / (ms_b2b * 1e-3), 1), **step_fracs(dec, ms_b2b),
            "scrubbed": {"scrub_mb": args.scrub_mb, "scrub": "read", "step_ms_median": round(med, 4),
                         "step_ms_min": round(float(np.min(per_s)), 4),
                         "step_hbm_frac_median": step_fracs(dec, med)["step_hbm_frac"],
                         "gate_up": roofline(dec, gu_s, dn_s)},
            "roofline": roofline(dec, gu, dn), "warmup_curve": dcurve,
            "settled": {"after_steps": args.warmup + 2 * args.steps + 100, "ms_per_step": round(ms_settled, 4),
                        "tokens_per_s": round(dec.sh.tokens / (ms_settled * 1e-3), 1),
                        **step_fracs(dec, ms_settled), "gate_up_avg_launch_ms": round(gu2, 4),
                        "down_avg_launch_ms": round(dn2, 4),
                        "startup_ms_per_5_steps": [round(float(np.mean(per_settle[i:i + 5])), 4)
                                                   for i in range(0, len(per_settle), 5)]}}
        for r in (result["decode"]["roofline"], result["decode"]["scrubbed"]["gate_up"]):
            r.pop("algorithmic_flops", None)
        dec.release()
        del dec

    ids = leg.inp["topk_idx"] if sh.routing == "precomputed" else leg.topk_idx.cpu().numpy()
    w = leg.inp["topk_weights"] if sh.routing == "precomputed" else leg.topk_w.cpu().numpy()
    leg.release()
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a bounded sample)")
        result["cpu_baseline"] = cpu_baseline(sh, leg.inp, ids, w, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
