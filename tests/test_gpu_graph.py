"""The entry points allocate nothing and never synchronise, so a step can be
captured into a HIP graph.  Each replay, with eager work and synchronisations
between them, must reproduce the eager step bit for bit (every kernel of the path
is deterministic)."""
import numpy as np
import pytest
import torch

import moe_synth
from gpu_util import device_inputs, make_moe, prepared

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt,routing,regime,I", [
    ("fp8_block128", "precomputed", "auto", 256), ("w4a8_mx", "from_logits", "auto", 256),
    ("nvfp4_w4a16", "precomputed", "auto", 256),
    # prefill tiles whose down leg splits over K (8 tiles, 17 K-steps: 5 pieces each):
    # the arrival counters must come back to zero within every replay
    ("fp8_block128", "precomputed", "prefill", 2176), ("bf16", "precomputed", "prefill", 1088)])
@pytest.mark.parametrize("plan_in_launch", [False, True])
def test_graph_replays_match_eager(fmt, routing, regime, I, plan_in_launch):
    """plan_in_launch: the step's plan and gate_up leg are moe_plan_ffn_gate_up (the
    plan built inside the gate_up launch where the tiles allow it)."""
    sh = moe_synth.MoEShape("graph_" + fmt, 41, 96, 512, I, 8, 2, fmt, routing)
    print(f"[graph] {fmt} {regime} I={I} plan_in_launch={plan_in_launch}", flush=True)
    inp = moe_synth.make_inputs(sh)
    moe = make_moe(sh, fuse_plan=2 if plan_in_launch else 0, tile_regime=regime)
    d = device_inputs(inp)
    w = prepared(moe, d)
    T, k = sh.tokens, sh.topk
    plan = moe.alloc_plan(T)
    ws = moe.alloc_workspace(T)
    h, hsf = moe.alloc_intermediate(T)
    y = torch.zeros((T * k, sh.hidden), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((T, sh.hidden), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()

    def step():
        if plan_in_launch:
            kw = (dict(topk_idx=d["topk_idx"]) if routing == "precomputed" else
                  dict(routing_logits=d["logits"], topk_idx_out=d["topk_idx"], topk_weights_out=d["topk_weights"]))
            moe.plan_ffn_gate_up(T, d["x"], d["x_sf"], w, plan, h, hsf, ws=ws, stream=s, **kw)
            moe.ffn_down(T, h, hsf, w, plan, y, stream=s)
            moe.combine(T, y, d["topk_weights"], plan, out, stream=s)
            return
        if routing == "precomputed":
            moe.plan(T, plan, topk_idx=d["topk_idx"], ws=ws, stream=s)
        else:
            moe.plan(T, plan, routing_logits=d["logits"], topk_idx_out=d["topk_idx"],
                     topk_weights_out=d["topk_weights"], ws=ws, stream=s)
        moe.ffn_gate_up(T, d["x"], d["x_sf"], w, plan, h, hsf, stream=s)
        moe.ffn_down(T, h, hsf, w, plan, y, stream=s)
        moe.combine(T, y, d["topk_weights"], plan, out, stream=s)

    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        out.zero_()
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager step"
        with torch.cuda.stream(s):  # eager work between replays
            step()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
    assert not torch.isnan(eager.float()).any()
