"""moe_forward_static (the entry point that allocates nothing: its workspace is the
library's per-device static scratch) against moe_forward with a caller-owned
workspace, through the C ABI: two calls in a row on the same scratch, the second
with fewer tokens, each bit-identical to moe_forward on the same inputs (the same
kernels run in the same order, so the results are equal bit for bit); and a token
count whose workspace exceeds the scratch is refused before any launch."""
import numpy as np
import pytest
import torch

import moe_synth
from gpu_util import device_inputs, make_moe, prepared
from mixture_experts_ffn_topk_amd import STATIC_SCRATCH_BYTES, MoEError

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,T1,T2", [("decode_fp8", 256, 100), ("tiny_fp8", 64, 17)])
def test_forward_static_matches_forward(name, T1, T2):
    sh = moe_synth.WORKLOADS[name]
    print(f"[no-alloc] {name}: T {T1} then {T2}", flush=True)
    inp = moe_synth.make_inputs(sh)
    moe = make_moe(sh)
    d = device_inputs(inp)
    w = prepared(moe, d)
    assert moe.workspace_size(T1) <= STATIC_SCRATCH_BYTES
    for T in (T1, T2):
        ref = torch.full((T, sh.hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
        ws = moe.alloc_workspace(T)
        moe.forward(T, d["x"][:T], d["x_sf"][:T], d["topk_idx"][:T], d["topk_weights"][:T], None, w, ref, ws)
        got = torch.full((T, sh.hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
        moe.forward_static(T, d["x"][:T], d["x_sf"][:T], d["topk_idx"][:T], d["topk_weights"][:T], None, w, got)
        torch.cuda.synchronize()
        assert torch.isfinite(got.float()).all()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"T={T}"
        del ws


def test_forward_static_refuses_beyond_its_scratch():
    sh = moe_synth.WORKLOADS["decode_fp8"]
    moe = make_moe(sh, max_tokens=4096)
    T = 4096
    assert moe.workspace_size(T) > STATIC_SCRATCH_BYTES
    x = torch.zeros((T, sh.hidden), dtype=torch.uint8, device="cuda")
    x_sf = torch.ones((T, sh.hidden // 128), dtype=torch.float32, device="cuda")
    ids = torch.zeros((T, sh.topk), dtype=torch.int64, device="cuda")
    tw = torch.zeros((T, sh.topk), dtype=torch.float32, device="cuda")
    wsz = moe.prepared_weights_size()
    w = {n: torch.empty(b, dtype=torch.uint8, device="cuda") for n, b in wsz.items()}
    out = torch.empty((T, sh.hidden), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(MoEError, match="WORKSPACE_TOO_SMALL"):
        moe.forward_static(T, x, x_sf, ids, tw, None, w, out)
