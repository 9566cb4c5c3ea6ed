"""The C ABI library on the CPU: it loads, exports every entry point that
include/moe_ffn.h declares, and validates arguments on the host before any
launch (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import mixture_experts_ffn_topk_amd as mx

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe_ffn.h")


def _lib():
    try:
        return mx.load_library()
    except ImportError as e:  # pragma: no cover
        pytest.fail(f"library not built: {e}")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\*\s]+?\b(moe_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("moe_plan", "moe_ffn", "moe_combine", "moe_forward", "moe_create", "moe_destroy",
              "moe_workspace_size"):
        assert n in names
    assert sorted(names) == sorted(mx.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert lib.moe_abi_version() == 11
    assert lib.moe_status_string(0) == b"ok"


def _cfg(**kw):
    base = dict(hidden=7168, intermediate_hidden=2048, num_experts=32, num_topk=8, max_num_tokens=256,
                activation_clamp=10.0, format=0, route_mode=0, topk_idx_bits=64, fast_math=1, tile_regime=0)
    base.update(kw)
    return mx._Config(**base)


@pytest.mark.parametrize("kw,expect", [
    ({}, 0),
    ({"hidden": 7168 + 64}, 1),                 # FP8: hidden % 128
    ({"intermediate_hidden": 2000}, 1),
    ({"num_topk": 33, "num_experts": 64}, 1),
    ({"num_topk": 9, "num_experts": 8}, 1),     # k > E
    ({"num_experts": 0}, 1),
    ({"activation_clamp": 0.0}, 1),
    ({"activation_clamp": float("nan")}, 1),
    ({"topk_idx_bits": 16}, 1),
    ({"format": 7}, 1),
    ({"route_mode": 3}, 1),
    ({"tile_regime": 5}, 1),
    ({"format": 1, "hidden": 4096, "intermediate_hidden": 14336 + 64}, 0),  # BF16: multiples of 64
    ({"format": 2, "hidden": 2880, "intermediate_hidden": 2880, "num_experts": 128, "num_topk": 4,
      "route_mode": 1}, 0),                    # MX: multiples of 32, logits routing
    ({"format": 2, "hidden": 2880 + 16, "intermediate_hidden": 2880}, 1),
    ({"format": 2, "hidden": 32768 + 32, "intermediate_hidden": 2880, "max_num_tokens": 16}, 2),  # MX scale rows in LDS
    ({"format": 3}, 0),                                          # NVFP4: multiples of 64
    ({"format": 3, "hidden": 7168 + 32}, 1),
    ({"format": 4}, 0),                                          # NVFP4 x NVFP4: multiples of 64
    ({"format": 4, "intermediate_hidden": 2048 + 32}, 1),
    ({"format": 5}, 1),
    ({"route_mode": 1, "num_experts": 600, "num_topk": 4}, 2),   # FromLogits over > 512 experts
    ({"max_num_tokens": -1}, 1),
    ({"hidden": 32768 + 128}, 2),                # FP8 weight scales of > 256 K-steps
    ({"intermediate_hidden": 32768 + 128}, 2),
    ({"hidden": 32768, "intermediate_hidden": 32768, "max_num_tokens": 16}, 2),  # 2 GiB of W13 per expert
    ({"max_num_tokens": 300000, "num_topk": 1, "num_experts": 8}, 2),  # x of 300000 x 7168 bytes
    ({"format": 1, "hidden": 4096, "intermediate_hidden": 14336, "num_experts": 8, "num_topk": 2,
      "max_num_tokens": 40000}, 2),              # bf16 intermediate of 80000 x 14336 x 2 bytes
])
def test_create_validation(kw, expect):
    lib = _lib()
    h = ctypes.c_void_p()
    st = lib.moe_create(ctypes.byref(_cfg(**kw)), ctypes.byref(h))
    assert st == expect
    if st == 0:
        assert h.value
        lib.moe_destroy(h)
    else:
        assert not h.value


def test_workspace_size_and_host_validation():
    lib = _lib()
    h = ctypes.c_void_p()
    assert lib.moe_create(ctypes.byref(_cfg()), ctypes.byref(h)) == 0
    ws0 = lib.moe_workspace_size(h, 0)
    ws = lib.moe_workspace_size(h, 256)
    assert ws > ws0 > 0
    # y [T*k, H] bf16 alone is part of the forward workspace
    assert ws >= 256 * 8 * 7168 * 2
    assert lib.moe_workspace_size(h, 257) == 0  # above capacity
    assert lib.moe_workspace_size(h, -1) == 0
    plan = mx._Plan(*([None] * 7))
    # invalid arguments are rejected before anything is launched
    assert lib.moe_plan(h, 300, None, None, None, None, ctypes.byref(plan), None, 0, None) == 1  # T > capacity
    assert lib.moe_plan(h, 10, None, None, None, None, ctypes.byref(plan), None, 0, None) == 1   # null plan bufs
    w = mx._Weights(None, None, None, None)
    assert lib.moe_forward(h, 10, None, None, None, None, None, ctypes.byref(w), None, None, 0, None) == 1
    w = mx._Weights(256, 256, 256, 256)
    assert lib.moe_forward(h, 10, 256, 256, 256, 256, None, ctypes.byref(w), 256, 256, 16, None) == 3  # ws too small
    assert lib.moe_forward(h, 10, 256, None, 256, 256, None, ctypes.byref(w), 256, 256, ws, None) == 1  # needs x_sf
    assert lib.moe_combine(h, 10, None, None, ctypes.byref(plan), None, None) == 1
    lib.moe_destroy(h)


def test_extended_entry_points_validate_on_host():
    """moe_plan_ex / moe_combine_ex / moe_forward_ex reject, before any launch: a
    routing bias with precomputed routing, and addends that are not 16-byte aligned;
    the timed legs reject what the untimed ones do."""
    lib = _lib()
    h = ctypes.c_void_p()
    assert lib.moe_create(ctypes.byref(_cfg()), ctypes.byref(h)) == 0  # PRECOMPUTED
    plan = mx._Plan(*([16] * 7))
    assert lib.moe_plan_ex(h, 10, 16, None, 16, None, None, ctypes.byref(plan), None, 0, None) == 1  # bias, precomputed
    assert lib.moe_combine_ex(h, 10, 16, 16, ctypes.byref(plan), 8, None, 16, None) == 1  # shared misaligned
    assert lib.moe_combine_ex(h, 10, 16, 16, ctypes.byref(plan), None, 24, 16, None) == 1  # residual misaligned
    w = mx._Weights(16, 16, 16, 16)
    assert lib.moe_forward_ex(h, 10, 16, 16, 16, 16, None, 16, ctypes.byref(w), None, None, 16, 16, 1 << 40,
                              None) == 1  # bias, precomputed
    assert lib.moe_forward_ex(h, 10, 16, 16, 16, 16, None, None, ctypes.byref(w), 4, None, 16, 16, 1 << 40,
                              None) == 1  # shared misaligned
    # the timed legs validate like the untimed ones; T = 0 launches nothing and records nothing
    assert lib.moe_ffn_gate_up_timed(h, 10, None, None, ctypes.byref(w), ctypes.byref(plan), 16, 16, None, None,
                                     None) == 1  # x missing
    assert lib.moe_ffn_down_timed(h, 10, 16, 16, ctypes.byref(w), ctypes.byref(plan), None, None, None,
                                  None) == 1  # y missing
    assert lib.moe_ffn_down_timed(h, 0, None, None, ctypes.byref(w), ctypes.byref(plan), None, None, None,
                                  None) == 0
    lib.moe_destroy(h)


def test_prepared_weight_sizes_and_validation():
    """Sizes follow the header's prepared layout: per expert, rows/16 row blocks x
    K-steps (128 elements; 64 for BF16) x 2048-byte tiles (1024 for MX), MX scale
    tiles of 64 bytes; FP8 scales unchanged."""
    lib = _lib()
    cases = [
        (dict(), (32 * 256 * 56 * 2048, 32 * 32 * 56 * 4, 32 * 448 * 16 * 2048, 32 * 56 * 16 * 4)),
        (dict(format=1, hidden=4096, intermediate_hidden=14336, num_experts=8, num_topk=2),
         (8 * 1792 * 64 * 2048, 0, 8 * 256 * 224 * 2048, 0)),
        # MX: K = 2880 -> 23 K-steps of 128 (the last one half empty, zero-padded)
        (dict(format=2, hidden=2880, intermediate_hidden=2880, num_experts=128, num_topk=4),
         (128 * 360 * 23 * 1024, 128 * 360 * 23 * 64, 128 * 180 * 23 * 1024, 128 * 180 * 23 * 64)),
        # NVFP4: 32-row tiles, K-steps of 64 -> 1024-byte data tiles and 128-byte scale tiles
        (dict(format=3, hidden=7168, intermediate_hidden=2048, num_experts=32, num_topk=8),
         (32 * 128 * 112 * 1024, 32 * 128 * 112 * 128, 32 * 224 * 32 * 1024, 32 * 224 * 32 * 128)),
    ]
    for kw, want in cases:
        h = ctypes.c_void_p()
        assert lib.moe_create(ctypes.byref(_cfg(**kw)), ctypes.byref(h)) == 0
        ps = mx._PreparedSizes()
        assert lib.moe_prepared_weights_size(h, ctypes.byref(ps)) == 0
        assert (ps.w13, ps.w13_sf, ps.w2, ps.w2_sf) == want
        lib.moe_destroy(h)
    h = ctypes.c_void_p()
    assert lib.moe_create(ctypes.byref(_cfg()), ctypes.byref(h)) == 0
    assert lib.moe_prepared_weights_size(h, None) == 1
    canon = mx._Weights(256, 512, 768, 1024)
    assert lib.moe_prepare_weights(h, ctypes.byref(canon), ctypes.byref(mx._Weights(None, 1, 1, 1)), None) == 1
    assert lib.moe_prepare_weights(h, ctypes.byref(canon), ctypes.byref(mx._Weights(4104, 16, 8192, 16)), None) == 1
    assert lib.moe_prepare_weights(h, ctypes.byref(canon), ctypes.byref(mx._Weights(256, 16, 8192, 16)), None) == 1
    lib.moe_destroy(h)
    # NVFP4 needs both per-expert global scales
    h = ctypes.c_void_p()
    assert lib.moe_create(ctypes.byref(_cfg(format=3)), ctypes.byref(h)) == 0
    no_gs = mx._Weights(256, 512, 768, 1024)
    with_gs = mx._Weights(256, 512, 768, 1024, 2048, 4096)
    out = mx._Weights(8192, 16384, 32768, 65536, 2048, 4096)
    assert lib.moe_prepare_weights(h, ctypes.byref(no_gs), ctypes.byref(out), None) == 1
    assert lib.moe_prepare_weights(h, ctypes.byref(with_gs), ctypes.byref(mx._Weights(8192, 16384, 32768, 65536)),
                                   None) == 1
    lib.moe_destroy(h)


def test_binding_raises_on_bad_config():
    with pytest.raises(mx.MoEError):
        mx.MoEFFN(7168 + 64, 2048, 32, 8, 256)


def test_misaligned_buffers_are_rejected_before_any_launch():
    """The kernels move activation, intermediate, y and output rows in 16-byte
    vectors, scales in 4-byte words, and carve the workspace at 256 bytes: a
    pointer off those alignments is MOE_ERR_INVALID_ARGUMENT (fake addresses;
    nothing is launched)."""
    lib = _lib()
    h = ctypes.c_void_p()
    assert lib.moe_create(ctypes.byref(_cfg()), ctypes.byref(h)) == 0
    A = 1 << 20  # an aligned fake address
    plan = mx._Plan(*([A] * 7))
    w = mx._Weights(A, A, A, A)
    big = 1 << 40
    # combine: y, out
    assert lib.moe_combine(h, 10, A + 8, A, ctypes.byref(plan), A, None) == 1
    assert lib.moe_combine(h, 10, A, A, ctypes.byref(plan), A + 2, None) == 1
    # ffn: x, x_sf, y, workspace
    assert lib.moe_ffn(h, 10, A + 4, A, ctypes.byref(w), ctypes.byref(plan), A, A, big, None) == 1
    assert lib.moe_ffn(h, 10, A, A + 2, ctypes.byref(w), ctypes.byref(plan), A, A, big, None) == 1
    assert lib.moe_ffn(h, 10, A, A, ctypes.byref(w), ctypes.byref(plan), A + 8, A, big, None) == 1
    assert lib.moe_ffn(h, 10, A, A, ctypes.byref(w), ctypes.byref(plan), A, A + 128, big, None) == 1
    # legs: h, h_sf
    assert lib.moe_ffn_gate_up(h, 10, A, A, ctypes.byref(w), ctypes.byref(plan), A + 8, A, None) == 1
    assert lib.moe_ffn_gate_up(h, 10, A, A, ctypes.byref(w), ctypes.byref(plan), A, A + 1, None) == 1
    assert lib.moe_ffn_down(h, 10, A + 8, A, ctypes.byref(w), ctypes.byref(plan), A, None) == 1
    assert lib.moe_ffn_down(h, 10, A, A, ctypes.byref(w), ctypes.byref(plan), A + 8, None) == 1
    # plan and forward workspaces
    assert lib.moe_plan(h, 10, A, None, None, None, ctypes.byref(plan), A + 64, big, None) == 1
    assert lib.moe_forward(h, 10, A, A, A, A, None, ctypes.byref(w), A, A + 16, big, None) == 1
    assert lib.moe_forward(h, 10, A, A, A, A, None, ctypes.byref(w), A + 8, A, big, None) == 1  # out
    lib.moe_destroy(h)


def test_out_fp32_config_is_validated():
    lib = _lib()
    h = ctypes.c_void_p()
    assert lib.moe_create(ctypes.byref(_cfg(out_fp32=1)), ctypes.byref(h)) == 0
    lib.moe_destroy(h)
    h = ctypes.c_void_p()
    assert lib.moe_create(ctypes.byref(_cfg(out_fp32=2)), ctypes.byref(h)) == 1


def test_binding_checks_tensors_before_the_call():
    """The binding refuses, before any address crosses the C ABI: an id tensor of the
    wrong width for topk_idx_bits (the plan kernels would read past it), weights of
    the wrong dtype, buffers that are too small, non-contiguous views, and host
    tensors."""
    import torch
    moe = mx.MoEFFN(256, 128, 8, 2, 64)  # FP8, 64-bit ids
    plan = {f: torch.zeros(n, dtype=torch.int32) for f, n in
            (("expert_counts", 8), ("expert_start_indices", 9), ("expert_ids", 8), ("num_active_experts", 1),
             ("src_info", 128), ("pair_row", 128), ("status", 1))}
    with pytest.raises(TypeError, match="topk_idx"):
        moe.plan(64, plan, topk_idx=torch.zeros((64, 2), dtype=torch.int32))
    with pytest.raises(ValueError, match="topk_idx holds"):
        moe.plan(64, plan, topk_idx=torch.zeros((32, 2), dtype=torch.int64))
    with pytest.raises(ValueError, match="contiguous"):
        moe.plan(64, plan, topk_idx=torch.zeros((2, 64), dtype=torch.int64).t())
    with pytest.raises(ValueError, match="GPU tensor"):
        moe.plan(64, plan, topk_idx=torch.zeros((64, 2), dtype=torch.int64))
    bad_plan = dict(plan, src_info=torch.zeros(128, dtype=torch.int64))
    with pytest.raises(TypeError, match="src_info"):
        moe.plan(64, bad_plan, topk_idx=torch.zeros((64, 2), dtype=torch.int64))
    y = torch.zeros((128, 256), dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="topk_weights"):
        moe.combine(64, y, torch.zeros((64, 2), dtype=torch.float64), plan, torch.zeros((64, 256), dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="out"):
        moe.combine(64, y, torch.zeros((64, 2)), plan, torch.zeros((64, 256), dtype=torch.float32))
    moe32 = mx.MoEFFN(256, 128, 8, 2, 64, topk_idx_bits=32, out_fp32=True)
    with pytest.raises(TypeError, match="topk_idx"):
        moe32.plan(64, plan, topk_idx=torch.zeros((64, 2), dtype=torch.int64))
    with pytest.raises(TypeError, match="out"):
        moe32.combine(64, y, torch.zeros((64, 2)), plan, torch.zeros((64, 256), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="x holds"):
        moe.ffn_gate_up(64, torch.zeros(100, dtype=torch.uint8), torch.zeros((64, 2)), {}, plan, None, None)


@pytest.mark.parametrize("kw,T,fuse_plan,expect", [
    ({}, 256, 1, 1),                                   # decode: weight-bound tiles, 2048 pairs, one round
    ({"max_num_tokens": 8192}, 8192, 1, 0),            # prefill: MFMA-bound tiles (2048 rows per expert)
    ({"max_num_tokens": 8192}, 8192, 2, 0),            # (not even where forced)
    ({"format": 2, "hidden": 2880, "intermediate_hidden": 2880, "num_experts": 128, "num_topk": 4,
      "max_num_tokens": 2048}, 2048, 1, 0),            # W4A8: 11 rounds x 8192 pairs > 4096
    ({"format": 2, "hidden": 2880, "intermediate_hidden": 2880, "num_experts": 128, "num_topk": 4,
      "max_num_tokens": 2048}, 2048, 2, 1),            # forced: the sizes allow it
    ({"hidden": 256, "intermediate_hidden": 128, "num_experts": 8, "num_topk": 2, "max_num_tokens": 64}, 64, 1, 1),
    ({"format": 1, "hidden": 4096, "intermediate_hidden": 14336, "num_experts": 8, "num_topk": 2,
      "max_num_tokens": 4096}, 4096, 1, 0),            # Mixtral: MFMA-bound tiles
    ({}, 0, 1, 0),                                     # no tokens
    ({}, 257, 1, 0),                                   # beyond max_num_tokens
])
def test_plan_in_gate_up_rule(kw, T, fuse_plan, expect):
    """The host's answer to whether the routing plan is built inside the gate_up
    launch: the weight-bound tile regime, at most 8192 pairs, and (unless forced)
    pairs x rounds of gate_up workgroups at most 4096."""
    lib = _lib()
    h = ctypes.c_void_p()
    assert lib.moe_create(ctypes.byref(_cfg(fuse_plan=fuse_plan, **kw)), ctypes.byref(h)) == 0
    assert lib.moe_plan_in_gate_up(h, T) == expect
    lib.moe_destroy(h)
    assert lib.moe_plan_in_gate_up(None, 16) == 0


SPLIT_BYTES = 256 * 4 + 256 * 512 * 128 * 4  # counters, then one fp32 partial tile per slot


@pytest.mark.parametrize("kw,expect", [
    ({}, 0),                                                   # decode: weight-bound tiles only
    ({"max_num_tokens": 8192}, SPLIT_BYTES),                   # FP8 reaching the prefill regime
    ({"tile_regime": 2}, SPLIT_BYTES),                         # forced prefill tiles
    ({"tile_regime": 1, "max_num_tokens": 8192}, 0),           # forced decode tiles
    ({"format": 1, "hidden": 4096, "intermediate_hidden": 14336, "num_experts": 8, "num_topk": 2,
      "max_num_tokens": 4096}, SPLIT_BYTES),                   # Mixtral BF16
    ({"format": 2, "hidden": 2880, "intermediate_hidden": 2880, "num_experts": 128, "num_topk": 4,
      "max_num_tokens": 8192}, 0),                             # W4A8: its down tiles never split
])
def test_down_split_size(kw, expect):
    """Bytes of the down leg's split-tail buffer: kSplitMaxSlots counters and partial
    tiles where the prefill tile regime can run an FP8 or BF16 down leg, else 0."""
    lib = _lib()
    h = ctypes.c_void_p()
    assert lib.moe_create(ctypes.byref(_cfg(**kw)), ctypes.byref(h)) == 0
    assert lib.moe_down_split_size(h) == expect
    lib.moe_destroy(h)
    assert lib.moe_down_split_size(None) == 0


def test_plan_down_split_must_be_aligned():
    """plan->down_split is optional but 256-byte aligned."""
    lib = _lib()
    h = ctypes.c_void_p()
    assert lib.moe_create(ctypes.byref(_cfg()), ctypes.byref(h)) == 0
    plan = mx._Plan(*([16] * 7), None, 128)
    assert lib.moe_plan(h, 10, 16, None, None, None, ctypes.byref(plan), None, 0, None) == 1
    lib.moe_destroy(h)


def test_plan_ffn_gate_up_validates_on_host():
    """moe_plan_ffn_gate_up checks what moe_plan and moe_ffn_gate_up check, before any
    launch; fuse_plan is 0, 1 or 2."""
    lib = _lib()
    h = ctypes.c_void_p()
    assert lib.moe_create(ctypes.byref(_cfg(fuse_plan=1)), ctypes.byref(h)) == 0  # PRECOMPUTED, FP8
    plan = mx._Plan(*([16] * 7))
    w = mx._Weights(16, 16, 16, 16)
    f = lib.moe_plan_ffn_gate_up
    assert f(h, 10, None, None, None, None, 16, 16, ctypes.byref(w), ctypes.byref(plan), 16, 16, None, 0,
             None) == 1  # ids missing
    assert f(h, 10, 16, None, None, None, None, 16, ctypes.byref(w), ctypes.byref(plan), 16, 16, None, 0,
             None) == 1  # x missing
    assert f(h, 10, 16, None, None, None, 16, None, ctypes.byref(w), ctypes.byref(plan), 16, 16, None, 0,
             None) == 1  # FP8 x_sf missing
    assert f(h, 10, 16, None, None, None, 16, 16, ctypes.byref(w), ctypes.byref(plan), None, 16, None, 0,
             None) == 1  # h missing
    assert f(h, 10, 16, None, None, None, 8, 16, ctypes.byref(w), ctypes.byref(plan), 16, 16, None, 0,
             None) == 1  # x misaligned
    assert f(h, 10, 16, None, None, None, 16, 16, ctypes.byref(w), ctypes.byref(plan), 16, 16, 128, 1 << 30,
             None) == 1  # workspace misaligned
    bad_plan = mx._Plan(*([16] * 6), None)  # status missing
    assert f(h, 10, 16, None, None, None, 16, 16, ctypes.byref(w), ctypes.byref(bad_plan), 16, 16, None, 0,
             None) == 1
    assert lib.moe_plan_ffn_gate_up_timed(h, 10, None, None, None, None, 16, 16, ctypes.byref(w), ctypes.byref(plan),
                                          16, 16, None, 0, None, None, None) == 1
    lib.moe_destroy(h)
    h = ctypes.c_void_p()
    assert lib.moe_create(ctypes.byref(_cfg(route_mode=1)), ctypes.byref(h)) == 0  # FROM_LOGITS
    assert f(h, 10, None, 16, None, 16, 16, 16, ctypes.byref(w), ctypes.byref(plan), 16, 16, None, 0,
             None) == 1  # topk_idx_out missing
    lib.moe_destroy(h)
    h = ctypes.c_void_p()
    assert lib.moe_create(ctypes.byref(_cfg(fuse_plan=2)), ctypes.byref(h)) == 0
    lib.moe_destroy(h)
    h = ctypes.c_void_p()
    assert lib.moe_create(ctypes.byref(_cfg(fuse_plan=3)), ctypes.byref(h)) == 1
