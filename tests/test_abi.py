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
    assert lib.moe_abi_version() == 5
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
    ({"format": 3}, 0),                                          # NVFP4: multiples of 64
    ({"format": 3, "hidden": 7168 + 32}, 1),
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
    w = mx._Weights(1, 1, 1, 1)
    assert lib.moe_forward(h, 10, 1, 1, 1, 1, None, ctypes.byref(w), 1, 1, 16, None) == 3  # workspace too small
    assert lib.moe_forward(h, 10, 1, None, 1, 1, None, ctypes.byref(w), 1, 1, ws, None) == 1  # FP8 needs x_sf
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
