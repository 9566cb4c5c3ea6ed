"""Python binding of libmoe_ffn.so — the routed MoE expert-FFN library for MI355X.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  torch supplies device memory and the HIP stream; the binding passes
``tensor.data_ptr()`` and sizes through ctypes to the C ABI of
``include/moe_ffn.h`` (same entry-point names).

The library must have been built (``python -m mixture_experts_ffn_topk_amd.build``
or ``__graft_entry__.build()``); if it is missing, loading fails loudly — there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_ffn.so")

# ------------------------------------------------------------------ enums (include/moe_ffn.h)
MOE_OK = 0
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARGUMENT", 2: "MOE_ERR_UNSUPPORTED",
                3: "MOE_ERR_WORKSPACE_TOO_SMALL", 4: "MOE_ERR_HIP"}
FORMATS = {"fp8_block128": 0, "bf16": 1, "w4a8_mx": 2, "nvfp4_w4a16": 3, "nvfp4": 4}
ROUTE_MODES = {"precomputed": 0, "from_logits": 1}
TILE_REGIMES = {"auto": 0, "decode": 1, "prefill": 2}


class MoEError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)}")
        self.status = status


class _Config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("intermediate_hidden", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("num_topk", ctypes.c_int32),
                ("max_num_tokens", ctypes.c_int32), ("activation_clamp", ctypes.c_float),
                ("format", ctypes.c_int32), ("route_mode", ctypes.c_int32),
                ("topk_idx_bits", ctypes.c_int32), ("fast_math", ctypes.c_int32),
                ("tile_regime", ctypes.c_int32), ("out_fp32", ctypes.c_int32), ("fuse_combine", ctypes.c_int32),
                ("fuse_plan", ctypes.c_int32)]


class _Weights(ctypes.Structure):
    _fields_ = [("w13", ctypes.c_void_p), ("w13_sf", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w2_sf", ctypes.c_void_p),
                ("w13_gs", ctypes.c_void_p), ("w2_gs", ctypes.c_void_p), ("c_input_scales", ctypes.c_void_p)]


class _Plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("expert_counts", "expert_start_indices", "expert_ids",
                                               "num_active_experts", "src_info", "pair_row", "status",
                                               "combine_counters", "down_split")]


class _PreparedSizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("w13", "w13_sf", "w2", "w2_sf")]


PLAN_FIELDS = [f for f, _ in _Plan._fields_]
EXPORTED = ["moe_create", "moe_destroy", "moe_workspace_size", "moe_down_split_size", "moe_plan_in_gate_up", "moe_prepared_weights_size", "moe_prepare_weights",
            "moe_plan", "moe_ffn", "moe_ffn_gate_up", "moe_ffn_down", "moe_combine", "moe_forward",
            "moe_plan_ex", "moe_combine_ex", "moe_forward_ex", "moe_ffn_gate_up_timed", "moe_ffn_down_timed",
            "moe_ffn_down_combine", "moe_ffn_down_combine_timed", "moe_plan_ffn_gate_up", "moe_plan_ffn_gate_up_timed",
            "moe_forward_static", "moe_status_string", "moe_abi_version"]
STATIC_SCRATCH_BYTES = 64 << 20  # MOE_STATIC_SCRATCH_BYTES

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoe_ffn.so and declare the C signatures.  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m mixture_experts_ffn_topk_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.moe_create.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(vp)]
    lib.moe_create.restype = i32
    lib.moe_destroy.argtypes = [vp]
    lib.moe_destroy.restype = None
    lib.moe_workspace_size.argtypes = [vp, i32]
    lib.moe_workspace_size.restype = sz
    lib.moe_down_split_size.argtypes = [vp]
    lib.moe_down_split_size.restype = sz
    lib.moe_plan_in_gate_up.argtypes = [vp, i32]
    lib.moe_plan_in_gate_up.restype = i32
    lib.moe_prepared_weights_size.argtypes = [vp, ctypes.POINTER(_PreparedSizes)]
    lib.moe_prepared_weights_size.restype = i32
    lib.moe_prepare_weights.argtypes = [vp, ctypes.POINTER(_Weights), ctypes.POINTER(_Weights), vp]
    lib.moe_prepare_weights.restype = i32
    lib.moe_plan.argtypes = [vp, i32, vp, vp, vp, vp, ctypes.POINTER(_Plan), vp, sz, vp]
    lib.moe_plan.restype = i32
    lib.moe_ffn.argtypes = [vp, i32, vp, vp, ctypes.POINTER(_Weights), ctypes.POINTER(_Plan), vp, vp, sz, vp]
    lib.moe_ffn.restype = i32
    lib.moe_ffn_gate_up.argtypes = [vp, i32, vp, vp, ctypes.POINTER(_Weights), ctypes.POINTER(_Plan), vp, vp, vp]
    lib.moe_ffn_gate_up.restype = i32
    lib.moe_ffn_down.argtypes = [vp, i32, vp, vp, ctypes.POINTER(_Weights), ctypes.POINTER(_Plan), vp, vp]
    lib.moe_ffn_down.restype = i32
    lib.moe_ffn_gate_up_timed.argtypes = lib.moe_ffn_gate_up.argtypes + [vp, vp]
    lib.moe_ffn_gate_up_timed.restype = i32
    lib.moe_plan_ffn_gate_up.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, ctypes.POINTER(_Weights),
                                         ctypes.POINTER(_Plan), vp, vp, vp, sz, vp]
    lib.moe_plan_ffn_gate_up.restype = i32
    lib.moe_plan_ffn_gate_up_timed.argtypes = lib.moe_plan_ffn_gate_up.argtypes + [vp, vp]
    lib.moe_plan_ffn_gate_up_timed.restype = i32
    lib.moe_ffn_down_timed.argtypes = lib.moe_ffn_down.argtypes + [vp, vp]
    lib.moe_ffn_down_timed.restype = i32
    lib.moe_ffn_down_combine.argtypes = [vp, i32, vp, vp, ctypes.POINTER(_Weights), ctypes.POINTER(_Plan), vp, vp,
                                         vp, vp, vp, vp]
    lib.moe_ffn_down_combine.restype = i32
    lib.moe_ffn_down_combine_timed.argtypes = lib.moe_ffn_down_combine.argtypes + [vp, vp]
    lib.moe_ffn_down_combine_timed.restype = i32
    lib.moe_combine.argtypes = [vp, i32, vp, vp, ctypes.POINTER(_Plan), vp, vp]
    lib.moe_combine.restype = i32
    lib.moe_forward.argtypes = [vp, i32, vp, vp, vp, vp, vp, ctypes.POINTER(_Weights), vp, vp, sz, vp]
    lib.moe_forward.restype = i32
    lib.moe_plan_ex.argtypes = [vp, i32, vp, vp, vp, vp, vp, ctypes.POINTER(_Plan), vp, sz, vp]
    lib.moe_plan_ex.restype = i32
    lib.moe_combine_ex.argtypes = [vp, i32, vp, vp, ctypes.POINTER(_Plan), vp, vp, vp, vp]
    lib.moe_combine_ex.restype = i32
    lib.moe_forward_ex.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, ctypes.POINTER(_Weights), vp, vp, vp, vp, sz, vp]
    lib.moe_forward_ex.restype = i32
    lib.moe_forward_static.argtypes = [vp, i32, vp, vp, vp, vp, vp, ctypes.POINTER(_Weights), vp, vp]
    lib.moe_forward_static.restype = i32
    lib.moe_status_string.argtypes = [i32]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_abi_version.argtypes = []
    lib.moe_abi_version.restype = i32
    _lib = lib
    return lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _event_handles(events):
    """hipEvent_t handles of a (start, stop) pair of torch.cuda.Event; torch creates
    an event at its first record, so an event never recorded has no handle yet."""
    hs = []
    for e in events:
        hv = int(e.cuda_event)
        if hv == 0:
            raise ValueError("a timing event must be created (recorded once) before it is passed to a launch")
        hs.append(ctypes.c_void_p(hv))
    return hs


def _stream(stream) -> int | None:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(st: int, what: str):
    if st != MOE_OK:
        raise MoEError(st, what)


def _need(t, what: str, nbytes: int, dtypes=None, elem: int | None = None, required: bool = True):
    """Check a tensor argument before its address crosses the C ABI, which cannot:
    of an allowed dtype (or element size), contiguous, and holding at least
    `nbytes` (its device is checked by _on_gpu).  A raw device address (int) is
    passed through unchecked."""
    if t is None:
        if required and nbytes > 0:
            raise ValueError(f"{what} is required")
        return
    if isinstance(t, int):
        return
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{what} must have dtype {' or '.join(str(d) for d in dtypes)} (got {t.dtype})")
    if elem is not None and t.element_size() != elem:
        raise TypeError(f"{what} must have {elem}-byte elements (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{what} holds {have} bytes; {nbytes} are needed")


def _on_gpu(**tensors):
    """Every tensor given (None and raw addresses aside) lives on the GPU; checked
    after the dtype and size checks of the same call."""
    for what, t in tensors.items():
        if isinstance(t, dict):
            _on_gpu(**{f"{what}['{k}']": v for k, v in t.items()})
        elif t is not None and not isinstance(t, int) and t.device.type != "cuda":
            raise ValueError(f"{what} must be a GPU tensor (got {t.device})")


class MoEFFN:
    """One GPU's share of experts with a fixed geometry (moe_create / moe_destroy).

    Tensors are torch tensors on the GPU (or raw device addresses as ints); their
    dtype and layout must match include/moe_ffn.h.  The binding checks each tensor
    it is given (device, contiguity, dtype where it decides how the kernels read
    it, size in bytes) and forwards its address; raw addresses are forwarded as
    they are."""

    def __init__(self, hidden: int, intermediate_hidden: int, num_experts: int, num_topk: int,
                 max_num_tokens: int, fmt: str = "fp8_block128", route_mode: str = "precomputed",
                 activation_clamp: float = 10.0, topk_idx_bits: int = 64, fast_math: bool = True,
                 tile_regime: str = "auto", out_fp32: bool = False, fuse_combine: bool = False,
                 fuse_plan: int = 0):
        self.lib = load_library()
        self.cfg = _Config(hidden, intermediate_hidden, num_experts, num_topk, max_num_tokens,
                           float(activation_clamp), FORMATS[fmt], ROUTE_MODES[route_mode], topk_idx_bits,
                           int(bool(fast_math)), TILE_REGIMES[tile_regime], int(bool(out_fp32)),
                           int(bool(fuse_combine)), int(fuse_plan))
        self.fuse_combine = bool(fuse_combine)
        self.fuse_plan = int(fuse_plan)  # 0, 1 (where it pays) or 2 (wherever the sizes allow)
        self.out_fp32 = bool(out_fp32)
        self.fmt, self.route_mode = fmt, route_mode
        self.hidden, self.inter, self.experts, self.topk = hidden, intermediate_hidden, num_experts, num_topk
        self.max_num_tokens = max_num_tokens
        self.topk_idx_bits = topk_idx_bits
        h = ctypes.c_void_p()
        _check(self.lib.moe_create(ctypes.byref(self.cfg), ctypes.byref(h)), "moe_create")
        self._h = h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            self.lib.moe_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---------------------------------------------------------------- argument checks
    def _x_bytes(self, n: int) -> int:
        """Bytes of an activation row of n elements."""
        return {"bf16": 2 * n, "nvfp4_w4a16": 2 * n, "nvfp4": n // 2}.get(self.fmt, n)

    def _x_sf_row(self) -> int:
        """Bytes of activation scales per token."""
        H = self.hidden
        return {"fp8_block128": H // 128 * 4, "w4a8_mx": H // 32, "nvfp4": H // 16}.get(self.fmt, 0)

    def _esz(self) -> int:
        """Bytes per intermediate element."""
        return 2 if self.fmt in ("bf16", "nvfp4_w4a16", "nvfp4") else 1

    def _sf_row(self, n: int) -> int:
        """Bytes of intermediate scales per row of n elements."""
        return {"fp8_block128": n // 128 * 4, "w4a8_mx": n // 32}.get(self.fmt, 0)

    def _idx_dtypes(self):
        import torch
        return (torch.int64,) if self.topk_idx_bits == 64 else (torch.int32,)

    def _check_plan(self, plan: dict, T: int):
        import torch
        E, n = self.experts, T * self.topk
        sizes = {"expert_counts": E, "expert_start_indices": E + 1, "expert_ids": E, "num_active_experts": 1,
                 "src_info": n, "pair_row": n, "status": 1, "combine_counters": T * self._cnt_stride(),
                 "down_split": self.down_split_size() // 4}
        for f in PLAN_FIELDS:
            _need(plan.get(f), f"plan['{f}']", 4 * sizes[f], (torch.int32,),
                  required=f not in ("combine_counters", "down_split"))

    def _check_x(self, x, x_sf, T: int):
        _need(x, "x", T * self._x_bytes(self.hidden))
        _need(x_sf, "x_sf", T * self._x_sf_row(), required=self._x_sf_row() > 0)

    def _check_weights(self, w: dict):
        import torch
        if not hasattr(self, "_psizes"):
            self._psizes = self.prepared_weights_size()
        for n, b in self._psizes.items():
            _need(w.get(n), f"weights['{n}']", b, required=b > 0)
        if self.fmt in ("nvfp4_w4a16", "nvfp4"):
            for g in ("w13_gs", "w2_gs") + (("c_input_scales",) if self.fmt == "nvfp4" else ()):
                _need(w.get(g), f"weights['{g}']", 4 * self.experts, (torch.float32,))

    def _check_routing_in(self, T: int, topk_idx, routing_logits, routing_bias):
        import torch
        if self.route_mode == "precomputed":
            _need(topk_idx, "topk_idx", T * self.topk * self.topk_idx_bits // 8, self._idx_dtypes())
        else:
            _need(routing_logits, "routing_logits", T * self.experts * 4, (torch.float32,))
            _need(routing_bias, "routing_bias", self.experts * 4, (torch.float32,), required=False)

    # ---------------------------------------------------------------- helpers (torch allocation)
    def workspace_size(self, num_tokens: int) -> int:
        return int(self.lib.moe_workspace_size(self._h, num_tokens))

    def down_split_size(self) -> int:
        """Bytes of plan['down_split'] (the down leg's split tail; 0: it never splits)."""
        return int(self.lib.moe_down_split_size(self._h))

    def plan_in_gate_up(self, num_tokens: int) -> bool:
        """Whether plan_ffn_gate_up (and forward with fuse_plan) builds the routing
        plan inside the gate_up launch for num_tokens tokens."""
        return bool(self.lib.moe_plan_in_gate_up(self._h, num_tokens))

    def alloc_workspace(self, num_tokens: int, device="cuda"):
        import torch
        return torch.empty(max(1, self.workspace_size(num_tokens)), dtype=torch.uint8, device=device)

    def prepared_weights_size(self) -> dict:
        ps = _PreparedSizes()
        _check(self.lib.moe_prepared_weights_size(self._h, ctypes.byref(ps)), "moe_prepared_weights_size")
        return {n: int(getattr(ps, n)) for n, _ in _PreparedSizes._fields_}

    def prepare_weights(self, weights: dict, out: dict | None = None, stream=None) -> dict:
        """moe_prepare_weights: canonical weights -> the prepared layout every FFN
        entry point reads.  Allocates the prepared tensors (uint8) unless `out`
        gives them."""
        import torch
        if out is None:
            dev = weights["w13"].device
            out = {n: (torch.empty(b, dtype=torch.uint8, device=dev) if b else None)
                   for n, b in self.prepared_weights_size().items()}
        for g in ("w13_gs", "w2_gs", "c_input_scales"):  # NVFP4 per-expert scales: read as given, no relayout
            if weights.get(g) is not None:
                out.setdefault(g, weights[g])
        cw, pw = self._weights_struct(weights), self._weights_struct(out)
        _check(self.lib.moe_prepare_weights(self._h, ctypes.byref(cw), ctypes.byref(pw), _stream(stream)),
               "moe_prepare_weights")
        return out

    def alloc_plan(self, num_tokens: int, device="cuda") -> dict:
        import torch
        E, np_ = self.experts, max(1, num_tokens * self.topk)
        sizes = {"expert_counts": E, "expert_start_indices": E + 1, "expert_ids": E, "num_active_experts": 1,
                 "src_info": np_, "pair_row": np_, "status": 1,
                 "combine_counters": max(1, num_tokens) * self._cnt_stride()}
        plan = {k: torch.empty(v, dtype=torch.int32, device=device) for k, v in sizes.items()}
        # the down leg's split tail (its counters start at zero; moe_plan zeroes them too)
        if self.down_split_size() > 0:
            plan["down_split"] = torch.zeros(self.down_split_size() // 4, dtype=torch.int32, device=device)
        return plan

    def _cnt_stride(self) -> int:
        """Fused-combine arrival counters per token: ceil(H / 128)."""
        return (self.hidden + 127) // 128

    @staticmethod
    def _plan_struct(plan: dict) -> _Plan:
        return _Plan(*[_ptr(plan.get(f)) for f in PLAN_FIELDS])

    @staticmethod
    def _weights_struct(w: dict) -> _Weights:
        return _Weights(_ptr(w["w13"]), _ptr(w.get("w13_sf")), _ptr(w["w2"]), _ptr(w.get("w2_sf")),
                        _ptr(w.get("w13_gs")), _ptr(w.get("w2_gs")), _ptr(w.get("c_input_scales")))

    @staticmethod
    def _nbytes(t) -> int:
        return 0 if t is None else (t.numel() * t.element_size())

    # ---------------------------------------------------------------- entry points
    def plan(self, num_tokens, plan: dict, topk_idx=None, routing_logits=None, topk_idx_out=None,
             topk_weights_out=None, ws=None, stream=None, routing_bias=None):
        import torch
        T = num_tokens
        self._check_plan(plan, T)
        self._check_routing_in(T, topk_idx, routing_logits, routing_bias)
        if self.route_mode == "from_logits":
            _need(topk_idx_out, "topk_idx_out", T * self.topk * self.topk_idx_bits // 8, self._idx_dtypes())
            _need(topk_weights_out, "topk_weights_out", T * self.topk * 4, (torch.float32,))
        _need(ws, "ws", 0, required=False)
        _on_gpu(plan=plan, topk_idx=topk_idx, routing_logits=routing_logits, topk_idx_out=topk_idx_out,
                topk_weights_out=topk_weights_out, ws=ws, routing_bias=routing_bias)
        ps = self._plan_struct(plan)
        if routing_bias is None:
            _check(self.lib.moe_plan(self._h, num_tokens, _ptr(topk_idx), _ptr(routing_logits), _ptr(topk_idx_out),
                                     _ptr(topk_weights_out), ctypes.byref(ps), _ptr(ws), self._nbytes(ws),
                                     _stream(stream)), "moe_plan")
        else:
            _check(self.lib.moe_plan_ex(self._h, num_tokens, _ptr(topk_idx), _ptr(routing_logits), _ptr(routing_bias),
                                        _ptr(topk_idx_out), _ptr(topk_weights_out), ctypes.byref(ps), _ptr(ws),
                                        self._nbytes(ws), _stream(stream)), "moe_plan_ex")

    def ffn(self, num_tokens, x, x_sf, weights: dict, plan: dict, y, ws, stream=None):
        T = num_tokens
        self._check_x(x, x_sf, T)
        self._check_weights(weights)
        self._check_plan(plan, T)
        _need(y, "y", T * self.topk * self.hidden * 2, elem=2)
        _need(ws, "ws", 0, required=False)
        _on_gpu(x=x, x_sf=x_sf, weights=weights, plan=plan, y=y, ws=ws)
        ws_ = self._weights_struct(weights)
        ps = self._plan_struct(plan)
        _check(self.lib.moe_ffn(self._h, num_tokens, _ptr(x), _ptr(x_sf), ctypes.byref(ws_), ctypes.byref(ps),
                                _ptr(y), _ptr(ws), self._nbytes(ws), _stream(stream)), "moe_ffn")

    def alloc_intermediate(self, num_tokens: int, device="cuda"):
        """(h, h_sf) buffers for moe_ffn_gate_up / moe_ffn_down."""
        import torch
        n = max(1, num_tokens * self.topk)
        if self.fmt in ("bf16", "nvfp4_w4a16", "nvfp4"):
            return torch.empty((n, self.inter), dtype=torch.bfloat16, device=device), None
        h = torch.empty((n, self.inter), dtype=torch.uint8, device=device)
        if self.fmt == "fp8_block128":
            return h, torch.empty((n, self.inter // 128), dtype=torch.float32, device=device)
        return h, torch.empty((n, self.inter // 32), dtype=torch.uint8, device=device)

    def ffn_gate_up(self, num_tokens, x, x_sf, weights: dict, plan: dict, h, h_sf, stream=None, events=None):
        """events: optional (start, stop) torch.cuda.Event pair (timing enabled, already
        created by one record) that the GEMM kernel's own launch updates
        (moe_ffn_gate_up_timed)."""
        T = num_tokens
        self._check_x(x, x_sf, T)
        self._check_weights(weights)
        self._check_plan(plan, T)
        _need(h, "h", T * self.topk * self.inter * self._esz())
        _need(h_sf, "h_sf", T * self.topk * self._sf_row(self.inter), required=self._sf_row(self.inter) > 0)
        _on_gpu(x=x, x_sf=x_sf, weights=weights, plan=plan, h=h, h_sf=h_sf)
        ws_ = self._weights_struct(weights)
        ps = self._plan_struct(plan)
        args = (self._h, num_tokens, _ptr(x), _ptr(x_sf), ctypes.byref(ws_), ctypes.byref(ps), _ptr(h), _ptr(h_sf),
                _stream(stream))
        if events is None:
            _check(self.lib.moe_ffn_gate_up(*args), "moe_ffn_gate_up")
        else:
            _check(self.lib.moe_ffn_gate_up_timed(*args, *_event_handles(events)), "moe_ffn_gate_up_timed")

    def plan_ffn_gate_up(self, num_tokens, x, x_sf, weights: dict, plan: dict, h, h_sf, topk_idx=None,
                         routing_logits=None, topk_idx_out=None, topk_weights_out=None, ws=None, stream=None,
                         events=None):
        """plan() followed by ffn_gate_up(), in one kernel launch where the sizes allow
        (moe_plan_ffn_gate_up); events as for ffn_gate_up."""
        import torch
        T = num_tokens
        self._check_plan(plan, T)
        self._check_routing_in(T, topk_idx, routing_logits, None)
        if self.route_mode == "from_logits":
            _need(topk_idx_out, "topk_idx_out", T * self.topk * self.topk_idx_bits // 8, self._idx_dtypes())
            _need(topk_weights_out, "topk_weights_out", T * self.topk * 4, (torch.float32,))
        _need(ws, "ws", 0, required=False)
        self._check_x(x, x_sf, T)
        self._check_weights(weights)
        _need(h, "h", T * self.topk * self.inter * self._esz())
        _need(h_sf, "h_sf", T * self.topk * self._sf_row(self.inter), required=self._sf_row(self.inter) > 0)
        _on_gpu(plan=plan, topk_idx=topk_idx, routing_logits=routing_logits, topk_idx_out=topk_idx_out,
                topk_weights_out=topk_weights_out, ws=ws, x=x, x_sf=x_sf, weights=weights, h=h, h_sf=h_sf)
        ws_ = self._weights_struct(weights)
        ps = self._plan_struct(plan)
        args = (self._h, num_tokens, _ptr(topk_idx), _ptr(routing_logits), _ptr(topk_idx_out), _ptr(topk_weights_out),
                _ptr(x), _ptr(x_sf), ctypes.byref(ws_), ctypes.byref(ps), _ptr(h), _ptr(h_sf), _ptr(ws),
                self._nbytes(ws), _stream(stream))
        if events is None:
            _check(self.lib.moe_plan_ffn_gate_up(*args), "moe_plan_ffn_gate_up")
        else:
            _check(self.lib.moe_plan_ffn_gate_up_timed(*args, *_event_handles(events)), "moe_plan_ffn_gate_up_timed")

    def ffn_down(self, num_tokens, h, h_sf, weights: dict, plan: dict, y, stream=None, events=None):
        """events: as for ffn_gate_up (moe_ffn_down_timed)."""
        T = num_tokens
        _need(h, "h", T * self.topk * self.inter * self._esz())
        _need(h_sf, "h_sf", T * self.topk * self._sf_row(self.inter), required=self._sf_row(self.inter) > 0)
        self._check_weights(weights)
        self._check_plan(plan, T)
        _need(y, "y", T * self.topk * self.hidden * 2, elem=2)
        _on_gpu(h=h, h_sf=h_sf, weights=weights, plan=plan, y=y)
        ws_ = self._weights_struct(weights)
        ps = self._plan_struct(plan)
        args = (self._h, num_tokens, _ptr(h), _ptr(h_sf), ctypes.byref(ws_), ctypes.byref(ps), _ptr(y),
                _stream(stream))
        if events is None:
            _check(self.lib.moe_ffn_down(*args), "moe_ffn_down")
        else:
            _check(self.lib.moe_ffn_down_timed(*args, *_event_handles(events)), "moe_ffn_down_timed")

    def ffn_down_combine(self, num_tokens, h, h_sf, weights: dict, plan: dict, topk_weights, y, out, stream=None,
                         shared=None, residual=None, events=None):
        """moe_ffn_down_combine(_timed): the down leg with the combine fused into its
        epilogue; plan must hold combine_counters zeroed by moe_plan."""
        import torch
        T = num_tokens
        _need(h, "h", T * self.topk * self.inter * self._esz())
        _need(h_sf, "h_sf", T * self.topk * self._sf_row(self.inter), required=self._sf_row(self.inter) > 0)
        self._check_weights(weights)
        self._check_plan(plan, T)
        _need(plan.get("combine_counters"), "plan['combine_counters']", 4 * T * self._cnt_stride(), (torch.int32,))
        _need(topk_weights, "topk_weights", T * self.topk * 4, (torch.float32,))
        _need(y, "y", T * self.topk * self.hidden * 2, elem=2)
        self._check_out(T, out, shared, residual)
        _on_gpu(h=h, h_sf=h_sf, weights=weights, plan=plan, topk_weights=topk_weights, y=y, out=out, shared=shared,
                residual=residual)
        ws_ = self._weights_struct(weights)
        ps = self._plan_struct(plan)
        args = (self._h, T, _ptr(h), _ptr(h_sf), ctypes.byref(ws_), ctypes.byref(ps), _ptr(topk_weights), _ptr(y),
                _ptr(shared), _ptr(residual), _ptr(out), _stream(stream))
        if events is None:
            _check(self.lib.moe_ffn_down_combine(*args), "moe_ffn_down_combine")
        else:
            _check(self.lib.moe_ffn_down_combine_timed(*args, *_event_handles(events)), "moe_ffn_down_combine_timed")

    def _check_out(self, T, out, shared, residual):
        _need(out, "out", T * self.hidden * (4 if self.out_fp32 else 2), elem=4 if self.out_fp32 else 2)
        _need(shared, "shared", T * self.hidden * 2, elem=2, required=False)
        _need(residual, "residual", T * self.hidden * 2, elem=2, required=False)

    def combine(self, num_tokens, y, topk_weights, plan: dict, out, stream=None, shared=None, residual=None):
        import torch
        T = num_tokens
        _need(y, "y", T * self.topk * self.hidden * 2, elem=2)
        _need(topk_weights, "topk_weights", T * self.topk * 4, (torch.float32,))
        _need(plan.get("pair_row"), "plan['pair_row']", T * self.topk * 4, (torch.int32,))
        self._check_out(T, out, shared, residual)
        _on_gpu(y=y, topk_weights=topk_weights, pair_row=plan.get("pair_row"), out=out, shared=shared,
                residual=residual)
        ps = self._plan_struct(plan)
        if shared is None and residual is None:
            _check(self.lib.moe_combine(self._h, num_tokens, _ptr(y), _ptr(topk_weights), ctypes.byref(ps), _ptr(out),
                                        _stream(stream)), "moe_combine")
        else:
            _check(self.lib.moe_combine_ex(self._h, num_tokens, _ptr(y), _ptr(topk_weights), ctypes.byref(ps),
                                           _ptr(shared), _ptr(residual), _ptr(out), _stream(stream)), "moe_combine_ex")

    def forward(self, num_tokens, x, x_sf, topk_idx, topk_weights, routing_logits, weights: dict, out, ws,
                stream=None, routing_bias=None, shared=None, residual=None):
        import torch
        T = num_tokens
        self._check_x(x, x_sf, T)
        self._check_weights(weights)
        self._check_routing_in(T, topk_idx, routing_logits, routing_bias)
        _need(topk_idx, "topk_idx", T * self.topk * self.topk_idx_bits // 8, self._idx_dtypes())
        _need(topk_weights, "topk_weights", T * self.topk * 4, (torch.float32,))
        self._check_out(T, out, shared, residual)
        _need(ws, "ws", 0, required=False)
        _on_gpu(x=x, x_sf=x_sf, weights=weights, topk_idx=topk_idx, topk_weights=topk_weights,
                routing_logits=routing_logits, routing_bias=routing_bias, out=out, ws=ws, shared=shared,
                residual=residual)
        ws_ = self._weights_struct(weights)
        if routing_bias is None and shared is None and residual is None:
            _check(self.lib.moe_forward(self._h, num_tokens, _ptr(x), _ptr(x_sf), _ptr(topk_idx), _ptr(topk_weights),
                                        _ptr(routing_logits), ctypes.byref(ws_), _ptr(out), _ptr(ws),
                                        self._nbytes(ws), _stream(stream)), "moe_forward")
        else:
            _check(self.lib.moe_forward_ex(self._h, num_tokens, _ptr(x), _ptr(x_sf), _ptr(topk_idx),
                                           _ptr(topk_weights), _ptr(routing_logits), _ptr(routing_bias),
                                           ctypes.byref(ws_), _ptr(shared), _ptr(residual), _ptr(out), _ptr(ws),
                                           self._nbytes(ws), _stream(stream)), "moe_forward_ex")

    def forward_static(self, num_tokens, x, x_sf, topk_idx, topk_weights, routing_logits, weights: dict, out,
                       stream=None):
        """moe_forward_static: moe_forward with the library's per-device static scratch
        as its workspace (no allocation; calls on one device share that scratch)."""
        import torch
        T = num_tokens
        self._check_x(x, x_sf, T)
        self._check_weights(weights)
        self._check_routing_in(T, topk_idx, routing_logits, None)
        _need(topk_idx, "topk_idx", T * self.topk * self.topk_idx_bits // 8, self._idx_dtypes())
        _need(topk_weights, "topk_weights", T * self.topk * 4, (torch.float32,))
        self._check_out(T, out, None, None)
        _on_gpu(x=x, x_sf=x_sf, weights=weights, topk_idx=topk_idx, topk_weights=topk_weights,
                routing_logits=routing_logits, out=out)
        ws_ = self._weights_struct(weights)
        _check(self.lib.moe_forward_static(self._h, num_tokens, _ptr(x), _ptr(x_sf), _ptr(topk_idx),
                                           _ptr(topk_weights), _ptr(routing_logits), ctypes.byref(ws_), _ptr(out),
                                           _stream(stream)), "moe_forward_static")


__all__ = ["MoEFFN", "MoEError", "load_library", "LIB_PATH", "EXPORTED", "FORMATS", "ROUTE_MODES", "TILE_REGIMES"]
