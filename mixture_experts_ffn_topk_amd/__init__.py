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
FORMATS = {"fp8_block128": 0, "bf16": 1, "w4a8_mx": 2, "nvfp4_w4a16": 3}
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
                ("tile_regime", ctypes.c_int32)]


class _Weights(ctypes.Structure):
    _fields_ = [("w13", ctypes.c_void_p), ("w13_sf", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w2_sf", ctypes.c_void_p),
                ("w13_gs", ctypes.c_void_p), ("w2_gs", ctypes.c_void_p)]


class _Plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("expert_counts", "expert_start_indices", "expert_ids",
                                               "num_active_experts", "src_info", "pair_row", "status")]


class _PreparedSizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("w13", "w13_sf", "w2", "w2_sf")]


PLAN_FIELDS = [f for f, _ in _Plan._fields_]
EXPORTED = ["moe_create", "moe_destroy", "moe_workspace_size", "moe_prepared_weights_size", "moe_prepare_weights",
            "moe_plan", "moe_ffn", "moe_ffn_gate_up", "moe_ffn_down", "moe_combine", "moe_forward",
            "moe_plan_ex", "moe_combine_ex", "moe_forward_ex", "moe_ffn_gate_up_timed", "moe_ffn_down_timed",
            "moe_status_string", "moe_abi_version"]

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
    lib.moe_ffn_down_timed.argtypes = lib.moe_ffn_down.argtypes + [vp, vp]
    lib.moe_ffn_down_timed.restype = i32
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


class MoEFFN:
    """One GPU's share of experts with a fixed geometry (moe_create / moe_destroy).

    Tensors are torch tensors on the GPU (or raw device addresses as ints); their
    dtype and layout must match include/moe_ffn.h — the binding only forwards
    pointers."""

    def __init__(self, hidden: int, intermediate_hidden: int, num_experts: int, num_topk: int,
                 max_num_tokens: int, fmt: str = "fp8_block128", route_mode: str = "precomputed",
                 activation_clamp: float = 10.0, topk_idx_bits: int = 64, fast_math: bool = True,
                 tile_regime: str = "auto"):
        self.lib = load_library()
        self.cfg = _Config(hidden, intermediate_hidden, num_experts, num_topk, max_num_tokens,
                           float(activation_clamp), FORMATS[fmt], ROUTE_MODES[route_mode], topk_idx_bits,
                           int(bool(fast_math)), TILE_REGIMES[tile_regime])
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

    # ---------------------------------------------------------------- helpers (torch allocation)
    def workspace_size(self, num_tokens: int) -> int:
        return int(self.lib.moe_workspace_size(self._h, num_tokens))

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
        for g in ("w13_gs", "w2_gs"):  # NVFP4 global scales: read as given, no relayout
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
                 "src_info": np_, "pair_row": np_, "status": 1}
        return {k: torch.empty(v, dtype=torch.int32, device=device) for k, v in sizes.items()}

    @staticmethod
    def _plan_struct(plan: dict) -> _Plan:
        return _Plan(*[_ptr(plan[f]) for f in PLAN_FIELDS])

    @staticmethod
    def _weights_struct(w: dict) -> _Weights:
        return _Weights(_ptr(w["w13"]), _ptr(w.get("w13_sf")), _ptr(w["w2"]), _ptr(w.get("w2_sf")),
                        _ptr(w.get("w13_gs")), _ptr(w.get("w2_gs")))

    @staticmethod
    def _nbytes(t) -> int:
        return 0 if t is None else (t.numel() * t.element_size())

    # ---------------------------------------------------------------- entry points
    def plan(self, num_tokens, plan: dict, topk_idx=None, routing_logits=None, topk_idx_out=None,
             topk_weights_out=None, ws=None, stream=None, routing_bias=None):
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
        ws_ = self._weights_struct(weights)
        ps = self._plan_struct(plan)
        _check(self.lib.moe_ffn(self._h, num_tokens, _ptr(x), _ptr(x_sf), ctypes.byref(ws_), ctypes.byref(ps),
                                _ptr(y), _ptr(ws), self._nbytes(ws), _stream(stream)), "moe_ffn")

    def alloc_intermediate(self, num_tokens: int, device="cuda"):
        """(h, h_sf) buffers for moe_ffn_gate_up / moe_ffn_down."""
        import torch
        n = max(1, num_tokens * self.topk)
        if self.fmt in ("bf16", "nvfp4_w4a16"):
            return torch.empty((n, self.inter), dtype=torch.bfloat16, device=device), None
        h = torch.empty((n, self.inter), dtype=torch.uint8, device=device)
        if self.fmt == "fp8_block128":
            return h, torch.empty((n, self.inter // 128), dtype=torch.float32, device=device)
        return h, torch.empty((n, self.inter // 32), dtype=torch.uint8, device=device)

    def ffn_gate_up(self, num_tokens, x, x_sf, weights: dict, plan: dict, h, h_sf, stream=None, events=None):
        """events: optional (start, stop) torch.cuda.Event pair (timing enabled, already
        created by one record) that the GEMM kernel's own launch updates
        (moe_ffn_gate_up_timed)."""
        ws_ = self._weights_struct(weights)
        ps = self._plan_struct(plan)
        args = (self._h, num_tokens, _ptr(x), _ptr(x_sf), ctypes.byref(ws_), ctypes.byref(ps), _ptr(h), _ptr(h_sf),
                _stream(stream))
        if events is None:
            _check(self.lib.moe_ffn_gate_up(*args), "moe_ffn_gate_up")
        else:
            _check(self.lib.moe_ffn_gate_up_timed(*args, *_event_handles(events)), "moe_ffn_gate_up_timed")

    def ffn_down(self, num_tokens, h, h_sf, weights: dict, plan: dict, y, stream=None, events=None):
        """events: as for ffn_gate_up (moe_ffn_down_timed)."""
        ws_ = self._weights_struct(weights)
        ps = self._plan_struct(plan)
        args = (self._h, num_tokens, _ptr(h), _ptr(h_sf), ctypes.byref(ws_), ctypes.byref(ps), _ptr(y),
                _stream(stream))
        if events is None:
            _check(self.lib.moe_ffn_down(*args), "moe_ffn_down")
        else:
            _check(self.lib.moe_ffn_down_timed(*args, *_event_handles(events)), "moe_ffn_down_timed")

    def combine(self, num_tokens, y, topk_weights, plan: dict, out, stream=None, shared=None, residual=None):
        ps = self._plan_struct(plan)
        if shared is None and residual is None:
            _check(self.lib.moe_combine(self._h, num_tokens, _ptr(y), _ptr(topk_weights), ctypes.byref(ps), _ptr(out),
                                        _stream(stream)), "moe_combine")
        else:
            _check(self.lib.moe_combine_ex(self._h, num_tokens, _ptr(y), _ptr(topk_weights), ctypes.byref(ps),
                                           _ptr(shared), _ptr(residual), _ptr(out), _stream(stream)), "moe_combine_ex")

    def forward(self, num_tokens, x, x_sf, topk_idx, topk_weights, routing_logits, weights: dict, out, ws,
                stream=None, routing_bias=None, shared=None, residual=None):
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


__all__ = ["MoEFFN", "MoEError", "load_library", "LIB_PATH", "EXPORTED", "FORMATS", "ROUTE_MODES", "TILE_REGIMES"]
