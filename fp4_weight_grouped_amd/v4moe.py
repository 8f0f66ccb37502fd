"""ctypes binding of libv4moe (``include/v4moe.h``).

Argument marshalling only: every function forwards torch device tensors'
pointers and the current HIP stream to the C entry point of the same name and
raises :class:`V4MoeError` on a non-zero return code.  PyTorch provides device
memory and streams; every step of the layer runs in the library's kernels.
The library must have been built (``fp4_weight_grouped_amd.build``); there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import re
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(HERE, "libv4moe.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "v4moe.h")

ROUTE_LEARNED = 0
ROUTE_HASH = 1

ACT_SWIGLU = 0
ACT_RELU2 = 1
ACT_RELU = 2


class V4MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libv4moe error {code}: {msg}")
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("topk", ctypes.c_int32), ("act", ctypes.c_int32)]


class Mat(ctypes.Structure):
    _fields_ = [("fp4", ctypes.c_void_p), ("e8m0", ctypes.c_void_p), ("blk", ctypes.c_void_p)]


class ExpertsC(ctypes.Structure):
    _fields_ = [("gate", Mat), ("up", Mat), ("down", Mat)]


_lib = None
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t
_DP = ctypes.POINTER(Dims)


def lib():
    """Load libv4moe.so; raise if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(SO):
            raise RuntimeError(f"{SO} is missing: build it with fp4_weight_grouped_amd.build.build()")
        L = ctypes.CDLL(SO)
        L.moe_workspace_bytes.argtypes = [_DP]
        L.moe_workspace_bytes.restype = _sz
        L.moe_strerror.argtypes = [ctypes.c_int]
        L.moe_strerror.restype = ctypes.c_char_p
        L.moe_route.argtypes = [_DP, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _sz, _vp]
        L.moe_permute.argtypes = [_DP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        L.moe_expert_ffn.argtypes = [_DP, _vp, _vp, _vp, _vp, ctypes.POINTER(ExpertsC), _vp, _vp, _sz, _vp]
        L.moe_combine.argtypes = [_DP, _vp, _vp, _vp, _vp]
        L.moe_layer_forward.argtypes = [_DP, _vp, _vp, _vp, _i32, _vp, ctypes.POINTER(ExpertsC),
                                        _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        L.moe_prepack_weights.argtypes = [_DP, ctypes.POINTER(ExpertsC), ctypes.POINTER(ExpertsC),
                                          _vp, _sz, _vp]
        L.moe_dequant_fp8.argtypes = [ctypes.POINTER(Mat), _i32, _i32, _i32, _vp, _vp]
        L.moe_quantize_weights.argtypes = [_i32, _i32, _i32, _vp, _i32, ctypes.POINTER(Mat), _vp, _vp]
        L.moe_backward_workspace_bytes.argtypes = [_DP]
        L.moe_backward_workspace_bytes.restype = _sz
        L.moe_transpose_weights.argtypes = [_DP, ctypes.POINTER(ExpertsC), _vp, _vp, _vp]
        L.moe_layer_backward.argtypes = [_DP, _vp, _vp, _vp, _i32, _vp, ctypes.POINTER(ExpertsC), _vp, _vp,
                                         _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        L.moe_layer_forward_noalloc.argtypes = [_DP, _vp, _vp, _vp, _i32, _vp, ctypes.POINTER(ExpertsC),
                                                _vp, _vp, _vp, _vp, _vp]
        L.moe_noalloc_max_workspace_bytes.argtypes = []
        L.moe_noalloc_max_workspace_bytes.restype = _sz
        L.moe_time_next_ffn.argtypes = [_vp, _vp]
        L.moe_time_next_ffn.restype = None
        for f in ("moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_layer_forward",
                  "moe_layer_forward_noalloc",
                  "moe_prepack_weights", "moe_dequant_fp8", "moe_quantize_weights", "moe_transpose_weights",
                  "moe_layer_backward"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def declared_functions() -> list:
    """Names of the functions declared in include/v4moe.h."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def strerror(code: int) -> str:
    return lib().moe_strerror(code).decode()


def _check(rc: int):
    if rc != 0:
        raise V4MoeError(rc, strerror(rc))


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def dims(T: int, H: int, I: int, E: int, topk: int, act: int = ACT_SWIGLU) -> Dims:
    return Dims(T, H, I, E, topk, act)


@dataclasses.dataclass
class DeviceMatrix:
    fp4: torch.Tensor   # uint8
    e8m0: torch.Tensor  # uint8
    blk: torch.Tensor   # float32

    def c(self) -> Mat:
        return Mat(self.fp4.data_ptr(), self.e8m0.data_ptr(), self.blk.data_ptr())


@dataclasses.dataclass
class DeviceExperts:
    gate: Optional[DeviceMatrix]   # None for the gate-less activations
    up: DeviceMatrix
    down: DeviceMatrix

    def c(self) -> ExpertsC:
        return ExpertsC(Mat() if self.gate is None else self.gate.c(), self.up.c(), self.down.c())


# ---- the C entry points ------------------------------------------------------------------
def moe_workspace_bytes(d: Dims) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(d)))


def moe_route(d: Dims, x, w_router, bias, mode, token_ids, topk_ids, topk_w, workspace):
    _check(lib().moe_route(ctypes.byref(d), _p(x), _p(w_router), _p(bias), mode, _p(token_ids),
                           _p(topk_ids), _p(topk_w), _p(workspace),
                           0 if workspace is None else workspace.numel(), _stream()))


def moe_permute(d: Dims, x, topk_ids, expert_offsets, sorted_pair, pair_pos, xq, xs, workspace):
    _check(lib().moe_permute(ctypes.byref(d), _p(x), _p(topk_ids), _p(expert_offsets), _p(sorted_pair),
                             _p(pair_pos), _p(xq), _p(xs), _p(workspace), workspace.numel(), _stream()))


def moe_expert_ffn(d: Dims, xq, xs, expert_offsets, sorted_pair, experts: DeviceExperts, y, workspace):
    ex = experts.c()
    _check(lib().moe_expert_ffn(ctypes.byref(d), _p(xq), _p(xs), _p(expert_offsets), _p(sorted_pair),
                                ctypes.byref(ex), _p(y), _p(workspace), workspace.numel(), _stream()))


def moe_combine(d: Dims, y, topk_w, out):
    _check(lib().moe_combine(ctypes.byref(d), _p(y), _p(topk_w), _p(out), _stream()))


def moe_layer_forward(d: Dims, x, w_router, bias, mode, token_ids, experts: DeviceExperts,
                      topk_ids, topk_w, expert_offsets, out, workspace):
    ex = experts.c()
    _check(lib().moe_layer_forward(ctypes.byref(d), _p(x), _p(w_router), _p(bias), mode, _p(token_ids),
                                   ctypes.byref(ex), _p(topk_ids), _p(topk_w), _p(expert_offsets),
                                   _p(out), _p(workspace), workspace.numel(), _stream()))


def moe_layer_forward_noalloc(d: Dims, x, w_router, bias, mode, token_ids, experts: DeviceExperts,
                              topk_ids, topk_w, expert_offsets, out):
    ex = experts.c()
    _check(lib().moe_layer_forward_noalloc(ctypes.byref(d), _p(x), _p(w_router), _p(bias), mode, _p(token_ids),
                                           ctypes.byref(ex), _p(topk_ids), _p(topk_w), _p(expert_offsets),
                                           _p(out), _stream()))


def moe_noalloc_max_workspace_bytes() -> int:
    return lib().moe_noalloc_max_workspace_bytes()


def moe_prepack_weights(d: Dims, canonical: DeviceExperts, packed: DeviceExperts, workspace):
    a, b = canonical.c(), packed.c()
    _check(lib().moe_prepack_weights(ctypes.byref(d), ctypes.byref(a), ctypes.byref(b), _p(workspace),
                                     workspace.numel(), _stream()))


def moe_dequant_fp8(m: DeviceMatrix, N: int, K: int, expert: int, out):
    mc = m.c()
    _check(lib().moe_dequant_fp8(ctypes.byref(mc), N, K, expert, _p(out), _stream()))


def moe_quantize_weights(w, out: DeviceMatrix, clamped=None, packed: bool = False):
    """w: fp32 [E][N][K] on the device -> out (fp4 and e8m0 in the canonical
    or the packed layout, blk [E][N/128][K/128]); clamped: int64 [1] device
    tensor the number of clamped sub-blocks is added to, or None."""
    E, N, K = w.shape
    oc = out.c()
    _check(lib().moe_quantize_weights(E, N, K, _p(w), 1 if packed else 0, ctypes.byref(oc), _p(clamped),
                                      _stream()))


def quantize_weights(w, clamped=None, packed: bool = False) -> DeviceMatrix:
    """Allocating convenience around moe_quantize_weights (the packed layout
    has the same byte counts as the canonical one)."""
    E, N, K = w.shape
    dev = w.device
    out = DeviceMatrix(fp4=torch.empty((E, N, K // 2), dtype=torch.uint8, device=dev),
                       e8m0=torch.empty((E, N, K // 32), dtype=torch.uint8, device=dev),
                       blk=torch.empty((E, N // 128, K // 128), dtype=torch.float32, device=dev))
    moe_quantize_weights(w, out, clamped, packed)
    return out


def moe_backward_workspace_bytes(d: Dims) -> int:
    return int(lib().moe_backward_workspace_bytes(ctypes.byref(d)))


def moe_transpose_weights(d: Dims, experts: DeviceExperts, wt_gu, wt_d):
    ex = experts.c()
    _check(lib().moe_transpose_weights(ctypes.byref(d), ctypes.byref(ex), _p(wt_gu), _p(wt_d), _stream()))


def moe_layer_backward(d: Dims, x, w_router, bias, mode, token_ids, experts: DeviceExperts, wt_gu, wt_d, dout,
                       dx, dw, dWg, dWu, dWd, workspace):
    ex = experts.c()
    _check(lib().moe_layer_backward(ctypes.byref(d), _p(x), _p(w_router), _p(bias), mode, _p(token_ids),
                                    ctypes.byref(ex), _p(wt_gu), _p(wt_d), _p(dout), _p(dx), _p(dw), _p(dWg),
                                    _p(dWu), _p(dWd), _p(workspace), workspace.numel(), _stream()))


def moe_time_next_ffn(start_event, stop_event):
    """start/stop: torch.cuda.Event(enable_timing=True) objects, or None."""
    a = None if start_event is None else ctypes.c_void_p(start_event.cuda_event)
    b = None if stop_event is None else ctypes.c_void_p(stop_event.cuda_event)
    lib().moe_time_next_ffn(a, b)


# ---- conveniences for callers holding host (numpy) weights ----------------------------------
def upload_matrix(m, device="cuda") -> DeviceMatrix:
    return DeviceMatrix(fp4=torch.from_numpy(m.fp4).to(device),
                        e8m0=torch.from_numpy(m.e8m0).to(device),
                        blk=torch.from_numpy(m.blk).to(device))


def prepack(d: Dims, canonical: DeviceExperts) -> DeviceExperts:
    """Canonical -> packed device weights (blk tensors are shared)."""
    def like(m: Optional[DeviceMatrix]) -> Optional[DeviceMatrix]:
        if m is None:
            return None
        return DeviceMatrix(torch.empty_like(m.fp4), torch.empty_like(m.e8m0), m.blk)
    packed = DeviceExperts(like(canonical.gate), like(canonical.up), like(canonical.down))
    ws = torch.empty(256, dtype=torch.uint8, device=canonical.up.fp4.device)
    moe_prepack_weights(d, canonical, packed, ws)
    return packed


def upload_experts(ex, d: Dims, device="cuda") -> DeviceExperts:
    """Host canonical weights (objects with gate/up/down, each fp4/e8m0/blk numpy
    arrays) -> packed device weights."""
    canon = DeviceExperts(None if ex.gate is None else upload_matrix(ex.gate, device), upload_matrix(ex.up, device),
                          upload_matrix(ex.down, device))
    packed = prepack(d, canon)
    del canon
    return packed


class MoELayer:
    """Device-resident layer: packed expert weights, router and a workspace."""

    def __init__(self, H: int, I: int, E: int, topk: int, experts: DeviceExperts,
                 w_router: torch.Tensor, device="cuda", act: int = ACT_SWIGLU):
        self.H, self.I, self.E, self.topk, self.act = H, I, E, topk, act
        self.experts = experts
        self.w_router = w_router
        self.device = device
        self._ws = None

    def dims(self, T: int) -> Dims:
        return Dims(T, self.H, self.I, self.E, self.topk, self.act)

    def workspace(self, T: int) -> torch.Tensor:
        n = moe_workspace_bytes(self.dims(T))
        if self._ws is None or self._ws.numel() < n:
            self._ws = torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    def forward(self, x: torch.Tensor, bias=None, mode=ROUTE_LEARNED, token_ids=None, out=None):
        """x: uint16 (bf16 bits) or bfloat16 [T][H] on the device.
        Returns (out bf16 bits [T][H], topk_ids, topk_w, expert_offsets)."""
        T = x.shape[0]
        d = self.dims(T)
        dev = self.device
        ids = torch.empty((T, self.topk), dtype=torch.int32, device=dev)
        w = torch.empty((T, self.topk), dtype=torch.float32, device=dev)
        off = torch.empty(self.E + 1, dtype=torch.int32, device=dev)
        if out is None:
            out = torch.empty((T, self.H), dtype=torch.int16, device=dev)
        moe_layer_forward(d, x, self.w_router, bias, mode, token_ids, self.experts, ids, w, off, out,
                          self.workspace(T))
        return out, ids, w, off

    def transposed_weights(self):
        """The transposed FP8 weight values (E4M3 bytes) the backward reads (made once)."""
        if getattr(self, "_wt", None) is None:
            d = self.dims(1)
            gI = 2 * self.I if self.act == ACT_SWIGLU else self.I
            wt_gu = torch.empty((self.E, self.H, gI), dtype=torch.uint8, device=self.device)
            wt_d = torch.empty((self.E, self.I, self.H), dtype=torch.uint8, device=self.device)
            moe_transpose_weights(d, self.experts, wt_gu, wt_d)
            self._wt = (wt_gu, wt_d)
        return self._wt

    def backward(self, x: torch.Tensor, dout: torch.Tensor, bias=None, mode=ROUTE_LEARNED, token_ids=None,
                 grads=None):
        """Gradients of sum(dout * out): dict(dx [T][H], dw [T][k], dWg / dWu [E][I][H], dWd [E][H][I])
        (fp32; dWg absent gate-less).  ``grads`` may hold preallocated outputs."""
        T = x.shape[0]
        d = self.dims(T)
        dev = self.device
        gated = self.act == ACT_SWIGLU
        g = grads or dict(
            dx=torch.empty((T, self.H), dtype=torch.float32, device=dev),
            dw=torch.empty((T, self.topk), dtype=torch.float32, device=dev),
            dWu=torch.empty((self.E, self.I, self.H), dtype=torch.float32, device=dev),
            dWd=torch.empty((self.E, self.H, self.I), dtype=torch.float32, device=dev),
            **({"dWg": torch.empty((self.E, self.I, self.H), dtype=torch.float32, device=dev)} if gated else {}))
        n = moe_backward_workspace_bytes(d)
        if getattr(self, "_bws", None) is None or self._bws.numel() < n:
            self._bws = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
        wt_gu, wt_d = self.transposed_weights()
        moe_layer_backward(d, x, self.w_router, bias, mode, token_ids, self.experts, wt_gu, wt_d, dout,
                           g["dx"], g["dw"], g.get("dWg"), g["dWu"], g["dWd"], self._bws)
        return g

    def forward_unfused(self, x: torch.Tensor, bias=None, mode=ROUTE_LEARNED, token_ids=None):
        """The same layer through the four separate entry points."""
        T = x.shape[0]
        d = self.dims(T)
        dev = self.device
        P = T * self.topk
        ids = torch.empty((T, self.topk), dtype=torch.int32, device=dev)
        w = torch.empty((T, self.topk), dtype=torch.float32, device=dev)
        off = torch.empty(self.E + 1, dtype=torch.int32, device=dev)
        sp = torch.empty(max(P, 1), dtype=torch.int32, device=dev)
        pp = torch.empty(max(P, 1), dtype=torch.int32, device=dev)
        xq = torch.empty((max(T, 1), self.H), dtype=torch.uint8, device=dev)
        xs = torch.empty((max(T, 1), self.H // 128), dtype=torch.float32, device=dev)
        y = torch.empty((max(P, 1), self.H), dtype=torch.int16, device=dev)
        out = torch.empty((T, self.H), dtype=torch.int16, device=dev)
        ws = self.workspace(T)
        moe_route(d, x, self.w_router, bias, mode, token_ids, ids, w, ws)
        moe_permute(d, x, ids, off, sp, pp, xq, xs, ws)
        moe_expert_ffn(d, xq, xs, off, sp, self.experts, y, ws)
        moe_combine(d, y, w, out)
        return dict(out=out, ids=ids, w=w, offsets=off, sorted_pair=sp[:P], pair_pos=pp[:P],
                    xq=xq[:T], xs=xs[:T], y=y[:P])
