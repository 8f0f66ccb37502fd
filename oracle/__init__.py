"""Python access to the CPU oracle (``oracle/v4moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark use it to check the HIP library; the library itself never
imports, loads or calls anything here.

The C source is compiled with gcc into ``oracle/liboracle.so`` by
:func:`build`; :func:`lib` builds it on first use if it is missing.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "v4moe_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

# -mfma: fmaf() is a single instruction (glibc's fmaf is also exact, only slower).
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-mfma", "-mavx2",
          "-fopenmp", "-fPIC", "-shared", "-fvisibility=hidden", "-std=c11"]


def build(force: bool = True) -> str:
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None

u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
vp = ctypes.c_void_p
ci = ctypes.c_int


# Activations (orc_layer_forward's act): SwiGLU, and the gate-less squared
# ReLU and ReLU.
ACT_SWIGLU = 0
ACT_RELU2 = 1
ACT_RELU = 2


class OrcWeights(ctypes.Structure):
    _fields_ = [("fp4", vp * 3), ("e8m0", vp * 3), ("blk", vp * 3)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_SO)
        L.orc_num_threads.argtypes = []
        L.orc_num_threads.restype = ci
        L.orc_e2m1_value.argtypes = [ci]; L.orc_e2m1_value.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [ci]; L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_encode.argtypes = [ctypes.c_double]; L.orc_e4m3_encode.restype = ci
        L.orc_bf16_encode.argtypes = [ctypes.c_float]; L.orc_bf16_encode.restype = ctypes.c_uint16
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]; L.orc_bf16_value.restype = ctypes.c_float
        L.orc_e4m3_encode_array.argtypes = [ctypes.c_int64, f64p, u8p]
        L.orc_e4m3_encode_array.restype = None
        L.orc_bf16_encode_array.argtypes = [ctypes.c_int64, f32p, u16p]
        L.orc_bf16_encode_array.restype = None
        L.orc_dequant_code.argtypes = [ci, ci]; L.orc_dequant_code.restype = ci
        L.orc_dequant_bitmap.argtypes = [ci, ci]; L.orc_dequant_bitmap.restype = ci
        L.orc_dequant_matrix.argtypes = [ci, ci, u8p, u8p, u8p]; L.orc_dequant_matrix.restype = None
        L.orc_router_logits.argtypes = [ci, ci, ci, u16p, f32p, vp, f32p]
        L.orc_router_logits.restype = None
        L.orc_splitmix64.argtypes = [ctypes.c_uint64]; L.orc_splitmix64.restype = ctypes.c_uint64
        L.orc_route.argtypes = [ci, ci, ci, ci, u16p, f32p, vp, ci, vp, i32p, f32p]
        L.orc_route.restype = None
        L.orc_quant_rows.argtypes = [ci, ci, f32p, u8p, f32p]; L.orc_quant_rows.restype = None
        L.orc_quant_x.argtypes = [ci, ci, u16p, u8p, f32p]; L.orc_quant_x.restype = None
        L.orc_permute.argtypes = [ci, ci, ci, i32p, i32p, i32p, i32p]; L.orc_permute.restype = None
        L.orc_e2m1_encode.argtypes = [ctypes.c_double]; L.orc_e2m1_encode.restype = ci
        L.orc_quantize_weights.argtypes = [ci, ci, ci, f32p, u8p, u8p, f32p]
        L.orc_quantize_weights.restype = ctypes.c_int64
        L.orc_layer_forward.argtypes = [ci, ci, ci, ci, ci, ci, u16p, f32p, vp, ci, vp,
                                        ctypes.POINTER(OrcWeights), i32p, f32p, i32p, i32p, i32p,
                                        u8p, f32p, vp, vp, vp, vp, ci]
        L.orc_layer_forward.restype = ci
        L.orc_layer_backward.argtypes = [ci, ci, ci, ci, ci, ci, u16p, f32p, vp, ci, vp,
                                         ctypes.POINTER(OrcWeights), u16p, vp, vp, vp, vp, vp, vp, ci, vp, ci]
        L.orc_layer_backward.restype = ci
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return lib().orc_num_threads()


# ---- scalar format helpers ----------------------------------------------------------
def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(code)


def e4m3_value(byte: int) -> float:
    return lib().orc_e4m3_value(byte)


def e4m3_encode(v: float) -> int:
    return lib().orc_e4m3_encode(float(v))


def bf16_encode(f: float) -> int:
    return lib().orc_bf16_encode(f)


def bf16_value(b: int) -> float:
    return lib().orc_bf16_value(b)


def dequant_code(code: int, b: int) -> int:
    return lib().orc_dequant_code(code, b)


def dequant_bitmap(code: int, b: int) -> int:
    return lib().orc_dequant_bitmap(code, b)


def splitmix64(v: int) -> int:
    return lib().orc_splitmix64(v)


# ---- array helpers ----------------------------------------------------------------
def e4m3_encode_array(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64).ravel()
    out = np.empty(v.size, np.uint8)
    lib().orc_e4m3_encode_array(v.size, v, out)
    return out


def bf16_encode_array(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32).ravel()
    out = np.empty(v.size, np.uint16)
    lib().orc_bf16_encode_array(v.size, v, out)
    return out


def dequant_matrix(fp4: np.ndarray, e8m0: np.ndarray) -> np.ndarray:
    """Canonical [N][K/2] FP4 + [N][K/32] E8M0 -> E4M3 bytes [N][K]."""
    N, K2 = fp4.shape
    out = np.empty((N, 2 * K2), np.uint8)
    lib().orc_dequant_matrix(N, 2 * K2, np.ascontiguousarray(fp4), np.ascontiguousarray(e8m0), out)
    return out


def router_logits(x, wr, bias=None) -> np.ndarray:
    T, H = x.shape
    E = wr.shape[1]
    z = np.empty((T, E), np.float32)
    lib().orc_router_logits(T, H, E, np.ascontiguousarray(x), np.ascontiguousarray(wr),
                            _ptr(bias), z)
    return z


def route(x, wr, k, bias=None, mode=0, token_ids=None, E=None):
    T, H = x.shape
    E = wr.shape[1] if E is None else E
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    tid = None if token_ids is None else np.ascontiguousarray(token_ids, dtype=np.int64)
    lib().orc_route(T, H, E, k, np.ascontiguousarray(x), np.ascontiguousarray(wr),
                    _ptr(bias), mode, _ptr(tid), ids, w)
    return ids, w


def quant_rows(v: np.ndarray):
    R, C = v.shape
    q = np.empty((R, C), np.uint8)
    s = np.empty((R, C // 128), np.float32)
    lib().orc_quant_rows(R, C, np.ascontiguousarray(v, dtype=np.float32), q, s)
    return q, s


def e2m1_encode(v: float) -> int:
    return lib().orc_e2m1_encode(float(v))


def quantize_weights(w: np.ndarray):
    """FP32 master weights [E][N][K] -> (fp4 [E][N][K/2], e8m0 [E][N][K/32],
    blk [E][N/128][K/128], clamped sub-block count), canonical layout."""
    E, N, K = w.shape
    fp4 = np.empty((E, N, K // 2), np.uint8)
    e8 = np.empty((E, N, K // 32), np.uint8)
    blk = np.empty((E, N // 128, K // 128), np.float32)
    clamped = lib().orc_quantize_weights(E, N, K, np.ascontiguousarray(w, dtype=np.float32), fp4, e8, blk)
    return fp4, e8, blk, int(clamped)


def quant_x(x: np.ndarray):
    T, H = x.shape
    q = np.empty((T, H), np.uint8)
    s = np.empty((T, H // 128), np.float32)
    lib().orc_quant_x(T, H, np.ascontiguousarray(x), q, s)
    return q, s


def permute(ids: np.ndarray, E: int):
    T, k = ids.shape
    off = np.empty(E + 1, np.int32)
    sp = np.empty(T * k, np.int32)
    pp = np.empty(T * k, np.int32)
    lib().orc_permute(T, k, E, np.ascontiguousarray(ids, dtype=np.int32), off, sp, pp)
    return off, sp, pp


def layer_forward(inp, subset=None, want_y=False, exact=False, k=None):
    """Run the whole layer on an :class:`fp4_weight_grouped_amd.inputs.Inputs`.

    Returns a dict with ids, w, offsets, sorted_pair, pair_pos, xq, xs, out
    (bf16 bits [T][H]) and, on request, y (bf16 bits [T*k][H]) and out_exact.
    With ``subset`` (token indices) only those rows of y/out are computed.
    """
    d = inp.dims
    T, H, I, E = d.T, d.H, d.I, d.E
    k = d.topk if k is None else k
    ex = inp.experts
    keep = []

    def c(a):
        a = np.ascontiguousarray(a)
        keep.append(a)
        return a.ctypes.data_as(ctypes.c_void_p)

    Wt = OrcWeights()
    for i, m in enumerate((ex.gate, ex.up, ex.down)):
        if m is None:            # gate-less activations: no gate matrix
            continue
        Wt.fp4[i] = c(m.fp4)
        Wt.e8m0[i] = c(m.e8m0)
        Wt.blk[i] = c(m.blk)
    res = dict(
        ids=np.empty((T, k), np.int32), w=np.empty((T, k), np.float32),
        offsets=np.empty(E + 1, np.int32), sorted_pair=np.empty(T * k, np.int32),
        pair_pos=np.empty(T * k, np.int32), xq=np.empty((T, H), np.uint8),
        xs=np.empty((T, H // 128), np.float32),
        out=np.zeros((T, H), np.uint16),
    )
    y = np.zeros((T * k, H), np.uint16) if want_y else None
    oex = np.zeros((T, H), np.float64) if exact else None
    sub = None if subset is None else np.ascontiguousarray(subset, dtype=np.int32)
    tid = None if inp.token_ids is None else np.ascontiguousarray(inp.token_ids, dtype=np.int64)
    bias = None if inp.bias is None else np.ascontiguousarray(inp.bias, dtype=np.float32)
    act = getattr(d, "act", ACT_SWIGLU)
    assert act != ACT_SWIGLU or ex.gate is not None
    lib().orc_layer_forward(T, H, I, E, k, act, np.ascontiguousarray(inp.x),
                            np.ascontiguousarray(inp.w_router), _ptr(bias), inp.mode, _ptr(tid),
                            ctypes.byref(Wt), res["ids"], res["w"], res["offsets"],
                            res["sorted_pair"], res["pair_pos"], res["xq"], res["xs"],
                            _ptr(y), _ptr(res["out"]), _ptr(oex),
                            _ptr(sub), 0 if sub is None else len(sub))
    if want_y:
        res["y"] = y
    if exact:
        res["out_exact"] = oex
    return res


def layer_backward(inp, dout, tokens=None, experts=None, want_dw=True):
    """Gradients of sum(dout * out) for the layer on ``inp`` (straight-through
    quantisation, the router not differentiated).  ``dout``: bf16 bits [T][H].

    Returns dict(dx [T][H] f64, dw [T][k] f64, dWg / dWu [n][I][H] and
    dWd [n][H][I] f64 for the listed experts (all experts if None; dWg is
    absent for the gate-less activations)).  With ``tokens`` only those rows
    of dx / dw are computed (others are zero)."""
    d = inp.dims
    T, H, I, E, k = d.T, d.H, d.I, d.E, d.topk
    act = getattr(d, "act", ACT_SWIGLU)
    ex = inp.experts
    keep = []

    def c(a):
        a = np.ascontiguousarray(a)
        keep.append(a)
        return a.ctypes.data_as(ctypes.c_void_p)

    Wt = OrcWeights()
    for i, m in enumerate((ex.gate, ex.up, ex.down)):
        if m is None:
            continue
        Wt.fp4[i] = c(m.fp4)
        Wt.e8m0[i] = c(m.e8m0)
        Wt.blk[i] = c(m.blk)
    elist = None if experts is None else np.ascontiguousarray(experts, dtype=np.int32)
    nE = E if elist is None else len(elist)
    res = dict(dx=np.zeros((T, H)), dw=np.zeros((T, k)))
    if want_dw:
        if act == ACT_SWIGLU:
            res["dWg"] = np.zeros((nE, I, H))
        res["dWu"] = np.zeros((nE, I, H))
        res["dWd"] = np.zeros((nE, H, I))
    tl = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    tid = None if inp.token_ids is None else np.ascontiguousarray(inp.token_ids, dtype=np.int64)
    bias = None if inp.bias is None else np.ascontiguousarray(inp.bias, dtype=np.float32)
    lib().orc_layer_backward(T, H, I, E, k, act, np.ascontiguousarray(inp.x),
                             np.ascontiguousarray(inp.w_router), _ptr(bias), inp.mode, _ptr(tid),
                             ctypes.byref(Wt), np.ascontiguousarray(dout, dtype=np.uint16),
                             _ptr(res["dx"]), _ptr(res["dw"]), _ptr(res.get("dWg")), _ptr(res.get("dWu")),
                             _ptr(res.get("dWd")), _ptr(tl), 0 if tl is None else len(tl),
                             _ptr(elist), nE if elist is not None else 0)
    return res
