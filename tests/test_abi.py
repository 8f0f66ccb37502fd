"""The C ABI without a GPU: the library loads, exports every function that
include/v4moe.h declares, sizes workspaces, and rejects bad arguments before
touching a device."""
import ctypes

import pytest

from fp4_weight_grouped_amd import v4moe


def test_exports_every_declared_function():
    names = v4moe.declared_functions()
    assert set(names) >= {"moe_route", "moe_permute", "moe_expert_ffn", "moe_combine",
                          "moe_layer_forward", "moe_workspace_bytes", "moe_prepack_weights",
                          "moe_dequant_fp8", "moe_quantize_weights", "moe_strerror", "moe_transpose_weights",
                          "moe_layer_backward", "moe_backward_workspace_bytes", "moe_layer_forward_noalloc",
                          "moe_noalloc_max_workspace_bytes"}
    L = v4moe.lib()
    for n in names:
        assert hasattr(L, n), n


def test_strerror():
    for c in range(0, -8, -1):
        assert v4moe.strerror(c) != "unknown error"
    assert v4moe.strerror(-99) == "unknown error"


def test_workspace_bytes():
    d = v4moe.dims(128, 4096, 2048, 256, 8)
    n = v4moe.moe_workspace_bytes(d)
    P = 128 * 8
    # at least the hq, y and xq buffers
    assert n >= P * 2048 + P * 4096 * 2 + 128 * 4096
    # and the router logits, fp32 [T][E]
    assert n >= 128 * 256 * 4 + P * 2048 + P * 4096 * 2 + 128 * 4096
    assert n % 256 == 0
    assert v4moe.moe_workspace_bytes(v4moe.dims(0, 4096, 2048, 256, 8)) > 0
    for bad in [v4moe.dims(1, 100, 2048, 256, 8), v4moe.dims(1, 4096, 100, 256, 8),
                v4moe.dims(1, 4096, 2048, 0, 1), v4moe.dims(1, 4096, 2048, 4, 8),
                v4moe.dims(-1, 4096, 2048, 256, 8), v4moe.dims(1, 4096, 2048, 256, 17)]:
        assert v4moe.moe_workspace_bytes(bad) == 0


def _call(name, *args):
    return getattr(v4moe.lib(), name)(*args)


def test_error_paths_without_device():
    L = v4moe.lib()
    d = v4moe.dims(4, 256, 128, 8, 2)
    bd = v4moe.dims(4, 255, 128, 8, 2)
    p = ctypes.c_void_p(4096)          # aligned, never dereferenced: every call below fails first
    mis = ctypes.c_void_p(4097)
    ex = v4moe.ExpertsC(v4moe.Mat(4096, 4096, 4096), v4moe.Mat(4096, 4096, 4096), v4moe.Mat(4096, 4096, 4096))
    assert L.moe_route(ctypes.byref(bd), p, p, None, 0, None, p, p, p, 1 << 30, None) == -2
    assert L.moe_route(ctypes.byref(d), p, p, None, 2, None, p, p, p, 1 << 30, None) == -2
    assert L.moe_route(ctypes.byref(d), None, p, None, 0, None, p, p, p, 1 << 30, None) == -1
    assert L.moe_route(ctypes.byref(d), mis, p, None, 0, None, p, p, p, 1 << 30, None) == -3
    assert L.moe_route(ctypes.byref(d), p, p, None, 0, None, p, p, p, 10, None) == -4
    assert L.moe_route(ctypes.byref(v4moe.dims(0, 256, 128, 8, 2)), p, p, None, 0, None, p, p, None, 0, None) == 0
    assert L.moe_permute(ctypes.byref(d), p, p, p, p, p, p, p, p, 10, None) == -4
    assert L.moe_permute(ctypes.byref(d), p, p, None, p, p, p, p, p, 1 << 30, None) == -1
    assert L.moe_permute(ctypes.byref(d), p, None, p, p, p, p, p, p, 1 << 30, None) == -1
    assert L.moe_expert_ffn(ctypes.byref(d), p, p, p, p, ctypes.byref(ex), p, p, 10, None) == -4
    assert L.moe_expert_ffn(ctypes.byref(d), p, p, p, p, None, p, p, 1 << 30, None) == -1
    bad_ex = v4moe.ExpertsC(v4moe.Mat(4096, 4097, 4096), v4moe.Mat(4096, 4096, 4096), v4moe.Mat(4096, 4096, 4096))
    assert L.moe_expert_ffn(ctypes.byref(d), p, p, p, p, ctypes.byref(bad_ex), p, p, 1 << 30, None) == -1
    assert L.moe_combine(ctypes.byref(d), p, p, mis, None) == -3
    assert L.moe_combine(ctypes.byref(v4moe.dims(0, 256, 128, 8, 2)), p, p, p, None) == 0
    assert L.moe_layer_forward(ctypes.byref(d), p, p, None, 0, None, ctypes.byref(ex), p, p, p, p, p, 10,
                               None) == -4
    assert L.moe_layer_forward(ctypes.byref(d), p, None, None, 0, None, ctypes.byref(ex), p, p, p, p, p,
                               1 << 30, None) == -1
    m = v4moe.Mat(4096, 4096, 4096)
    assert L.moe_dequant_fp8(ctypes.byref(m), 15, 128, 0, p, None) == -2
    assert L.moe_dequant_fp8(ctypes.byref(m), 16, 100, 0, p, None) == -2
    assert L.moe_prepack_weights(ctypes.byref(d), ctypes.byref(ex), ctypes.byref(ex), p, 8, None) == -4
    assert L.moe_backward_workspace_bytes(ctypes.byref(bd)) == 0
    assert L.moe_backward_workspace_bytes(ctypes.byref(d)) > L.moe_workspace_bytes(ctypes.byref(d))
    assert L.moe_transpose_weights(ctypes.byref(bd), ctypes.byref(ex), p, p, None) == -2
    assert L.moe_transpose_weights(ctypes.byref(d), ctypes.byref(ex), None, p, None) == -1
    assert L.moe_transpose_weights(ctypes.byref(d), ctypes.byref(ex), mis, p, None) == -3
    nb = L.moe_backward_workspace_bytes(ctypes.byref(d))
    assert L.moe_layer_backward(ctypes.byref(d), p, p, None, 0, None, ctypes.byref(ex), p, p, p, p, p, p, p, p, p,
                                nb - 1, None) == -4
    assert L.moe_layer_backward(ctypes.byref(d), p, p, None, 0, None, ctypes.byref(ex), p, p, p, p, p, None, p, p,
                                p, nb, None) == -1
    assert L.moe_layer_backward(ctypes.byref(d), p, p, None, 3, None, ctypes.byref(ex), p, p, p, p, p, p, p, p, p,
                                nb, None) == -2
    assert L.moe_layer_backward(ctypes.byref(d), mis, p, None, 0, None, ctypes.byref(ex), p, p, p, p, p, p, p, p, p,
                                nb, None) == -3
    assert L.moe_quantize_weights(1, 100, 128, p, 0, ctypes.byref(m), None, None) == -2
    assert L.moe_quantize_weights(1, 128, 64, p, 0, ctypes.byref(m), None, None) == -2
    assert L.moe_quantize_weights(0, 128, 128, p, 1, ctypes.byref(m), None, None) == -2
    assert L.moe_quantize_weights(1, 128, 128, None, 0, ctypes.byref(m), None, None) == -1
    assert L.moe_quantize_weights(1, 128, 128, mis, 0, ctypes.byref(m), None, None) == -3
    assert L.moe_quantize_weights(1, 128, 128, p, 0, ctypes.byref(v4moe.Mat(4096, 0, 4096)), None, None) == -1


def test_noalloc_limits_without_device():
    """The allocation-free layer forward checks dimensions and its static
    scratch size before touching a device."""
    L = v4moe.lib()
    cap = L.moe_noalloc_max_workspace_bytes()
    assert cap == 16 << 20
    p = ctypes.c_void_p(4096)
    ex = v4moe.ExpertsC(v4moe.Mat(4096, 4096, 4096), v4moe.Mat(4096, 4096, 4096), v4moe.Mat(4096, 4096, 4096))
    bad = v4moe.dims(4, 255, 128, 8, 2)
    assert L.moe_layer_forward_noalloc(ctypes.byref(bad), p, p, None, 0, None, ctypes.byref(ex), p, p, p, p,
                                       None) == -2
    # the decode layer fits up to T = 189; T = 190 does not
    fits = v4moe.dims(189, 4096, 2048, 256, 8)
    over = v4moe.dims(190, 4096, 2048, 256, 8)
    assert L.moe_workspace_bytes(ctypes.byref(fits)) <= cap < L.moe_workspace_bytes(ctypes.byref(over))
    assert L.moe_layer_forward_noalloc(ctypes.byref(over), p, p, None, 0, None, ctypes.byref(ex), p, p, p, p,
                                       None) == -4
