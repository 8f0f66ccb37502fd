"""moe_layer_forward_noalloc (the layer forward on the library's static
per-GPU scratch array, for callers that cannot allocate) against
moe_layer_forward on a caller workspace, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from fp4_weight_grouped_amd import inputs, v4moe

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _bf16_f64(bits):
    return (np.asarray(bits).view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _outputs(T, d):
    return (torch.empty((T, d.topk), dtype=torch.int32, device=DEV),
            torch.empty((T, d.topk), dtype=torch.float32, device=DEV),
            torch.empty(d.E + 1, dtype=torch.int32, device=DEV),
            torch.empty((T, d.H), dtype=torch.int16, device=DEV))


def test_noalloc_matches_layer_forward_two_calls():
    inp = inputs.make("decode")
    d = inp.dims
    dims = v4moe.dims(d.T, d.H, d.I, d.E, d.topk)
    experts = v4moe.upload_experts(inp.experts, dims, DEV)
    wr = torch.from_numpy(inp.w_router).to(DEV)
    x_all = torch.from_numpy(inp.x.view(np.int16)).to(DEV)
    assert v4moe.moe_noalloc_max_workspace_bytes() == 16 << 20
    for T in (128, 37):                      # the second call smaller than the first
        print(f"[noalloc] T={T} H={d.H} I={d.I} E={d.E} k={d.topk}", flush=True)
        dt = v4moe.dims(T, d.H, d.I, d.E, d.topk)
        x = x_all[:T].contiguous()
        ids_a, w_a, off_a, out_a = _outputs(T, d)
        ws = torch.empty(v4moe.moe_workspace_bytes(dt), dtype=torch.uint8, device=DEV)
        v4moe.moe_layer_forward(dt, x, wr, None, 0, None, experts, ids_a, w_a, off_a, out_a, ws)
        ids_b, w_b, off_b, out_b = _outputs(T, d)
        v4moe.moe_layer_forward_noalloc(dt, x, wr, None, 0, None, experts, ids_b, w_b, off_b, out_b)
        torch.cuda.synchronize()
        for a, b in ((ids_a, ids_b), (w_a, w_b), (off_a, off_b), (out_a, out_b)):
            assert torch.equal(a, b)
    # the second (smaller) call against the oracle as well
    sub = inputs.Inputs(dims=inputs.Dims(37, d.H, d.I, d.E, d.topk), mode=0, x=inp.x[:37].copy(),
                        w_router=inp.w_router, bias=None, token_ids=None, experts=inp.experts)
    ref = oracle.layer_forward(sub)
    assert np.array_equal(ids_b.cpu().numpy(), ref["ids"])
    assert np.array_equal(off_b.cpu().numpy(), ref["offsets"])
    g, r = _bf16_f64(out_b.cpu().numpy()), _bf16_f64(ref["out"])
    rel = np.linalg.norm(g - r) / np.linalg.norm(r)
    mx = np.abs(g - r).max() / np.abs(r).max()
    print(f"  T=37 vs oracle rel_l2={rel:.3e} max_rel={mx:.3e}", flush=True)
    assert rel <= 2e-3 and mx <= 1e-2


def test_noalloc_rejects_batches_beyond_the_scratch():
    """A batch whose workspace exceeds the static array is refused before
    anything is enqueued: the outputs keep their contents."""
    H, I, E, k = 4096, 2048, 256, 8
    T = 512
    dt = v4moe.dims(T, H, I, E, k)
    assert v4moe.moe_workspace_bytes(dt) > v4moe.moe_noalloc_max_workspace_bytes()
    p = torch.zeros(64, dtype=torch.uint8, device=DEV)
    mat = v4moe.Mat(p.data_ptr(), p.data_ptr(), p.data_ptr())
    c = v4moe.ExpertsC(mat, mat, mat)
    ids = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    off = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    rc = v4moe.lib().moe_layer_forward_noalloc(
        v4moe.ctypes.byref(dt), v4moe._p(p), v4moe._p(p), None, 0, None, v4moe.ctypes.byref(c),
        v4moe._p(ids), v4moe._p(p), v4moe._p(off), v4moe._p(p), v4moe._stream())
    torch.cuda.synchronize()
    assert rc == -4
    assert int(ids.min()) == -7 and int(ids.max()) == -7 and int(off.min()) == -7
