"""Pins of the oracle's layer backward (P1 section 3 and P4 section 3:
deterministic MoE backward; P1 section 4 and P4 section 4: gradients taken with
the forward's FP8 weights and passed straight to the FP32 master weights).

The reference here is torch autograd in fp64 over a dense restatement of the
forward: for every (token, expert) pair the expert FFN on the dequantised
weights, with every rounding the forward makes (G and U to fp32, h to fp32
then E4M3 per 128 channels, Y to bf16) written as value + (rounded - value)
.detach(), i.e. straight through.  Autograd differentiates that graph by a
mechanism that shares nothing with the oracle's hand-written chain rule, so a
wrong derivative, a transposed weight, a dropped term or a mis-ordered index in
the oracle fails here.
"""
import numpy as np
import pytest
import torch

import oracle
from fp4_weight_grouped_amd import inputs
from test_oracle_ffn import bf16_to_f64, quant_real, real_matrix

torch.set_default_dtype(torch.float64)


def ste(v, rounded):
    return v + (rounded - v).detach()


def to_f32(v):
    return ste(v, v.detach().float().double())


def to_bf16(v):
    return ste(v, v.detach().float().to(torch.bfloat16).double())


def quant_e4m3_rows(v):
    q = torch.from_numpy(quant_real(v.detach().float().numpy()))
    return ste(v, q)


def autograd_backward(inp, dout_bits):
    d = inp.dims
    T, H, I, E, k = d.T, d.H, d.I, d.E, d.topk
    act = d.act
    f = oracle.layer_forward(inp)
    ids, w = f["ids"], f["w"]
    xhat = torch.from_numpy(quant_real(bf16_to_f64(inp.x).astype(np.float32))).requires_grad_(True)
    wt = torch.from_numpy(w.astype(np.float64)).requires_grad_(True)
    mats = {}
    for name in ("gate", "up", "down"):
        m = getattr(inp.experts, name)
        if m is not None:
            mats[name] = torch.from_numpy(np.stack([real_matrix(m, e) for e in range(E)])).requires_grad_(True)
    out = torch.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            U = to_f32(mats["up"][e] @ xhat[t])
            if act == inputs.ACT_SWIGLU:
                G = to_f32(mats["gate"][e] @ xhat[t])
                h = G / (1 + torch.exp(-G)) * U
            elif act == inputs.ACT_RELU2:
                h = torch.clamp(U, min=0) ** 2
            else:
                h = torch.clamp(U, min=0)
            hq = quant_e4m3_rows(to_f32(h)[None, :])[0]
            Y = to_bf16(mats["down"][e] @ hq)
            out = out.index_add(0, torch.tensor([t]), (wt[t, j] * Y)[None, :])
    dout = torch.from_numpy(bf16_to_f64(dout_bits))
    (out * dout).sum().backward()
    return dict(dx=xhat.grad.numpy(), dw=wt.grad.numpy(),
                **{f"dW{n[0]}": mats[n].grad.numpy() for n in mats})


def rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


def small(act, T=24, H=256, I=256, E=4, k=2, seed=21):
    ex = inputs.gen_experts(seed, E, H, I, gated=act == inputs.ACT_SWIGLU)
    return inputs.Inputs(dims=inputs.Dims(T, H, I, E, k, act), mode=0, x=inputs.gen_x(seed, T, H),
                         w_router=inputs.gen_router(seed, H, E), bias=None, token_ids=None, experts=ex)


def dout_for(inp, seed=5):
    r = np.random.default_rng(seed)
    return inputs.to_bf16_bits(r.standard_normal((inp.dims.T, inp.dims.H)).astype(np.float32))


@pytest.mark.parametrize("act", [inputs.ACT_SWIGLU, inputs.ACT_RELU2, inputs.ACT_RELU])
def test_backward_matches_autograd(act):
    inp = small(act)
    dout = dout_for(inp)
    got = oracle.layer_backward(inp, dout)
    ref = autograd_backward(inp, dout)
    assert rel(got["dx"], ref["dx"]) < 1e-9
    assert rel(got["dw"], ref["dw"]) < 1e-9
    for key in ("dWu", "dWd") + (("dWg",) if act == inputs.ACT_SWIGLU else ()):
        assert rel(got[key], ref[key]) < 1e-9, key


def test_subsets_match_full_run():
    inp = small(inputs.ACT_SWIGLU, T=32, E=8, k=3, seed=22)
    dout = dout_for(inp, 6)
    full = oracle.layer_backward(inp, dout)
    toks = [0, 7, 31]
    exps = [5, 2]
    part = oracle.layer_backward(inp, dout, tokens=toks, experts=exps)
    assert np.array_equal(part["dx"][toks], full["dx"][toks])
    assert np.array_equal(part["dw"][toks], full["dw"][toks])
    for key in ("dWg", "dWu", "dWd"):
        assert np.array_equal(part[key], full[key][exps])


def test_linearity_in_dout_and_unused_expert_zero():
    """Gradients are linear in dout (2*dout gives exactly twice, dout = 0
    gives zero), and an expert that receives no token has zero weight
    gradients."""
    inp = small(inputs.ACT_SWIGLU, T=8, E=8, k=1, seed=23)
    inp.bias = np.full(inp.dims.E, -30.0, np.float32)
    inp.bias[[1, 3]] = 0.0                           # only experts 1 and 3 are ever picked
    dout = dout_for(inp, 7)
    g1 = oracle.layer_backward(inp, dout)
    d2 = inputs.to_bf16_bits(2.0 * bf16_to_f64(dout).astype(np.float32))
    g2 = oracle.layer_backward(inp, d2)
    for key in ("dx", "dw", "dWg", "dWu", "dWd"):
        assert np.array_equal(g2[key], 2.0 * g1[key]), key
    z = oracle.layer_backward(inp, np.zeros_like(dout))
    assert all(np.all(z[key] == 0) for key in ("dx", "dw", "dWg", "dWu", "dWd"))
    used = {1, 3}
    for e in range(inp.dims.E):
        if e not in used:
            assert np.all(g1["dWd"][e] == 0) and np.all(g1["dWg"][e] == 0)
        else:
            assert np.abs(g1["dWd"][e]).max() > 0
