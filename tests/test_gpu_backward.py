"""GPU parity of moe_layer_backward against the CPU oracle's layer backward
(straight-through quantisation, gradients on the forward's FP8 weights, fixed
accumulation order; P1 section 3 and 4, P4 section 3 and 4).

Bar.  The oracle is exact (fp64).  The GPU rounds dout * w, the row gradients
(dG, dU) and the weight-gradient activations (E4M3 code x fp32 scale) to bf16
before its matrix products (unit roundoff u = 2^-9), accumulating in fp32.
Each output element carries at most three such roundings on its path, each a
relative perturbation of at most u of one factor, so the per-element relative
error stays below ~3u ~ 6e-3 before cancellation; over a whole tensor the
errors are independent in sign and the relative L2 error is a fraction of
that.  Tested: relative L2 <= 5e-3 and max|d| <= 3e-2 * max|ref| for every
gradient; bitwise equality across repeated runs; dx of a request alone equal
bitwise to its rows inside a larger batch.
"""
import numpy as np
import pytest
import torch

import oracle
from fp4_weight_grouped_amd import inputs, v4moe

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REL_L2 = 5e-3
MAX_REL = 3e-2


def check(got, ref, what):
    got = np.asarray(got, np.float64)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    mx = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-300)
    print(f"  {what}: rel_l2={rel:.3e} max_rel={mx:.3e}", flush=True)
    assert rel <= REL_L2, (what, rel)
    assert mx <= MAX_REL, (what, mx)


def make(T, H, I, E, k, act=inputs.ACT_SWIGLU, seed=31, mode=0, bias=False):
    ex = inputs.gen_experts(seed, E, H, I, gated=act == inputs.ACT_SWIGLU)
    return inputs.Inputs(dims=inputs.Dims(T, H, I, E, k, act), mode=mode, x=inputs.gen_x(seed, T, H),
                         w_router=inputs.gen_router(seed, H, E),
                         bias=inputs.zipf_bias(seed, E) if bias else None,
                         token_ids=np.arange(T, dtype=np.int64) * 5 + 2 if mode == 1 else None, experts=ex)


def dout_for(inp, seed=9):
    r = np.random.default_rng(seed)
    return inputs.to_bf16_bits(r.standard_normal((inp.dims.T, inp.dims.H)).astype(np.float32))


def gpu_layer(inp):
    d = inp.dims
    ex = v4moe.upload_experts(inp.experts, v4moe.dims(max(d.T, 1), d.H, d.I, d.E, d.topk, d.act), DEV)
    return v4moe.MoELayer(d.H, d.I, d.E, d.topk, ex, torch.from_numpy(inp.w_router).to(DEV), DEV, act=d.act)


def gpu_backward(layer, inp, dout):
    x = torch.from_numpy(inp.x.view(np.int16)).to(DEV)
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).to(DEV)
    tid = None if inp.token_ids is None else torch.from_numpy(inp.token_ids).to(DEV)
    g = layer.backward(x, torch.from_numpy(dout.view(np.int16)).to(DEV), bias, inp.mode, tid)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in g.items()}


def full_check(inp, label, runs=2):
    print(f"[{label}] dims={inp.dims} mode={inp.mode}", flush=True)
    dout = dout_for(inp)
    ref = oracle.layer_backward(inp, dout)
    layer = gpu_layer(inp)
    g = gpu_backward(layer, inp, dout)
    check(g["dx"], ref["dx"], f"{label} dx")
    check(g["dw"], ref["dw"], f"{label} dw")
    keys = ("dWu", "dWd") + (("dWg",) if inp.dims.act == inputs.ACT_SWIGLU else ())
    for key in keys:
        check(g[key], ref[key], f"{label} {key}")
    for _ in range(runs - 1):
        g2 = gpu_backward(layer, inp, dout)
        for key in ("dx", "dw") + keys:
            assert np.array_equal(g2[key], g[key]), f"{key} differs between runs"
    return g, layer, dout


@pytest.mark.parametrize("act", [inputs.ACT_SWIGLU, inputs.ACT_RELU2, inputs.ACT_RELU])
def test_backward_small(act):
    full_check(make(24, 256, 256, 4, 2, act), f"small act{act}")


@pytest.mark.parametrize("T,H,I,E,k,mode,bias", [
    (37, 256, 128, 8, 2, 0, False),     # ragged rows, several m-tiles
    (200, 512, 384, 8, 3, 0, True),     # 3 chunks of I, skewed load, partial 64-row tiles
    (300, 256, 256, 16, 1, 1, False),   # hash routing, k = 1
    (64, 256, 128, 64, 4, 0, True),     # many experts, some empty (zero weight gradients)
    (1200, 256, 384, 4, 2, 0, True),    # large-batch weight gradients: experts of 1199 / 1046 rows in
                                        # 288-column chunks (ragged last chunk) next to experts of 29 / 126
])
def test_backward_shapes(T, H, I, E, k, mode, bias):
    g, _, _ = full_check(make(T, H, I, E, k, mode=mode, bias=bias), f"T{T}H{H}I{I}E{E}k{k}")


def test_backward_dx_batch_invariant():
    """A request's dx computed alone equals its rows in the batched call."""
    inp = make(64, 256, 256, 8, 2, seed=33)
    dout = dout_for(inp)
    layer = gpu_layer(inp)
    full = gpu_backward(layer, inp, dout)
    for lo, hi in [(0, 1), (5, 29), (40, 64)]:
        sub = inputs.Inputs(dims=inputs.Dims(hi - lo, 256, 256, 8, 2), mode=0,
                            x=np.ascontiguousarray(inp.x[lo:hi]), w_router=inp.w_router, bias=None,
                            token_ids=None, experts=inp.experts)
        alone = gpu_backward(layer, sub, np.ascontiguousarray(dout[lo:hi]))
        assert np.array_equal(alone["dx"], full["dx"][lo:hi])
        assert np.array_equal(alone["dw"], full["dw"][lo:hi])


@pytest.mark.parametrize("act", [inputs.ACT_SWIGLU, inputs.ACT_RELU2])
def test_transposed_weights_are_the_fp8_bytes(act):
    """moe_transpose_weights writes each weight's E4M3 byte, the byte the
    oracle's dequantisation gives (every sub-block exponent of the lossless
    window, so E4M3 subnormals and both zero signs occur), transposed:
    wt_gu[e][h] = [gate(e, :, h) | up(e, :, h)], wt_d[e][i] = down(e, :, i)."""
    E, H, I = 3, 256, 256
    gated = act == inputs.ACT_SWIGLU
    ex = inputs.gen_experts(47, E, H, I, b_range=(-8, 6), gated=gated)
    inp = inputs.Inputs(dims=inputs.Dims(8, H, I, E, 2, act), mode=0, x=inputs.gen_x(47, 8, H),
                        w_router=inputs.gen_router(47, H, E), bias=None, token_ids=None, experts=ex)
    wt_gu, wt_d = gpu_layer(inp).transposed_weights()
    torch.cuda.synchronize()
    wt_gu, wt_d = wt_gu.cpu().numpy(), wt_d.cpu().numpy()
    for e in range(E):
        cols = ([oracle.dequant_matrix(ex.gate.fp4[e], ex.gate.e8m0[e]).T] if gated else []) + \
               [oracle.dequant_matrix(ex.up.fp4[e], ex.up.e8m0[e]).T]
        assert np.array_equal(wt_gu[e], np.concatenate(cols, axis=1)), e
        assert np.array_equal(wt_d[e], oracle.dequant_matrix(ex.down.fp4[e], ex.down.e8m0[e]).T), e


def test_backward_zero_tokens():
    inp = make(0, 256, 128, 4, 2)
    layer = gpu_layer(inp)
    g = gpu_backward(layer, inp, np.zeros((0, 256), np.uint16))
    assert all(np.all(g[key] == 0) for key in ("dWg", "dWu", "dWd"))


def sampled(name, n_tok, n_exp):
    inp = inputs.make(name)
    d = inp.dims
    print(f"[{name}] backward T={d.T}", flush=True)
    dout = dout_for(inp)
    layer = gpu_layer(inp)
    g = gpu_backward(layer, inp, dout)
    ids = oracle.route(inp.x, inp.w_router, d.topk, inp.bias, inp.mode, inp.token_ids, d.E)[0]
    cnt = np.bincount(ids.ravel(), minlength=d.E)
    rng = np.random.default_rng(1)
    toks = np.unique(np.concatenate([rng.choice(d.T, n_tok, replace=False), [0, d.T - 1]]))
    exps = [int(np.argmax(cnt))] + [int(e) for e in rng.choice(np.nonzero(cnt)[0], n_exp - 1, replace=False)]
    exps = list(dict.fromkeys(exps))
    ref = oracle.layer_backward(inp, dout, tokens=toks, experts=exps)
    check(g["dx"][toks], ref["dx"][toks], f"{name} dx[sample]")
    check(g["dw"][toks], ref["dw"][toks], f"{name} dw[sample]")
    keys = ("dWu", "dWd") + (("dWg",) if d.act == inputs.ACT_SWIGLU else ())
    for key in keys:
        check(g[key][exps], ref[key], f"{name} {key}[experts {exps}]")
    idle = np.nonzero(cnt == 0)[0]
    if len(idle):
        assert np.all(g["dWd"][idle] == 0)


@pytest.mark.slow
def test_backward_decode_full_size():
    sampled("decode", 6, 3)


@pytest.mark.slow
def test_backward_decode_gateless_full_size():
    sampled("decode_relu2", 4, 2)


@pytest.mark.slow
def test_backward_prefill_full_size():
    sampled("prefill", 3, 1)


@pytest.mark.slow
def test_backward_largest_hidden_and_intermediate():
    """H = I = 16384: 256 chunks in the [dG dU] contraction, the largest
    transposes and weight gradients; every token to both experts."""
    full_check(make(2, 16384, 16384, 2, 2, seed=35), "T2H16384I16384E2k2", runs=1)


def test_qat_step_from_fp32_master_weights():
    """One QAT step end to end: FP32 master weights -> moe_quantize_weights
    straight into the packed layout -> layer forward and backward on the GPU;
    the gradients (straight through to the master weights) match the oracle's
    backward on the oracle's own quantisation of the same master weights."""
    T, H, I, E, k = 48, 256, 256, 4, 2
    rng = np.random.default_rng(41)
    masters = [rng.standard_normal((E, I, H)).astype(np.float32) * np.float32(0.05),
               rng.standard_normal((E, I, H)).astype(np.float32) * np.float32(0.05),
               rng.standard_normal((E, H, I)).astype(np.float32) * np.float32(0.05)]
    mats = []
    for m in masters:
        fp4, e8, blk, _ = oracle.quantize_weights(m)
        mats.append(inputs.Matrix(fp4=fp4, e8m0=e8, blk=blk))
    inp = inputs.Inputs(dims=inputs.Dims(T, H, I, E, k), mode=0, x=inputs.gen_x(41, T, H),
                        w_router=inputs.gen_router(41, H, E), bias=None, token_ids=None,
                        experts=inputs.Experts(*mats))
    dout = dout_for(inp)
    ref = oracle.layer_backward(inp, dout)
    packed = v4moe.DeviceExperts(*[v4moe.quantize_weights(torch.from_numpy(m).to(DEV), packed=True)
                                   for m in masters])
    layer = v4moe.MoELayer(H, I, E, k, packed, torch.from_numpy(inp.w_router).to(DEV), DEV)
    g = gpu_backward(layer, inp, dout)
    check(g["dx"], ref["dx"], "qat dx")
    check(g["dw"], ref["dw"], "qat dw")
    for key in ("dWg", "dWu", "dWd"):
        check(g[key], ref[key], f"qat {key}")
        assert g[key].shape == masters[("dWg", "dWu", "dWd").index(key)].shape
