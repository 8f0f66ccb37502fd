"""Pins of the oracle's expert FFN and combine.

* Closed form: with every weight code = 1.0, b = 0 and x = 1, every stage has
  a value that can be written down (P1 section 1.4 for the SwiGLU gate/up/down
  structure; section 4 for FP4 weights used as FP8).
* Dense equivalence: when every token is routed to every expert, the
  permuted, chunk-promoted, combined result equals a plain dense computation
  done with library matmuls on the real (dequantised, block-scaled) tensors;
  with equal weights 1/E it is one dense SwiGLU FFN of width E*I.
"""
import json
import os

import numpy as np
import torch

import oracle
from fp4_weight_grouped_amd import inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")
E2M1 = np.array(json.load(open(os.path.join(GOLD, "formats.json")))["e2m1_positive_values_by_code"])


def bf16_to_f64(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def const_matrix(E, N, K, code, b, blk):
    return inputs.Matrix(
        fp4=np.full((E, N, K // 2), code | (code << 4), np.uint8),
        e8m0=np.full((E, N, K // 32), 127 + b, np.uint8),
        blk=np.full((E, N // 128, K // 128), blk, np.float32))


def make_inputs(T, H, I, E, k, experts, x=None, mode=0, seed=7):
    x = inputs.gen_x(seed, T, H) if x is None else x
    return inputs.Inputs(dims=inputs.Dims(T, H, I, E, k), mode=mode, x=x,
                         w_router=inputs.gen_router(seed, H, E), bias=None,
                         token_ids=None, experts=experts)


def test_closed_form_all_ones():
    T, H, I, E = 8, 256, 256, 4
    sg, sd = 2.0 ** -5, 0.0375
    ex = inputs.Experts(gate=const_matrix(E, I, H, 0x2, 0, sg), up=const_matrix(E, I, H, 0x2, 0, sg),
                        down=const_matrix(E, H, I, 0x2, 0, sd))
    x = np.full((T, H), 0x3F80, np.uint16)                 # bf16 1.0
    for k in (1, 2, 4):
        r = oracle.layer_forward(make_inputs(T, H, I, E, k, ex, x=x), want_y=True)
        assert np.all(r["xq"] == 0x7E)                         # 1 / (1/448) -> 448
        assert np.all(r["xs"] == np.float32(1.0 / 448.0))
        G = H * sg                                             # = H * (1/448) * 448 * sg
        h = G / (1 + np.exp(-G)) * G
        Y = I * sd * h
        y = bf16_to_f64(r["y"])
        out = bf16_to_f64(r["out"])
        np.testing.assert_allclose(y, Y, rtol=2 ** -8)         # bf16 rounding
        np.testing.assert_allclose(out, Y, rtol=2 ** -8)
        if k == 1:
            assert np.array_equal(r["out"], r["y"])          # w = a/a = 1 exactly


def real_matrix(m, e):
    """Real weight values e2m1(code) * 2^b * blk, straight from the MXFP4 definition."""
    N, K2 = m.fp4.shape[1:]
    K = 2 * K2
    b = m.fp4[e]
    codes = np.empty((N, K), np.int64)
    codes[:, 0::2] = b & 15
    codes[:, 1::2] = b >> 4
    val = E2M1[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    val *= np.exp2(np.repeat(m.e8m0[e].astype(np.float64) - 127, 32, axis=1))
    val *= np.repeat(np.repeat(m.blk[e].astype(np.float64), 128, 0), 128, 1)
    return val


def quant_real(v32):
    """Per (row, 128) group: s = fp32(amax/448); q = E4M3 cast (torch) of fp32(v/s).
    Returns the real value q * s."""
    R, C = v32.shape
    g = v32.reshape(R, C // 128, 128)
    amax = np.abs(g).max(-1)
    s = np.where(amax > 0, (amax / np.float32(448.0)).astype(np.float32), np.float32(1.0))
    y = (g / s[..., None]).astype(np.float32)
    q = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    return (q * s[..., None].astype(np.float64)).reshape(R, C)


def dense_expert(xr, ex, e):
    G = (xr @ real_matrix(ex.gate, e).T).astype(np.float32).astype(np.float64)
    U = (xr @ real_matrix(ex.up, e).T).astype(np.float32).astype(np.float64)
    h = (G / (1 + np.exp(-G)) * U).astype(np.float32)
    return quant_real(h) @ real_matrix(ex.down, e).T


def test_dense_equivalence_learned_weights():
    T, H, I, E = 24, 256, 256, 4
    ex = inputs.gen_experts(11, E, H, I)
    inp = make_inputs(T, H, I, E, E, ex, seed=11)
    r = oracle.layer_forward(inp, exact=True)
    xr = quant_real(bf16_to_f64(inp.x).astype(np.float32))
    ref = np.zeros((T, H))
    ref_bf = np.zeros((T, H))
    for e in range(E):
        we = (r["w"].astype(np.float64) * (r["ids"] == e)).sum(1)
        ye = dense_expert(xr, ex, e)
        ref += we[:, None] * ye
        # normal mode: Y rounded fp64 -> fp32 -> bf16 before the weighted sum
        yb = torch.from_numpy(ye.astype(np.float32)).to(torch.bfloat16).double().numpy()
        ref_bf += we[:, None] * yb
    err = np.abs(r["out_exact"] - ref).max() / np.abs(ref).max()
    assert err < 1e-12, err
    ref_bf = torch.from_numpy(ref_bf.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.mean(r["out"] != ref_bf) < 1e-3


def test_dense_equivalence_one_wide_ffn():
    """Hash routing with k = E gives every expert weight 1/E; E*out is then a
    single SwiGLU FFN whose gate/up rows and down columns are the experts'
    concatenated (h's 128-channel groups align with experts since I%128 == 0)."""
    T, H, I, E = 16, 256, 128, 8
    ex = inputs.gen_experts(12, E, H, I)
    inp = make_inputs(T, H, I, E, E, ex, mode=1, seed=12)
    r = oracle.layer_forward(inp, exact=True)
    assert np.all(r["w"] == np.float32(1.0 / E))
    xr = quant_real(bf16_to_f64(inp.x).astype(np.float32))
    Wg = np.concatenate([real_matrix(ex.gate, e) for e in range(E)], 0)
    Wu = np.concatenate([real_matrix(ex.up, e) for e in range(E)], 0)
    Wd = np.concatenate([real_matrix(ex.down, e) for e in range(E)], 1)
    G = (xr @ Wg.T).astype(np.float32).astype(np.float64)
    U = (xr @ Wu.T).astype(np.float32).astype(np.float64)
    h = (G / (1 + np.exp(-G)) * U).astype(np.float32)
    Y = quant_real(h) @ Wd.T
    err = np.abs(E * r["out_exact"] - Y).max() / np.abs(Y).max()
    assert err < 1e-12, err


def test_subset_rows_match_full_run():
    inp = inputs.make("tiny")
    full = oracle.layer_forward(inp, want_y=True)
    sub = [0, 5, 63, 17]
    part = oracle.layer_forward(inp, subset=sub, want_y=True)
    assert np.array_equal(part["out"][sub], full["out"][sub])
    for key in ("ids", "w", "offsets", "sorted_pair", "pair_pos", "xq", "xs"):
        assert np.array_equal(part[key], full[key])


def test_batch_invariance_oracle():
    """A token's output does not depend on its batch mates (P1 section 3.1)."""
    inp = inputs.make("tiny")
    full = oracle.layer_forward(inp)
    for lo, hi in [(0, 1), (10, 30), (63, 64)]:
        sub = inputs.Inputs(dims=inputs.Dims(hi - lo, 256, 128, 8, 2), mode=0,
                            x=np.ascontiguousarray(inp.x[lo:hi]), w_router=inp.w_router,
                            bias=None, token_ids=None, experts=inp.experts)
        alone = oracle.layer_forward(sub)
        assert np.array_equal(alone["out"], full["out"][lo:hi])


# ---- the gate-less activations (the pages' cheap alternative to SwiGLU) ------------------
ACTS = {oracle.ACT_RELU2: lambda u: np.maximum(u, 0.0) ** 2, oracle.ACT_RELU: lambda u: np.maximum(u, 0.0)}


def make_gateless(T, H, I, E, k, act, up, down, x=None, mode=0, seed=7):
    x = inputs.gen_x(seed, T, H) if x is None else x
    return inputs.Inputs(dims=inputs.Dims(T, H, I, E, k, act), mode=mode, x=x,
                         w_router=inputs.gen_router(seed, H, E), bias=None, token_ids=None,
                         experts=inputs.Experts(gate=None, up=up, down=down))


def test_closed_form_gateless():
    """x = 1, every up weight +-1.0 * sg and every down weight 1.0 * sd:
    U = +-H*sg, h = act(U), and with a constant h row the E4M3 round trip is
    exact, so Y = I * sd * act(U).  Negative pre-activations give exactly 0."""
    T, H, I, E = 8, 256, 256, 4
    sg, sd = 2.0 ** -6, 0.0375
    x = np.full((T, H), 0x3F80, np.uint16)
    for act, f in ACTS.items():
        for code, sign in ((0x2, 1.0), (0xA, -1.0)):
            inp = make_gateless(T, H, I, E, 2, act, const_matrix(E, I, H, code, 0, sg),
                                const_matrix(E, H, I, 0x2, 0, sd), x=x)
            r = oracle.layer_forward(inp, want_y=True)
            Y = I * sd * f(sign * H * sg)
            if sign < 0:
                assert np.all(r["y"] == 0) and np.all(r["out"] == 0)
            else:
                np.testing.assert_allclose(bf16_to_f64(r["y"]), Y, rtol=2 ** -8)
                np.testing.assert_allclose(bf16_to_f64(r["out"]), Y, rtol=2 ** -8)


def test_dense_equivalence_gateless():
    """Every token routed to every expert: the exact-mode output equals the
    dense per-expert computation act(x W_up^T) quantised, times W_down^T,
    weighted by the routing weights."""
    T, H, I, E = 24, 256, 256, 4
    for act, f in ACTS.items():
        ex = inputs.gen_experts(13, E, H, I, gated=False)
        assert ex.gate is None
        inp = make_gateless(T, H, I, E, E, act, ex.up, ex.down, seed=13)
        r = oracle.layer_forward(inp, exact=True)
        xr = quant_real(bf16_to_f64(inp.x).astype(np.float32))
        ref = np.zeros((T, H))
        for e in range(E):
            we = (r["w"].astype(np.float64) * (r["ids"] == e)).sum(1)
            U = (xr @ real_matrix(ex.up, e).T).astype(np.float32).astype(np.float64)
            h = f(U).astype(np.float32)
            ref += we[:, None] * (quant_real(h) @ real_matrix(ex.down, e).T)
        err = np.abs(r["out_exact"] - ref).max() / np.abs(ref).max()
        assert err < 1e-12, (act, err)
        # about half the pre-activations are negative and contribute nothing
        U0 = xr @ real_matrix(ex.up, 0).T
        assert 0.3 < np.mean(U0 < 0) < 0.7


def test_tiny_gateless_workload_runs():
    """The tiny_relu2 workload runs end to end with no gate matrix."""
    inp = inputs.make("tiny_relu2")
    assert inp.experts.gate is None and inp.dims.act == oracle.ACT_RELU2
    r = oracle.layer_forward(inp)
    assert np.abs(bf16_to_f64(r["out"])).max() > 0
