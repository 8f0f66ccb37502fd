"""GPU parity of moe_quantize_weights (FP32 master weights -> canonical MXFP4
under fp32 128x128 block scales; P1 section 4 and P4 section 4) against the
CPU oracle's quantiser.  Codes, sub-block exponents, block scales and the
clamped count are integer or exactly rounded fp32 results: the bar is
bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from fp4_weight_grouped_amd import v4moe

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def master_weights(rng, E, N, K):
    """Normal weights with a per-row log-normal magnitude, plus the cases the
    method has: an all-zero block, an all-zero sub-block, sub-blocks far below
    their block (clamped), fp32 subnormals, signed zeros, exact E2M1 ties,
    values that saturate at 6, and blocks of tiny magnitude (both ways of
    forming w / s)."""
    w = (rng.standard_normal((E, N, K)) * np.exp(rng.standard_normal((E, N, 1)))).astype(np.float32)
    if N >= 256 and K >= 256:
        w[0, :128, :128] = 0.0                                # all-zero block: s = 1
        w[0, 128, 128:160] = 0.0                              # all-zero sub-block: b = 0
        w[0, 129, 128:160] = -0.0                             # signed zeros keep code 8
        w[0, 130, 160:192] *= np.float32(1e-9)                # below the window: clamped
        w[0, 131, 192:224] = np.float32(1e-41) * rng.standard_normal(32).astype(np.float32)  # subnormals
    if N >= 384 and K >= 256:
        w[0, 256:384, :128] *= np.float32(1e-30)            # block max below 2^-84: the divide path
        tiny = w[0, 256:384, 128:256]                         # block max just above 2^-84 ...
        tiny *= np.float32(2.0 ** -80)
        tiny[5, :32] = np.float32(1e-38) * rng.standard_normal(32).astype(np.float32)   # ... with w < 2^-103
        tiny[6, 32:48] = np.float32(3e-44)                   # subnormal weights
        tiny[6, 48:64] = -np.float32(3e-44)
    # ties: a block whose max is 384 (s = 1) and a sub-block with max 4 (b = 0)
    # holding every E2M1 midpoint and both signs
    kb = 2 if K >= 384 else 0
    blkw = w[-1, -128:, kb * 128:(kb + 1) * 128]
    blkw[:] = np.clip(blkw, -300, 300)
    blkw[0, 0] = 384.0
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0,
                     4.0, 0.5, -0.0, 0.0, 3.0, 2.0, 1.0, 1.5, -6.0 + 2.0 ** -20, 5.5, 5.25,
                     4.75, 0.125, -0.375, 2.25, 2.75, 3.25, 3.75], np.float32)
    blkw[1, 32:64] = mids
    blkw[2, 64:96] = mids * np.float32(0.5)                  # same ties one exponent down (b = -1)
    return w


def run_gpu(w, clamped=True):
    wd = torch.from_numpy(w).to(DEV)
    c = torch.zeros(1, dtype=torch.int64, device=DEV) if clamped else None
    out = v4moe.quantize_weights(wd, c)
    torch.cuda.synchronize()
    return (out.fp4.cpu().numpy(), out.e8m0.cpu().numpy(), out.blk.cpu().numpy(),
            None if c is None else int(c.item()))


@pytest.mark.parametrize("E,N,K,seed", [(2, 256, 384, 0), (1, 128, 128, 1), (3, 384, 256, 2)])
def test_quantizer_bit_exact(E, N, K, seed):
    print(f"quantize E={E} N={N} K={K} seed={seed}", flush=True)
    w = master_weights(np.random.default_rng(seed), E, N, K)
    fp4, e8, blk, cl = oracle.quantize_weights(w)
    g4, g8, gb, gc = run_gpu(w)
    assert np.array_equal(gb.view(np.uint32), blk.view(np.uint32))
    assert np.array_equal(g8, e8), np.argwhere(g8 != e8)[:5]
    assert np.array_equal(g4, fp4), np.argwhere(g4 != fp4)[:5]
    assert gc == cl
    assert cl >= 1 or N < 256 or K < 256
    # the tie rows really hold ties (the pins of the oracle fix their codes)
    if K >= 384:
        codes = np.stack([fp4 & 15, fp4 >> 4], -1).reshape(E, N, K)
        assert list(codes[-1, N - 127, 256 + 32:256 + 39]) == [0, 2, 2, 4, 4, 6, 6]


def test_quantizer_full_expert_shape_and_clamp_counter_accumulates():
    """One expert's gate matrix at 2048 x 7168 against the oracle, and the
    clamped counter adds across calls instead of overwriting."""
    E, N, K = 1, 2048, 7168
    print(f"quantize E={E} N={N} K={K}", flush=True)
    rng = np.random.default_rng(5)
    w = master_weights(rng, E, N, K)
    fp4, e8, blk, cl = oracle.quantize_weights(w)
    wd = torch.from_numpy(w).to(DEV)
    c = torch.zeros(1, dtype=torch.int64, device=DEV)
    out = v4moe.quantize_weights(wd, c)
    v4moe.moe_quantize_weights(wd, out, c)
    torch.cuda.synchronize()
    assert np.array_equal(out.blk.cpu().numpy().view(np.uint32), blk.view(np.uint32))
    assert np.array_equal(out.e8m0.cpu().numpy(), e8)
    assert np.array_equal(out.fp4.cpu().numpy(), fp4)
    assert int(c.item()) == 2 * cl


def test_quantized_weights_feed_the_layer():
    """Quantiser output passes the prepack window check, and the packed
    weights read back through the matrix kernels' path as the oracle's
    lossless E4M3 dequantisation of the oracle's own quantisation."""
    E, H, I = 2, 256, 128
    rng = np.random.default_rng(7)
    ws = [master_weights(rng, E, I, H), master_weights(rng, E, I, H), master_weights(rng, E, H, I)]
    d = v4moe.dims(1, H, I, E, 1)
    mats = [v4moe.quantize_weights(torch.from_numpy(w).to(DEV)) for w in ws]
    packed = v4moe.prepack(d, v4moe.DeviceExperts(*mats))
    for w, m in zip(ws, [packed.gate, packed.up, packed.down]):
        fp4, e8, _, _ = oracle.quantize_weights(w)
        N, K = w.shape[1], w.shape[2]
        for e in range(E):
            out = torch.empty((N, K), dtype=torch.uint8, device=DEV)
            v4moe.moe_dequant_fp8(m, N, K, e, out)
            torch.cuda.synchronize()
            want = oracle.dequant_matrix(fp4[e], e8[e])
            assert np.array_equal(out.cpu().numpy(), want)


@pytest.mark.parametrize("E,H,I,seed", [(2, 256, 384, 3), (1, 512, 128, 4)])
def test_packed_output_equals_prepacked_canonical(E, H, I, seed):
    """packed=1 writes byte for byte what moe_prepack_weights makes of the
    canonical output (gate/up: N = I, K = H; down: N = H, K = I, so both an
    odd and an even number of 128-wide chunks occur)."""
    print(f"quantize packed E={E} H={H} I={I}", flush=True)
    rng = np.random.default_rng(seed)
    wg = torch.from_numpy(master_weights(rng, E, I, H)).to(DEV)
    wd = torch.from_numpy(master_weights(rng, E, H, I)).to(DEV)
    canon = v4moe.DeviceExperts(v4moe.quantize_weights(wg), v4moe.quantize_weights(wg), v4moe.quantize_weights(wd))
    ref = v4moe.prepack(v4moe.dims(1, H, I, E, 1), canon)
    pg, pd = v4moe.quantize_weights(wg, packed=True), v4moe.quantize_weights(wd, packed=True)
    torch.cuda.synchronize()
    for got, want in ((pg, ref.gate), (pd, ref.down)):
        assert torch.equal(got.fp4, want.fp4)
        assert torch.equal(got.e8m0, want.e8m0)
        assert torch.equal(got.blk, want.blk)
