"""Pins of the oracle's weight quantiser (FP32 master weights -> MXFP4 under
fp32 128x128 block scales; P1 section 4 and P4 section 4, FP4 quantisation-aware
training, with the OCP MX shared-exponent rule for the 1x32 sub-blocks).

Each check compares against something other than the quantiser's own code:
brute-force nearest-value search for the E2M1 encoder, exact round trips of
blocks built from known codes and exponents, a constructed clamping case, a
brute-force nearest-grid check on random weights, and the lossless FP4 -> FP8
map of the pages applied to the quantiser's output.
"""
import numpy as np
import pytest

import oracle

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def brute_e2m1(x: float) -> int:
    """Nearest of the 8 magnitudes; on a tie the even code; >= 6 -> 6; sign kept."""
    m = abs(x)
    if m >= 6.0:
        idx = 7
    else:
        d = np.abs(GRID - m)
        cands = np.flatnonzero(d == d.min())
        idx = int(cands[0]) if len(cands) == 1 else int([c for c in cands if c % 2 == 0][0])
    return idx | (8 if np.signbit(x) else 0)


def e2m1_values(codes: np.ndarray) -> np.ndarray:
    c = codes.astype(np.int64)
    v = GRID[c & 7]
    return np.where(c & 8, -v, v)


def unpack_codes(fp4: np.ndarray) -> np.ndarray:
    lo = fp4 & 15
    hi = fp4 >> 4
    return np.stack([lo, hi], axis=-1).reshape(*fp4.shape[:-1], fp4.shape[-1] * 2)


def test_e2m1_encode_matches_brute_force():
    rng = np.random.default_rng(0)
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    xs = list(GRID) + mids + [m * (1 + s * 2.0 ** -40) for m in mids for s in (-1, 1)]
    xs += [6.0, 6.5, 7.0, 1e6, 0.0]
    xs += list(rng.uniform(-8, 8, 20000)) + list(rng.uniform(-0.4, 0.4, 2000))
    xs += [-x for x in xs]
    for x in xs:
        assert oracle.e2m1_encode(x) == brute_e2m1(x), x
    assert oracle.e2m1_encode(-0.0) == 8 and oracle.e2m1_encode(0.0) == 0


def test_known_ties():
    # halfway cases go to the even code: 0.25->0, 0.75->1.0, 1.25->1.0,
    # 1.75->2.0, 2.5->2.0, 3.5->4.0, 5->4.0
    want = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for x, c in want.items():
        assert oracle.e2m1_encode(x) == c
        assert oracle.e2m1_encode(-x) == c | 8


def build_representable(rng, E, N, K):
    """Weights w = blk * e2m1(code) * 2^b with known codes, b and blk: every
    128x128 block holds one element 6 * 2^6 (so amax/384 recovers blk exactly),
    and every sub-block holds an element of magnitude 4 or 6 (so the shared
    exponent rule recovers b)."""
    NB, KB = N // 128, K // 128
    blk = (2.0 ** rng.integers(-12, 4, (E, NB, KB))).astype(np.float32)
    b = rng.integers(-8, 7, (E, N, K // 32))
    codes = rng.integers(0, 16, (E, N, K)).astype(np.uint8)
    # one magnitude-4 or -6 element per sub-block
    pos = rng.integers(0, 32, (E, N, K // 32))
    big = rng.choice(np.array([6, 7, 14, 15], np.uint8), (E, N, K // 32))
    cv = codes.reshape(E, N, K // 32, 32)
    np.put_along_axis(cv, pos[..., None], big[..., None], axis=-1)
    # block maxima: row 0 of each block, first sub-block, b = 6, code 7
    for nb in range(NB):
        for kb in range(KB):
            b[:, nb * 128, kb * 4] = 6
            cv[:, nb * 128, kb * 4, 0] = 7
    codes = cv.reshape(E, N, K)
    scale = np.repeat(np.repeat(blk.astype(np.float64), 128, axis=1), 128, axis=2)
    w = e2m1_values(codes) * np.ldexp(1.0, np.repeat(b, 32, axis=2)) * scale
    w = w.astype(np.float32)
    assert np.array_equal(w.astype(np.float64), e2m1_values(codes) * np.ldexp(1.0, np.repeat(b, 32, axis=2)) * scale)
    return w, codes, b, blk


def test_roundtrip_of_representable_weights():
    rng = np.random.default_rng(1)
    w, codes, b, blk = build_representable(rng, 2, 256, 384)
    fp4, e8, s, clamped = oracle.quantize_weights(w)
    assert clamped == 0
    assert np.array_equal(s, blk)
    assert np.array_equal(e8.astype(np.int64) - 127, b)
    got = unpack_codes(fp4)
    # a zero element keeps its sign: -0.0 encodes as 0x8, +0.0 as 0x0
    assert np.array_equal(got, codes)


def test_clamped_subblock_is_counted():
    w = np.zeros((1, 128, 128), np.float32)
    w[0, 0, 0] = 384.0                      # block scale 1.0
    w[0, 5, 32:64] = 2.0 ** -20             # wants b = -22: below the window
    w[0, 7, 64:96] = 3.0 * 2.0 ** -7        # floor(log2(3 * 2^-7)) - 2 = -8: the window's edge
    fp4, e8, s, clamped = oracle.quantize_weights(w)
    assert s[0, 0, 0] == 1.0
    assert clamped == 1
    assert e8[0, 5, 1] == 127 - 8 and e8[0, 7, 2] == 127 - 8
    assert np.all(unpack_codes(fp4)[0, 5, 32:64] == 0)            # 2^-12 rounds to zero
    assert np.all(unpack_codes(fp4)[0, 7, 64:96] == 7)            # 3 * 2^-7 * 2^8 = 6 exactly
    assert e8[0, 0, 0] == 127 + 6 and unpack_codes(fp4)[0, 0, 0] == 7
    assert e8[0, 1, 0] == 127                                     # all-zero sub-block: b = 0


def test_random_weights_nearest_code_and_block_max():
    rng = np.random.default_rng(2)
    E, N, K = 2, 256, 256
    w = (rng.standard_normal((E, N, K)) * np.exp(rng.standard_normal((E, N, 1)))).astype(np.float32)
    w[0, :128, :128] *= 1e-3                 # a quiet block
    fp4, e8, s, clamped = oracle.quantize_weights(w)
    codes = unpack_codes(fp4)
    b = e8.astype(np.int64) - 127
    assert clamped == 0
    for e in range(E):
        for nb in range(N // 128):
            for kb in range(K // 128):
                blkw = w[e, nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
                amax = np.abs(blkw).max()
                assert s[e, nb, kb] == np.float32(amax / np.float32(384.0))
                r, c = np.unravel_index(np.abs(blkw).argmax(), blkw.shape)
                assert codes[e, nb * 128 + r, kb * 128 + c] & 7 == 7     # the block max lands on 6
    # every element: brute-force nearest code of v * 2^-b, v = w / s in fp32
    idx = rng.integers(0, E * N * K, 3000)
    for i in idx:
        e, n, k = np.unravel_index(i, (E, N, K))
        v = np.float32(w[e, n, k] / s[e, n // 128, k // 128])
        assert codes[e, n, k] == brute_e2m1(float(v) * 2.0 ** -int(b[e, n, k // 32]))
    # the shared exponent: 4 <= max |v| * 2^-b < 8 for every non-zero sub-block
    v = w / np.repeat(np.repeat(s, 128, axis=1), 128, axis=2)
    am = np.abs(v).reshape(E, N, K // 32, 32).max(axis=-1) * np.ldexp(1.0, -b)
    assert np.all((am >= 4) & (am < 8))


def test_quantised_weights_dequantise_losslessly():
    """The quantiser's codes and exponents, through the pages' FP4 -> E4M3 map,
    give exactly e2m1 * 2^b (P1 section 4: the conversion loses nothing)."""
    rng = np.random.default_rng(3)
    w = rng.standard_normal((1, 128, 256)).astype(np.float32)
    w[0, 3, :32] *= 1e-4
    fp4, e8, s, _ = oracle.quantize_weights(w)
    q = oracle.dequant_matrix(fp4[0], e8[0])
    got = np.vectorize(oracle.e4m3_value)(q.astype(np.int64))
    want = e2m1_values(unpack_codes(fp4)[0]) * np.ldexp(1.0, np.repeat(e8[0].astype(np.int64) - 127, 32, axis=1))
    assert np.array_equal(got, want)


def test_reconstruction_error_within_e2m1_half_step():
    """|w - blk * e2m1(code) * 2^b| <= blk * 2^b * (half the E2M1 spacing at
    |v| 2^-b), or the saturation excess above 6, for every element: the
    quantiser picks the nearest representable value under its own scales."""
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((2, 256, 384)) * np.exp(2 * rng.standard_normal((2, 256, 1)))).astype(np.float32)
    fp4, e8, s, clamped = oracle.quantize_weights(w)
    codes = unpack_codes(fp4)
    b = np.repeat(e8.astype(np.int64) - 127, 32, axis=2)
    blk = np.repeat(np.repeat(s.astype(np.float64), 128, 1), 128, 2)
    deq = e2m1_values(codes) * np.ldexp(1.0, b) * blk
    m = np.abs(w.astype(np.float64) / blk) * np.ldexp(1.0, -b)        # |v| 2^-b (fp64)
    spacing = np.where(m < 2, 0.5, np.where(m < 4, 1.0, 2.0))
    bound = np.where(m <= 6, spacing / 2, m - 6) * np.ldexp(1.0, b) * blk
    err = np.abs(w - deq)
    assert np.all(err <= bound * (1 + 1e-6) + 1e-30), np.max(err / np.maximum(bound, 1e-300))
    # on these weights the MXFP4 map keeps about 88% of the signal
    assert np.linalg.norm(w - deq) / np.linalg.norm(w) < 0.15


def test_layer_from_fp32_master_weights():
    """Dense equivalence starting from FP32 master weights: quantise with the
    oracle, run the layer with every token routed to every expert (exact
    mode), and compare with a dense SwiGLU FFN on the same master weights in
    fp64.  The only differences are the FP4 weight and FP8 activation
    quantisation: about 12% relative error per MXFP4 matrix on Gaussian
    weights, about 21% through the three matrices and SwiGLU here, far below
    what a wrong scale or transposition gives (> 100%)."""
    from fp4_weight_grouped_amd import inputs
    T, H, I, E = 16, 256, 128, 4
    rng = np.random.default_rng(5)
    wg, wu = (rng.standard_normal((E, I, H)).astype(np.float32) * np.float32(0.05) for _ in range(2))
    wd = rng.standard_normal((E, H, I)).astype(np.float32) * np.float32(0.05)
    mats = []
    for wm in (wg, wu, wd):
        fp4, e8, s, clamped = oracle.quantize_weights(wm)
        assert clamped == 0
        mats.append(inputs.Matrix(fp4=fp4, e8m0=e8, blk=s))
    x = inputs.gen_x(5, T, H)
    inp = inputs.Inputs(dims=inputs.Dims(T, H, I, E, E), mode=1, x=x, w_router=inputs.gen_router(5, H, E),
                        bias=None, token_ids=None, experts=inputs.Experts(*mats))
    r = oracle.layer_forward(inp, exact=True)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = np.zeros((T, H))
    for e in range(E):
        G = xf @ wg[e].T.astype(np.float64)
        U = xf @ wu[e].T.astype(np.float64)
        ref += (1.0 / E) * ((G / (1 + np.exp(-G)) * U) @ wd[e].T.astype(np.float64))
    rel = np.linalg.norm(r["out_exact"] - ref) / np.linalg.norm(ref)
    assert rel < 0.3, rel
    # a transposed down matrix or a dropped block scale is far off
    bad = np.zeros((T, H))
    for e in range(E):
        G = xf @ wg[e].T.astype(np.float64)
        U = xf @ wu[e].T.astype(np.float64)
        bad += (1.0 / E) * ((G / (1 + np.exp(-G)) * U) @ wd[e].reshape(I, H).astype(np.float64))
    assert np.linalg.norm(r["out_exact"] - bad) / np.linalg.norm(ref) > 1.0
