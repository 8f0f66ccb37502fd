"""Pins of the oracle's number formats and of the FP4 -> FP8 dequantisation.

The lossless-dequant claim (P1 section 4, FP4 quantisation-aware training; P4
section 4): E4M3 has two more exponent bits than E2M1, so e2m1(code) * 2^b is
exactly representable for a bounded range of sub-block exponents b.  The tests
enumerate every code and exponent and check the oracle's byte against exact
arithmetic, and the encoders against torch's casts and a brute-force search.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_e2m1_table_matches_spec():
    g = _gold("formats.json")
    for code in range(8):
        assert oracle.e2m1_value(code) == g["e2m1_positive_values_by_code"][code]
        assert oracle.e2m1_value(code | 8) == -g["e2m1_positive_values_by_code"][code]


def test_e4m3_decode_matches_spec():
    g = _gold("formats.json")
    for hexcode, v in g["e4m3_examples"].items():
        assert oracle.e4m3_value(int(hexcode, 16)) == v
    for c in g["e4m3_nan_codes"]:
        assert np.isnan(oracle.e4m3_value(c))
    finite = [oracle.e4m3_value(c) for c in range(256) if c not in g["e4m3_nan_codes"]]
    assert max(finite) == g["e4m3_max_normal"]
    pos = sorted(v for v in finite if v > 0)
    assert pos[0] == g["e4m3_min_subnormal"]
    assert g["e4m3_exponent_bits"] - g["e2m1_exponent_bits"] == 2


def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    tv = codes.to(torch.float64).numpy()
    for c in range(256):
        ov = oracle.e4m3_value(c)
        if np.isnan(tv[c]):
            assert np.isnan(ov)
        else:
            assert ov == tv[c], c


def test_e4m3_encode_decode_identity():
    for c in range(256):
        v = oracle.e4m3_value(c)
        if np.isnan(v):
            continue
        assert oracle.e4m3_encode(v) == c, hex(c)


def _brute_e4m3(vals):
    """Nearest finite E4M3 code by exhaustive search; ties to the even code;
    anything above the largest finite magnitude saturates."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    cv = np.array([oracle.e4m3_value(int(c)) for c in codes])
    out = np.empty(len(vals), np.uint8)
    for i, v in enumerate(vals):
        if abs(v) > 448.0:
            out[i] = 0x7E | (0x80 if v < 0 else 0)
            continue
        same_sign = codes[(cv != 0) & (np.sign(cv) == np.sign(v))] if v != 0 else np.array([], int)
        cand = np.concatenate([same_sign, [0x80 if np.signbit(v) else 0x00]])
        d = np.abs(np.array([oracle.e4m3_value(int(c)) for c in cand]) - v)
        best = cand[d == d.min()]
        if len(best) > 1:
            best = best[(best & 1) == 0]
        out[i] = best[0]
    return out


def test_e4m3_encode_brute_force():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(1500) * 10.0,
        rng.uniform(-0.02, 0.02, 800),                 # subnormal neighbourhood
        rng.uniform(400, 500, 200) * rng.choice([-1, 1], 200),
        # exact midpoints between neighbouring codes (ties)
        [(oracle.e4m3_value(c) + oracle.e4m3_value(c + 1)) / 2 for c in range(0, 0x7E)],
        [-(oracle.e4m3_value(c) + oracle.e4m3_value(c + 1)) / 2 for c in range(0, 0x7E)],
    ])
    got = oracle.e4m3_encode_array(v)
    ref = _brute_e4m3(v)
    assert np.array_equal(got, ref)


def test_e4m3_encode_matches_torch_cast():
    # every bf16 value whose magnitude is below the saturation threshold, at a few scales
    b = np.arange(65536, dtype=np.uint32).astype(np.uint32) << 16
    f = b.view(np.float32)
    for scale in (1.0, 3.0, 1 / 7.0, 2.0 ** -8):
        v = (f * np.float32(scale)).astype(np.float32)
        v = v[np.isfinite(v) & (np.abs(v) < 464.0)]
        got = oracle.e4m3_encode_array(v.astype(np.float64))
        ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        # torch keeps the sign of a value that rounds to zero; so does the oracle
        assert np.array_equal(got, ref)
    rng = np.random.default_rng(2)
    v = (rng.standard_normal(2_000_000) * 60).astype(np.float32)
    v = v[np.abs(v) < 464.0]
    got = oracle.e4m3_encode_array(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates():
    assert oracle.e4m3_encode(1e9) == 0x7E
    assert oracle.e4m3_encode(-500.0) == 0xFE
    assert oracle.e4m3_encode(470.0) == 0x7E
    assert oracle.e4m3_encode(448.0) == 0x7E


def test_bf16_encode_matches_torch_cast():
    rng = np.random.default_rng(3)
    v = np.concatenate([
        rng.standard_normal(1_000_000).astype(np.float32),
        (rng.standard_normal(100_000) * 1e-30).astype(np.float32),
        # exact ties: bf16 value + half a bf16 ulp
        ((rng.integers(0, 2 ** 15, 50_000).astype(np.uint32) << 16) | 0x8000).view(np.float32),
    ])
    v = v[np.isfinite(v)]
    got = oracle.bf16_encode_array(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    for u in (0x3F80, 0xBF80, 0x4120, 0x0001):
        assert oracle.bf16_encode(oracle.bf16_value(u)) == u


def test_dequant_lossless_window_exhaustive():
    """Every code times 2^b is exactly representable in E4M3 iff b in [-8, 6]."""
    exact_b = []
    for b in range(-12, 11):
        ok = True
        for code in range(16):
            want = oracle.e2m1_value(code) * 2.0 ** b
            got = oracle.e4m3_value(oracle.dequant_code(code, b))
            ok &= (got == want) and (np.signbit(got) == np.signbit(want))
        if ok:
            exact_b.append(b)
    assert exact_b == list(range(-8, 7))


def test_dequant_negative_zero_kept():
    assert oracle.dequant_code(0x8, 0) == 0x80
    assert oracle.dequant_code(0x0, 0) == 0x00


def test_dequant_bitmap_equals_encoder_in_normal_window():
    for b in range(-5, 7):
        for code in range(16):
            assert oracle.dequant_bitmap(code, b) == oracle.dequant_code(code, b), (code, b)
    # below the window the bit formula is wrong for the smallest magnitudes
    assert any(oracle.dequant_bitmap(c, -6) != oracle.dequant_code(c, -6) for c in range(16))


def test_dequant_matrix_layout():
    """Canonical layout: row-major [N][K/2], even k in the low nibble, one E8M0
    byte per 32 consecutive k."""
    rng = np.random.default_rng(4)
    N, K = 8, 128
    fp4 = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    e8 = (127 + rng.integers(-4, 1, (N, K // 32))).astype(np.uint8)
    out = oracle.dequant_matrix(fp4, e8)
    for n in range(N):
        for k in range(K):
            code = (fp4[n, k // 2] >> (4 * (k & 1))) & 15
            b = int(e8[n, k // 32]) - 127
            assert oracle.e4m3_value(int(out[n, k])) == oracle.e2m1_value(int(code)) * 2.0 ** b
