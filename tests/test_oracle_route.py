"""Pins of the oracle's routing (P2, DeepSeekMoE notes: sqrt(softplus)
affinity replacing sigmoid; hash routing in the early layers) and of the
permutation that stands in for the dispatch (P1 sections 1.1-1.2)."""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from fp4_weight_grouped_amd import inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def bf16_bits(a):
    return inputs.to_bf16_bits(np.asarray(a, np.float32))


def bf16_vals(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_topk_brute_force_tiny():
    """E=8, k=2: the selection equals the best ordered pair under the order
    (logit descending, expert id ascending), found by enumerating all pairs."""
    inp = inputs.make("tiny")
    z = oracle.router_logits(inp.x, inp.w_router)
    ids, w = oracle.route(inp.x, inp.w_router, 2)
    E = 8
    for t in range(inp.dims.T):
        key = lambda e: (float(z[t, e]), -e)
        best = max(itertools.permutations(range(E), 2), key=lambda pr: tuple(key(e) for e in pr))
        assert tuple(ids[t]) == best


def _tie_inputs(T=32, H=256, E=8, seed=5):
    rng = np.random.default_rng(seed)
    x = rng.choice([-1.0, 0.0, 1.0], size=(T, H)).astype(np.float32)
    base = rng.choice([0.0, 0.5, 1.0], size=(H, 3)).astype(np.float32)
    wr = base[:, rng.integers(0, 3, E)]          # many identical columns -> exact logit ties
    return bf16_bits(x), np.ascontiguousarray(wr)


@pytest.mark.parametrize("k", [1, 2, 3, 5])
def test_topk_ties_go_to_lower_id(k):
    x, wr = _tie_inputs()
    z = oracle.router_logits(x, wr)
    ids, _ = oracle.route(x, wr, k)
    n_ties = 0
    for t in range(x.shape[0]):
        S = set(ids[t].tolist())
        assert len(S) == k
        for i in S:
            for j in set(range(8)) - S:
                assert z[t, i] > z[t, j] or (z[t, i] == z[t, j] and i < j)
                n_ties += z[t, i] == z[t, j]
        # slots are ranked: non-increasing logits, ties by increasing id
        for a, b in zip(ids[t][:-1], ids[t][1:]):
            assert z[t, a] > z[t, b] or (z[t, a] == z[t, b] and a < b)
    assert n_ties > 0          # the inputs really exercise ties


def test_weights_sum_to_one_and_follow_affinity():
    inp = inputs.make("tiny")
    z = oracle.router_logits(inp.x, inp.w_router)
    for k in (1, 2, 4, 8):
        ids, w = oracle.route(inp.x, inp.w_router, k)
        assert np.all(w > 0)
        s = w.astype(np.float64).sum(1)
        assert np.all(np.abs(s - 1.0) <= k * 2.0 ** -23)
        # w_j proportional to sqrt(softplus(z_j)) (fp64 textbook softplus via log(1+exp))
        zz = np.take_along_axis(z, ids, 1).astype(np.float64)
        a = np.sqrt(np.log1p(np.exp(zz)))
        np.testing.assert_allclose(w, a / a.sum(1, keepdims=True), rtol=3e-7)
        if k == 1:
            assert np.all(w == 1.0)


def test_logits_within_recursive_summation_bound():
    """|z - z_exact| <= gamma_H * sum_h |x_h w_h| (Higham, recursive summation
    with one rounding per step), z_exact from exact products and fsum."""
    inp = inputs.make("tiny")
    z = oracle.router_logits(inp.x, inp.w_router)
    xv = bf16_vals(inp.x).astype(np.float64)
    W = inp.w_router.astype(np.float64)
    H = xv.shape[1]
    u = 2.0 ** -24
    gamma = H * u / (1 - H * u)
    for t in range(0, inp.dims.T, 7):
        for e in range(inp.dims.E):
            prods = xv[t] * W[:, e]          # exact: 8-bit x 24-bit significands
            ex = math.fsum(prods)
            assert abs(float(z[t, e]) - ex) <= gamma * np.abs(prods).sum()


def test_logits_sequential_fma_order():
    """Closed form that fixes the order: 1*2^24 + 1*1 + 1*(-2^24) is 0 when summed
    left to right in fp32 (2^24 + 1 rounds to 2^24) but 1 exactly; a bias is one
    fp32 add after the chain."""
    H, E = 128, 2
    x = bf16_bits(np.ones((1, H), np.float32))
    wr = np.zeros((H, E), np.float32)
    wr[0, 0], wr[1, 0], wr[2, 0] = 2.0 ** 24, 1.0, -(2.0 ** 24)
    wr[0, 1], wr[1, 1], wr[2, 1] = 1.0, 2.0 ** 24, -(2.0 ** 24)   # 1 + 2^24 -> 2^24 + 1 lost too
    wr[3, 1] = 3.0
    z = oracle.router_logits(x, wr)
    assert z[0, 0] == 0.0
    assert z[0, 1] == 3.0
    # a fused multiply-add keeps the exact product: -3 + 3*(1+2^-23) = 3*2^-23,
    # where a separately rounded product would give 2^-21
    wr2 = np.zeros((H, 1), np.float32)
    xx = np.zeros((1, H), np.float32)
    xx[0, 0], wr2[0, 0] = 1.0, -3.0
    xx[0, 1], wr2[1, 0] = 3.0, np.float32(1 + 2.0 ** -23)
    z2 = oracle.router_logits(bf16_bits(xx), wr2)
    assert z2[0, 0] == np.float32(3 * 2.0 ** -23)
    b = np.array([0.25, -0.5], np.float32)
    zb = oracle.router_logits(x, wr, b)
    assert zb[0, 0] == np.float32(0.25) and zb[0, 1] == np.float32(2.5)


def test_logits_single_chain_order():
    """One h-ascending chain over all of H, however long.  With x = 1:
    expert 0 holds 2^24 at h = 0 and 1 at h = 512 and h = 513: every partial
    sum 2^24 + 1 rounds (to even) back to 2^24, so the chain gives 2^24, where
    any split of h into blocks of 512 or fewer summed separately gives 2^24 + 2;
    expert 1 holds 2^24 at h = 0, 1 at h = 1 .. H-2 and -2^24 at h = H-1: the
    chain loses every 1 and ends at 0, while an order that adds the ones
    first gives H - 2; expert 2 holds 1 everywhere (every partial sum exact),
    so its logit is H.  Error bound gamma_H * sum |x_h w_h| against exact sums
    at H = 4096 on random data."""
    for H in (1024, 640, 4096):
        x = bf16_bits(np.ones((1, H), np.float32))
        wr = np.zeros((H, 3), np.float32)
        wr[0, 0], wr[512, 0], wr[513, 0] = 2.0 ** 24, 1.0, 1.0
        wr[0, 1], wr[1:H - 1, 1], wr[H - 1, 1] = 2.0 ** 24, 1.0, -(2.0 ** 24)
        wr[:, 2] = 1.0
        z = oracle.router_logits(x, wr)
        assert z[0, 0] == np.float32(2.0 ** 24)
        assert z[0, 1] == 0.0
        assert z[0, 2] == np.float32(H)
    rng = np.random.default_rng(7)
    H, E = 4096, 8
    x = bf16_bits(rng.standard_normal((3, H)).astype(np.float32))
    wr = rng.standard_normal((H, E)).astype(np.float32)
    z = oracle.router_logits(x, wr)
    xv = bf16_vals(x).astype(np.float64)
    u = 2.0 ** -24
    gamma = H * u / (1 - H * u)
    for t in range(3):
        for e in range(E):
            prods = xv[t] * wr[:, e].astype(np.float64)
            assert abs(float(z[t, e]) - math.fsum(prods)) <= gamma * np.abs(prods).sum()


def test_splitmix64_published_output():
    g = json.load(open(os.path.join(GOLD, "splitmix64.json")))
    gamma = int(g["golden_gamma"], 16)
    for i, h in enumerate(g["seed0_outputs"]):
        assert oracle.splitmix64((i * gamma) % 2 ** 64) == int(h, 16)


def test_hash_routing():
    T, H, E, k = 200, 128, 16, 4
    x = bf16_bits(np.zeros((T, H), np.float32))
    wr = np.zeros((H, E), np.float32)
    tid = np.arange(T, dtype=np.int64) * 7 + 3
    ids, w = oracle.route(x, wr, k, mode=1, token_ids=tid)
    assert np.all(w == np.float32(1.0 / k))
    hits = 0
    for t in range(T):
        assert len(set(ids[t].tolist())) == k
        first = oracle.splitmix64(int(tid[t]) * k) % E
        assert ids[t, 0] == first
        for j in range(k):
            c = oracle.splitmix64(int(tid[t]) * k + j) % E
            hits += ids[t, j] == c
    assert hits > 0.6 * T * k      # probing past a collision is the exception
    # k = E: every expert exactly once
    ids, w = oracle.route(x[:5], wr, E, mode=1)
    assert all(sorted(r.tolist()) == list(range(E)) for r in ids)


def _hash_ids(token_id, k, E):
    x = bf16_bits(np.zeros((1, 128), np.float32))
    ids, w = oracle.route(x, np.zeros((128, E), np.float32), k, mode=1,
                          token_ids=np.array([token_id], np.int64))
    assert np.all(w == np.float32(1.0 / k))
    return ids[0].tolist()


def test_hash_collision_probe_steps_up():
    """A raw hash that repeats an earlier pick moves to the next free expert id
    going up, wrapping from E-1 to 0 (P2's hash routing needs k distinct
    experts; the probe direction is the stated reading).  Raw hashes
    splitmix64(id*k + j) mod E are checked against the pinned generator, then
    the stored ids against sequences worked out by hand from them:
      E=16, k=4, id 17: raw 10 7 15 15 -> 15 taken, 15+1 wraps to 0;
      E=16, k=4, id 47: raw 6 1 5 5 -> 5 taken, 6 taken, 7;
      E=8,  k=8, id 0:  raw 7 1 6 5 2 2 0 7 -> slot 5: 2 taken, 3;
                        slot 7: 7, 0, 1, 2, 3 taken, 4.
    A probe stepping down (15 -> 14, 5 -> 4) or re-hashing gives other ids."""
    cases = [
        (17, 4, 16, [10, 7, 15, 15], [10, 7, 15, 0]),
        (47, 4, 16, [6, 1, 5, 5], [6, 1, 5, 7]),
        (0, 8, 8, [7, 1, 6, 5, 2, 2, 0, 7], [7, 1, 6, 5, 2, 3, 0, 4]),
    ]
    for tid, k, E, raw, want in cases:
        assert [oracle.splitmix64(tid * k + j) % E for j in range(k)] == raw
        assert _hash_ids(tid, k, E) == want, (tid, k, E)
    # k = E: the hand-worked sequence is a permutation of all experts
    assert sorted(cases[2][4]) == list(range(8))


def test_permutation_matches_stable_sort():
    rng = np.random.default_rng(6)
    for T, k, E in [(64, 2, 8), (37, 8, 256), (1, 1, 1), (300, 4, 16)]:
        ids = rng.integers(0, E, (T, k)).astype(np.int32)
        if E == 16:
            ids[:] = np.minimum(ids, 3)          # most experts empty
        off, sp, pp = oracle.permute(ids, E)
        flat = ids.ravel()
        ref = np.argsort(flat, kind="stable")
        assert np.array_equal(sp, ref)
        assert np.array_equal(pp[sp], np.arange(T * k))
        assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
        assert off[-1] == T * k and np.all(np.diff(off) >= 0)
