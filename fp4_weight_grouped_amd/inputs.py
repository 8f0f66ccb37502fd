"""Seeded synthetic inputs for the MoE layer forward.

This module only draws random numbers and lays them out in the byte formats the
layer consumes.  It holds none of the layer's arithmetic (no routing, no
quantisation, no dequantisation): both the CPU oracle under ``oracle/`` and the
HIP library read the arrays produced here.

Workloads (all seed 0 unless stated):

* ``tiny``     T=64,   H=256,  I=128,  E=8,   k=2  (oracle finishes in seconds)
* ``decode``   T=128,  H=4096, I=2048, E=256, k=8  (long-tail small batch)
* ``prefill``  T=8192, H=4096, I=2048, E=256, k=8
* ``zipf``     T=4096, same dims, per-expert router bias -1.2*ln(rank)
* ``hash``     T=4096, same dims, hash routing, equal weights
* ``ragged``   64 requests with lognormal(5, 1.2) lengths clipped to [1, 4096]
* ``tiny_relu2``, ``decode_relu2``, ``prefill_relu2``: the gate-less expert
  FFN with squared ReLU; the large ones at I=3072, the parameter count of the
  SwiGLU experts at I=2048 (2*H*3072 = 3*H*2048); ``tiny_relu2`` at I=256.

Distributions: x ~ N(0,1) rounded to bf16; router W_r ~ N(0, 0.02) fp32 [H][E];
FP4 codes uniform over all 16 nibbles; the power-of-two sub-block exponent b is
uniform over the integers in [-4, 0] and stored as the E8M0 byte 127+b; the
fp32 scale of every 128x128 weight block ~ U(0.01, 0.05).

Weight layout handed to the library ("canonical"): for a matrix with N output
rows and K inputs, ``fp4`` is uint8 [E][N][K/2] (K contiguous, even k in the low
nibble), ``e8m0`` is uint8 [E][N][K/32], ``blk`` is fp32 [E][N/128][K/128].
gate and up have N=I, K=H; down has N=H, K=I.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import functools
import os
from typing import Optional

import numpy as np

# One random stream per tensor (per expert for the weights), keyed by a fixed
# tag, so that every tensor of a workload is reproducible on its own.
_TAG = {
    "x": 1, "w_router": 2,
    "gate": 3, "up": 4, "down": 5,
    "zipf_perm": 6, "lengths": 7,
}

ROUTE_LEARNED = 0
ROUTE_HASH = 1

# Expert activations: SwiGLU (gate, up, down) or a gate-less one (up, down).
ACT_SWIGLU = 0
ACT_RELU2 = 1
ACT_RELU = 2


@dataclasses.dataclass(frozen=True)
class Dims:
    T: int
    H: int
    I: int
    E: int
    topk: int
    act: int = ACT_SWIGLU


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dims: Dims
    mode: int = ROUTE_LEARNED
    zipf_bias: bool = False
    ragged_requests: int = 0       # >0: T is the sum of this many request lengths
    b_range: tuple = (-4, 0)


_BIG = dict(H=4096, I=2048, E=256, topk=8)

WORKLOADS = {
    "tiny": Workload("tiny", Dims(T=64, H=256, I=128, E=8, topk=2)),
    "decode": Workload("decode", Dims(T=128, **_BIG)),
    "prefill": Workload("prefill", Dims(T=8192, **_BIG)),
    "zipf": Workload("zipf", Dims(T=4096, **_BIG), zipf_bias=True),
    "hash": Workload("hash", Dims(T=4096, **_BIG), mode=ROUTE_HASH),
    "ragged": Workload("ragged", Dims(T=0, **_BIG), ragged_requests=64),
    "tiny_relu2": Workload("tiny_relu2", Dims(T=64, H=256, I=256, E=8, topk=2, act=ACT_RELU2)),
    "decode_relu2": Workload("decode_relu2", Dims(T=128, H=4096, I=3072, E=256, topk=8, act=ACT_RELU2)),
    "prefill_relu2": Workload("prefill_relu2", Dims(T=8192, H=4096, I=3072, E=256, topk=8, act=ACT_RELU2)),
}


def _rng(seed: int, tag: str) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, _TAG[tag]]))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16) using torch's round-to-nearest-even cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


@dataclasses.dataclass
class Matrix:
    """One weight matrix for all experts, canonical layout (see module docstring)."""
    fp4: np.ndarray    # uint8 [E][N][K/2]
    e8m0: np.ndarray   # uint8 [E][N][K/32]
    blk: np.ndarray    # fp32  [E][N/128][K/128]

    @property
    def nbytes(self) -> int:
        return self.fp4.nbytes + self.e8m0.nbytes + self.blk.nbytes


@dataclasses.dataclass
class Experts:
    gate: Optional[Matrix]   # N=I, K=H; None for the gate-less activations
    up: Matrix     # N=I, K=H
    down: Matrix   # N=H, K=I


def gen_matrix(seed: int, tag: str, E: int, N: int, K: int,
               b_range=(-4, 0), blk_range=(0.01, 0.05)) -> Matrix:
    """One random stream per (matrix, expert); experts are drawn in parallel
    threads, which does not change the values."""
    fp4 = np.empty((E, N, K // 2), np.uint8)
    e8m0 = np.empty((E, N, K // 32), np.uint8)
    blk = np.empty((E, N // 128, K // 128), np.float32)

    def one(e):
        r = np.random.default_rng(np.random.SeedSequence([seed, _TAG[tag], e]))
        n = N * K // 2
        # uniform FP4 codes: raw 64-bit generator output viewed as bytes (two codes per byte)
        fp4[e] = r.bit_generator.random_raw((n + 7) // 8).view(np.uint8)[:n].reshape(N, K // 2)
        b = r.integers(b_range[0], b_range[1] + 1, size=(N, K // 32), dtype=np.int16)
        e8m0[e] = (b + 127).astype(np.uint8)
        blk[e] = r.uniform(blk_range[0], blk_range[1], size=(N // 128, K // 128))

    with concurrent.futures.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(one, range(E)))
    return Matrix(fp4=fp4, e8m0=e8m0, blk=blk)


@functools.lru_cache(maxsize=2)
def gen_experts(seed: int, E: int, H: int, I: int, b_range=(-4, 0), gated: bool = True) -> Experts:
    return Experts(
        gate=gen_matrix(seed, "gate", E, I, H, b_range) if gated else None,
        up=gen_matrix(seed, "up", E, I, H, b_range),
        down=gen_matrix(seed, "down", E, H, I, b_range),
    )


def ragged_lengths(seed: int, n: int = 64) -> np.ndarray:
    r = _rng(seed, "lengths")
    L = np.rint(r.lognormal(mean=5.0, sigma=1.2, size=n))
    return np.clip(L, 1, 4096).astype(np.int64)


@dataclasses.dataclass
class Inputs:
    dims: Dims
    mode: int
    x: np.ndarray                    # uint16 bf16 bits [T][H]
    w_router: np.ndarray             # fp32 [H][E]
    bias: Optional[np.ndarray]       # fp32 [E] or None
    token_ids: Optional[np.ndarray]  # int64 [T] or None (hash routing keys)
    experts: Experts
    lengths: Optional[np.ndarray] = None   # ragged workload: request lengths


def gen_x(seed: int, T: int, H: int) -> np.ndarray:
    r = _rng(seed, "x")
    return to_bf16_bits(r.standard_normal((T, H), dtype=np.float32))


def gen_router(seed: int, H: int, E: int) -> np.ndarray:
    r = _rng(seed, "w_router")
    return (r.standard_normal((H, E), dtype=np.float32) * np.float32(0.02)).astype(np.float32)


def zipf_bias(seed: int, E: int, s: float = 1.2) -> np.ndarray:
    """log of a Zipf(s) popularity over a random expert order: b_e = -s*ln(rank_e)."""
    r = _rng(seed, "zipf_perm")
    rank = r.permutation(E).astype(np.float64) + 1.0
    return (-s * np.log(rank)).astype(np.float32)


def make(name_or_wl, seed: int = 0, T: Optional[int] = None) -> Inputs:
    """Build the inputs of a named workload (optionally overriding T)."""
    wl = WORKLOADS[name_or_wl] if isinstance(name_or_wl, str) else name_or_wl
    d = wl.dims
    lengths = None
    if wl.ragged_requests:
        lengths = ragged_lengths(seed, wl.ragged_requests)
        Tn = int(lengths.sum())
    else:
        Tn = d.T
    if T is not None:
        Tn = T
    dims = Dims(T=Tn, H=d.H, I=d.I, E=d.E, topk=d.topk, act=d.act)
    x = gen_x(seed, Tn, d.H)
    wr = gen_router(seed, d.H, d.E)
    bias = zipf_bias(seed, d.E) if wl.zipf_bias else None
    token_ids = np.arange(Tn, dtype=np.int64) if wl.mode == ROUTE_HASH else None
    ex = gen_experts(seed, d.E, d.H, d.I, wl.b_range, d.act == ACT_SWIGLU)
    return Inputs(dims=dims, mode=wl.mode, x=x, w_router=wr, bias=bias,
                  token_ids=token_ids, experts=ex, lengths=lengths)

