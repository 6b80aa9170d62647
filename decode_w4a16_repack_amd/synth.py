"""Seeded synthetic inputs in the canonical storage format.

Shared by the tests, the benchmark and the oracle's callers.  It draws random
numbers and packs them into the input format; it holds none of the method's
arithmetic (no dequantization, no product).

Canonical format (the ONNX MatMulNBits reading used throughout):
  A        fp16 [M][K] row-major
  qweight  u8 [N][K/2]; code k of column n in nibble (k mod 2) of byte k/2,
           even k in the low nibble
  scales   fp16 or fp32 [N][G], G = K/group
  zeros    u8 [N][ceil(G/2)]; group i of column n in nibble (i mod 2),
           even i in the low nibble; None for the symmetric case

Value distributions follow the workload recipe: A ~ N(0,1); codes and
zero-points uniform over 0..15; scales uniform on [0.001, 0.02] (drawn in
double, rounded once to the storage dtype); bias ~ N(0, 0.1); gamma ~ N(1, 0.1).
Draw order from one numpy PCG64 generator: A, codes, scales, zero-points,
then bias or gamma, then a second weight set when one is asked for.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np


def pack_nibbles_rows(vals: np.ndarray) -> np.ndarray:
    """u8 [R][C] of 4-bit values -> u8 [R][ceil(C/2)], even column low nibble."""
    vals = np.asarray(vals, dtype=np.uint8)
    R, C = vals.shape
    if C % 2:
        vals = np.concatenate([vals, np.zeros((R, 1), np.uint8)], axis=1)
    return (vals[:, 0::2] | (vals[:, 1::2] << 4)).astype(np.uint8)


@dataclass
class QuantWeight:
    K: int
    N: int
    group: int
    codes: np.ndarray            # u8 [K][N], the raw draws (for pins)
    qweight: np.ndarray          # u8 [N][K/2]
    scales: np.ndarray           # fp16/fp32 [N][G]
    zp: Optional[np.ndarray]     # u8 [N][G] raw draws, None if symmetric
    zeros: Optional[np.ndarray]  # u8 [N][ceil(G/2)], None if symmetric


def draw_weight(rng: np.random.Generator, K: int, N: int, group: int,
                scale_dtype=np.float16, asym: bool = True,
                scale_lo: float = 0.001, scale_hi: float = 0.02) -> QuantWeight:
    G = K // group
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    scales = rng.uniform(scale_lo, scale_hi, size=(N, G)).astype(scale_dtype)
    zp = rng.integers(0, 16, size=(N, G), dtype=np.uint8) if asym else None
    qweight = pack_nibbles_rows(codes.T)
    zeros = pack_nibbles_rows(zp) if asym else None
    return QuantWeight(K, N, group, codes, qweight, scales, zp, zeros)


def weight_from_codes(codes: np.ndarray, scales: np.ndarray,
                      zp: Optional[np.ndarray], group: int) -> QuantWeight:
    """Canonical storage of given codes u8[K][N] and zero-points u8[N][G]."""
    codes = np.asarray(codes, dtype=np.uint8)
    K, N = codes.shape
    zeros = None if zp is None else pack_nibbles_rows(zp)
    return QuantWeight(K, N, group, codes, pack_nibbles_rows(codes.T),
                       np.ascontiguousarray(scales), zp, zeros)


@dataclass
class Problem:
    M: int
    K: int
    N: int
    group: int
    A: np.ndarray                  # fp16 [M][K]
    w: QuantWeight
    bias: Optional[np.ndarray] = None    # fp16 [N]
    gamma: Optional[np.ndarray] = None   # fp16 [K]
    w_up: Optional[QuantWeight] = None   # second weight set (gate_up)


def make_problem(M: int, K: int, N: int, group: int, *, seed: int = 0,
                 scale_dtype=np.float16, asym: bool = True, bias: bool = False,
                 gamma: bool = False, gate_up: bool = False) -> Problem:
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((M, K)).astype(np.float16)
    w = draw_weight(rng, K, N, group, scale_dtype, asym)
    b = rng.normal(0.0, 0.1, size=N).astype(np.float16) if bias else None
    g = rng.normal(1.0, 0.1, size=K).astype(np.float16) if gamma else None
    wu = draw_weight(rng, K, N, group, scale_dtype, asym) if gate_up else None
    return Problem(M, K, N, group, A, w, b, g, wu)


def draw_activations(seed: int, M: int, K: int) -> np.ndarray:
    return np.random.default_rng(seed).standard_normal((M, K)).astype(np.float16)
