"""Helpers for the GPU parity tests: run one seeded case through the C ABI
(via the binding) and through the oracle, and compare.

Tolerances:
  * the judged bound (onnx-genai PR "Marlin-style fused fp16xint4 tensor-core
    GEMM", "Validation"): |gpu - oracle| <= 2e-2 * max|oracle| per shape;
  * a strict secondary bound derived from the arithmetic: the GPU rounds the
    fp32 result to fp16 once (<= 1/2 ulp), fp32 summation of K terms adds
    far less than 1e-3 * max|out| at these sizes, and the RMSNorm prologue
    rounds A*gamma to fp16 once per element (relative 2^-11, a random walk
    over K terms), so |gpu - oracle| <= ulp16(|oracle|) + 1e-3 * max|out|.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import decode_w4a16_repack_amd as w4
from decode_w4a16_repack_amd import synth


def to_dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def nan_out(M: int, N: int) -> torch.Tensor:
    """Output buffer pre-filled with NaN, so an output the kernel never wrote
    fails the comparison instead of passing on stale memory."""
    return torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")


def ulp16(x):
    """fp16 unit in the last place at |x| (normal range)."""
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def repack_dev(w: synth.QuantWeight):
    return w4.repack(to_dev(w.qweight), to_dev(w.scales), to_dev(w.zeros), w.K, w.N, w.group)


def check_close(gpu, ref, what, strict=True):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    mx = float(np.abs(ref).max())
    err = np.abs(gpu - ref)
    tol = 2e-2 * mx
    assert err.max() <= tol, f"{what}: max err {err.max():.4g} > tol {tol:.4g}"
    if strict:
        bound = ulp16(ref) + 1e-3 * mx
        bad = err > bound
        assert not bad.any(), (f"{what}: {int(bad.sum())} outputs above the strict bound; "
                               f"worst {err.max():.4g} (max|out| {mx:.4g})")
    return float(err.max()), tol


def sample_cols(N: int, count: int, seed: int = 1) -> np.ndarray:
    """Columns spread over every 16-column tile boundary region and random ones."""
    rng = np.random.default_rng(seed)
    edge = np.array([0, 1, 15, 16, 31, N // 2, N - 17, N - 16, N - 1])
    return np.unique(np.concatenate([edge, rng.choice(N, size=count, replace=False)]))
