"""CPU oracle for the W4A16 group-quantized GEMM (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the GPU library
(``decode_w4a16_repack_amd``) and neither imports the other.

What it computes follows the onnx-genai pull request "Marlin-style fused
fp16xint4 tensor-core GEMM": the dequantized weight is (q - zp) * scale per
(column, group) ("What's landed"), checked there against an f64
dequant -> GEMM oracle ("Validation"); the RMSNorm prologue ("fused RMS-norm
epilogue" update) and the paired gate/up SwiGLU ("gate_up SwiGLU MLP fusion"
update).  The bias + ReLU epilogue and the fused/unfused byte model follow the
"Fusion benchmark" page; the skip + RMSNorm residual sum (``skip_sum``)
follows the SkipSimplifiedLayerNormalization op named in the "Stage 2 of
spec-capture" update.

Every value is computed in IEEE double by ``w4a16_oracle.c`` and
``repack_oracle.c``; this module only widens inputs to double (exact for fp16
and fp32) and marshals arrays.

Pinned by ``tests/test_oracle_pins.py``.  Parity unpinned: absolute output
values beyond the closed forms, invariants and brute-force cases listed there
(the pages print no worked numeric example).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SOURCES = ["w4a16_oracle.c", "repack_oracle.c"]

EPILOGUES = {"none": 0, "bias": 1, "bias_relu": 2}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    if not force and os.path.exists(_SO):
        return _SO
    srcs = [os.path.join(_HERE, s) for s in _SOURCES]
    tmp = _SO + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", "-o", tmp] + srcs + ["-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        lib.oracle_dequant.argtypes = [P, P, P, I, I, I, P]
        lib.oracle_gemm.argtypes = [P, I, I, I, P, P, P, I, P, D, I, P, P, I, P, P]
        lib.oracle_gate_up.argtypes = [P, I, I, I, P, P, P, P, P, P, I, P, D, P, I, P, P]
        lib.oracle_packed_layout.argtypes = [I, I, I, I, I, P, P, P]
        lib.oracle_weight_nibble_index.argtypes = [I, I, I]
        lib.oracle_weight_nibble_index.restype = ctypes.c_long
        lib.oracle_rmsnorm.argtypes = [P, I, I, P, D, P, P]
        lib.oracle_rmsnorm.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [I]
        lib.oracle_set_threads.restype = None
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_repack.argtypes = [P, P, P, I, I, I, I, P]
        lib.oracle_unrepack.argtypes = [P, I, I, I, I, I, P, P, P]
        for f in (lib.oracle_dequant, lib.oracle_gemm, lib.oracle_gate_up,
                  lib.oracle_packed_layout, lib.oracle_repack, lib.oracle_unrepack):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a), dtype=np.float64)


def _u8(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a), dtype=np.uint8)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def set_threads(n: int) -> None:
    """Threads for the oracle's parallel loops in this process."""
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    """OpenMP threads the oracle's parallel loops use in this process."""
    return int(_load().oracle_max_threads())


def dequant(qweight, scales, zeros, K: int, N: int, group: int) -> np.ndarray:
    """Dense f64 W[K][N] with W[k][n] = (q - z) * s."""
    lib = _load()
    q, s, z = _u8(qweight), _f64(scales), _u8(zeros)
    W = np.empty((K, N), dtype=np.float64)
    _check(lib.oracle_dequant(_ptr(q), _ptr(s), _ptr(z), K, N, group, _ptr(W)), "dequant")
    return W


def gemm(A, qweight, scales, zeros, group: int, N: int, *, gamma=None,
         eps: float = 1e-6, epilogue: str = "none", bias=None, cols=None) -> np.ndarray:
    """f64 output [M][len(cols) or N] of the fused GEMM (see module doc)."""
    lib = _load()
    A = _f64(A)
    M, K = A.shape
    q, s, z = _u8(qweight), _f64(scales), _u8(zeros)
    g, b = _f64(gamma), _f64(bias)
    c = None if cols is None else np.ascontiguousarray(cols, dtype=np.int32)
    nc = N if c is None else len(c)
    out = np.empty((M, nc), dtype=np.float64)
    xw = np.empty((M, K), dtype=np.float64)
    rc = lib.oracle_gemm(_ptr(A), M, K, N, _ptr(q), _ptr(s), _ptr(z), group,
                         _ptr(g), float(eps), EPILOGUES[epilogue], _ptr(b),
                         _ptr(c), nc, _ptr(xw), _ptr(out))
    _check(rc, "gemm")
    return out


def gate_up(A, gate, up, group: int, N: int, *, gamma=None, eps: float = 1e-6,
            cols=None) -> np.ndarray:
    """f64 silu(X.Wg) * (X.Wu); ``gate``/``up`` are (qweight, scales, zeros)."""
    lib = _load()
    A = _f64(A)
    M, K = A.shape
    qg, sg, zg = _u8(gate[0]), _f64(gate[1]), _u8(gate[2])
    qu, su, zu = _u8(up[0]), _f64(up[1]), _u8(up[2])
    g = _f64(gamma)
    c = None if cols is None else np.ascontiguousarray(cols, dtype=np.int32)
    nc = N if c is None else len(c)
    out = np.empty((M, nc), dtype=np.float64)
    xw = np.empty((M, K), dtype=np.float64)
    rc = lib.oracle_gate_up(_ptr(A), M, K, N, _ptr(qg), _ptr(sg), _ptr(zg),
                            _ptr(qu), _ptr(su), _ptr(zu), group, _ptr(g),
                            float(eps), _ptr(c), nc, _ptr(xw), _ptr(out))
    _check(rc, "gate_up")
    return out


def rmsnorm(A, gamma, eps: float = 1e-6):
    """(X, r): the f64 RMSNorm prologue X[m][k] = A[m][k] * gamma[k] * r[m],
    r[m] = 1 / sqrt(mean_k A[m][k]^2 + eps) (eps inside the root, mean over
    the whole row)."""
    lib = _load()
    A = _f64(A)
    M, K = A.shape
    g = _f64(gamma)
    X = np.empty((M, K), dtype=np.float64)
    r = np.empty(M, dtype=np.float64)
    _check(lib.oracle_rmsnorm(_ptr(A), M, K, _ptr(g), float(eps), _ptr(X), _ptr(r)), "rmsnorm")
    return X, r


def gemm_rms_staged(A, qweight, scales, zeros, group: int, N: int, gamma, *,
                    eps: float = 1e-6, staging: str = "normalized",
                    epilogue: str = "none", bias=None, cols=None) -> np.ndarray:
    """The fused GEMM with the RMSNorm prologue under the staged readings
    of the "fused RMS-norm epilogue" update, which keeps the prologue's
    result in fp16 scratch between the norm and the product:

    * ``staging="normalized"``: X16 = fp16(X) (X as in :func:`rmsnorm`),
      then the product and epilogue on X16;
    * ``staging="scaled"``: X16 = fp16(A * gamma) (each product rounded
      once), the product on X16, each row times r[m], then the epilogue.

    Every other step is the canonical oracle's, in f64; only the one fp16
    rounding of the staged row differs, so the gap to :func:`gemm` with
    ``gamma`` is bounded by that rounding (pinned in the tests)."""
    A64 = _f64(A)
    X, r = rmsnorm(A64, gamma, eps)
    if staging == "normalized":
        return gemm(to_fp16(X), qweight, scales, zeros, group, N, epilogue=epilogue,
                    bias=bias, cols=cols)
    if staging != "scaled":
        raise ValueError(f"unknown staging {staging!r}")
    xg = to_fp16(A64 * _f64(gamma)[None, :])
    y = gemm(xg, qweight, scales, zeros, group, N, cols=cols) * r[:, None]
    if epilogue == "none":
        return y
    b = _f64(bias)
    b = b if cols is None else b[np.asarray(cols)]
    y = y + b[None, :]
    return np.maximum(y, 0.0) if epilogue == "bias_relu" else y


def packed_layout(K: int, N: int, group: int, esize: int, has_zp: bool):
    """(scales offset, zeros offset, total bytes) of the packed buffer."""
    lib = _load()
    so, zo, tot = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    rc = lib.oracle_packed_layout(K, N, group, esize, int(bool(has_zp)),
                                  ctypes.byref(so), ctypes.byref(zo), ctypes.byref(tot))
    _check(rc, "packed_layout")
    return so.value, zo.value, tot.value


def weight_nibble_index(K: int, k: int, n: int) -> int:
    return int(_load().oracle_weight_nibble_index(K, k, n))


def repack(qweight, scales, zeros, K: int, N: int, group: int) -> np.ndarray:
    """Packed bytes (u8) of the canonical inputs; scales keep their dtype's bytes."""
    lib = _load()
    scales = np.ascontiguousarray(scales)
    esize = scales.dtype.itemsize
    q, z = _u8(qweight), _u8(zeros)
    _, _, total = packed_layout(K, N, group, esize, zeros is not None)
    out = np.empty(total, dtype=np.uint8)
    rc = lib.oracle_repack(_ptr(q), _ptr(scales.view(np.uint8)), _ptr(z), K, N,
                           group, esize, _ptr(out))
    _check(rc, "repack")
    return out


def unrepack(packed, K: int, N: int, group: int, scale_dtype, has_zp: bool):
    """Inverse of :func:`repack`: (qweight, scales, zeros-or-None)."""
    lib = _load()
    p = _u8(packed)
    G = K // group
    sdt = np.dtype(scale_dtype)
    q = np.empty((N, K // 2), dtype=np.uint8)
    s = np.empty((N, G), dtype=sdt)
    z = np.empty((N, (G + 1) // 2), dtype=np.uint8) if has_zp else None
    rc = lib.oracle_unrepack(_ptr(p), K, N, group, sdt.itemsize, int(bool(has_zp)),
                             _ptr(q), _ptr(s.view(np.uint8)), _ptr(z))
    _check(rc, "unrepack")
    return q, s, z


def skip_sum(A, residual) -> np.ndarray:
    """fp16 residual sum S = A + residual of the skip + RMSNorm prologue
    (SkipSimplifiedLayerNormalization, named in the "Stage 2 of
    spec-capture" update): the exact sum of two fp16 values, rounded once
    to fp16 (nearest-even).  The norm and the product then take S as the
    activation: ``gemm(skip_sum(A, R), ..., gamma=gamma)``.  A sum beyond
    the fp16 range rounds to infinity, as IEEE rounding defines."""
    with np.errstate(over="ignore"):
        return (np.asarray(A, dtype=np.float64) +
                np.asarray(residual, dtype=np.float64)).astype(np.float16)


def to_fp16(y: np.ndarray) -> np.ndarray:
    """Round the f64 result to fp16, nearest-even (IEEE default; beyond the
    fp16 range, to infinity)."""
    with np.errstate(over="ignore"):
        return np.asarray(y, dtype=np.float64).astype(np.float16)


def mlp(A, gate, up, down, group: int, I: int, H: int, *, gamma=None,
        eps: float = 1e-6, cols=None) -> np.ndarray:
    """f64 output [M][len(cols) or H] of the MLP block that the "gate_up
    SwiGLU MLP fusion" update names as the bulk of the decode cost: the
    paired gate/up projection (K = A's width, N = I, optional RMSNorm
    prologue), its result rounded once to fp16 (the intermediate is an fp16
    tensor handed from one projection to the next), then the plain down
    projection of that intermediate (K = I, N = H).  ``gate``, ``up`` and
    ``down`` are (qweight, scales, zeros); all three share ``group``."""
    h = to_fp16(gate_up(A, gate, up, group, I, gamma=gamma, eps=eps))
    return gemm(h, down[0], down[1], down[2], group, H, cols=cols)
