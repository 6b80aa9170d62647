"""Analytic byte model (test infrastructure only).

Follows the "Fusion benchmark" page ("Report bytes beside time"): for f32
matmul followed by bias and ReLU over an M x N output, the unfused chain
moves 20 bytes per output element (matmul writes 4; the bias pass reads 4 and
writes 4; the ReLU pass reads 4 and writes 4), the fused path 4 (one write),
and the operand traffic of A and B is common to both and excluded, so fusion
saves at most 16*M*N bytes.  With e bytes per output element the same count
gives 5e (unfused) and e (fused) per element.

The GEMM's own algorithmic bytes are what the method must move once: the
packed int4 weights (K*N/2), the per-(column, group) scales and zero-points,
the activations read once and the output written once.
"""
from __future__ import annotations


def epilogue_chain_bytes(M: int, N: int, elem_bytes: int, fused: bool) -> int:
    """Output-side bytes of matmul -> bias -> relu, excluding A/B traffic."""
    passes_unfused = 1 + 2 + 2  # matmul write; bias read+write; relu read+write
    return M * N * elem_bytes * (1 if fused else passes_unfused)


def epilogue_saved_bytes(M: int, N: int, elem_bytes: int) -> int:
    return (epilogue_chain_bytes(M, N, elem_bytes, fused=False)
            - epilogue_chain_bytes(M, N, elem_bytes, fused=True))


def rmsnorm_a_side_bytes(M: int, K: int, fused: bool) -> int:
    """Activation-side bytes (fp16): fused reads A once; unfused reads A,
    writes the normalized A to scratch and reads it back in the GEMM."""
    return 2 * M * K * (1 if fused else 3)


def gemm_bytes(M: int, K: int, N: int, group: int, scale_bytes: int = 2,
               has_zp: bool = True, bias: bool = False, gamma: bool = False,
               n_weights: int = 1) -> int:
    """Algorithmic bytes of one fused call (fp16 A and out)."""
    G = K // group
    per_weight = K * N // 2 + N * G * scale_bytes + (N * G // 2 if has_zp else 0)
    return (n_weights * per_weight + 2 * M * K + 2 * M * N
            + (2 * N if bias else 0) + (2 * K if gamma else 0))


def gemm_flops(M: int, K: int, N: int, n_weights: int = 1) -> int:
    """2*M*N*K per weight matrix (one multiply and one add per term)."""
    return 2 * M * N * K * n_weights
