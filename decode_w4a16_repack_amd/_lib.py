"""ctypes loader for libw4a16.so (the C ABI declared in include/w4a16.h).

Argument marshalling only: no computation happens here.  torch is imported
first so that the library binds to the HIP runtime torch already loaded (one
runtime per process, so torch streams are valid handles for the library).
Loading fails loudly when the shared library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the process's HIP runtime first)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libw4a16.so")

# status codes (w4a16_status)
OK = 0
ERR_NULL = -1
ERR_SHAPE = -2
ERR_GROUP = -3
ERR_DTYPE = -4
ERR_EPILOGUE = -5
ERR_WORKSPACE = -6
ERR_ALIGN = -7
ERR_LAUNCH = -8
ERR_SPLIT = -9
ERR_SCRATCH = -10

# bytes of split-K arrival counters at the start of every workspace
# (W4A16_COUNTER_BYTES)
COUNTER_BYTES = 16384
# the static scratch of w4a16_gemm_noalloc (W4A16_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 8 << 20

KERNEL_STREAM = 1
KERNEL_TILE = 2
KERNEL_PANEL = 3

SCALE_F16 = 0
SCALE_F32 = 1
EPI = {"none": 0, "bias": 1, "bias_relu": 2}

EXPORTS = [
    "w4a16_packed_bytes", "w4a16_repack", "w4a16_workspace_bytes", "w4a16_gemm",
    "w4a16_gemm_gate_up", "w4a16_status_string", "w4a16_layout_version",
    "w4a16_add_bias", "w4a16_relu", "w4a16_rmsnorm", "w4a16_probe_read",
    "w4a16_probe_copy", "w4a16_probe_lds_read", "w4a16_probe_lds_copy", "w4a16_probe_read_tiles",
    "w4a16_probe_mfma_valu",
    "w4a16_plan", "w4a16_gemm_split", "w4a16_gemm_gate_up_split",
    "w4a16_gemm_skip_rmsnorm", "w4a16_gemm_gate_up_skip_rmsnorm",
    "w4a16_mlp_workspace_bytes", "w4a16_mlp", "w4a16_gemm_noalloc",
]


class PlanInfo(ctypes.Structure):
    """w4a16_plan_info."""
    _fields_ = [("kernel", ctypes.c_int), ("split", ctypes.c_int),
                ("k_tiles_per_split", ctypes.c_int), ("grid", ctypes.c_int * 3),
                ("block", ctypes.c_int), ("lds_bytes", ctypes.c_int),
                ("workspace_bytes", ctypes.c_size_t), ("col_tiles", ctypes.c_int),
                ("k_tiles_per_wave", ctypes.c_int)]


class W4A16Error(RuntimeError):
    def __init__(self, status: int, what: str, text: str):
        super().__init__(f"{what} failed with status {status}: {text}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with decode_w4a16_repack_amd.build.build() "
            "(there is no fallback path)")
    L = ctypes.CDLL(LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    sig = {
        "w4a16_packed_bytes": (Z, [I, I, I, I, I]),
        "w4a16_repack": (I, [P, P, P, I, I, I, I, P, P]),
        "w4a16_workspace_bytes": (Z, [I, I, I, I, I]),
        "w4a16_gemm": (I, [P, I, I, I, I, I, I, P, I, P, P, F, P, P, Z, P]),
        "w4a16_gemm_gate_up": (I, [P, I, I, I, I, I, I, P, P, P, F, P, P, Z, P]),
        "w4a16_status_string": (ctypes.c_char_p, [I]),
        "w4a16_layout_version": (I, []),
        "w4a16_add_bias": (I, [P, P, I, I, P, P]),
        "w4a16_relu": (I, [P, I, I, P, P]),
        "w4a16_rmsnorm": (I, [P, P, F, I, I, P, P]),
        "w4a16_probe_read": (I, [P, Z, P, P]),
        "w4a16_probe_copy": (I, [P, P, Z, P]),
        "w4a16_probe_lds_read": (I, [I, I, P, P]),
        "w4a16_probe_lds_copy": (I, [P, Z, I, I, P, P]),
        "w4a16_probe_read_tiles": (I, [P, I, I, I, I, P, Z, P]),
        "w4a16_probe_mfma_valu": (I, [I, I, I, I, P, Z, P]),
        "w4a16_plan": (I, [I, I, I, I, I, I, I, ctypes.POINTER(PlanInfo)]),
        "w4a16_gemm_split": (I, [P, I, I, I, I, I, I, P, I, P, P, F, P, P, Z, I, P]),
        "w4a16_gemm_gate_up_split": (I, [P, I, I, I, I, I, I, P, P, P, F, P, P, Z, I, P]),
        "w4a16_gemm_skip_rmsnorm": (I, [P, P, P, I, I, I, I, I, I, P, I, P, P, F, P, P, Z, P]),
        "w4a16_gemm_gate_up_skip_rmsnorm": (I, [P, P, P, I, I, I, I, I, I, P, P, P, F, P, P, Z, P]),
        "w4a16_mlp_workspace_bytes": (Z, [I, I, I, I]),
        "w4a16_mlp": (I, [P, P, P, I, I, I, I, I, I, P, P, P, P, F, P, P, P, Z, P]),
        "w4a16_gemm_noalloc": (I, [P, I, I, I, I, I, I, P, I, P, P, F, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def check(status: int, what: str) -> None:
    if status != OK:
        text = lib().w4a16_status_string(status).decode()
        raise W4A16Error(status, what, text)
