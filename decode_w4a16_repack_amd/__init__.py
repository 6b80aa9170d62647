"""MI355X-native W4A16 group-quantized GEMM/GEMV.

Thin torch binding over the C ABI of ``libw4a16.so`` (include/w4a16.h):
argument marshalling only; every step runs in the library's HIP kernels on
the caller's current torch stream.  There is no CPU fallback: calling an op
without the built library or without a GPU raises.

    pw = repack(qweight, scales, zeros, K, N, group)   # one time, on the GPU
    y = gemm(A, pw)                                     # fp16 [M][N]
    y = gemm(A, pw, epilogue="bias_relu", bias=b)
    y = gemm(A, pw, gamma=g, eps=1e-6)                  # RMSNorm prologue
    y = gemm_gate_up(A, pw_gate, pw_up)                 # silu(A.Wg) * (A.Wu)
    y = mlp(A, pw_gate, pw_up, pw_down)                 # (silu(A.Wg) * (A.Wu)) . Wd
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import W4A16Error

__all__ = [
    "PackedWeight", "repack", "gemm", "gemm_gate_up", "packed_bytes",
    "workspace_bytes", "layout_version", "add_bias", "relu", "rmsnorm",
    "probe_read", "probe_copy", "probe_lds_read", "probe_lds_copy", "probe_read_tiles",
    "probe_mfma_valu", "Workspace", "plan", "Plan", "W4A16Error",
    "mlp", "mlp_workspace_bytes", "gemm_noalloc",
]


def _stream():
    return ctypes_stream(torch.cuda.current_stream())


def ctypes_stream(s: torch.cuda.Stream):
    return s.cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need_gpu(t: torch.Tensor, name: str, dtype=None, device=None, shape=None):
    _need_form(t, name, dtype, shape)
    _need_device(t, name, device)


def _need_form(t: torch.Tensor, name: str, dtype=None, shape=None):
    """dtype, shape and contiguity (checked before the device, so a wrong
    shape is reported as such on any host)."""
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_device(t: torch.Tensor, name: str, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the activations on {device}")


def _check_operands(A: torch.Tensor, weights, *, out=None, bias=None, gamma=None,
                    residual=None, residual_out=None):
    """Everything the library reads or writes besides the workspace, checked
    before the call: the library trusts its pointers, so a short ``out`` or
    ``bias`` would be overrun on the device.  Shapes first, then devices."""
    _need_form(A, "A", torch.float16)
    if A.dim() != 2:
        raise ValueError(f"A must be 2-D [M][K], got shape {tuple(A.shape)}")
    M, K = A.shape
    N = weights[0].N
    for i, w in enumerate(weights):
        _need_form(w.data, f"packed weight {i}", torch.uint8)
        if w.data.numel() < packed_bytes(w.K, w.N, w.group, w.scale_dtype, w.has_zp):
            raise ValueError(f"packed weight {i} is shorter than its layout")
    if out is not None:
        _need_form(out, "out", torch.float16, shape=(M, N))
    if bias is not None:
        _need_form(bias, "bias", torch.float16)
        if bias.numel() != N:
            raise ValueError(f"bias must have N={N} elements, got {bias.numel()}")
    if gamma is not None:
        _need_form(gamma, "gamma", torch.float16)
        if gamma.numel() != K:
            raise ValueError(f"gamma must have K={K} elements, got {gamma.numel()}")
    for t, n in ((residual, "residual"), (residual_out, "residual_out")):
        if t is not None:
            _need_form(t, n, torch.float16, shape=(M, K))
    _need_device(A, "A")
    dev = A.device
    for i, w in enumerate(weights):
        _need_device(w.data, f"packed weight {i}", dev)
    for t, n in ((out, "out"), (bias, "bias"), (gamma, "gamma"), (residual, "residual"),
                 (residual_out, "residual_out")):
        if t is not None:
            _need_device(t, n, dev)


@dataclass
class PackedWeight:
    """A repacked int4 weight (layout version 1) and its shape."""
    data: torch.Tensor  # uint8, w4a16_packed_bytes long
    K: int
    N: int
    group: int
    scale_dtype: int    # _lib.SCALE_F16 / SCALE_F32
    has_zp: bool


def layout_version() -> int:
    return _lib.lib().w4a16_layout_version()


def packed_bytes(K: int, N: int, group: int, scale_dtype: int, has_zp: bool) -> int:
    return _lib.lib().w4a16_packed_bytes(K, N, group, scale_dtype, int(has_zp))


def workspace_bytes(M: int, K: int, N: int, group: int, gate_up: bool = False) -> int:
    return _lib.lib().w4a16_workspace_bytes(M, K, N, group, int(gate_up))


@dataclass
class Plan:
    """The launch a call of one shape makes (w4a16_plan_info)."""
    kernel: str          # "stream" (M <= 16), "panel" (M <= 32) or "tile"
    split: int           # workgroups along K per output tile
    k_tiles_per_split: int
    grid: tuple
    block: int
    lds_bytes: int
    workspace_bytes: int
    col_tiles: int          # 16-column weight tiles per workgroup
    k_tiles_per_wave: int   # 128-wide k tiles per wavefront and column tile


def plan(M: int, K: int, N: int, group: int, scale_dtype: int = _lib.SCALE_F16,
         gate_up: bool = False, split: int = 0) -> Plan:
    """Host-only query of the plan; split > 0 forces that split-K factor."""
    info = _lib.PlanInfo()
    st = _lib.lib().w4a16_plan(M, K, N, group, scale_dtype, int(gate_up), split, info)
    _lib.check(st, "w4a16_plan")
    kind = {_lib.KERNEL_STREAM: "stream", _lib.KERNEL_PANEL: "panel"}.get(info.kernel, "tile")
    return Plan(kind, info.split,
                info.k_tiles_per_split, tuple(info.grid), info.block, info.lds_bytes,
                info.workspace_bytes, info.col_tiles, info.k_tiles_per_wave)


class Workspace:
    """Zero-filled device workspace reused across calls on one device.

    The library leaves its arrival counters at zero after every call, so the
    buffer is zero-filled only when it is (re)allocated.  Calls that share a
    workspace must be ordered on one stream.
    """

    def __init__(self):
        self._buf = {}

    def get(self, nbytes: int, device) -> Optional[torch.Tensor]:
        if nbytes == 0:
            return None
        key = torch.device(device)
        buf = self._buf.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=key)
            self._buf[key] = buf
        return buf


_default_ws = Workspace()


def repack(qweight: torch.Tensor, scales: torch.Tensor, zeros: Optional[torch.Tensor],
           K: int, N: int, group: int) -> PackedWeight:
    """Repack canonical weights (u8 [N][K/2], fp16/fp32 scales [N][G],
    u8 zeros [N][ceil(G/2)] or None) into the packed layout, on the GPU."""
    if scales.dtype == torch.float16:
        sdt = _lib.SCALE_F16
    elif scales.dtype == torch.float32:
        sdt = _lib.SCALE_F32
    else:
        raise ValueError("scales must be float16 or float32")
    if K % 2 or group <= 0 or K % group:
        _lib.check(_lib.ERR_SHAPE, "w4a16_repack")
    G = K // group
    _need_form(qweight, "qweight", torch.uint8, shape=(N, K // 2))
    _need_form(scales, "scales", shape=(N, G))
    if zeros is not None:
        _need_form(zeros, "zeros", torch.uint8, shape=(N, (G + 1) // 2))
    _need_device(qweight, "qweight")
    _need_device(scales, "scales", qweight.device)
    if zeros is not None:
        _need_device(zeros, "zeros", qweight.device)
    nbytes = packed_bytes(K, N, group, sdt, zeros is not None)
    if nbytes == 0:
        _lib.check(_lib.ERR_SHAPE, "w4a16_packed_bytes")
    out = torch.empty(nbytes, dtype=torch.uint8, device=qweight.device)
    st = _lib.lib().w4a16_repack(_ptr(qweight), _ptr(scales), _ptr(zeros), K, N, group,
                                 sdt, _ptr(out), _stream())
    _lib.check(st, "w4a16_repack")
    return PackedWeight(out, K, N, group, sdt, zeros is not None)


def gemm(A: torch.Tensor, w: PackedWeight, *, epilogue: str = "none",
         bias: Optional[torch.Tensor] = None, gamma: Optional[torch.Tensor] = None,
         eps: float = 1e-6, out: Optional[torch.Tensor] = None,
         workspace: Optional[Workspace] = None, split: int = 0,
         residual: Optional[torch.Tensor] = None,
         residual_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp16 [M][N] = epilogue(X . dequant(W)), X = A or RMSNorm(A; gamma, eps),
    or with ``residual`` X = RMSNorm(A + residual) (w4a16_gemm_skip_rmsnorm;
    the sum is written to ``residual_out`` when given).  split > 0 forces
    that split-K factor (w4a16_gemm_split)."""
    _check_operands(A, [w], out=out, bias=bias, gamma=gamma, residual=residual,
                    residual_out=residual_out)
    M, K = A.shape
    if K != w.K:
        raise ValueError(f"A has K={K}, weight has K={w.K}")
    if epilogue not in _lib.EPI:
        raise ValueError(f"unknown epilogue {epilogue!r}")
    _check_residual(A, gamma, residual, residual_out, split)
    if out is None:
        out = torch.empty((M, w.N), dtype=torch.float16, device=A.device)
    if split:
        ws_n = plan(M, K, w.N, w.group, w.scale_dtype, False, split).workspace_bytes
    else:
        ws_n = workspace_bytes(M, K, w.N, w.group, False)
    ws = (workspace or _default_ws).get(ws_n, A.device)
    args = (_ptr(A), M, K, w.N, w.group, w.scale_dtype, int(w.has_zp), _ptr(w.data),
            _lib.EPI[epilogue], _ptr(bias), _ptr(gamma), float(eps), _ptr(out), _ptr(ws), ws_n)
    if residual is not None:
        st = _lib.lib().w4a16_gemm_skip_rmsnorm(_ptr(A), _ptr(residual), _ptr(residual_out),
                                                *args[1:], _stream())
    elif split:
        st = _lib.lib().w4a16_gemm_split(*args, split, _stream())
    else:
        st = _lib.lib().w4a16_gemm(*args, _stream())
    _lib.check(st, "w4a16_gemm")
    return out


def gemm_noalloc(A: torch.Tensor, w: PackedWeight, *, epilogue: str = "none",
                 bias: Optional[torch.Tensor] = None, gamma: Optional[torch.Tensor] = None,
                 eps: float = 1e-6, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """gemm() through w4a16_gemm_noalloc: no workspace argument; the library's
    static per-device scratch holds what the workspace would (calls that
    overlap on one GPU race).  Raises W4A16Error (W4A16_ERR_SCRATCH) for a
    shape that needs more than that scratch."""
    _check_operands(A, [w], out=out, bias=bias, gamma=gamma)
    M, K = A.shape
    if K != w.K:
        raise ValueError(f"A has K={K}, weight has K={w.K}")
    if epilogue not in _lib.EPI:
        raise ValueError(f"unknown epilogue {epilogue!r}")
    if out is None:
        out = torch.empty((M, w.N), dtype=torch.float16, device=A.device)
    st = _lib.lib().w4a16_gemm_noalloc(_ptr(A), M, K, w.N, w.group, w.scale_dtype,
                                       int(w.has_zp), _ptr(w.data), _lib.EPI[epilogue],
                                       _ptr(bias), _ptr(gamma), float(eps), _ptr(out), _stream())
    _lib.check(st, "w4a16_gemm_noalloc")
    return out


def _check_residual(A, gamma, residual, residual_out, split):
    if residual is None:
        if residual_out is not None:
            raise ValueError("residual_out needs residual")
        return
    if gamma is None:
        raise ValueError("the residual (skip) prologue needs gamma")
    if split:
        raise ValueError("split is not available with the residual prologue")
    if residual.shape != A.shape or (residual_out is not None and residual_out.shape != A.shape):
        raise ValueError("residual and residual_out must have A's shape")


def gemm_gate_up(A: torch.Tensor, w_gate: PackedWeight, w_up: PackedWeight, *,
                 gamma: Optional[torch.Tensor] = None, eps: float = 1e-6,
                 out: Optional[torch.Tensor] = None,
                 workspace: Optional[Workspace] = None, split: int = 0,
                 residual: Optional[torch.Tensor] = None,
                 residual_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp16 [M][N] = silu(X . Wg) * (X . Wu); split, residual and
    residual_out as in gemm()."""
    for w in (w_gate, w_up):
        if (w.K, w.N, w.group, w.scale_dtype, w.has_zp) != (
                w_gate.K, w_gate.N, w_gate.group, w_gate.scale_dtype, w_gate.has_zp):
            raise ValueError("gate and up weights must share K, N, group, scale dtype, zp")
    _check_operands(A, [w_gate, w_up], out=out, gamma=gamma, residual=residual,
                    residual_out=residual_out)
    M, K = A.shape
    _check_residual(A, gamma, residual, residual_out, split)
    if K != w_gate.K:
        raise ValueError(f"A has K={K}, weights have K={w_gate.K}")
    if out is None:
        out = torch.empty((M, w_gate.N), dtype=torch.float16, device=A.device)
    if split:
        ws_n = plan(M, K, w_gate.N, w_gate.group, w_gate.scale_dtype, True, split).workspace_bytes
    else:
        ws_n = workspace_bytes(M, K, w_gate.N, w_gate.group, True)
    ws = (workspace or _default_ws).get(ws_n, A.device)
    args = (_ptr(A), M, K, w_gate.N, w_gate.group, w_gate.scale_dtype, int(w_gate.has_zp),
            _ptr(w_gate.data), _ptr(w_up.data), _ptr(gamma), float(eps), _ptr(out),
            _ptr(ws), ws_n)
    if residual is not None:
        st = _lib.lib().w4a16_gemm_gate_up_skip_rmsnorm(_ptr(A), _ptr(residual),
                                                        _ptr(residual_out), *args[1:], _stream())
    elif split:
        st = _lib.lib().w4a16_gemm_gate_up_split(*args, split, _stream())
    else:
        st = _lib.lib().w4a16_gemm_gate_up(*args, _stream())
    _lib.check(st, "w4a16_gemm_gate_up")
    return out


def mlp_workspace_bytes(M: int, H: int, I: int, group: int) -> int:
    return _lib.lib().w4a16_mlp_workspace_bytes(M, H, I, group)


def mlp(A: torch.Tensor, w_gate: PackedWeight, w_up: PackedWeight, w_down: PackedWeight, *,
        gamma: Optional[torch.Tensor] = None, eps: float = 1e-6,
        inter: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
        workspace: Optional[Workspace] = None,
        residual: Optional[torch.Tensor] = None,
        residual_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """MLP block (w4a16_mlp): inter = fp16 silu(X . Wg) * (X . Wu) [M][I],
    then fp16 [M][H] = inter . Wd.  A is [M][H]; w_gate and w_up have K = H,
    N = I; w_down has K = I, N = H.  X, gamma, residual and residual_out as
    in gemm_gate_up().  ``inter`` receives the intermediate when given."""
    _need_form(A, "A", torch.float16)
    if A.dim() != 2:
        raise ValueError(f"A must be 2-D [M][H], got shape {tuple(A.shape)}")
    M, H = A.shape
    key = (w_gate.group, w_gate.scale_dtype, w_gate.has_zp)
    for w in (w_up, w_down):
        if (w.group, w.scale_dtype, w.has_zp) != key:
            raise ValueError("gate, up and down weights must share group, scale dtype, zp")
    I = w_gate.N
    if (w_gate.K, w_up.K, w_up.N, w_down.K, w_down.N) != (H, H, I, I, H):
        raise ValueError(f"weights do not chain: A has H={H}; gate {w_gate.K}x{w_gate.N}, "
                         f"up {w_up.K}x{w_up.N}, down {w_down.K}x{w_down.N}")
    _need_form(w_down.data, "packed down weight", torch.uint8)
    if w_down.data.numel() < packed_bytes(w_down.K, w_down.N, w_down.group,
                                          w_down.scale_dtype, w_down.has_zp):
        raise ValueError("packed down weight is shorter than its layout")
    for t, n, shp in ((inter, "inter", (M, I)), (out, "out", (M, H))):
        if t is not None:
            _need_form(t, n, torch.float16, shape=shp)
    _check_operands(A, [w_gate, w_up], gamma=gamma, residual=residual,
                    residual_out=residual_out)
    _need_device(w_down.data, "packed down weight", A.device)
    _check_residual(A, gamma, residual, residual_out, 0)
    if inter is None:
        inter = torch.empty((M, I), dtype=torch.float16, device=A.device)
    if out is None:
        out = torch.empty((M, H), dtype=torch.float16, device=A.device)
    _need_device(inter, "inter", A.device)
    _need_device(out, "out", A.device)
    ws_n = mlp_workspace_bytes(M, H, I, w_gate.group)
    ws = (workspace or _default_ws).get(ws_n, A.device)
    st = _lib.lib().w4a16_mlp(_ptr(A), _ptr(residual), _ptr(residual_out), M, H, I,
                              w_gate.group, w_gate.scale_dtype, int(w_gate.has_zp),
                              _ptr(w_gate.data), _ptr(w_up.data), _ptr(w_down.data),
                              _ptr(gamma), float(eps), _ptr(inter), _ptr(out), _ptr(ws), ws_n,
                              _stream())
    _lib.check(st, "w4a16_mlp")
    return out


def add_bias(x: torch.Tensor, bias: torch.Tensor, out: Optional[torch.Tensor] = None):
    """Unfused-chain pass: fp16(x + bias)."""
    _need_form(x, "x", torch.float16)
    M, N = x.shape
    _need_form(bias, "bias", torch.float16)
    if bias.numel() != N:
        raise ValueError(f"bias must have N={N} elements, got {bias.numel()}")
    if out is not None:
        _need_form(out, "out", torch.float16, shape=(M, N))
    for t, n in ((x, "x"), (bias, "bias"), (out, "out")):
        if t is not None:
            _need_device(t, n, x.device)
    out = torch.empty_like(x) if out is None else out
    _lib.check(_lib.lib().w4a16_add_bias(_ptr(x), _ptr(bias), M, N, _ptr(out), _stream()),
               "w4a16_add_bias")
    return out


def relu(x: torch.Tensor, out: Optional[torch.Tensor] = None):
    """Unfused-chain pass: max(x, 0)."""
    _need_form(x, "x", torch.float16)
    M, N = x.shape
    if out is not None:
        _need_form(out, "out", torch.float16, shape=(M, N))
        _need_device(out, "out", x.device)
    _need_device(x, "x", x.device)
    out = torch.empty_like(x) if out is None else out
    _lib.check(_lib.lib().w4a16_relu(_ptr(x), M, N, _ptr(out), _stream()), "w4a16_relu")
    return out


def rmsnorm(A: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6,
            out: Optional[torch.Tensor] = None):
    """Unfused-chain pass: fp16(A * gamma / sqrt(mean(A^2) + eps))."""
    _need_form(A, "A", torch.float16)
    M, K = A.shape
    _need_form(gamma, "gamma", torch.float16)
    if gamma.numel() != K:
        raise ValueError(f"gamma must have K={K} elements, got {gamma.numel()}")
    if out is not None:
        _need_form(out, "out", torch.float16, shape=(M, K))
    for t, n in ((A, "A"), (gamma, "gamma"), (out, "out")):
        if t is not None:
            _need_device(t, n, A.device)
    out = torch.empty_like(A) if out is None else out
    _lib.check(_lib.lib().w4a16_rmsnorm(_ptr(A), _ptr(gamma), float(eps), M, K, _ptr(out),
                                        _stream()), "w4a16_rmsnorm")
    return out


def probe_read(buf: torch.Tensor, sink: torch.Tensor) -> None:
    _need_gpu(buf, "buf")
    _need_gpu(sink, "sink", device=buf.device)
    if sink.numel() * sink.element_size() < 4096 * 4:
        raise ValueError("sink must hold at least 4096 32-bit values")
    _lib.check(_lib.lib().w4a16_probe_read(_ptr(buf), buf.numel() * buf.element_size(),
                                           _ptr(sink), _stream()), "w4a16_probe_read")


def probe_copy(src: torch.Tensor, dst: torch.Tensor) -> None:
    _need_gpu(src, "src")
    _need_gpu(dst, "dst", device=src.device)
    if dst.numel() * dst.element_size() < src.numel() * src.element_size():
        raise ValueError("dst is smaller than src")
    _lib.check(_lib.lib().w4a16_probe_copy(_ptr(src), _ptr(dst),
                                           src.numel() * src.element_size(), _stream()),
               "w4a16_probe_copy")


def probe_lds_read(workgroups: int, iters: int, sink: torch.Tensor) -> None:
    """w4a16_probe_lds_read: workgroups x 512 threads read iters x 16 KiB of
    LDS per wavefront; sink (device, >= workgroups * 512 int32) gets one word
    per thread."""
    _need_gpu(sink, "sink")
    if sink.numel() * sink.element_size() < workgroups * 512 * 4:
        raise ValueError("sink needs workgroups * 512 * 4 bytes")
    _lib.check(_lib.lib().w4a16_probe_lds_read(int(workgroups), int(iters), _ptr(sink), _stream()),
               "w4a16_probe_lds_read")


def probe_lds_copy(buf: torch.Tensor, workgroups: int, steps: int, sink: torch.Tensor) -> None:
    """w4a16_probe_lds_copy: copies of the 64-row fp16 matrix in buf
    (device, a multiple of 16 KiB) into LDS, 32 KiB per workgroup and step."""
    _need_gpu(buf, "buf")
    _need_gpu(sink, "sink", device=buf.device)
    if sink.numel() * sink.element_size() < workgroups * 512 * 4:
        raise ValueError("sink needs workgroups * 512 * 4 bytes")
    _lib.check(_lib.lib().w4a16_probe_lds_copy(_ptr(buf), buf.numel() * buf.element_size(),
                                               int(workgroups), int(steps), _ptr(sink), _stream()),
               "w4a16_probe_lds_copy")


def probe_mfma_valu(valu_per_8_mfma: int, waves_per_simd: int, workgroups: int, iters: int,
                    sink: torch.Tensor) -> None:
    """w4a16_probe_mfma_valu: every wavefront runs iters rounds of 8 MFMAs and
    valu_per_8_mfma independent fp32 FMAs; workgroups of 256 * waves_per_simd
    threads; sink (device, >= workgroups * threads fp32) gets one value per
    thread."""
    _need_gpu(sink, "sink")
    if sink.numel() * sink.element_size() < workgroups * 256 * waves_per_simd * 4:
        raise ValueError("sink needs workgroups * 256 * waves_per_simd * 4 bytes")
    _lib.check(_lib.lib().w4a16_probe_mfma_valu(int(valu_per_8_mfma), int(waves_per_simd),
                                                int(workgroups), int(iters), _ptr(sink),
                                                sink.numel() * sink.element_size(), _stream()),
               "w4a16_probe_mfma_valu")


def probe_read_tiles(w: PackedWeight, mode: int, workgroups: int, sink: torch.Tensor) -> None:
    """w4a16_probe_read_tiles: plain reads of w's packed weight tiles, in the
    streaming kernel's decomposition (mode 0) or split evenly over
    `workgroups` workgroups (mode 1); sink gets one word per thread."""
    _need_form(w.data, "w.data", torch.uint8)
    if w.data.numel() < w.K * w.N // 2:
        raise ValueError("w.data is shorter than the weight tiles of a K x N matrix")
    _need_form(sink, "sink")
    grid = (w.N // 16 + 3) // 4 if mode == 0 else int(workgroups)
    if sink.numel() * sink.element_size() < grid * 512 * 4:
        raise ValueError(f"sink needs {grid * 512 * 4} bytes")
    _need_device(w.data, "w.data")
    _need_device(sink, "sink", device=w.data.device)
    _lib.check(_lib.lib().w4a16_probe_read_tiles(_ptr(w.data), int(w.K), int(w.N), int(mode),
                                                 int(workgroups), _ptr(sink),
                                                 sink.numel() * sink.element_size(), _stream()),
               "w4a16_probe_read_tiles")
