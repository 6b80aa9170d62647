"""The Python binding on a host without a GPU: every op refuses CPU tensors
(there is no CPU path) and a missing shared library fails loudly."""
import pytest
import torch

import decode_w4a16_repack_amd as w4
from decode_w4a16_repack_amd import _lib


def _pw(K=256, N=32, group=128):
    return w4.PackedWeight(torch.zeros(w4.packed_bytes(K, N, group, _lib.SCALE_F16, True),
                                       dtype=torch.uint8),
                           K, N, group, _lib.SCALE_F16, True)


def test_ops_refuse_cpu_tensors():
    A = torch.zeros((2, 256), dtype=torch.float16)
    pw = _pw()
    with pytest.raises(ValueError, match="GPU tensor"):
        w4.gemm(A, pw)
    with pytest.raises(ValueError, match="GPU tensor"):
        w4.gemm_gate_up(A, pw, pw)
    with pytest.raises(ValueError, match="GPU tensor"):
        w4.mlp(A, _pw(256, 128), _pw(256, 128), _pw(128, 256))
    q = torch.zeros((32, 128), dtype=torch.uint8)
    s = torch.zeros((32, 2), dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU tensor"):
        w4.repack(q, s, None, 256, 32, 128)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libw4a16.so"))
    with pytest.raises(ImportError, match="no fallback"):
        _lib.lib()


def test_ops_refuse_wrong_shapes_before_any_call():
    """The library trusts its pointers, so the binding checks every operand's
    shape against the call before it calls: a short ``out``, ``bias`` or
    ``gamma`` would otherwise be overrun on the device.  Shapes are checked
    before devices, so these checks run on any host."""
    A = torch.zeros((2, 256), dtype=torch.float16)
    pw = _pw()
    with pytest.raises(ValueError, match="out must have shape"):
        w4.gemm(A, pw, out=torch.zeros((1, 32), dtype=torch.float16))
    with pytest.raises(ValueError, match="out must have shape"):
        w4.gemm(A, pw, out=torch.zeros((2, 16), dtype=torch.float16))
    with pytest.raises(ValueError, match="bias must have N=32"):
        w4.gemm(A, pw, epilogue="bias", bias=torch.zeros(16, dtype=torch.float16))
    with pytest.raises(ValueError, match="gamma must have K=256"):
        w4.gemm(A, pw, gamma=torch.zeros(128, dtype=torch.float16))
    with pytest.raises(ValueError, match="residual must have shape"):
        w4.gemm(A, pw, gamma=torch.zeros(256, dtype=torch.float16),
                residual=torch.zeros((2, 128), dtype=torch.float16))
    with pytest.raises(ValueError, match="out must have shape"):
        w4.gemm_gate_up(A, pw, pw, out=torch.zeros((2, 16), dtype=torch.float16))
    with pytest.raises(ValueError, match="gamma must have K=256"):
        w4.gemm_gate_up(A, pw, pw, gamma=torch.zeros(255, dtype=torch.float16))
    short = w4.PackedWeight(pw.data[:-256], pw.K, pw.N, pw.group, pw.scale_dtype, pw.has_zp)
    with pytest.raises(ValueError, match="shorter than its layout"):
        w4.gemm(A, short)
    with pytest.raises(ValueError, match="inter must have shape"):
        w4.mlp(A, _pw(256, 128), _pw(256, 128), _pw(128, 256),
               inter=torch.zeros((2, 64), dtype=torch.float16))
    with pytest.raises(ValueError, match="out must have shape"):
        w4.mlp(A, _pw(256, 128), _pw(256, 128), _pw(128, 256),
               out=torch.zeros((2, 128), dtype=torch.float16))
    with pytest.raises(ValueError, match="bias must have N=256"):
        w4.add_bias(A, torch.zeros(128, dtype=torch.float16))
    with pytest.raises(ValueError, match="gamma must have K=256"):
        w4.rmsnorm(A, torch.zeros(128, dtype=torch.float16))
    q = torch.zeros((32, 128), dtype=torch.uint8)
    s = torch.zeros((32, 2), dtype=torch.float16)
    with pytest.raises(ValueError, match="qweight must have shape"):
        w4.repack(q[:16], s, None, 256, 32, 128)
    with pytest.raises(ValueError, match="scales must have shape"):
        w4.repack(q, s[:, :1], None, 256, 32, 128)
    with pytest.raises(ValueError, match="zeros must have shape"):
        w4.repack(q, s, torch.zeros((32, 2), dtype=torch.uint8), 256, 32, 128)
    # the tile-read probe: the weight region and the sink are checked too
    tiny = w4.PackedWeight(torch.zeros(100, dtype=torch.uint8), 256, 32, 128, _lib.SCALE_F16, True)
    with pytest.raises(ValueError, match="shorter than the weight tiles"):
        w4.probe_read_tiles(tiny, 0, 0, torch.zeros(512, dtype=torch.int32))
    with pytest.raises(ValueError, match="sink needs 8192 bytes"):
        w4.probe_read_tiles(pw, 1, 4, torch.zeros(100, dtype=torch.int32))


def test_plan_reports_the_kernel_configuration():
    """w4a16_plan names the configuration a shape runs (column tiles per
    workgroup, k tiles per wavefront), which the GPU tests use to pin each
    case to the configuration it is meant to cover."""
    p = w4.plan(1, 5120, 13824, 128)
    assert (p.kernel, p.col_tiles, p.k_tiles_per_wave, p.grid) == ("stream", 4, 5, (216, 1, 1))
    p = w4.plan(8, 5120, 13824, 128, gate_up=True)
    assert (p.kernel, p.col_tiles, p.k_tiles_per_wave, p.block) == ("stream", 4, 5, 512)
    p = w4.plan(1, 5120, 8192, 128)
    assert (p.kernel, p.col_tiles, p.k_tiles_per_wave, p.grid) == ("stream", 2, 5, (256, 1, 1))
    p = w4.plan(8, 13696, 4096, 128)
    assert (p.kernel, p.col_tiles, p.k_tiles_per_wave, p.grid) == ("stream", 1, 14, (256, 1, 1))
    p = w4.plan(32, 5120, 13824, 128)
    assert (p.kernel, p.col_tiles, p.k_tiles_per_wave) == ("panel", 4, 5)
    p = w4.plan(128, 5120, 13824, 128)
    assert (p.kernel, p.col_tiles, p.k_tiles_per_wave, p.grid) == ("tile", 8, 20, (108, 1, 2))
