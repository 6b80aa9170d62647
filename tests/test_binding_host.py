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
