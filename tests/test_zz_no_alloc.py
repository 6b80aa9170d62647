"""w4a16_gemm_noalloc, the entry point for callers that cannot allocate: the
same result as w4a16_gemm with a caller workspace, through the C ABI.

Its workspace (split-K partial sums and arrival counters, RMSNorm staging
rows) is the library's static per-device scratch, which keeps the last
call's contents: so each case makes two calls in a row, the second on a
smaller input, and both must equal w4a16_gemm bit for bit and meet the
oracle.  A shape that needs more than the scratch is refused on the host.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import decode_w4a16_repack_amd as w4
from decode_w4a16_repack_amd import _lib, synth

from gpu_cases import check_close, nan_out, repack_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)


def _noalloc(A, pw, out, *, epilogue="none", bias=None, gamma=None, eps=1e-6):
    M, K = A.shape
    return _lib.lib().w4a16_gemm_noalloc(
        A.data_ptr(), M, K, pw.N, pw.group, pw.scale_dtype, int(pw.has_zp), pw.data.data_ptr(),
        _lib.EPI[epilogue], None if bias is None else bias.data_ptr(),
        None if gamma is None else gamma.data_ptr(), ctypes.c_float(eps), out.data_ptr(),
        torch.cuda.current_stream().cuda_stream)


def _case(M, K, N, g, seed, epilogue="none", rms=False, sdt=np.float16):
    p = synth.make_problem(M, K, N, g, seed=seed, bias=epilogue != "none", gamma=rms,
                           scale_dtype=sdt)
    return p, repack_dev(p.w), to_dev(p.A), to_dev(p.bias), to_dev(p.gamma)


# (first call, second smaller call): kernel, and what of the scratch it uses
PAIRS = [
    # streaming kernel, narrow N: split-K partials and counters; RMSNorm in registers
    ((16, 5120, 1024, 128, "bias_relu", True), (3, 1024, 256, 32, "none", False)),
    # tile then panel kernel with the staged RMSNorm prologue (staging rows,
    # and split-K partials on the panel call)
    ((72, 2048, 512, 64, "bias", True), (20, 1024, 256, 128, "none", True)),
    # deep k (107 k tiles) split over workgroups, then a plain small call
    ((12, 13696, 4096, 128, "none", False), (1, 5120, 256, 128, "bias", False)),
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_workspace_entry_point(first, second):
    ws = w4.Workspace()
    for i, (M, K, N, g, epi, rms) in enumerate((first, second)):
        p, pw, A, b, gm = _case(M, K, N, g, seed=1000 * i + M + N, epilogue=epi, rms=rms,
                                sdt=np.float32 if i else np.float16)
        plan = w4.plan(M, K, N, g, pw.scale_dtype)
        assert 0 < plan.workspace_bytes <= _lib.NOALLOC_SCRATCH_BYTES, (M, K, N, plan)
        out = nan_out(M, N)
        st = _noalloc(A, pw, out, epilogue=epi, bias=b if epi != "none" else None,
                      gamma=gm if rms else None)
        assert st == _lib.OK, _lib.lib().w4a16_status_string(st)
        want = w4.gemm(A, pw, epilogue=epi, bias=b if epi != "none" else None,
                       gamma=gm if rms else None, workspace=ws, out=nan_out(M, N))
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"call {i}: differs from w4a16_gemm"
        ref = oracle.gemm(p.A, p.w.qweight, p.w.scales, p.w.zeros, g, N,
                          gamma=p.gamma if rms else None, epilogue=epi,
                          bias=p.bias if epi != "none" else None)
        check_close(out.cpu().numpy(), ref, f"noalloc call {i} M={M} K={K} N={N}")


def test_noalloc_repeats_bit_identically_and_without_allocating():
    """Consecutive calls on one stream reuse the scratch (each leaves its
    counters at zero) and take no device memory."""
    p, pw, A, b, gm = _case(8, 5120, 512, 128, seed=7, rms=True)
    outs = [nan_out(8, 512) for _ in range(3)]
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats()["allocation.all.allocated"]
    for o in outs:
        assert _noalloc(A, pw, o, gamma=gm) == _lib.OK
    torch.cuda.synchronize()
    assert torch.cuda.memory_stats()["allocation.all.allocated"] == before
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])
    check_close(outs[0].cpu().numpy(),
                oracle.gemm(p.A, p.w.qweight, p.w.scales, p.w.zeros, 128, 512, gamma=p.gamma),
                "noalloc repeated")


def test_noalloc_refuses_shapes_beyond_the_scratch():
    """A call whose workspace need exceeds the scratch is refused on the host
    (W4A16_ERR_SCRATCH) and writes nothing."""
    M, K, N = 640, 8192, 256   # staged RMSNorm rows alone: 640 * 8192 * 2 = 10 MiB
    assert w4.workspace_bytes(M, K, N, 128) > _lib.NOALLOC_SCRATCH_BYTES
    A = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    gm = torch.ones(K, dtype=torch.float16, device="cuda")
    pw = w4.PackedWeight(torch.zeros(w4.packed_bytes(K, N, 128, 0, True), dtype=torch.uint8,
                                     device="cuda"), K, N, 128, 0, True)
    out = nan_out(M, N)
    assert _noalloc(A, pw, out, gamma=gm) == _lib.ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    # the same shape without the prologue needs no workspace and runs
    assert _noalloc(A, pw, out) == _lib.OK
    torch.cuda.synchronize()
    assert torch.equal(out, torch.zeros_like(out))
