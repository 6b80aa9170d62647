"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every input is seeded and synthetic (decode_w4a16_repack_amd.synth); expected
values come only from ``oracle``.  Sizes: small shapes compared element by
element (several 16x128 tiles and ragged M), and the K=5120 N=13824 g=128
decode shape compared on sampled columns in the launch configuration the
benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
import decode_w4a16_repack_amd as w4
from decode_w4a16_repack_amd import synth

from gpu_cases import check_close, nan_out, repack_dev, sample_cols, to_dev

pytestmark = pytest.mark.gpu

F16, F32 = np.float16, np.float32


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import oracle as o
    o.build(force=False)
    torch.manual_seed(0)


def run_gemm(p, **kw):
    w = repack_dev(p.w)
    A = to_dev(p.A)
    out = w4.gemm(A, w, bias=to_dev(p.bias) if kw.get("epilogue", "none") != "none" else None,
                  gamma=to_dev(p.gamma) if kw.get("rms") else None,
                  epilogue=kw.get("epilogue", "none"), eps=kw.get("eps", 1e-6),
                  out=nan_out(p.M, p.N))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def ref_gemm(p, cols=None, **kw):
    return oracle.gemm(p.A, p.w.qweight, p.w.scales, p.w.zeros, p.group, p.N,
                       gamma=p.gamma if kw.get("rms") else None, eps=kw.get("eps", 1e-6),
                       epilogue=kw.get("epilogue", "none"),
                       bias=p.bias if kw.get("epilogue", "none") != "none" else None,
                       cols=cols)


# ------------------------------------------------------------------- repack


@pytest.mark.parametrize("K,N,g,sdt,asym", [
    (512, 512, 32, F16, True), (4096, 4096, 16, F32, False),
    (256, 48, 64, F32, True), (5120, 13824, 128, F16, True), (1024, 4096, 128, F16, False)])
def test_device_repack_is_byte_identical_to_host(K, N, g, sdt, asym):
    p = synth.make_problem(1, K, N, g, seed=0, scale_dtype=sdt, asym=asym)
    host = oracle.repack(p.w.qweight, p.w.scales, p.w.zeros, K, N, g)
    dev = repack_dev(p.w).data.cpu().numpy()
    assert dev.shape == host.shape
    assert np.array_equal(dev, host)


# ------------------------------------------------------------- small shapes


def test_tiny_config_full_output():
    """M=2 K=512 N=512 g=32, asymmetric zp, fp16 scales, seed 0: every output."""
    p = synth.make_problem(2, 512, 512, 32, seed=0)
    check_close(run_gemm(p), ref_gemm(p), "tiny")


# (4 | 5: activation rows through LDS | loaded per k tile; 16 | 17 and 32 | 33:
# the next kernel)
SMALL_M = [1, 2, 3, 4, 5, 7, 8, 12, 16, 17, 24, 32, 33, 64, 65, 128, 130]


@pytest.mark.parametrize("M", SMALL_M)
@pytest.mark.parametrize("g", [16, 32, 64, 128])
def test_small_shapes_all_outputs(M, g):
    i = SMALL_M.index(M) + g
    sdt = F32 if i % 2 else F16
    asym = (i // 2) % 2 == 0
    p = synth.make_problem(M, 1024, 384, g, seed=M * 7 + g, scale_dtype=sdt, asym=asym)
    check_close(run_gemm(p), ref_gemm(p), f"M={M} g={g} {sdt.__name__} asym={asym}")


@pytest.mark.parametrize("M,g,epi", [(65, 32, "none"), (100, 64, "bias"), (128, 128, "bias_relu"),
                                     (129, 128, "none"), (256, 64, "bias_relu"), (300, 32, "bias")])
def test_large_m_all_outputs(M, g, epi):
    """Several 64-row blocks with ragged rows (M % 64) and ragged column
    blocks (N = 400 is 25 column tiles), every output against the oracle,
    and the result repeats bit-identically."""
    sdt = F32 if M % 2 else F16
    p = synth.make_problem(M, 1536, 400, g, seed=M + g, scale_dtype=sdt, asym=M != 129, bias=True)
    got = run_gemm(p, epilogue=epi)
    check_close(got, ref_gemm(p, epilogue=epi), f"M={M} g={g} {epi}")
    assert np.array_equal(got, run_gemm(p, epilogue=epi)), "not repeatable"


@pytest.mark.parametrize("sdt", [F16, F32])
@pytest.mark.parametrize("asym", [True, False])
@pytest.mark.parametrize("M", [1, 16, 29, 40, 90])
def test_scale_dtype_and_zp_variants(sdt, asym, M):
    p = synth.make_problem(M, 2048, 256, 64, seed=3, scale_dtype=sdt, asym=asym)
    check_close(run_gemm(p), ref_gemm(p), f"M={M} {sdt.__name__} asym={asym}")


def test_rows_beyond_m_untouched():
    for M in (7, 33):
        p = synth.make_problem(M, 1024, 256, 32, seed=M)
        w = repack_dev(p.w)
        big = torch.full((M + 3, 256), 1234.0, dtype=torch.float16, device="cuda")
        w4.gemm(to_dev(p.A), w, out=big[:M])
        torch.cuda.synchronize()
        got = big.cpu().numpy()
        assert np.all(got[M:] == np.float16(1234.0))
        check_close(got[:M], ref_gemm(p), f"canary M={M}")


# ----------------------------------------------- decode shape, sampled columns


DECODE_M = [1, 2, 4, 7, 8, 16, 32, 33, 64, 128]


@pytest.mark.parametrize("M", DECODE_M)
def test_decode_shape_sampled(M):
    K, N, g = 5120, 13824, 128
    p = synth.make_problem(M, K, N, g, seed=0)
    got = run_gemm(p)
    cols = sample_cols(N, 160 if M <= 32 else 64, seed=M)
    err, tol = check_close(got[:, cols], ref_gemm(p, cols=cols), f"decode M={M}")
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("sdt,asym", [(F16, False), (F32, True), (F32, False)])
def test_decode_shape_variants_sampled(sdt, asym):
    K, N, g, M = 5120, 13824, 128, 16
    p = synth.make_problem(M, K, N, g, seed=1, scale_dtype=sdt, asym=asym)
    got = run_gemm(p)
    cols = sample_cols(N, 96, seed=2)
    check_close(got[:, cols], ref_gemm(p, cols=cols), f"decode {sdt.__name__} asym={asym}")


# ------------------------------------------------------- exactness properties


@pytest.mark.parametrize("M", [1, 16, 64])
def test_run_to_run_bit_identical(M):
    p = synth.make_problem(M, 5120, 13824, 128, seed=4)
    w = repack_dev(p.w)
    A = to_dev(p.A)
    y1 = w4.gemm(A, w, out=nan_out(M, p.N))
    y2 = w4.gemm(A, w, out=nan_out(M, p.N))
    assert not torch.isnan(y1).any()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_explicit_zp8_bit_identical_to_symmetric():
    p = synth.make_problem(16, 1024, 512, 32, seed=6, asym=False)
    G = p.K // p.group
    z8 = synth.pack_nibbles_rows(np.full((p.N, G), 8, np.uint8))
    A = to_dev(p.A)
    w_sym = w4.repack(to_dev(p.w.qweight), to_dev(p.w.scales), None, p.K, p.N, p.group)
    w_z8 = w4.repack(to_dev(p.w.qweight), to_dev(p.w.scales), to_dev(z8), p.K, p.N, p.group)
    assert torch.equal(w4.gemm(A, w_sym), w4.gemm(A, w_z8))


def test_unit_scale_integer_case_exact():
    """s = 1, zp = 0, small integer A: the fp32 sums are exact integers, so the
    GPU result equals the int64 product rounded once to fp16."""
    rng = np.random.default_rng(8)
    K, N, M, g = 1024, 256, 5, 128
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    w = synth.weight_from_codes(codes, np.ones((N, K // g), F16), np.zeros((N, K // g), np.uint8), g)
    A = rng.integers(-2, 3, size=(M, K)).astype(F16)
    dev = w4.gemm(to_dev(A), repack_dev(w))
    ref = (A.astype(np.int64) @ codes.astype(np.int64)).astype(np.float64).astype(F16)
    assert np.array_equal(dev.cpu().numpy(), ref)


def test_workspace_reuse_across_shapes():
    """Split-K counters must be left at zero: alternate shapes on one workspace."""
    ws = w4.Workspace()
    cases = [synth.make_problem(M, K, N, 128, seed=M)
             for M, K, N in ((1, 5120, 4096), (4, 5120, 4096), (2, 1024, 512),
                             (1, 5120, 4096), (8, 5120, 4096), (1, 1024, 512))]
    for p in cases:
        w = repack_dev(p.w)
        got = w4.gemm(to_dev(p.A), w, workspace=ws, out=nan_out(p.M, p.N)).cpu().numpy()
        cols = sample_cols(p.N, 64, seed=p.M)
        check_close(got[:, cols], ref_gemm(p, cols=cols), f"reuse M={p.M}")


# ------------------------------------------------------------------ epilogues


@pytest.mark.parametrize("g", [16, 32, 64, 128])
@pytest.mark.parametrize("epi", ["bias", "bias_relu"])
def test_bias_epilogues_group_sweep(g, epi):
    p = synth.make_problem(16, 4096, 4096, g, seed=g, bias=True)
    got = run_gemm(p, epilogue=epi)
    cols = sample_cols(p.N, 512, seed=g)
    check_close(got[:, cols], ref_gemm(p, cols=cols, epilogue=epi), f"{epi} g={g}")
    if epi == "bias_relu":
        assert (got >= 0).all()


@pytest.mark.parametrize("g", [16, 32, 64, 128])
def test_rmsnorm_prologue_group_sweep(g):
    p = synth.make_problem(16, 4096, 4096, g, seed=100 + g, gamma=True)
    got = run_gemm(p, rms=True)
    cols = sample_cols(p.N, 512, seed=g)
    check_close(got[:, cols], ref_gemm(p, cols=cols, rms=True), f"rmsnorm g={g}")


@pytest.mark.parametrize("M", [1, 5, 40])
def test_rmsnorm_prologue_small(M):
    p = synth.make_problem(M, 1024, 256, 32, seed=M, gamma=True)
    check_close(run_gemm(p, rms=True), ref_gemm(p, rms=True), f"rmsnorm M={M}")


@pytest.mark.parametrize("M,g,gu", [(5, 64, False), (20, 64, False), (70, 128, False),
                                    (130, 32, False), (40, 16, True), (9, 128, True)])
def test_rmsnorm_odd_k_tile_count(M, g, gu):
    """K = 1152 is 9 k tiles: the two k slices of a workgroup get 5 and 4, so
    one slice runs a step past K.  That step must add nothing, neither to
    the product nor to the sums of squares of the RMSNorm prologue."""
    p = synth.make_problem(M, 1152, 256, g, seed=M + g, gamma=True, gate_up=gu)
    if gu:
        check_close(run_gate_up(p, rms=True), ref_gate_up(p, rms=True), f"odd-k gate_up M={M}")
    else:
        check_close(run_gemm(p, rms=True), ref_gemm(p, rms=True), f"odd-k rmsnorm M={M} g={g}")
        check_close(run_gemm(p), ref_gemm(p), f"odd-k M={M} g={g}")


def test_staging_and_split_calls_share_one_workspace():
    """Calls with the RMSNorm prologue above M = 16 stage their rows in the
    workspace; split-K calls count arrivals at its start.  Alternating them on
    one workspace must leave every result right (the staging never overlaps
    the counters, which every call leaves at zero)."""
    ws = w4.Workspace()
    cases = [synth.make_problem(70, 1152, 256, 128, seed=1, gamma=True),   # tile, staged
             synth.make_problem(5, 1152, 256, 64, seed=2, gamma=True),     # stream, split-K
             synth.make_problem(20, 1152, 256, 64, seed=3, gamma=True),    # panel, split-K + staged
             synth.make_problem(9, 1152, 256, 128, seed=4)]                # stream, split-K
    dev = [(to_dev(p.A), repack_dev(p.w), to_dev(p.gamma)) for p in cases]
    for rep in range(2):
        for p, (A, w, gm) in zip(cases, dev):
            y = w4.gemm(A, w, gamma=gm, out=nan_out(p.M, p.N), workspace=ws)
            torch.cuda.synchronize()
            check_close(y.cpu().numpy(), ref_gemm(p, rms=p.gamma is not None),
                        f"shared workspace M={p.M} pass {rep}")


def test_unfused_chain_matches_fused():
    """FUSED=0 chain (GEMM -> bias pass -> ReLU pass; RMSNorm pass -> GEMM)
    computes the same as the fused kernels, within the tolerance."""
    p = synth.make_problem(16, 4096, 4096, 64, seed=7, bias=True, gamma=True)
    w = repack_dev(p.w)
    A, b, gm = to_dev(p.A), to_dev(p.bias), to_dev(p.gamma)
    y = w4.relu(w4.add_bias(w4.gemm(A, w), b))
    fused = w4.gemm(A, w, epilogue="bias_relu", bias=b)
    cols = sample_cols(p.N, 256)
    ref = ref_gemm(p, cols=cols, epilogue="bias_relu")
    check_close(y.cpu().numpy()[:, cols], ref, "unfused bias_relu", strict=False)
    check_close(fused.cpu().numpy()[:, cols], ref, "fused bias_relu")
    xn = w4.rmsnorm(A, gm, 1e-6)
    y2 = w4.gemm(xn, w)
    ref2 = ref_gemm(p, cols=cols, rms=True)
    check_close(y2.cpu().numpy()[:, cols], ref2, "unfused rmsnorm", strict=False)


def test_unfused_passes_exact():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 256)).astype(F16)
    b = rng.normal(0, 0.1, 256).astype(F16)
    got_b = w4.add_bias(to_dev(x), to_dev(b)).cpu().numpy()
    assert np.array_equal(got_b, (x.astype(F32) + b.astype(F32)).astype(F16))
    got_r = w4.relu(to_dev(x)).cpu().numpy()
    assert np.array_equal(got_r, np.maximum(x, F16(0)))


# -------------------------------------------------------------------- gate_up


def run_gate_up(p, rms=False):
    wg, wu = repack_dev(p.w), repack_dev(p.w_up)
    out = w4.gemm_gate_up(to_dev(p.A), wg, wu, gamma=to_dev(p.gamma) if rms else None,
                          out=nan_out(p.M, p.N))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def ref_gate_up(p, cols=None, rms=False):
    return oracle.gate_up(p.A, (p.w.qweight, p.w.scales, p.w.zeros),
                          (p.w_up.qweight, p.w_up.scales, p.w_up.zeros), p.group, p.N,
                          gamma=p.gamma if rms else None, cols=cols)


def test_gate_up_config_sampled():
    """M=32, K=5120, N=13824, g=128 asym: silu(A.Wg) * (A.Wu)."""
    p = synth.make_problem(32, 5120, 13824, 128, seed=0, gate_up=True)
    got = run_gate_up(p)
    cols = sample_cols(p.N, 128)
    check_close(got[:, cols], ref_gate_up(p, cols=cols), "gate_up M=32")


@pytest.mark.parametrize("M,g,rms", [(1, 128, False), (8, 16, True), (3, 32, False), (70, 64, True),
                                     (25, 16, True), (32, 128, False)])
def test_gate_up_small_all_outputs(M, g, rms):
    p = synth.make_problem(M, 1024, 256, g, seed=M + g, gate_up=True, gamma=rms)
    check_close(run_gate_up(p, rms), ref_gate_up(p, rms=rms), f"gate_up M={M} g={g} rms={rms}")


@pytest.mark.parametrize("M,rms", [(1, False), (8, True), (16, False)])
def test_gate_up_group16_fp32_scales_narrow_config(M, rms):
    """Group 16 with fp32 scales and two weight streams: the 4-column-tile
    streaming configuration's metadata exceeds the LDS, so the planner takes
    a narrower one (not the tile kernel)."""
    p = synth.make_problem(M, 1024, 512, 16, seed=70 + M, scale_dtype=F32, gate_up=True,
                           gamma=rms)
    assert w4.plan(M, 1024, 512, 16, 1, True).kernel == "stream"
    check_close(run_gate_up(p, rms), ref_gate_up(p, rms=rms), f"gate_up g16 fp32 M={M}")


# ------------------------------------------------- skip + RMSNorm prologue


@pytest.mark.parametrize("M,K,N,g,gu", [(1, 1024, 384, 128, False), (8, 1152, 256, 32, False),
                                        (16, 1024, 512, 64, True), (20, 1152, 256, 64, False),
                                        (27, 1024, 256, 32, True),
                                        (64, 2048, 512, 16, False), (130, 1024, 256, 128, True),
                                        (3, 1024, 256, 128, True), (4, 1152, 256, 64, False),
                                        (5, 1152, 256, 128, True), (12, 1024, 384, 32, False)])
def test_skip_rmsnorm_prologue_all_outputs(M, K, N, g, gu):
    """X = RMSNorm(A + residual): every output against the oracle, and the
    residual sum written out bit-exactly (one fp16 rounding per element)."""
    p = synth.make_problem(M, K, N, g, seed=M * 3 + K, gamma=True, gate_up=gu)
    R = np.random.default_rng(M + K).standard_normal((M, K)).astype(F16)
    S = oracle.skip_sum(p.A, R)
    A, Rd, gm = to_dev(p.A), to_dev(R), to_dev(p.gamma)
    w = repack_dev(p.w)
    s_out = torch.full((M, K), float("nan"), dtype=torch.float16, device="cuda")
    if gu:
        wu = repack_dev(p.w_up)
        y = w4.gemm_gate_up(A, w, wu, gamma=gm, residual=Rd, residual_out=s_out, out=nan_out(M, N))
        ref = oracle.gate_up(S, (p.w.qweight, p.w.scales, p.w.zeros),
                             (p.w_up.qweight, p.w_up.scales, p.w_up.zeros), g, N, gamma=p.gamma)
    else:
        y = w4.gemm(A, w, gamma=gm, residual=Rd, residual_out=s_out, out=nan_out(M, N))
        ref = oracle.gemm(S, p.w.qweight, p.w.scales, p.w.zeros, g, N, gamma=p.gamma)
    torch.cuda.synchronize()
    check_close(y.cpu().numpy(), ref, f"skip rmsnorm M={M} K={K} gu={gu}")
    assert np.array_equal(s_out.cpu().numpy().view(np.uint16), S.view(np.uint16))
    # the same without writing the sum
    y2 = (w4.gemm_gate_up(A, w, wu, gamma=gm, residual=Rd) if gu
          else w4.gemm(A, w, gamma=gm, residual=Rd))
    assert torch.equal(y2, y)


@pytest.mark.parametrize("M", [1, 32])
def test_skip_rmsnorm_decode_shape_sampled(M):
    K, N, g = 5120, 13824, 128
    p = synth.make_problem(M, K, N, g, seed=40 + M, gamma=True, bias=True)
    R = np.random.default_rng(M).standard_normal((M, K)).astype(F16)
    S = oracle.skip_sum(p.A, R)
    s_out = torch.full((M, K), float("nan"), dtype=torch.float16, device="cuda")
    y = w4.gemm(to_dev(p.A), repack_dev(p.w), gamma=to_dev(p.gamma), residual=to_dev(R),
                residual_out=s_out, epilogue="bias", bias=to_dev(p.bias), out=nan_out(M, N))
    cols = sample_cols(N, 96, seed=M)
    ref = oracle.gemm(S, p.w.qweight, p.w.scales, p.w.zeros, g, N, gamma=p.gamma,
                      epilogue="bias", bias=p.bias, cols=cols)
    torch.cuda.synchronize()
    check_close(y.cpu().numpy()[:, cols], ref, f"skip rmsnorm decode M={M}")
    assert np.array_equal(s_out.cpu().numpy().view(np.uint16), S.view(np.uint16))


# ------------------------------------- M=8 decode shapes and split-K control

# The shapes the "Small-M split-K retune" update tunes at M=8: o/q
# 4096x4096, down 13696x4096 (107 k tiles: deeper than one workgroup
# covers, so always split), gate_up 4096 x 2*13696 and 5120 x 2*13824.


@pytest.mark.parametrize("K,N", [(4096, 4096), (13696, 4096)])
def test_split_sweep_gemm_shapes_sampled(K, N):
    p = synth.make_problem(8, K, N, 128, seed=K + N, gamma=True, bias=True)
    cols = sample_cols(N, 96, seed=K)
    got = run_gemm(p)
    check_close(got[:, cols], ref_gemm(p, cols=cols), f"M=8 K={K} N={N}")
    got = run_gemm(p, rms=True, epilogue="bias_relu")
    check_close(got[:, cols], ref_gemm(p, cols=cols, rms=True, epilogue="bias_relu"),
                f"M=8 K={K} N={N} rms+bias_relu")


@pytest.mark.parametrize("K,N", [(4096, 13696), (5120, 13824)])
def test_split_sweep_gate_up_shapes_sampled(K, N):
    p = synth.make_problem(8, K, N, 128, seed=K, gate_up=True)
    got = run_gate_up(p)
    cols = sample_cols(N, 96, seed=N)
    check_close(got[:, cols], ref_gate_up(p, cols=cols), f"gate_up M=8 K={K} N={N}")


def test_forced_splits_match_oracle_and_repeat():
    """Every forced split of the deep down_proj shape (with the RMSNorm
    prologue, whose sums of squares are also split) meets the oracle on
    sampled columns, and repeats bit-identically."""
    K, N, M = 13696, 4096, 8
    p = synth.make_problem(M, K, N, 128, seed=11, gamma=True)
    w = repack_dev(p.w)
    A, gm = to_dev(p.A), to_dev(p.gamma)
    cols = sample_cols(N, 64, seed=3)
    ref = ref_gemm(p, cols=cols, rms=True)
    # (1 and 2: the 14-tile slices of one column tile; 3 and more: 5-tile
    # slices of 4 column tiles)
    for sk in (1, 2, 3, 4, 8, 16, 107):
        y1 = w4.gemm(A, w, gamma=gm, out=nan_out(M, N), split=sk)
        y2 = w4.gemm(A, w, gamma=gm, out=nan_out(M, N), split=sk)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2), f"split {sk} not repeatable"
        check_close(y1.cpu().numpy()[:, cols], ref, f"down_proj split={sk}")


@pytest.mark.parametrize("M,gu", [(2, False), (3, True)])
def test_deep_k_skip_rmsnorm_staged_sampled(M, gu):
    """K = 13696 at M <= 4 runs on 14-tile slices, which cannot hold the
    residual in registers: the skip + RMSNorm prologue is staged; outputs on
    sampled columns, the sum bit-exact."""
    K, N, g = 13696, 4096, 128
    p = synth.make_problem(M, K, N, g, seed=60 + M, gamma=True, gate_up=gu)
    R = np.random.default_rng(M).standard_normal((M, K)).astype(F16)
    S = oracle.skip_sum(p.A, R)
    s_out = torch.full((M, K), float("nan"), dtype=torch.float16, device="cuda")
    A, Rd, gm, w = to_dev(p.A), to_dev(R), to_dev(p.gamma), repack_dev(p.w)
    cols = sample_cols(N, 64, seed=M)
    if gu:
        y = w4.gemm_gate_up(A, w, repack_dev(p.w_up), gamma=gm, residual=Rd, residual_out=s_out,
                            out=nan_out(M, N))
        ref = oracle.gate_up(S, (p.w.qweight, p.w.scales, p.w.zeros),
                             (p.w_up.qweight, p.w_up.scales, p.w_up.zeros), g, N,
                             gamma=p.gamma, cols=cols)
    else:
        y = w4.gemm(A, w, gamma=gm, residual=Rd, residual_out=s_out, out=nan_out(M, N))
        ref = oracle.gemm(S, p.w.qweight, p.w.scales, p.w.zeros, g, N, gamma=p.gamma, cols=cols)
    torch.cuda.synchronize()
    check_close(y.cpu().numpy()[:, cols], ref, f"deep-k skip rmsnorm M={M} gu={gu}")
    assert np.array_equal(s_out.cpu().numpy().view(np.uint16), S.view(np.uint16))


@pytest.mark.parametrize("M", [1, 8, 16, 17, 32])
def test_forced_splits_all_outputs_small(M):
    """Small shape, every output, every feasible split (1 .. 8 k tiles)."""
    p = synth.make_problem(M, 1024, 384, 32, seed=M, gate_up=True, gamma=True)
    ref = ref_gemm(p, rms=True)
    ref_gu = ref_gate_up(p, rms=True)
    w, wu = repack_dev(p.w), repack_dev(p.w_up)
    A, gm = to_dev(p.A), to_dev(p.gamma)
    for sk in range(1, 9):
        y = w4.gemm(A, w, gamma=gm, out=nan_out(M, p.N), split=sk)
        check_close(y.cpu().numpy(), ref, f"M={M} split={sk}")
        y = w4.gemm_gate_up(A, w, wu, gamma=gm, out=nan_out(M, p.N), split=sk)
        check_close(y.cpu().numpy(), ref_gu, f"gate_up M={M} split={sk}")


# --------------------------------------------------------------------- probes


def test_probes():
    src = torch.randint(0, 255, (1 << 22,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    w4.probe_copy(src, dst)
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    w4.probe_read(src, sink)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    # the compute-unit probes: small launches that must complete cleanly
    sink2 = torch.zeros(8 * 512, dtype=torch.int32, device="cuda")
    w4.probe_lds_read(8, 4, sink2)
    rows = torch.randn(64, 1024, device="cuda").half()
    w4.probe_lds_copy(rows, 8, 5, sink2)
    torch.cuda.synchronize()
    # the issue probe: every FMA count and wavefront count runs, and the
    # folded registers are finite and the same from run to run
    fs = torch.zeros(8 * 512, dtype=torch.float32, device="cuda")
    for waves in (1, 2):
        for x in (0, 8, 16, 32, 48, 64):
            w4.probe_mfma_valu(x, waves, 8, 3, fs)
            first = fs.clone()
            w4.probe_mfma_valu(x, waves, 8, 3, fs)
            torch.cuda.synchronize()
            assert torch.isfinite(first[: 8 * 256 * waves]).all()
            assert torch.equal(first, fs)



@pytest.mark.parametrize("K,N,mode,wgs", [(5120, 13824, 0, 0), (5120, 13824, 1, 256),
                                          (1024, 400, 0, 0), (1024, 400, 1, 7), (384, 48, 1, 300)])
def test_probe_read_tiles_reads_every_tile_once(K, N, mode, wgs):
    # each 16-byte chunk of the weight region is folded by exactly one lane,
    # so the xor of every word the probe writes is the xor of every word of
    # the region (ragged shapes: a 1-tile last column block, fewer k tiles
    # than wavefronts, more workgroups than tiles)
    g = torch.Generator(device="cuda")
    g.manual_seed(K + N + mode)
    wreg = torch.randint(0, 256, (K * N // 2,), dtype=torch.uint8, device="cuda", generator=g)
    pw = w4.PackedWeight(wreg, K, N, 128, 0, False)
    grid = (N // 16 + 3) // 4 if mode == 0 else wgs
    sink = torch.zeros(grid * 512, dtype=torch.int32, device="cuda")
    w4.probe_read_tiles(pw, mode, wgs, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(wreg.cpu().numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want


# ------------------------------------------------------- deepest k range

_DEEP = {}


def _deep_weight():
    """K = 28672, N = 8192, group 128 (a 70B-class down projection): drawn
    once per module, packed once."""
    if not _DEEP:
        w = synth.draw_weight(np.random.default_rng(2024), 28672, 8192, 128)
        _DEEP["w"], _DEEP["pw"] = w, repack_dev(w)
    return _DEEP["w"], _DEEP["pw"]


@pytest.mark.parametrize("M,rms", [(1, False), (8, True), (24, False), (40, True)])
def test_deepest_k_sampled(M, rms):
    """224 k tiles: the streaming and panel kernels split them 6 ways, the
    tile kernel runs them in one workgroup; sampled columns against the
    oracle, and a repeated call bit-identical."""
    w, pw = _deep_weight()
    rng = np.random.default_rng(M)
    A = rng.standard_normal((M, w.K)).astype(F16)
    gm = rng.normal(1.0, 0.1, size=w.K).astype(F16) if rms else None
    Ad, gd = to_dev(A), to_dev(gm)
    y = w4.gemm(Ad, pw, gamma=gd, out=nan_out(M, w.N))
    y2 = w4.gemm(Ad, pw, gamma=gd, out=nan_out(M, w.N))
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    cols = sample_cols(w.N, 96, seed=M)
    ref = oracle.gemm(A, w.qweight, w.scales, w.zeros, 128, w.N, gamma=gm, cols=cols)
    check_close(y.cpu().numpy()[:, cols], ref, f"K=28672 M={M} rms={rms}")


# ------------------------------------------------------------ MLP chain


def _mlp_case(M, H, I, g, seed, gamma=False, resid=False, asym=True, sdt=F16):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((M, H)).astype(F16)
    ws = [synth.draw_weight(rng, H, I, g, sdt, asym), synth.draw_weight(rng, H, I, g, sdt, asym),
          synth.draw_weight(rng, I, H, g, sdt, asym)]
    gm = rng.normal(1.0, 0.1, size=H).astype(F16) if gamma or resid else None
    R = rng.standard_normal((M, H)).astype(F16) if resid else None
    return A, ws, gm, R


def _mlp_ref(A, ws, gm, R, g, I, H, cols=None):
    X = A if R is None else oracle.skip_sum(A, R)
    t = [(w.qweight, w.scales, w.zeros) for w in ws]
    return X, oracle.mlp(X, t[0], t[1], t[2], g, I, H, gamma=gm, cols=cols)


@pytest.mark.parametrize("M,H,I,g,gamma,resid,asym,sdt", [
    (1, 512, 1024, 128, False, False, True, F16), (8, 512, 1536, 64, True, False, True, F16),
    (13, 384, 768, 32, False, False, True, F16), (24, 512, 1024, 128, True, True, True, F16),
    (64, 256, 512, 16, False, False, True, F16), (129, 256, 384, 128, True, False, True, F16),
    (3, 1024, 256, 64, False, True, True, F16), (16, 512, 1024, 32, True, False, False, F32),
    (40, 384, 768, 128, False, False, False, F32), (2, 256, 512, 16, True, True, True, F32)])
def test_mlp_chain_all_outputs(M, H, I, g, gamma, resid, asym, sdt):
    """w4a16_mlp: the intermediate against the oracle's gate_up, the output
    against the oracle's chain (both every element), the residual sum
    bit-exact, and the output bit-identical to the two separate calls."""
    A, ws, gm, R = _mlp_case(M, H, I, g, seed=M * 7 + I, gamma=gamma, resid=resid, asym=asym,
                             sdt=sdt)
    X, ref = _mlp_ref(A, ws, gm, R, g, I, H)
    pg, pu, pd = (repack_dev(w) for w in ws)
    Ad, gd, Rd = to_dev(A), to_dev(gm), to_dev(R)
    inter = nan_out(M, I)
    s_out = torch.full((M, H), float("nan"), dtype=torch.float16, device="cuda") if resid else None
    y = w4.mlp(Ad, pg, pu, pd, gamma=gd, residual=Rd, residual_out=s_out, inter=inter,
               out=nan_out(M, H))
    torch.cuda.synchronize()
    t = [(w.qweight, w.scales, w.zeros) for w in ws]
    check_close(inter.cpu().numpy(), oracle.gate_up(X, t[0], t[1], g, I, gamma=gm),
                f"mlp intermediate M={M} H={H} I={I}")
    check_close(y.cpu().numpy(), ref, f"mlp M={M} H={H} I={I} g={g}")
    if resid:
        assert np.array_equal(s_out.cpu().numpy().view(np.uint16), X.view(np.uint16))
    h = w4.gemm_gate_up(Ad, pg, pu, gamma=gd, residual=Rd)
    y2 = w4.gemm(h, pd)
    torch.cuda.synchronize()
    assert torch.equal(h, inter) and torch.equal(y2, y)


@pytest.mark.parametrize("M,H,I", [(8, 4096, 13696), (1, 5120, 13824), (32, 4096, 13696)])
def test_mlp_decode_shapes_sampled(M, H, I):
    """The decode MLP shapes (gate_up H x 2*I, down I x H; the down
    projection is the deep-k split-K shape) with the RMSNorm prologue: the
    intermediate and the output on sampled columns."""
    g = 128
    A, ws, gm, R = _mlp_case(M, H, I, g, seed=H + I + M, gamma=True)
    cols = sample_cols(H, 96, seed=M)
    X, ref = _mlp_ref(A, ws, gm, R, g, I, H, cols=cols)
    inter = nan_out(M, I)
    y = w4.mlp(to_dev(A), *(repack_dev(w) for w in ws), gamma=to_dev(gm), inter=inter,
               out=nan_out(M, H))
    torch.cuda.synchronize()
    icols = sample_cols(I, 96, seed=M + 1)
    t = [(w.qweight, w.scales, w.zeros) for w in ws]
    check_close(inter.cpu().numpy()[:, icols],
                oracle.gate_up(X, t[0], t[1], g, I, gamma=gm, cols=icols), f"mlp inter M={M}")
    check_close(y.cpu().numpy()[:, cols], ref, f"mlp decode M={M} H={H} I={I}")
    assert torch.isfinite(y).all()
