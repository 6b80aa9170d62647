"""GPU parity of every kernel configuration, element by element.

Each case names the configuration it is meant to run (kernel, 16-column
tiles per workgroup, k tiles per wavefront, grid) and asserts it through the
host-only plan query first, so a planner change cannot move a case off the
configuration it covers.  The cases include ragged last column blocks
(N / 16 not a multiple of the workgroup's column tiles), where the last
workgroup clamps its tile reads and its finishing wavefronts past N exit,
and the headline K=5120 N=13824 g=128 shape and the paired gate/up at M=32
compared on every output.  Expected values come only from ``oracle``.
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
    oracle.build(force=False)


def expect_plan(M, K, N, g, *, kernel, col_tiles, grid=None, gate_up=False, sdt=0,
                kpw=None, split=None):
    p = w4.plan(M, K, N, g, sdt, gate_up)
    assert p.kernel == kernel, p
    assert p.col_tiles == col_tiles, p
    if grid is not None:
        assert p.grid == grid, p
    if kpw is not None:
        assert p.k_tiles_per_wave == kpw, p
    if split is not None:
        assert p.split == split, p
    return p


def ragged(N, col_tiles):
    """Column tiles of the last workgroup (col_tiles when N is not ragged)."""
    t = N // 16
    return t - (t + col_tiles - 1) // col_tiles * col_tiles + col_tiles


def run(p, *, gate_up=False, epilogue="none", rms=False):
    A = to_dev(p.A)
    w = repack_dev(p.w)
    gm = to_dev(p.gamma) if rms else None
    if gate_up:
        y = w4.gemm_gate_up(A, w, repack_dev(p.w_up), gamma=gm, out=nan_out(p.M, p.N))
    else:
        y = w4.gemm(A, w, epilogue=epilogue, bias=to_dev(p.bias) if epilogue != "none" else None,
                    gamma=gm, out=nan_out(p.M, p.N))
    torch.cuda.synchronize()
    return y.cpu().numpy()


def ref(p, *, gate_up=False, epilogue="none", rms=False, cols=None):
    gm = p.gamma if rms else None
    if gate_up:
        return oracle.gate_up(p.A, (p.w.qweight, p.w.scales, p.w.zeros),
                              (p.w_up.qweight, p.w_up.scales, p.w_up.zeros), p.group, p.N,
                              gamma=gm, cols=cols)
    return oracle.gemm(p.A, p.w.qweight, p.w.scales, p.w.zeros, p.group, p.N, gamma=gm,
                       epilogue=epilogue, bias=p.bias if epilogue != "none" else None, cols=cols)


# ------------------------------------------ the streaming kernel (M <= 16)


@pytest.mark.parametrize("M", [1, 4, 8, 16])
def test_stream_four_tile_blocks_ragged_last_block(M):
    """4 column tiles per workgroup at N = 13808 (863 tiles): 216 workgroups,
    the last one covering 3 tiles.  Rows through LDS (M <= 4) and loaded per
    k tile (M > 4); every output."""
    expect_plan(M, 5120, 13808, 128, kernel="stream", col_tiles=4, grid=(216, 1, 1), split=1,
                kpw=5)
    assert ragged(13808, 4) == 3
    p = synth.make_problem(M, 5120, 13808, 128, seed=500 + M, bias=True)
    check_close(run(p, epilogue="bias"), ref(p, epilogue="bias"), f"N=13808 M={M}")


@pytest.mark.parametrize("M", [2, 7])
def test_stream_four_tiles_group16_gate_up(M):
    """The four-tile configuration with two weight streams and group 16 (the
    largest scale tables it takes), rows through LDS (M <= 4) and in
    registers, with the ragged last block; every output."""
    expect_plan(M, 5120, 13808, 16, kernel="stream", col_tiles=4, grid=(216, 1, 1), split=1,
                kpw=5, gate_up=True)
    p = synth.make_problem(M, 5120, 13808, 16, seed=600 + M, gate_up=True)
    check_close(run(p, gate_up=True), ref(p, gate_up=True), f"k-sliced g16 gate_up M={M}")


@pytest.mark.parametrize("M,K,N,grid", [(1, 4096, 8192, (256, 1, 1)), (1, 5120, 8192, (256, 1, 1)),
                                        (1, 1024, 6416, (201, 1, 1)), (8, 5120, 6416, (201, 1, 1)),
                                        (16, 5120, 6416, (201, 1, 1)), (3, 4096, 8192, (256, 1, 1))])
def test_stream_two_tile_blocks(M, K, N, grid):
    """2 column tiles per workgroup: N = 8192 fills 256 workgroups exactly;
    N = 6416 (401 tiles) leaves the last workgroup one tile; every output."""
    expect_plan(M, K, N, 128, kernel="stream", col_tiles=2, grid=grid, split=1)
    p = synth.make_problem(M, K, N, 128, seed=M + N, asym=(N != 8192))
    check_close(run(p), ref(p), f"two-tile M={M} K={K} N={N}")


@pytest.mark.parametrize("M,rms", [(1, False), (8, True), (16, False)])
def test_stream_one_tile_blocks(M, rms):
    """1 column tile per workgroup: N = 3200 gives 200 workgroups."""
    expect_plan(M, 5120, 3200, 128, kernel="stream", col_tiles=1, grid=(200, 1, 1), split=1)
    p = synth.make_problem(M, 5120, 3200, 128, seed=M + 3200, gamma=rms)
    check_close(run(p, rms=rms), ref(p, rms=rms), f"one-tile M={M} rms={rms}")


@pytest.mark.parametrize("M", [1, 2, 4, 8, 16])
def test_headline_shape_every_output(M):
    """K=5120 N=13824 g=128, asymmetric zero-points, fp16 scales: the
    configuration the benchmark times, compared on all 13824 columns."""
    expect_plan(M, 5120, 13824, 128, kernel="stream", col_tiles=4, grid=(216, 1, 1), split=1)
    p = synth.make_problem(M, 5120, 13824, 128, seed=0)
    check_close(run(p), ref(p), f"headline M={M}")


@pytest.mark.parametrize("M,gu", [(1, False), (1, True), (8, False)])
def test_wide_n_streams_with_split_k(M, gu):
    """A 70B-class projection (K=8192, N=28672: 1792 column tiles) stays on
    the streaming kernel with a 2-way k split (one arrival counter per column
    tile); sampled columns across the whole range, and a repeat is
    bit-identical."""
    K, N = 8192, 28672 if M == 1 else 22016
    expect_plan(M, K, N, 128, kernel="stream", col_tiles=4, gate_up=gu, split=2)
    p = synth.make_problem(M, K, N, 128, seed=700 + M, gate_up=gu)
    A, w = to_dev(p.A), repack_dev(p.w)
    wu = repack_dev(p.w_up) if gu else None
    call = (lambda: w4.gemm_gate_up(A, w, wu, out=nan_out(M, N))) if gu else \
        (lambda: w4.gemm(A, w, out=nan_out(M, N)))
    y1, y2 = call(), call()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    cols = sample_cols(N, 256, seed=M)
    check_close(y1.cpu().numpy()[:, cols], ref(p, gate_up=gu, cols=cols), f"wide N M={M} gu={gu}")


# ------------------------------------------- the panel kernel (16 < M <= 32)


@pytest.mark.parametrize("M,K,N,split", [(17, 1024, 400, None), (32, 1024, 400, None),
                                         (24, 4096, 4112, 3), (17, 5120, 13808, 1),
                                         (32, 5120, 13808, 1)])
def test_panel_ragged_last_block(M, K, N, split):
    """4 column tiles per workgroup with a ragged last block (N = 400: 25
    tiles; N = 4112: 257; N = 13808: 863), with and without a k split across
    workgroups; every output."""
    pl = expect_plan(M, K, N, 128, kernel="panel", col_tiles=4, split=split)
    assert pl.grid[0] == (N // 16 + 3) // 4 and ragged(N, 4) < 4
    p = synth.make_problem(M, K, N, 128, seed=M * 3 + N, bias=True)
    check_close(run(p, epilogue="bias_relu"), ref(p, epilogue="bias_relu"),
                f"panel ragged M={M} K={K} N={N}")


def test_gate_up_config_every_output():
    """M=32 K=5120 N=13824 g=128 asymmetric: silu(A.Wg) * (A.Wu) on every
    output, on the panel kernel."""
    expect_plan(32, 5120, 13824, 128, kernel="panel", col_tiles=4, gate_up=True, split=1)
    p = synth.make_problem(32, 5120, 13824, 128, seed=0, gate_up=True)
    check_close(run(p, gate_up=True), ref(p, gate_up=True), "gate_up M=32 every output")


@pytest.mark.parametrize("M", [17, 32])
def test_panel_gate_up_ragged(M):
    expect_plan(M, 1024, 400, 64, kernel="panel", col_tiles=4, gate_up=True)
    p = synth.make_problem(M, 1024, 400, 64, seed=M + 64, gate_up=True, gamma=True)
    check_close(run(p, gate_up=True, rms=True), ref(p, gate_up=True, rms=True),
                f"panel gate_up ragged M={M}")


@pytest.mark.parametrize("M,K,N,g,gu", [(24, 1152, 13808, 64, False), (17, 1024, 13824, 128, True),
                                        (32, 1024, 13824, 16, True), (32, 5120, 13824, 128, False),
                                        (32, 5120, 13824, 128, True)])
def test_panel_rmsnorm_prologue_in_kernel(M, K, N, g, gu):
    """The panel kernel's own RMSNorm prologue (no k split across workgroups,
    so nothing is staged): x * gamma in the fragments, the slices' sums of
    squares through LDS, the row scale in the epilogue.  K = 1152 has 9 k
    tiles, so one slice ends past K; N = 13808 a ragged last block; every
    output at K <= 1152, a sample of them at K = 5120."""
    expect_plan(M, K, N, g, kernel="panel", col_tiles=4, gate_up=gu, split=1)
    p = synth.make_problem(M, K, N, g, seed=M * 7 + K + g, gamma=True, gate_up=gu)
    got = run(p, gate_up=gu, rms=True)
    cols = None if K <= 1152 else np.unique(np.concatenate([np.arange(N - 32, N),
                                                            sample_cols(N, 160, seed=K)]))
    want = ref(p, gate_up=gu, rms=True, cols=cols)
    check_close(got if cols is None else got[:, cols], want, f"panel rmsnorm M={M} K={K} gu={gu}")


# ------------------------------------------------ the tile kernel (M > 32)


@pytest.mark.parametrize("M,N", [(64, 13808), (128, 13808)])
def test_tile_ragged_last_block_sampled(M, N):
    """The tile kernel's column blocks (64 or 128 columns) with a ragged last
    block at the decode depth; the last block's columns and a sample of the
    rest against the oracle."""
    pl = w4.plan(M, 5120, N, 128)
    assert pl.kernel == "tile" and (N // 16) % pl.col_tiles != 0
    p = synth.make_problem(M, 5120, N, 128, seed=M + 1)
    got = run(p)
    cols = np.unique(np.concatenate([np.arange(N - 128, N), sample_cols(N, 128, seed=M)]))
    check_close(got[:, cols], ref(p, cols=cols), f"tile ragged M={M} N={N}")


@pytest.mark.parametrize("M,g,epi,rms", [(128, 128, "bias_relu", False), (100, 32, "bias", False),
                                         (128, 64, "none", True), (70, 16, "bias", True)])
def test_tile_epilogue_wide_ragged_sampled(M, g, epi, rms):
    """The tile kernel's epilogue with two 64-row blocks (two column tiles per
    wavefront), a ragged last column block and a ragged last row block: bias
    and ReLU, the staged RMSNorm row scales, every group size's path; the
    last block's columns and a sample of the rest against the oracle."""
    N = 13808
    pl = w4.plan(M, 1024, N, g)
    assert pl.kernel == "tile" and pl.grid[2] == 2 and (N // 16) % pl.col_tiles != 0
    p = synth.make_problem(M, 1024, N, g, seed=M + g, gamma=rms, bias=epi != "none")
    got = run(p, epilogue=epi, rms=rms)
    cols = np.unique(np.concatenate([np.arange(N - 160, N), sample_cols(N, 128, seed=M + g)]))
    check_close(got[:, cols], ref(p, epilogue=epi, rms=rms, cols=cols),
                f"tile epilogue M={M} g={g} {epi} rms={rms}")
