"""Capture contract ("Stage 2 of spec-capture" and "What's landed" updates on
the onnx-genai pull request: a warmed call is capture-safe when its launch
grid is static, nothing is allocated on replay and nothing is read back to
the host).

A warm call of each entry point is captured into a HIP graph (through
torch.cuda.CUDAGraph) and replayed several times, with eager work of the
program (other library calls on other inputs, torch ops, synchronizations)
between the replays; every replay must reproduce the eager result
bit-for-bit and meet the oracle's result within the parity tolerance (the
pull request's "Validation" section pairs its capture-safety checks with
f64-oracle parity).  The shapes include the split-K path, whose arrival
counters must be back at zero after every replay.
"""
import numpy as np
import pytest
import torch

import oracle
import decode_w4a16_repack_amd as w4
from decode_w4a16_repack_amd import synth

from gpu_cases import check_close, repack_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)


def _oracle_of(p, kind, R):
    """f64 oracle result of one capture case (every output)."""
    t = (p.w.qweight, p.w.scales, p.w.zeros)
    if kind == "skip":
        return oracle.gemm(oracle.skip_sum(p.A, R), *t, p.group, p.N, gamma=p.gamma)
    if kind == "gate_up":
        return oracle.gate_up(p.A, t, (p.w_up.qweight, p.w_up.scales, p.w_up.zeros), p.group,
                              p.N, gamma=p.gamma)
    if kind == "rms":
        return oracle.gemm(p.A, *t, p.group, p.N, gamma=p.gamma)
    if kind == "bias_relu":
        return oracle.gemm(p.A, *t, p.group, p.N, epilogue="bias_relu", bias=p.bias)
    return oracle.gemm(p.A, *t, p.group, p.N)


def _capture(fn):
    """Warm fn eagerly, then capture one call of it on a side stream."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.synchronize()
    return g


# (M, K, N, group, kind): stream kernel without and with split-K, tile
# kernel with one and two 64-row blocks, gate_up, RMSNorm and bias epilogues
CASES = [
    (1, 5120, 13824, 128, "gemm"),
    (1, 5120, 256, 128, "gemm"),          # split-K across workgroups
    (8, 13696, 4096, 128, "gemm"),        # deep k: 14-tile slices, no split
    (12, 13696, 4096, 128, "gemm"),       # deep k: split-K
    (16, 1024, 384, 32, "rms"),
    (64, 1024, 512, 64, "bias_relu"),
    (130, 2048, 512, 128, "gemm"),
    (8, 1024, 256, 128, "gate_up"),       # split-K gate_up with RMSNorm
    (40, 1024, 256, 16, "gate_up"),
    (32, 1024, 512, 64, "rms"),           # panel kernel on staged rows (split over k)
    (24, 1024, 13824, 128, "rms"),        # panel kernel, its own RMSNorm prologue
    (32, 1152, 13808, 64, "gate_up"),     # panel gate_up, its own prologue, ragged block
    (70, 1024, 256, 128, "skip"),         # tile kernel, staged skip + RMSNorm
    (12, 1024, 384, 32, "skip"),          # stream kernel, staged skip + RMSNorm
    (3, 1024, 384, 128, "skip"),          # stream kernel, skip + RMSNorm in registers
]


@pytest.mark.parametrize("M,K,N,g,kind", CASES)
def test_graph_replay_is_bit_identical_to_eager(M, K, N, g, kind):
    p = synth.make_problem(M, K, N, g, seed=M + N, gamma=True, bias=True, gate_up=(kind == "gate_up"))
    w = repack_dev(p.w)
    wu = repack_dev(p.w_up) if kind == "gate_up" else None
    A, gm, b = to_dev(p.A), to_dev(p.gamma), to_dev(p.bias)
    ws = w4.Workspace()
    ws.get(8 << 20, "cuda")  # sized once: no reallocation can move it after capture
    out = torch.empty((M, N), dtype=torch.float16, device="cuda")
    R_host = np.random.default_rng(M).standard_normal((M, K)).astype(np.float16)
    R = to_dev(R_host)
    S = torch.empty((M, K), dtype=torch.float16, device="cuda")
    expect = _oracle_of(p, kind, R_host)

    def call():
        if kind == "skip":
            w4.gemm(A, w, gamma=gm, residual=R, residual_out=S, out=out, workspace=ws)
        elif kind == "gate_up":
            w4.gemm_gate_up(A, w, wu, gamma=gm, out=out, workspace=ws)
        elif kind == "rms":
            w4.gemm(A, w, gamma=gm, out=out, workspace=ws)
        elif kind == "bias_relu":
            w4.gemm(A, w, epilogue="bias_relu", bias=b, out=out, workspace=ws)
        else:
            w4.gemm(A, w, out=out, workspace=ws)

    call()
    torch.cuda.synchronize()
    eager, eager_s = out.clone(), S.clone()
    g_ = _capture(call)
    # other eager work on the same workspace between replays: a different
    # shape that also splits k (its counters share the workspace)
    q = synth.make_problem(2, 1024, 512, 128, seed=99)
    wq, Aq = repack_dev(q.w), to_dev(q.A)
    ref_q = w4.gemm(Aq, wq, workspace=ws).clone()
    for r in range(4):
        out.fill_(float("nan"))
        S.fill_(float("nan"))
        g_.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager call"
        check_close(out.cpu().numpy(), expect, f"replay {r} {kind} M={M} K={K} N={N}")
        if kind == "skip":
            assert torch.equal(S, eager_s), f"replay {r}: residual sum differs"
            assert np.array_equal(S.cpu().numpy().view(np.uint16),
                                  oracle.skip_sum(p.A, R_host).view(np.uint16))
        assert torch.equal(w4.gemm(Aq, wq, workspace=ws), ref_q)
        torch.cuda.synchronize()


@pytest.mark.parametrize("M", [8, 24])
def test_mlp_block_replay_is_bit_identical_to_eager(M):
    """w4a16_mlp (gate_up with the RMSNorm prologue, staged at 24 rows, then
    the down projection, split over k) captured and replayed: intermediate
    and output equal the eager call every time."""
    H, I, g = 512, 1536, 64
    rng = np.random.default_rng(M)
    ws_ = [synth.draw_weight(rng, H, I, g), synth.draw_weight(rng, H, I, g),
           synth.draw_weight(rng, I, H, g)]
    pw = [repack_dev(x) for x in ws_]
    A_host = rng.standard_normal((M, H)).astype(np.float16)
    gm_host = rng.normal(1.0, 0.1, size=H).astype(np.float16)
    A, gm = to_dev(A_host), to_dev(gm_host)
    t = [(x.qweight, x.scales, x.zeros) for x in ws_]
    expect_inter = oracle.gate_up(A_host, t[0], t[1], g, I, gamma=gm_host)
    expect_out = oracle.mlp(A_host, t[0], t[1], t[2], g, I, H, gamma=gm_host)
    ws = w4.Workspace()
    ws.get(8 << 20, "cuda")
    inter = torch.empty((M, I), dtype=torch.float16, device="cuda")
    out = torch.empty((M, H), dtype=torch.float16, device="cuda")

    def call():
        w4.mlp(A, *pw, gamma=gm, inter=inter, out=out, workspace=ws)

    call()
    torch.cuda.synchronize()
    e_inter, e_out = inter.clone(), out.clone()
    g_ = _capture(call)
    for r in range(4):
        inter.fill_(float("nan"))
        out.fill_(float("nan"))
        g_.replay()
        torch.cuda.synchronize()
        assert torch.equal(inter, e_inter) and torch.equal(out, e_out), f"replay {r}"
        check_close(inter.cpu().numpy(), expect_inter, f"replay {r} mlp intermediate M={M}")
        check_close(out.cpu().numpy(), expect_out, f"replay {r} mlp output M={M}")
        w4.gemm(A, pw[0], gamma=gm, workspace=ws)  # other eager work on the workspace
        torch.cuda.synchronize()


def test_replay_reads_current_inputs():
    """The graph holds pointers, not values: new input data written into the
    captured buffers is what the next replay computes on."""
    p1 = synth.make_problem(4, 1024, 256, 64, seed=1)
    p2 = synth.make_problem(4, 1024, 256, 64, seed=2)
    w = repack_dev(p1.w)
    A = to_dev(p1.A)
    ws = w4.Workspace()
    ws.get(1 << 20, "cuda")
    out = torch.empty((4, 256), dtype=torch.float16, device="cuda")
    g_ = _capture(lambda: w4.gemm(A, w, out=out, workspace=ws))
    ref2 = w4.gemm(to_dev(p2.A), w, workspace=ws).clone()
    A.copy_(to_dev(p2.A))
    g_.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, ref2)
    check_close(out.cpu().numpy(),
                oracle.gemm(p2.A, p1.w.qweight, p1.w.scales, p1.w.zeros, 64, 256),
                "replay on new inputs")


def test_replay_allocates_nothing():
    """No device memory is taken on replay (the library never allocates; the
    workspace is the caller's)."""
    p = synth.make_problem(1, 5120, 256, 128, seed=5)
    w = repack_dev(p.w)
    A = to_dev(p.A)
    ws = w4.Workspace()
    ws.get(1 << 20, "cuda")
    out = torch.empty((1, 256), dtype=torch.float16, device="cuda")
    g_ = _capture(lambda: w4.gemm(A, w, out=out, workspace=ws))
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats()
    for _ in range(8):
        g_.replay()
    torch.cuda.synchronize()
    after = torch.cuda.memory_stats()
    assert after["allocation.all.allocated"] == before["allocation.all.allocated"]
    assert after["allocated_bytes.all.current"] == before["allocated_bytes.all.current"]
    check_close(out.cpu().numpy(), oracle.gemm(p.A, p.w.qweight, p.w.scales, p.w.zeros, 128, 256),
                "replayed split-K call")
