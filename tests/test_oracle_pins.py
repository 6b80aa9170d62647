"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

None of these compares the oracle with itself through a retyped formula.  Each
pin is a hand-worked example, a closed form, an exact special case that
reduces to an integer/library matmul built from the raw draws (not from the
packed bytes the oracle reads), or an invariant.  Chosen so that a dropped
term, a wrong sign, a swapped nibble, a transposed operand or a wrong group
index fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import bytemodel
from decode_w4a16_repack_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- hand-worked


def test_handworked_dequant_and_epilogues(oracle_lib):
    g = _load("handworked_tiny.json")
    K, N, grp = g["K"], g["N"], g["group"]
    q = np.array(g["qweight_bytes"], np.uint8)
    s = np.array(g["scales"], np.float64)
    z = np.array(g["zeros_bytes"], np.uint8)
    A = np.array(g["A"], np.float64)
    b = np.array(g["bias"], np.float64)
    # the fixture's bytes are the canonical packing of its codes
    assert (synth.pack_nibbles_rows(np.array(g["codes_by_column"])) == q).all()
    assert (synth.pack_nibbles_rows(np.array(g["zp_by_column"])) == z).all()
    W = oracle.dequant(q, s, z, K, N, grp)
    assert np.array_equal(W, np.array(g["W"]))
    for epi, key in [("none", "expected_none"), ("bias", "expected_bias"),
                     ("bias_relu", "expected_bias_relu")]:
        y = oracle.gemm(A, q, s, z, grp, N, epilogue=epi, bias=b)
        assert np.array_equal(y, np.array(g[key])), epi


# ------------------------------------------------- exact integer special cases


@pytest.mark.parametrize("group", [16, 32, 64, 128])
def test_unit_scale_zero_zp_is_integer_matmul(oracle_lib, group):
    """s = 1, zp = 0, integer A: the result is the int64 product A @ codes."""
    rng = np.random.default_rng(11)
    K, N, M = 256, 48, 3
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    G = K // group
    w = synth.weight_from_codes(codes, np.ones((N, G), np.float16),
                                np.zeros((N, G), np.uint8), group)
    A = rng.integers(-8, 9, size=(M, K))
    y = oracle.gemm(A.astype(np.float64), w.qweight, w.scales, w.zeros, group, N)
    assert np.array_equal(y, (A.astype(np.int64) @ codes.astype(np.int64)).astype(np.float64))


def test_symmetric_is_codes_minus_eight(oracle_lib):
    """zeros=None means zero-point 8: s = 1 gives A @ (codes - 8) exactly."""
    rng = np.random.default_rng(12)
    K, N, M, group = 128, 32, 2, 32
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    w = synth.weight_from_codes(codes, np.ones((N, K // group), np.float32), None, group)
    A = rng.integers(-8, 9, size=(M, K))
    y = oracle.gemm(A.astype(np.float64), w.qweight, w.scales, None, group, N)
    ref = A.astype(np.int64) @ (codes.astype(np.int64) - 8)
    assert np.array_equal(y, ref.astype(np.float64))


def test_explicit_zp8_bit_identical_to_symmetric(oracle_lib):
    p = synth.make_problem(3, 256, 32, 64, seed=5, asym=False)
    G = p.K // p.group
    z8 = synth.pack_nibbles_rows(np.full((p.N, G), 8, np.uint8))
    y_sym = oracle.gemm(p.A, p.w.qweight, p.w.scales, None, p.group, p.N)
    y_z8 = oracle.gemm(p.A, p.w.qweight, p.w.scales, z8, p.group, p.N)
    assert np.array_equal(y_sym, y_z8)


# ---------------------------------------- brute force vs a library matmul


@pytest.mark.parametrize("group", [16, 32, 64, 128])
@pytest.mark.parametrize("sdt", [np.float16, np.float32])
@pytest.mark.parametrize("asym", [True, False])
def test_tiny_vs_numpy_matmul_from_raw_draws(oracle_lib, group, sdt, asym):
    """Dense W rebuilt from the raw (unpacked) draws, then numpy's matmul."""
    M, K, N = 3, 256, 32
    p = synth.make_problem(M, K, N, group, seed=7, scale_dtype=sdt, asym=asym)
    G = K // group
    kgrp = np.arange(K) // group
    zp = p.w.zp if asym else np.full((N, G), 8, np.uint8)
    W = (p.w.codes.astype(np.float64) - zp.T[kgrp, :]) * \
        p.w.scales.astype(np.float64).T[kgrp, :]
    ref = p.A.astype(np.float64) @ W
    y = oracle.gemm(p.A, p.w.qweight, p.w.scales, p.w.zeros, group, N)
    assert np.allclose(y, ref, rtol=0, atol=1e-12 * np.abs(ref).max())
    Wo = oracle.dequant(p.w.qweight, p.w.scales, p.w.zeros, K, N, group)
    assert np.array_equal(Wo, W)


def test_column_subset_matches_full(oracle_lib):
    p = synth.make_problem(2, 256, 64, 32, seed=3)
    full = oracle.gemm(p.A, p.w.qweight, p.w.scales, p.w.zeros, p.group, p.N)
    cols = np.array([63, 0, 17, 17, 5])
    sub = oracle.gemm(p.A, p.w.qweight, p.w.scales, p.w.zeros, p.group, p.N, cols=cols)
    assert np.array_equal(sub, full[:, cols])


# ------------------------------------------------------------------ invariants


def test_power_of_two_scale_scales_output_exactly(oracle_lib):
    p = synth.make_problem(2, 256, 32, 64, seed=9, scale_dtype=np.float32)
    y = oracle.gemm(p.A, p.w.qweight, p.w.scales, p.w.zeros, p.group, p.N)
    y8 = oracle.gemm(p.A, p.w.qweight, p.w.scales * np.float32(8), p.w.zeros, p.group, p.N)
    assert np.array_equal(y8, 8 * y)


@pytest.mark.parametrize("group", [16, 32, 128])
def test_group_knockout(oracle_lib, group):
    """Codes equal to the zero-point over group i remove exactly that group:
    identical to zeroing A's columns of group i."""
    rng = np.random.default_rng(21)
    K, N, M = 256, 32, 2
    p = synth.make_problem(M, K, N, group, seed=21)
    i = (K // group) - 1 if group == 128 else 1
    codes = p.w.codes.copy()
    ks = slice(i * group, (i + 1) * group)
    codes[ks, :] = p.w.zp[:, i][None, :]
    w_ko = synth.weight_from_codes(codes, p.w.scales, p.w.zp, group)
    A0 = p.A.astype(np.float64).copy()
    A0[:, ks] = 0.0
    y_ko = oracle.gemm(p.A, w_ko.qweight, w_ko.scales, w_ko.zeros, group, N)
    y_a0 = oracle.gemm(A0, p.w.qweight, p.w.scales, p.w.zeros, group, N)
    assert np.array_equal(y_ko, y_a0)
    # and the group did contribute before
    y = oracle.gemm(p.A, p.w.qweight, p.w.scales, p.w.zeros, group, N)
    assert not np.array_equal(y, y_a0)
    del rng


def test_column_permutation(oracle_lib):
    p = synth.make_problem(2, 128, 48, 32, seed=4)
    perm = np.random.default_rng(0).permutation(p.N)
    w = synth.weight_from_codes(p.w.codes[:, perm], p.w.scales[perm], p.w.zp[perm], p.group)
    y = oracle.gemm(p.A, p.w.qweight, p.w.scales, p.w.zeros, p.group, p.N)
    yp = oracle.gemm(p.A, w.qweight, w.scales, w.zeros, p.group, p.N)
    assert np.array_equal(yp, y[:, perm])


def test_bias_and_relu_compose(oracle_lib):
    p = synth.make_problem(4, 256, 64, 64, seed=13, bias=True)
    y = oracle.gemm(p.A, p.w.qweight, p.w.scales, p.w.zeros, p.group, p.N)
    b = p.bias.astype(np.float64)
    yb = oracle.gemm(p.A, p.w.qweight, p.w.scales, p.w.zeros, p.group, p.N,
                     epilogue="bias", bias=p.bias)
    ybr = oracle.gemm(p.A, p.w.qweight, p.w.scales, p.w.zeros, p.group, p.N,
                      epilogue="bias_relu", bias=p.bias)
    assert np.array_equal(yb, y + b)
    assert np.array_equal(ybr, np.maximum(y + b, 0.0))
    assert (ybr == 0).any() and (ybr > 0).any()


# --------------------------------------------------------------------- RMSNorm


def test_rmsnorm_constant_row_closed_form(oracle_lib):
    """A row of constant c with gamma = 1 normalizes to c / sqrt(c^2 + eps)."""
    K, N, group = 256, 32, 32
    p = synth.make_problem(1, K, N, group, seed=2)
    for c, eps in [(0.75, 1e-6), (1e-3, 1e-6), (-2.0, 0.5)]:
        A = np.full((1, K), c)
        W = oracle.dequant(p.w.qweight, p.w.scales, p.w.zeros, K, N, group)
        x = c / np.sqrt(c * c + eps)
        ref = x * W.sum(axis=0, keepdims=True)
        y = oracle.gemm(A, p.w.qweight, p.w.scales, p.w.zeros, group, N,
                        gamma=np.ones(K), eps=eps)
        assert np.allclose(y, ref, rtol=1e-13, atol=1e-13), (c, eps)
    # eps inside the root: c = 1e-3, eps = 1e-6 gives 1/sqrt(2), not 1
    assert abs(1e-3 / np.sqrt(1e-6 + 1e-6) - 0.7071067811865476) < 1e-15


def test_rmsnorm_scale_invariant_at_zero_eps(oracle_lib):
    """With eps = 0 the prologue is invariant to scaling A by a power of two,
    and gamma acts per k (a one-hot gamma selects one row of W)."""
    p = synth.make_problem(2, 128, 16, 32, seed=8)
    g = np.ones(p.K)
    y1 = oracle.gemm(p.A, p.w.qweight, p.w.scales, p.w.zeros, p.group, p.N, gamma=g, eps=0.0)
    y4 = oracle.gemm(4.0 * p.A.astype(np.float64), p.w.qweight, p.w.scales, p.w.zeros,
                     p.group, p.N, gamma=g, eps=0.0)
    assert np.array_equal(y1, y4)
    k0 = 37
    onehot = np.zeros(p.K)
    onehot[k0] = 1.0
    A = p.A.astype(np.float64)
    W = oracle.dequant(p.w.qweight, p.w.scales, p.w.zeros, p.K, p.N, p.group)
    y = oracle.gemm(A, p.w.qweight, p.w.scales, p.w.zeros, p.group, p.N, gamma=onehot, eps=0.0)
    r = 1.0 / np.sqrt((A * A).mean(axis=1))
    assert np.allclose(y, (A[:, k0] * r)[:, None] * W[k0][None, :], rtol=1e-14, atol=0)


@pytest.mark.parametrize("staging", ["normalized", "scaled"])
def test_rms_staged_exact_when_the_staged_row_is_representable(oracle_lib, staging):
    """A row of +-1 with eps = 0 has mean square exactly 1, so X = +-gamma
    and A * gamma = +-gamma are fp16 values already: the staged readings
    round nothing and equal the canonical oracle bit for bit."""
    rng = np.random.default_rng(41)
    K, N, group = 256, 32, 64
    p = synth.make_problem(1, K, N, group, seed=42, gamma=True, bias=True)
    A = rng.choice([-1.0, 1.0], size=(3, K)).astype(np.float16)
    w = (p.w.qweight, p.w.scales, p.w.zeros)
    for epi in ("none", "bias_relu"):
        ref = oracle.gemm(A, *w, group, N, gamma=p.gamma, eps=0.0, epilogue=epi, bias=p.bias)
        got = oracle.gemm_rms_staged(A, *w, group, N, p.gamma, eps=0.0, staging=staging,
                                     epilogue=epi, bias=p.bias)
        assert np.array_equal(got, ref), (staging, epi)


@pytest.mark.parametrize("staging", ["normalized", "scaled"])
def test_rms_staged_gap_within_the_fp16_rounding_bound(oracle_lib, staging):
    """The staged row differs from the exact one only by one round-to-nearest
    to fp16: relative error at most 2^-11 for a normal result, absolute at
    most 2^-25 below 2^-14.  So |Y_staged - Y| <= sum_k (2^-11 |X_k| +
    2^-25) |W_kn| (for the scaled reading the row factor r > 0 carries the
    bound over unchanged), and the gap must also be far inside the parity
    tolerance 2e-2 max|Y| (a twentieth of it here; about a hundredth is
    measured); a staging that rounds nothing would show no gap at all."""
    K, N, group = 1024, 64, 128
    p = synth.make_problem(4, K, N, group, seed=43, gamma=True)
    w = (p.w.qweight, p.w.scales, p.w.zeros)
    ref = oracle.gemm(p.A, *w, group, N, gamma=p.gamma, eps=1e-6)
    got = oracle.gemm_rms_staged(p.A, *w, group, N, p.gamma, eps=1e-6, staging=staging)
    X, r = oracle.rmsnorm(p.A, p.gamma, 1e-6)
    assert np.allclose(X, p.A.astype(np.float64) * p.gamma.astype(np.float64) * r[:, None],
                       rtol=1e-15, atol=0)
    W = np.abs(oracle.dequant(p.w.qweight, p.w.scales, p.w.zeros, K, N, group))
    bound = (2.0 ** -11) * (np.abs(X) @ W) + (2.0 ** -25) * W.sum(axis=0)[None, :]
    gap = np.abs(got - ref)
    assert (gap <= bound * (1 + 1e-9) + 1e-12).all(), staging
    assert gap.max() > 0.0
    assert gap.max() < 0.05 * 2e-2 * np.abs(ref).max()


# --------------------------------------------------------------------- gate_up


def test_gate_up_equal_weights_is_silu_y_times_y(oracle_lib):
    p = synth.make_problem(2, 256, 32, 64, seed=17)
    w = (p.w.qweight, p.w.scales, p.w.zeros)
    y = oracle.gemm(p.A, *w, p.group, p.N)
    out = oracle.gate_up(p.A, w, w, p.group, p.N)
    assert np.allclose(out, y * y / (1.0 + np.exp(-y)), rtol=1e-14, atol=1e-14)


def test_gate_up_integer_gate_silu_values(oracle_lib):
    """Integer gate outputs let silu be checked at known points:
    silu(0) = 0 and silu(v) = v * sigmoid(v) (sigmoid from scipy)."""
    from scipy.special import expit
    rng = np.random.default_rng(31)
    K, N, group = 128, 16, 32
    G = K // group
    codes = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    codes[:, 0] = 8  # column 0: every code at the zero-point -> gate 0
    gate = synth.weight_from_codes(codes, np.ones((N, G), np.float16),
                                   np.full((N, G), 8, np.uint8), group)
    up = synth.make_problem(1, K, N, group, seed=32).w
    A = rng.integers(-2, 3, size=(2, K)).astype(np.float64)
    yg = A @ (codes.astype(np.float64) - 8)
    yu = oracle.gemm(A, up.qweight, up.scales, up.zeros, group, N)
    out = oracle.gate_up(A, (gate.qweight, gate.scales, gate.zeros),
                         (up.qweight, up.scales, up.zeros), group, N)
    assert np.all(out[:, 0] == 0.0)
    assert np.allclose(out, yg * expit(yg) * yu, rtol=1e-13, atol=1e-12)


def test_gate_up_rmsnorm_matches_prenormalized(oracle_lib):
    """The prologue applies to the shared activation of both projections."""
    p = synth.make_problem(2, 128, 16, 32, seed=19, gamma=True, gate_up=True)
    g, u = (p.w.qweight, p.w.scales, p.w.zeros), (p.w_up.qweight, p.w_up.scales, p.w_up.zeros)
    A = p.A.astype(np.float64)
    gam = p.gamma.astype(np.float64)
    X = A * gam / np.sqrt((A * A).mean(axis=1, keepdims=True) + 1e-6)
    a = oracle.gate_up(p.A, g, u, p.group, p.N, gamma=p.gamma, eps=1e-6)
    b = oracle.gate_up(X, g, u, p.group, p.N)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ MLP chain


def test_mlp_permutation_down_returns_rounded_intermediate(oracle_lib):
    """A down projection whose dequantized weight is a permutation matrix
    (code 9 on one entry per row, 8 elsewhere, zero-point 8, scale 1) moves
    intermediate column i to output column perm[i] unchanged: the chain's
    output is then exactly the fp16-rounded gate_up result, permuted.  The
    permutation is not an involution, so a transposed down operand fails."""
    p = synth.make_problem(2, 256, 128, 32, seed=41, gate_up=True)
    g, u = (p.w.qweight, p.w.scales, p.w.zeros), (p.w_up.qweight, p.w_up.scales, p.w_up.zeros)
    I = H = 128
    perm = np.roll(np.arange(H), 5)
    codes = np.full((I, H), 8, np.uint8)
    codes[np.arange(I), perm] = 9
    G = I // p.group
    d = synth.weight_from_codes(codes, np.ones((H, G), np.float16), None, p.group)
    y = oracle.mlp(p.A, g, u, (d.qweight, d.scales, None), p.group, I, H)
    h = oracle.gate_up(p.A, g, u, p.group, I).astype(np.float16).astype(np.float64)
    ref = np.empty_like(h)
    ref[:, perm] = h
    assert np.array_equal(y, ref)


@pytest.mark.parametrize("asym", [True, False])
def test_mlp_tiny_vs_numpy_from_raw_draws(oracle_lib, asym):
    """Dense gate, up and down weights rebuilt from the raw draws; silu from
    scipy; the intermediate rounded to fp16 by numpy; numpy's matmul."""
    from scipy.special import expit
    rng = np.random.default_rng(43)
    M, K, I, H, group = 3, 256, 128, 48, 32
    A = rng.standard_normal((M, K)).astype(np.float16)
    ws = [synth.draw_weight(rng, K, I, group, asym=asym),
          synth.draw_weight(rng, K, I, group, asym=asym),
          synth.draw_weight(rng, I, H, group, asym=asym)]

    def dense(w):
        kg = np.arange(w.K) // group
        zp = w.zp if asym else np.full((w.N, w.K // group), 8, np.uint8)
        return (w.codes.astype(np.float64) - zp.T[kg, :]) * w.scales.astype(np.float64).T[kg, :]
    Wg, Wu, Wd = (dense(w) for w in ws)
    a = A.astype(np.float64)
    yg, yu = a @ Wg, a @ Wu
    h = (yg * expit(yg) * yu).astype(np.float16).astype(np.float64)
    ref = h @ Wd
    t = [(w.qweight, w.scales, w.zeros) for w in ws]
    y = oracle.mlp(A, t[0], t[1], t[2], group, I, H)
    assert np.allclose(y, ref, rtol=0, atol=1e-12 * np.abs(ref).max())
    cols = np.array([47, 0, 16, 31])
    ys = oracle.mlp(A, t[0], t[1], t[2], group, I, H, cols=cols)
    assert np.array_equal(ys, y[:, cols])


# ------------------------------------------------------------------ byte model


def test_fusion_byte_model_page_numbers():
    """'Fusion benchmark' page: f32 matmul+bias+relu moves 20 B per output
    unfused and 4 fused; fusion saves at most 16*M*N."""
    M = N = 512
    assert bytemodel.epilogue_chain_bytes(M, N, 4, fused=False) == 20 * M * N
    assert bytemodel.epilogue_chain_bytes(M, N, 4, fused=True) == 4 * M * N
    assert bytemodel.epilogue_saved_bytes(M, N, 4) == 16 * M * N
    # fp16 at M=16, N=4096: 131,072 B fused vs 655,360 B unfused
    assert bytemodel.epilogue_chain_bytes(16, 4096, 2, fused=True) == 131072
    assert bytemodel.epilogue_chain_bytes(16, 4096, 2, fused=False) == 655360
    assert bytemodel.rmsnorm_a_side_bytes(16, 4096, True) == 131072
    assert bytemodel.rmsnorm_a_side_bytes(16, 4096, False) == 393216


def test_gemm_byte_count_decode_shape():
    # K=5120 N=13824 g=128, fp16 scales, 4-bit zero-points, M=1
    assert bytemodel.gemm_bytes(1, 5120, 13824, 128) == 36809728
    assert bytemodel.gemm_bytes(128, 5120, 13824, 128) == 41621504
    assert bytemodel.gemm_flops(1, 1, 1) == 2
    # 8192^3 GEMM is 2*8192^3 ~ 1.1 TFLOP (croqtile tutorial, "TFLOPS")
    assert bytemodel.gemm_flops(8192, 8192, 8192) == 1099511627776


# ------------------------------------------------------------------- repack


def test_repack_index_golden(oracle_lib):
    for c in _load("repack_index.json")["cases"]:
        assert oracle.weight_nibble_index(c["K"], c["k"], c["n"]) == c["index"], c


@pytest.mark.parametrize("K,N", [(128, 16), (256, 32), (384, 48)])
def test_repack_map_is_bijection(oracle_lib, K, N):
    idx = np.array([oracle.weight_nibble_index(K, k, n) for n in range(N) for k in range(K)])
    assert np.array_equal(np.sort(idx), np.arange(K * N))


def test_repack_word_semantics(oracle_lib):
    """Word d of lane l in tile (t, kc) holds codes k = 128kc+32d+8kq+j of
    column 16t + l%16 (kq = l//16): even j in bits 4(j/2), odd j in bits
    16+4(j/2)."""
    K, N, group = 256, 32, 128
    p = synth.make_problem(1, K, N, group, seed=23)
    packed = oracle.repack(p.w.qweight, p.w.scales, p.w.zeros, K, N, group)
    words = packed[: K * N // 2].view(np.uint32)  # little-endian host
    KC = K // 128
    for t in range(N // 16):
        for kc in range(KC):
            for lane in range(64):
                for d in range(4):
                    wv = int(words[((t * KC + kc) * 64 + lane) * 4 + d])
                    n = 16 * t + lane % 16
                    for j in range(8):
                        k = 128 * kc + 32 * d + 8 * (lane // 16) + j
                        sh = 4 * (j // 2) + (16 if j % 2 else 0)
                        assert (wv >> sh) & 15 == p.w.codes[k, n]


@pytest.mark.parametrize("sdt", [np.float16, np.float32])
@pytest.mark.parametrize("asym", [True, False])
@pytest.mark.parametrize("K,N,group", [(512, 512, 32), (256, 48, 16), (1024, 64, 128)])
def test_repack_round_trip(oracle_lib, sdt, asym, K, N, group):
    p = synth.make_problem(1, K, N, group, seed=29, scale_dtype=sdt, asym=asym)
    packed = oracle.repack(p.w.qweight, p.w.scales, p.w.zeros, K, N, group)
    q, s, z = oracle.unrepack(packed, K, N, group, sdt, asym)
    assert np.array_equal(q, p.w.qweight)
    assert np.array_equal(s.view(np.uint8), p.w.scales.view(np.uint8))
    if asym:
        assert np.array_equal(z, p.w.zeros)
    # scale and zero-point regions: element (t, i, c) is (n = 16t + c, group i)
    so, zo, total = oracle.packed_layout(K, N, group, np.dtype(sdt).itemsize, asym)
    G = K // group
    sreg = packed[so: so + N * G * np.dtype(sdt).itemsize].view(sdt).reshape(N // 16, G, 16)
    assert np.array_equal(sreg.transpose(0, 2, 1).reshape(N, G).view(np.uint8),
                          p.w.scales.view(np.uint8))
    if asym:
        zb = packed[zo: zo + N * G // 2]
        zn = np.stack([zb & 15, zb >> 4], axis=1).reshape(N // 16, G, 16)
        assert np.array_equal(zn.transpose(0, 2, 1).reshape(N, G), p.w.zp)
    assert not packed[K * N // 2: so].any()


@pytest.mark.parametrize("esize", [2, 4])
@pytest.mark.parametrize("has_zp", [True, False])
def test_repack_metadata_positions_golden(oracle_lib, esize, has_zp):
    """Scale and zero-point positions worked out by hand from the layout's
    text (tests/golden/repack_meta_index.json): one marked scale and one
    marked zero-point at a time, every other byte of both regions zero."""
    g = _load("repack_meta_index.json")
    K, N, group = g["K"], g["N"], g["group"]
    G = K // group
    lay = next(x for x in g["layout"] if x["esize"] == esize and x["has_zp"] == has_zp)
    so, zo, total = oracle.packed_layout(K, N, group, esize, has_zp)
    assert so == lay["scales_offset"] and total == lay["total"]
    if has_zp:
        assert zo == lay["zeros_offset"]
    sdt = np.float16 if esize == 2 else np.float32
    q = np.zeros((N, K // 2), np.uint8)
    marker = np.array(1.5, sdt)  # 0x3E00 / 0x3FC00000: nonzero high byte
    for c in g["scales"]:
        s = np.zeros((N, G), sdt)
        s[c["n"], c["i"]] = marker
        z = np.zeros((N, (G + 1) // 2), np.uint8) if has_zp else None
        packed = oracle.repack(q, s, z, K, N, group)
        at = so + c["index"] * esize
        assert packed[at: at + esize].tobytes() == marker.tobytes(), c
        region = packed[so: so + N * G * esize].copy()
        region[c["index"] * esize: (c["index"] + 1) * esize] = 0
        assert not region.any(), c
    if not has_zp:
        return
    for c in g["zeros"]:
        z = np.zeros((N, (G + 1) // 2), np.uint8)
        i = c["i"]
        z[c["n"], i // 2] = 0xA << (4 * (i % 2))  # zero-point 10 in its canonical nibble
        packed = oracle.repack(q, np.zeros((N, G), sdt), z, K, N, group)
        b = packed[zo + c["byte"]]
        assert b == (0xA0 if c["high"] else 0x0A), c
        region = packed[zo: zo + N * G // 2].copy()
        region[c["byte"]] = 0
        assert not region.any(), c


def test_packed_sizes_decode_shape(oracle_lib):
    so, zo, total = oracle.packed_layout(5120, 13824, 128, 2, True)
    assert so == 35389440 and zo == 35389440 + 1105920 and total == 36771840
    assert oracle.packed_layout(5120, 13824, 128, 2, False)[2] == 36495360


# ------------------------------------------------------ magnitude plausibility


def test_output_magnitude_matches_page_tolerance_scale(oracle_lib):
    """The page's parity line (worst_abs 0.013 against tol 0.67 = 2e-2*max|out|)
    implies max|out| ~ 33.5 at K=5120 N=13824 g=128.  The workload recipe
    (A ~ N(0,1), codes and zp uniform, scales U[0.001, 0.02]) must land in the
    same range, or the inputs are not the page's kind."""
    p = synth.make_problem(2, 5120, 13824, 128, seed=0)
    cols = np.arange(0, 13824, 3)
    y = oracle.gemm(p.A, p.w.qweight, p.w.scales, p.w.zeros, 128, 13824, cols=cols)
    assert 15.0 < np.abs(y).max() < 60.0


def test_skip_sum_rounds_once_to_nearest_even():
    """S = A + R in fp16 (IEEE 754 binary16, round to nearest, ties to even):
    exact when representable; 2048 + 1 and 2050 + 1 are ties between
    neighbours 2 apart and go to the even significand (2048, 2052); a sum
    past the largest finite value 65504 by half an ulp or more overflows."""
    import oracle
    f = np.float16
    A = np.array([3, -7.5, 2048, 2050, 0.25, 65504, 1e-7], dtype=f)
    R = np.array([5, 7.5, 1, 1, 0.125, 16, 0], dtype=f)
    S = oracle.skip_sum(A, R)
    assert S.dtype == np.float16
    assert list(S[:5]) == [8, 0, 2048, 2052, 0.375]
    assert np.isinf(S[5])                      # 65520 is the tie with 2^16: rounds up
    assert S[6] == A[6]                        # adding zero is the identity
    rng = np.random.default_rng(0)
    x = rng.standard_normal((4, 64)).astype(f)
    y = rng.standard_normal((4, 64)).astype(f)
    assert np.array_equal(oracle.skip_sum(x, y), oracle.skip_sum(y, x))
