"""C-ABI checks that need no GPU: the library loads, exports every function
include/w4a16.h declares, and rejects bad arguments on the host before any
HIP call (every error status is forced here)."""
import ctypes
import os
import re

import pytest

from decode_w4a16_repack_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")
CB = _lib.COUNTER_BYTES  # split-K arrival counters at the start of every workspace


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a16_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libw4a16.so is not built; run __graft_entry__.build()")
    return _lib.lib()


def test_exports_every_header_function(L):
    names = header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.EXPORTS)


def test_header_is_plain_c_and_cxx(tmp_path):
    """The header compiles as strict C99 and as C++17 with no warning: a C
    caller needs nothing from C++ or from HIP's headers."""
    import shutil
    import subprocess
    src = tmp_path / "use.c"
    src.write_text('#include "w4a16.h"\nint main(void) { return w4a16_layout_version() > 0 ? 0 : 1; }\n')
    inc = os.path.join(ROOT, "include")
    for cc, std, lang in (("gcc", "-std=c99", "c"), ("g++", "-std=c++17", "c++")):
        if shutil.which(cc) is None:
            pytest.skip(f"{cc} not found")
        r = subprocess.run([cc, std, "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                            "-x", lang, "-I", inc, str(src)], capture_output=True, text=True)
        assert r.returncode == 0, (cc, r.stderr)


def test_header_enums_match_binding():
    text = open(HEADER).read()
    for name, val in [("W4A16_ERR_NULL", -1), ("W4A16_ERR_SHAPE", -2),
                      ("W4A16_ERR_GROUP", -3), ("W4A16_ERR_DTYPE", -4),
                      ("W4A16_ERR_EPILOGUE", -5), ("W4A16_ERR_WORKSPACE", -6),
                      ("W4A16_ERR_ALIGN", -7), ("W4A16_ERR_LAUNCH", -8),
                      ("W4A16_ERR_SPLIT", -9), ("W4A16_ERR_SCRATCH", -10)]:
        assert re.search(rf"{name}\s*=\s*{val}\b", text), name
        assert getattr(_lib, name[6:]) == val
    assert re.search(r"W4A16_EPI_BIAS_RELU\s*=\s*2", text)
    assert re.search(rf"#define W4A16_COUNTER_BYTES {_lib.COUNTER_BYTES}\b", text)
    assert re.search(r"W4A16_SCALE_F32\s*=\s*1", text)


def test_layout_version_and_status_strings(L):
    assert L.w4a16_layout_version() == 1
    for st in range(-10, 1):
        assert len(L.w4a16_status_string(st)) > 0
    assert L.w4a16_status_string(-99) == b"unknown status"


def test_packed_bytes_matches_oracle_layout(L, oracle_lib):
    import oracle
    for K, N, g, sdt, zp in [(5120, 13824, 128, 0, 1), (5120, 13824, 128, 0, 0),
                             (512, 512, 32, 1, 1), (4096, 4096, 16, 0, 1),
                             (128, 16, 16, 1, 0), (384, 48, 128, 0, 1)]:
        esize = 2 if sdt == 0 else 4
        assert L.w4a16_packed_bytes(K, N, g, sdt, zp) == oracle.packed_layout(K, N, g, esize, zp)[2]


def test_packed_bytes_rejects_bad_shapes(L):
    assert L.w4a16_packed_bytes(100, 16, 16, 0, 1) == 0
    assert L.w4a16_packed_bytes(128, 15, 16, 0, 1) == 0
    assert L.w4a16_packed_bytes(128, 16, 8, 0, 1) == 0
    assert L.w4a16_packed_bytes(128, 16, 16, 7, 1) == 0


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def gemm(L, A=FAKE, M=2, K=512, N=512, group=32, sdt=0, zp=1, packed=FAKE, epi=0,
         bias=None, gamma=None, out=FAKE, ws=None, ws_n=0):
    return L.w4a16_gemm(A, M, K, N, group, sdt, zp, packed, epi, bias, gamma, 1e-6, out,
                        ws, ws_n, None)


def test_gemm_validation_statuses(L):
    assert gemm(L, A=None) == _lib.ERR_NULL
    assert gemm(L, packed=None) == _lib.ERR_NULL
    assert gemm(L, out=None) == _lib.ERR_NULL
    assert gemm(L, M=0) == _lib.ERR_SHAPE
    assert gemm(L, K=500) == _lib.ERR_SHAPE
    assert gemm(L, N=24) == _lib.ERR_SHAPE
    assert gemm(L, group=48) == _lib.ERR_GROUP
    assert gemm(L, group=256) == _lib.ERR_GROUP
    assert gemm(L, sdt=2) == _lib.ERR_DTYPE
    assert gemm(L, epi=3) == _lib.ERR_EPILOGUE
    assert gemm(L, epi=1, bias=None) == _lib.ERR_EPILOGUE
    assert gemm(L, epi=2, bias=None) == _lib.ERR_EPILOGUE
    assert gemm(L, A=FAKE + 2) == _lib.ERR_ALIGN
    assert gemm(L, out=FAKE + 8) == _lib.ERR_ALIGN
    assert gemm(L, epi=1, bias=FAKE + 4) == _lib.ERR_ALIGN
    # a shape that needs split-K partials must get a workspace
    M, K, N, g = 4, 5120, 512, 128   # a narrow grid: the plan splits k across workgroups
    need = L.w4a16_workspace_bytes(M, K, N, g, 0)
    assert need > 0
    assert gemm(L, M=M, K=K, N=N, group=g, ws=None) == _lib.ERR_WORKSPACE
    assert gemm(L, M=M, K=K, N=N, group=g, ws=FAKE, ws_n=need - 1) == _lib.ERR_WORKSPACE
    assert gemm(L, M=M, K=K, N=N, group=g, ws=FAKE + 4, ws_n=need) == _lib.ERR_ALIGN


def test_gate_up_and_repack_validation(L):
    f = L.w4a16_gemm_gate_up
    assert f(FAKE, 2, 512, 512, 32, 0, 1, FAKE, None, None, 1e-6, FAKE, None, 0, None) == _lib.ERR_NULL
    assert f(FAKE, 2, 512, 512, 33, 0, 1, FAKE, FAKE, None, 1e-6, FAKE, None, 0, None) == _lib.ERR_GROUP
    assert f(FAKE, 2, 512, 512, 32, 0, 1, FAKE, FAKE + 1, None, 1e-6, FAKE, None, 0, None) == _lib.ERR_ALIGN
    r = L.w4a16_repack
    assert r(None, FAKE, None, 512, 512, 32, 0, FAKE, None) == _lib.ERR_NULL
    assert r(FAKE, FAKE, None, 512, 520, 32, 0, FAKE, None) == _lib.ERR_SHAPE
    assert r(FAKE, FAKE, None, 512, 512, 32, 5, FAKE, None) == _lib.ERR_DTYPE
    assert r(FAKE, FAKE, FAKE + 8, 512, 512, 32, 0, FAKE, None) == _lib.ERR_ALIGN


def test_aux_validation(L):
    assert L.w4a16_add_bias(FAKE, None, 2, 16, FAKE, None) == _lib.ERR_NULL
    assert L.w4a16_relu(FAKE, 2, 20, FAKE, None) == _lib.ERR_SHAPE
    assert L.w4a16_rmsnorm(FAKE, FAKE, 1e-6, 2, 100, FAKE, None) == _lib.ERR_SHAPE
    assert L.w4a16_probe_read(FAKE, 15, FAKE, None) == _lib.ERR_SHAPE
    assert L.w4a16_probe_copy(FAKE, FAKE + 4, 16, None) == _lib.ERR_ALIGN
    assert L.w4a16_probe_lds_read(4, 10, None, None) == _lib.ERR_NULL
    assert L.w4a16_probe_lds_read(0, 10, FAKE, None) == _lib.ERR_SHAPE
    assert L.w4a16_probe_lds_read(4, 0, FAKE, None) == _lib.ERR_SHAPE
    assert L.w4a16_probe_lds_read(4, 10, FAKE + 4, None) == _lib.ERR_ALIGN
    assert L.w4a16_probe_lds_copy(None, 16384, 4, 10, FAKE, None) == _lib.ERR_NULL
    assert L.w4a16_probe_lds_copy(FAKE, 16000, 4, 10, FAKE, None) == _lib.ERR_SHAPE
    assert L.w4a16_probe_lds_copy(FAKE, 8192, 4, 10, FAKE, None) == _lib.ERR_SHAPE
    assert L.w4a16_probe_lds_copy(FAKE, 16384, 70000, 10, FAKE, None) == _lib.ERR_SHAPE
    assert L.w4a16_probe_lds_copy(FAKE, 16384, 4, 0, FAKE, None) == _lib.ERR_SHAPE
    assert L.w4a16_probe_lds_copy(FAKE + 4, 16384, 4, 10, FAKE, None) == _lib.ERR_ALIGN
    sb = 256 * 512 * 4
    assert L.w4a16_probe_mfma_valu(16, 2, 256, 100, None, sb, None) == _lib.ERR_NULL
    assert L.w4a16_probe_mfma_valu(12, 2, 256, 100, FAKE, sb, None) == _lib.ERR_SHAPE
    assert L.w4a16_probe_mfma_valu(16, 3, 256, 100, FAKE, sb, None) == _lib.ERR_SHAPE
    assert L.w4a16_probe_mfma_valu(16, 2, 0, 100, FAKE, sb, None) == _lib.ERR_SHAPE
    assert L.w4a16_probe_mfma_valu(16, 2, 256, 0, FAKE, sb, None) == _lib.ERR_SHAPE
    assert L.w4a16_probe_mfma_valu(16, 2, 256, 100, FAKE, sb - 4, None) == _lib.ERR_SHAPE
    assert L.w4a16_probe_mfma_valu(16, 2, 256, 100, FAKE + 4, sb, None) == _lib.ERR_ALIGN
    big = 1 << 30
    assert L.w4a16_probe_read_tiles(None, 5120, 13824, 0, 0, FAKE, big, None) == _lib.ERR_NULL
    assert L.w4a16_probe_read_tiles(FAKE, 5000, 13824, 0, 0, FAKE, big, None) == _lib.ERR_SHAPE
    assert L.w4a16_probe_read_tiles(FAKE, 5120, 13820, 0, 0, FAKE, big, None) == _lib.ERR_SHAPE
    assert L.w4a16_probe_read_tiles(FAKE, 5120, 13824, 2, 0, FAKE, big, None) == _lib.ERR_SHAPE
    assert L.w4a16_probe_read_tiles(FAKE, 5120, 13824, 1, 0, FAKE, big, None) == _lib.ERR_SHAPE
    assert L.w4a16_probe_read_tiles(FAKE, 5120, 13824, 1, 70000, FAKE, big, None) == _lib.ERR_SHAPE
    # the sink holds one word per thread of the grid: 216 workgroups in mode 0
    assert L.w4a16_probe_read_tiles(FAKE, 5120, 13824, 0, 0, FAKE, 216 * 2048 - 4, None) == _lib.ERR_SHAPE
    assert L.w4a16_probe_read_tiles(FAKE, 5120, 13824, 1, 256, FAKE, 255 * 2048, None) == _lib.ERR_SHAPE
    assert L.w4a16_probe_read_tiles(FAKE + 4, 5120, 13824, 0, 0, FAKE, big, None) == _lib.ERR_ALIGN


def test_workspace_only_for_narrow_grids(L):
    # wide N fills the chip without k splits across workgroups.  M <= 4 (the
    # streaming kernel, RMSNorm prologue in registers): no workspace.  Above
    # that the workspace holds only the RMSNorm staging (fp16 [M][K] rows,
    # fp32 [M] sums of squares, each 256-byte aligned), which only calls that
    # stage their prologue need.  It starts after the split-K arrival
    # counters (W4A16_COUNTER_BYTES) that every plan shares (and leaves at
    # zero): staged rows written there would corrupt the next split-K call.
    a256 = lambda v: (v + 255) // 256 * 256
    for M in (1, 2, 4):
        assert L.w4a16_workspace_bytes(M, 5120, 13824, 128, 0) == 0
        assert L.w4a16_workspace_bytes(M, 5120, 13824, 128, 1) == 0
    # M = 5..32: the streaming and panel kernels stage only the skip + RMSNorm
    # prologue (the panel kernel also with a k split across workgroups, which
    # wide N does not need); the tile kernel (M > 32) stages every prologue
    for M in (5, 16, 17, 32, 64, 128):
        stage = CB + a256(M * 5120 * 2) + a256(M * 4)
        assert L.w4a16_workspace_bytes(M, 5120, 13824, 128, 0) == stage
        assert L.w4a16_workspace_bytes(M, 5120, 13824, 128, 1) == stage
        # a call that stages checks for the staging before any launch
        if M > 32:
            assert gemm(L, M=M, K=5120, N=13824, group=128, gamma=FAKE) == _lib.ERR_WORKSPACE
            assert gemm(L, M=M, K=5120, N=13824, group=128, gamma=FAKE, ws=FAKE,
                        ws_n=stage - 1) == _lib.ERR_WORKSPACE
        skip = L.w4a16_gemm_skip_rmsnorm(FAKE, FAKE, None, M, 5120, 13824, 128, 0, 1, FAKE, 0,
                                         None, FAKE, 1e-6, FAKE, FAKE, stage - 1, None)
        assert skip == _lib.ERR_WORKSPACE
    assert L.w4a16_workspace_bytes(0, 5120, 13824, 128, 0) == 0
    w1 = L.w4a16_workspace_bytes(1, 5120, 256, 128, 0)
    w1g = L.w4a16_workspace_bytes(1, 5120, 256, 128, 1)
    assert 0 < w1 < w1g


def test_single_hip_runtime_after_load(L):
    """The library must bind to the HIP runtime torch loaded (one per process)."""
    maps = open("/proc/self/maps").read()
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(libs) <= 1, libs


def plan(L, M, K, N, g=128, sdt=0, gu=0, split=0):
    info = _lib.PlanInfo()
    st = L.w4a16_plan(M, K, N, g, sdt, gu, split, ctypes.byref(info))
    return st, info


def test_plan_query_matches_workspace_and_kernel_choice(L):
    """Stream kernel for M <= 16, panel kernel to M = 32, tile kernel above; the plan's workspace is
    what w4a16_workspace_bytes reports; the grid covers every column tile."""
    for M, K, N, gu in [(1, 5120, 13824, 0), (8, 13696, 4096, 0), (16, 4096, 4096, 0),
                        (8, 4096, 13696, 1), (17, 5120, 13824, 0), (128, 1024, 384, 1),
                        (1, 1024, 384, 0)]:
        st, info = plan(L, M, K, N, gu=gu)
        assert st == _lib.OK
        assert info.kernel == (_lib.KERNEL_STREAM if M <= 16 else
                               _lib.KERNEL_PANEL if M <= 32 else _lib.KERNEL_TILE)
        assert info.block in (256, 512)
        assert info.k_tiles_per_split * info.split >= K // 128
        assert info.k_tiles_per_split * (info.split - 1) < K // 128  # no empty split
        assert info.grid[1] == info.split
        ws = max(plan(L, M, K, N, sdt=s, gu=gu)[1].workspace_bytes for s in (0, 1))
        assert ws == L.w4a16_workspace_bytes(M, K, N, 128, gu)
        # split-K exchange, plus the RMSNorm staging rows above M = 16
        stage = 0 if M <= 4 else CB + (M * K * 2 + 255) // 256 * 256 + (M * 4 + 255) // 256 * 256
        assert (info.workspace_bytes > stage) == (info.split > 1)
        assert info.workspace_bytes >= stage


def test_plan_deep_k_splits_and_forced_splits(L):
    """K = 13696 (107 k tiles) is deeper than an 8 x 5-tile workgroup
    covers.  Up to 8 rows the automatic plan takes slices of 14 k tiles with
    one column tile per workgroup (256 workgroups, no split); above that it
    splits k, and a forced split below that minimum, above the tile count,
    or on the tile kernel (M > 32) is rejected; a forced split rounds so
    that no slice is empty."""
    st, auto = plan(L, 8, 13696, 4096)
    assert st == _lib.OK and auto.split == 1 and auto.k_tiles_per_split == 107
    assert tuple(auto.grid) == (256, 1, 1)
    st, f = plan(L, 8, 13696, 4096, split=1)
    assert st == _lib.OK and f.split == 1
    st, auto = plan(L, 16, 13696, 4096)
    assert st == _lib.OK and auto.split >= 3
    for sk in (1, 2):
        assert plan(L, 16, 13696, 4096, split=sk)[0] == _lib.ERR_SPLIT
    assert plan(L, 8, 1024, 384, split=9)[0] == _lib.ERR_SPLIT    # 8 k tiles
    st, f = plan(L, 17, 4096, 4096, split=2)                      # panel kernel, M > 16
    assert st == _lib.OK and f.kernel == _lib.KERNEL_PANEL and f.split == 2
    assert plan(L, 17, 4096, 4096, split=33)[0] == _lib.ERR_SPLIT  # 32 k tiles
    assert plan(L, 33, 4096, 4096, split=2)[0] == _lib.ERR_SPLIT   # tile kernel
    st, f = plan(L, 8, 5120, 13824, split=9)   # 40 tiles: 5 per split -> 8 splits
    assert st == _lib.OK and (f.split, f.k_tiles_per_split) == (8, 5)
    for sk in (3, 4, 8, 16):
        st, f = plan(L, 16, 13696, 4096, split=sk)
        assert st == _lib.OK and f.split <= sk and f.workspace_bytes > 0
    st, f = plan(L, 8, 4096, 4096, split=1)
    # no split-K exchange: only the skip + RMSNorm staging (after the counters)
    assert st == _lib.OK and f.split == 1 and f.workspace_bytes == CB + 8 * 4096 * 2 + 256
    assert L.w4a16_plan(8, 4096, 4096, 128, 0, 0, 0, None) == _lib.ERR_NULL
    assert plan(L, 8, 4000, 4096)[0] == _lib.ERR_SHAPE


def test_forced_split_workspace_checked_before_launch(L):
    """A forced split needs its own workspace size; a smaller one is refused
    on the host (FAKE pointers are never dereferenced)."""
    FAKE = 1 << 20
    st, f = plan(L, 8, 13696, 4096, split=8)
    # the reported size ends with the skip + RMSNorm staging rows; a call
    # without that prologue needs the split-K part before them
    staging = (8 * 13696 * 2 + 255) // 256 * 256 + 256
    split_part = f.workspace_bytes - staging
    assert split_part > CB
    assert L.w4a16_gemm_split(FAKE, 8, 13696, 4096, 128, 0, 1, FAKE, 0, None, None, 1e-6,
                              FAKE, FAKE, split_part - 1, 8, None) == _lib.ERR_WORKSPACE
    # above 8 rows the 107 k tiles need at least 3 splits: 2 is refused
    assert L.w4a16_gemm_split(FAKE, 16, 13696, 4096, 128, 0, 1, FAKE, 0, None, None, 1e-6,
                              FAKE, FAKE, 1 << 30, 2, None) == _lib.ERR_SPLIT
    assert L.w4a16_gemm_gate_up_split(FAKE, 20, 4096, 4096, 128, 0, 1, FAKE, FAKE, None, 1e-6,
                                      FAKE, FAKE, 1 << 30, 33, None) == _lib.ERR_SPLIT


def test_library_sources_never_allocate_sync_or_memset():
    """Capture safety by construction: no allocation, free, host
    synchronization, copy or memset call anywhere in the library sources
    (a memset node in a captured graph is also avoided this way)."""
    csrc = os.path.join(ROOT, "decode_w4a16_repack_amd", "csrc")
    banned = re.compile(r"\b(hipMalloc\w*|hipFree\w*|hipHostMalloc|hipMemset\w*|hipMemcpy\w*|"
                        r"hipDeviceSynchronize|hipStreamSynchronize|hipEventSynchronize)\s*\(")
    for name in sorted(os.listdir(csrc)):
        text = re.sub(r"//[^\n]*|/\*.*?\*/", "", open(os.path.join(csrc, name)).read(), flags=re.S)
        hits = banned.findall(text)
        assert not hits, (name, hits)


def test_skip_rmsnorm_validation(L):
    """The skip prologue needs residual and gamma; 16-byte aligned buffers."""
    FAKE = 1 << 20
    args = (8, 1024, 256, 128, 0, 1, FAKE, 0, None)
    assert L.w4a16_gemm_skip_rmsnorm(FAKE, None, None, *args, FAKE, 1e-6, FAKE, FAKE,
                                     1 << 30, None) == _lib.ERR_NULL
    assert L.w4a16_gemm_skip_rmsnorm(FAKE, FAKE, None, *args, None, 1e-6, FAKE, FAKE,
                                     1 << 30, None) == _lib.ERR_NULL
    assert L.w4a16_gemm_skip_rmsnorm(FAKE, FAKE + 8, None, *args, FAKE, 1e-6, FAKE, FAKE,
                                     1 << 30, None) == _lib.ERR_ALIGN
    assert L.w4a16_gemm_skip_rmsnorm(FAKE, FAKE, FAKE + 4, *args, FAKE, 1e-6, FAKE, FAKE,
                                     1 << 30, None) == _lib.ERR_ALIGN
    assert L.w4a16_gemm_gate_up_skip_rmsnorm(FAKE, None, None, 8, 1024, 256, 128, 0, 1, FAKE,
                                             FAKE, FAKE, 1e-6, FAKE, FAKE, 1 << 30,
                                             None) == _lib.ERR_NULL
    assert L.w4a16_gemm_gate_up_skip_rmsnorm(FAKE, FAKE, None, 8, 1000, 256, 128, 0, 1, FAKE,
                                             FAKE, FAKE, 1e-6, FAKE, FAKE, 1 << 30,
                                             None) == _lib.ERR_SHAPE


def test_mlp_validation_before_any_launch(L):
    """w4a16_mlp checks both projections on the host before it enqueues
    either: a bad down projection (or workspace) fails with nothing run."""
    FAKE = 1 << 20
    M, H, I, g = 8, 1024, 2048, 128
    need = L.w4a16_mlp_workspace_bytes(M, H, I, g)
    assert need == max(L.w4a16_workspace_bytes(M, H, I, g, 1),
                       L.w4a16_workspace_bytes(M, I, H, g, 0))
    assert L.w4a16_mlp_workspace_bytes(M, H, I + 1, g) == 0

    def mlp(A=FAKE, res=None, res_out=None, M=M, H=H, I=I, g=g, gate=FAKE, up=FAKE,
            down=FAKE, gamma=None, inter=FAKE, out=FAKE, ws=FAKE, ws_n=1 << 30):
        return L.w4a16_mlp(A, res, res_out, M, H, I, g, 0, 1, gate, up, down, gamma, 1e-6,
                           inter, out, ws, ws_n, None)
    assert mlp(inter=None) == _lib.ERR_NULL
    assert mlp(down=None) == _lib.ERR_NULL
    assert mlp(I=2048 + 64) == _lib.ERR_SHAPE        # down projection's K = I
    assert mlp(H=1024 + 16) == _lib.ERR_SHAPE        # gate_up's K = H
    assert mlp(inter=FAKE + 8) == _lib.ERR_ALIGN
    assert mlp(down=FAKE + 4) == _lib.ERR_ALIGN
    assert mlp(res=FAKE) == _lib.ERR_NULL            # residual needs gamma
    assert mlp(res_out=FAKE) == _lib.ERR_NULL        # residual_out needs residual
    # the skip prologue of gate_up is staged above 4 rows: its staging rows
    # (M*H fp16 after the counter bytes) are required, whatever else
    stage = CB + M * H * 2 + 256
    assert need >= stage
    assert mlp(res=FAKE, gamma=FAKE, ws=None, ws_n=0) == _lib.ERR_WORKSPACE
    assert mlp(res=FAKE, gamma=FAKE, ws=FAKE, ws_n=stage - 1) == _lib.ERR_WORKSPACE
    # sizes only (no call): the decode MLP block at M=1
    d = L.w4a16_workspace_bytes(1, 13696, 4096, 128, 0)
    u = L.w4a16_workspace_bytes(1, 4096, 13696, 128, 1)
    assert L.w4a16_mlp_workspace_bytes(1, 4096, 13696, 128) == max(d, u)


def test_plan_invariants_over_many_shapes(L):
    """Host-only sweep of the planner over M, K, N, group, scale width,
    gate_up and forced splits: every automatic plan exists and is
    consistent (kernel by M, LDS within the 160 KiB of a compute unit, the k
    range covered with no empty split, the grid over every column tile, the
    workspace at least the staging it needs), and every forced split either
    plans with at most that many splits or is refused, never anything else."""
    import itertools
    KS = [128, 1024, 1152, 4096, 5120, 8192, 13696, 13824, 14336, 16384, 28672]
    NS = [16, 256, 4096, 5120, 13824, 22016, 28672]
    MS = [1, 2, 4, 5, 8, 9, 16, 17, 24, 32, 33, 64, 128, 129]
    n = 0
    for M, K, N, g, sdt, gu in itertools.product(MS, KS, NS, (16, 128), (0, 1), (0, 1)):
        st, info = plan(L, M, K, N, g, sdt, gu)
        assert st == _lib.OK, (M, K, N, g, sdt, gu, st)
        KC = K // 128
        want = (_lib.KERNEL_STREAM if M <= 16 else _lib.KERNEL_PANEL if M <= 32
                else _lib.KERNEL_TILE)
        # every M <= 16 shape runs on the streaming kernel (the split-K
        # counters cover N up to 65536), never on the 64-row tile kernel; the
        # panel kernel takes every 16 < M <= 32 shape but one whose scale
        # tables exceed its LDS (group 16, fp32 scales, two weight streams)
        panel_lds = g == 16 and sdt == 1 and gu == 1
        assert info.kernel == want or (want == _lib.KERNEL_PANEL and panel_lds
                                       and info.kernel == _lib.KERNEL_TILE), \
            (M, K, N, g, sdt, gu, info.kernel)
        assert 0 < info.lds_bytes <= 160 * 1024
        assert info.block in (256, 512)
        assert info.split >= 1 and info.grid[1] == info.split
        assert info.k_tiles_per_split * info.split >= KC
        assert info.k_tiles_per_split * (info.split - 1) < KC
        assert all(x >= 1 for x in info.grid)
        if info.kernel != _lib.KERNEL_TILE:
            rows = 16 if info.kernel == _lib.KERNEL_STREAM else 32
            assert info.grid[2] == (M + rows - 1) // rows
        stage = CB + M * K * 2 if M > 4 else 0
        assert info.workspace_bytes >= stage
        assert info.workspace_bytes == max(plan(L, M, K, N, g, s, gu)[1].workspace_bytes
                                           for s in (sdt,))
        n += 1
        if M <= 32 and K in (1152, 13696) and N in (256, 4096):
            for sk in (1, 2, 3, 5, 8, KC, KC + 1):
                st, f = plan(L, M, K, N, g, sdt, gu, split=sk)
                assert st in (_lib.OK, _lib.ERR_SPLIT), (M, K, N, sk, st)
                if st == _lib.OK:
                    assert 1 <= f.split <= sk and f.grid[1] == f.split
                    assert f.k_tiles_per_split * f.split >= KC
                    assert f.k_tiles_per_split * (f.split - 1) < KC
                    assert f.kernel != _lib.KERNEL_TILE
    assert n == len(MS) * len(KS) * len(NS) * 8


def test_noalloc_validates_and_refuses_before_any_hip_call(L):
    """w4a16_gemm_noalloc reports argument errors like w4a16_gemm, and a shape
    whose workspace need exceeds its static scratch with W4A16_ERR_SCRATCH,
    all on the host (FAKE pointers are never dereferenced)."""
    f = L.w4a16_gemm_noalloc
    assert re.search(rf"#define W4A16_NOALLOC_SCRATCH_BYTES \(8u << 20\)", open(HEADER).read())
    assert _lib.NOALLOC_SCRATCH_BYTES == 8 << 20
    assert f(None, 2, 512, 512, 32, 0, 1, FAKE, 0, None, None, 1e-6, FAKE, None) == _lib.ERR_NULL
    assert f(FAKE, 2, 500, 512, 32, 0, 1, FAKE, 0, None, None, 1e-6, FAKE, None) == _lib.ERR_SHAPE
    assert f(FAKE, 2, 512, 512, 32, 0, 1, FAKE, 1, None, None, 1e-6, FAKE, None) == _lib.ERR_EPILOGUE
    assert f(FAKE + 4, 2, 512, 512, 32, 0, 1, FAKE, 0, None, None, 1e-6, FAKE, None) == _lib.ERR_ALIGN
    # staged RMSNorm rows of 640 x 8192 fp16 (10 MiB) exceed the 8 MiB scratch
    M, K, N = 640, 8192, 256
    assert L.w4a16_workspace_bytes(M, K, N, 128, 0) > _lib.NOALLOC_SCRATCH_BYTES
    assert f(FAKE, M, K, N, 128, 0, 1, FAKE, 0, None, FAKE, 1e-6, FAKE, None) == _lib.ERR_SCRATCH
    # split-K partials of 16 x 65536 over 2 splits (8 MiB + counters) exceed it too
    st, info = plan(L, 16, 8192, 65536)
    assert st == _lib.OK and info.split > 1 and info.workspace_bytes > _lib.NOALLOC_SCRATCH_BYTES
    assert f(FAKE, 16, 8192, 65536, 128, 0, 1, FAKE, 0, None, None, 1e-6, FAKE, None) \
        == _lib.ERR_SCRATCH
