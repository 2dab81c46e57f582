"""The C interface on the host: exports, argument checks and kernel-family choice.

None of these calls reaches the GPU: tg_gemm_plan is pure host code, and
tg_gemm returns before any HIP call when its arguments are invalid or there is
nothing to compute.  Pointers here are made-up integers that are never
dereferenced.
"""
import ctypes
import os
import re

import pytest

import tiled_dense_gemm_tg_amd as tg
from tiled_dense_gemm_tg_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tg_gemm.h")

# made-up, suitably aligned device addresses in disjoint ranges
PA, PB, PC, PBIAS = 0x7F0000000000, 0x7F1000000000, 0x7F2000000000, 0x7F3000000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(tg_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tg.LIBRARY):
        pytest.fail("libtg_gemm.so is not built (run __graft_entry__.build())")
    return tg.load_library()


def test_header_declares_the_interface():
    assert declared_functions() == sorted(tg.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_and_status_strings(lib):
    assert "gfx950" in tg.tg_version()
    assert tg.tg_status_string(tg.TG_OK) == "TG_OK"
    assert tg.tg_status_string(tg.TG_ERR_INVALID_ARG) == "TG_ERR_INVALID_ARG"
    assert tg.tg_status_string(tg.TG_ERR_UNSUPPORTED) == "TG_ERR_UNSUPPORTED"
    assert tg.tg_status_string(tg.TG_ERR_LAUNCH) == "TG_ERR_LAUNCH"
    assert tg.tg_status_string(99) == "TG_UNKNOWN_STATUS"


def plan(M, N, K, dtype=I.F16, A=PA, B=PB, bias=None, epi=I.EPI_NONE, C=PC):
    return tg.tg_gemm_plan(M, N, K, dtype, A, B, bias, epi, C)


@pytest.mark.parametrize("args,status", [
    (dict(M=-1, N=4, K=4), tg.TG_ERR_INVALID_ARG),
    (dict(M=4, N=-1, K=4), tg.TG_ERR_INVALID_ARG),
    (dict(M=4, N=4, K=-1), tg.TG_ERR_INVALID_ARG),
    (dict(M=4, N=4, K=4, dtype=2), tg.TG_ERR_INVALID_ARG),
    (dict(M=4, N=4, K=4, epi=3), tg.TG_ERR_INVALID_ARG),
    (dict(M=4, N=4, K=4, A=None), tg.TG_ERR_INVALID_ARG),
    (dict(M=4, N=4, K=4, B=None), tg.TG_ERR_INVALID_ARG),
    (dict(M=4, N=4, K=4, C=None), tg.TG_ERR_INVALID_ARG),
    (dict(M=4, N=4, K=4, epi=I.EPI_BIAS), tg.TG_ERR_INVALID_ARG),            # bias missing
    (dict(M=4, N=4, K=4, epi=I.EPI_BIAS_GELU_TANH), tg.TG_ERR_INVALID_ARG),
    (dict(M=4, N=4, K=4, bias=PBIAS), tg.TG_ERR_INVALID_ARG),                # bias without epilogue
    (dict(M=4, N=4, K=4, C=PA + 8), tg.TG_ERR_INVALID_ARG),                  # C overlaps A
    (dict(M=4, N=4, K=4, C=PB - 8), tg.TG_ERR_INVALID_ARG),                  # C overlaps B
    (dict(M=4, N=4, K=4, epi=I.EPI_BIAS, bias=PC + 30), tg.TG_ERR_INVALID_ARG),  # bias inside C
    (dict(M=1 << 16, N=1 << 15, K=8), tg.TG_ERR_UNSUPPORTED),              # C has 2^31 elements
    (dict(M=8, N=8, K=(1 << 30) + 8), tg.TG_ERR_UNSUPPORTED),
])
def test_invalid_arguments(lib, args, status):
    st, _ = plan(**args)
    assert st == status
    # tg_gemm rejects them the same way, before any HIP call
    a = dict(dtype=I.F16, A=PA, B=PB, bias=None, epi=I.EPI_NONE, C=PC)
    a.update(args)
    st2 = tg.tg_gemm(a["M"], a["N"], a["K"], a["dtype"], a["A"], a["B"], a["bias"], a["epi"], a["C"], None)
    assert st2 == status


def test_plan_rejects_null_output_pointer(lib):
    assert lib.tg_gemm_plan(4, 4, 4, 0, PA, PB, None, 0, PC, None) == tg.TG_ERR_INVALID_ARG


def test_unknown_path_is_invalid(lib):
    assert tg.tg_gemm_path(7, 4, 4, 4, I.F16, PA, PB, None, I.EPI_NONE, PC, None) == tg.TG_ERR_INVALID_ARG
    assert tg.tg_gemm_path(tg.TG_PATH_NONE, 4, 4, 4, I.F16, PA, PB, None, I.EPI_NONE, PC, None) \
        == tg.TG_ERR_INVALID_ARG


@pytest.mark.parametrize("M,N,K", [(0, 5, 5), (5, 0, 5), (0, 0, 0)])
def test_empty_output_is_a_noop(lib, M, N, K):
    assert plan(M, N, K, A=None, B=None, C=None) == (tg.TG_OK, tg.TG_PATH_NONE)
    # nothing is launched, so this is safe without a GPU
    assert tg.tg_gemm(M, N, K, I.F16, None, None, None, I.EPI_NONE, None, None) == tg.TG_OK


def test_empty_K_allows_null_operands(lib):
    assert plan(80, 64, 0, A=None, B=None, bias=PBIAS, epi=I.EPI_BIAS) == (tg.TG_OK, tg.TG_PATH_TILED)
    assert plan(64, 64, 0, A=None, B=None, bias=PBIAS, epi=I.EPI_BIAS) == (tg.TG_OK, tg.TG_PATH_SKINNY)


@pytest.mark.parametrize("M,N,K,ptrs,path", [
    (16, 11008, 4096, {}, tg.TG_PATH_SKINNY),          # decode shape
    (1, 4, 8, {}, tg.TG_PATH_SKINNY),
    (16, 12, 8, {}, tg.TG_PATH_SKINNY),                 # N % 4 == 0 is enough
    (17, 11008, 4096, {}, tg.TG_PATH_SKINNY),          # two row blocks per workgroup
    (48, 16384, 4096, {}, tg.TG_PATH_SKINNY),          # three, 256 slabs: one round on 256 CUs
    (64, 16384, 4096, {}, tg.TG_PATH_SKINNY),          # four
    (48, 16388, 4096, {}, tg.TG_PATH_TILED),           # a second round of slabs: tiled is faster
    (17, 28672, 4096, {}, tg.TG_PATH_TILED),
    (16, 28672, 4096, {}, tg.TG_PATH_SKINNY),          # one row block: skinny at any width
    (65, 11008, 4096, {}, tg.TG_PATH_TILED),
    (16, 11008, 4100, {}, tg.TG_PATH_TILED),            # K % 8 != 0: not skinny, tiled takes any shape
    (16, 11010, 4096, {}, tg.TG_PATH_TILED),            # N % 4 != 0
    (16, 11008, 4096, {"A": PA + 8}, tg.TG_PATH_TILED),
    (4096, 4096, 4096, {}, tg.TG_PATH_TILED),
    (8192, 8192, 8192, {"bias": PBIAS, "epi": I.EPI_BIAS_GELU_TANH}, tg.TG_PATH_TILED),
    (4000, 4093, 4111, {"bias": PBIAS, "epi": I.EPI_BIAS_GELU_TANH, "dtype": I.BF16}, tg.TG_PATH_TILED),
    (4000, 4096, 4104, {}, tg.TG_PATH_TILED),           # ragged M is fine for the vector path
    (130808, 256, 8192, {}, tg.TG_PATH_TILED),          # 2 (M + 256) K just below 2^31 - 64 Ki
    (130812, 256, 8192, {}, tg.TG_PATH_TILED_GENERIC),  # ... and at it
    (256, 129792, 8192, {}, tg.TG_PATH_TILED),          # 2 (K + 64) (N + 256) just below
    (256, 129800, 8192, {}, tg.TG_PATH_TILED_GENERIC),
    (256, 256, 256, {"C": PC + 8}, tg.TG_PATH_TILED),
    (256, 256, 256, {"B": PB + 2}, tg.TG_PATH_TILED),
    (256, 256, 256, {"bias": PBIAS + 2, "epi": I.EPI_BIAS}, tg.TG_PATH_TILED),
    (256, 257, 255, {"A": PA + 2, "C": PC + 6}, tg.TG_PATH_TILED),
])
def test_kernel_family_choice(lib, M, N, K, ptrs, path):
    assert plan(M, N, K, **ptrs) == (tg.TG_OK, path)


def test_explicit_path_requirements(lib):
    # the skinny family needs M <= 64, K % 8 == 0, N % 4 == 0 and alignment;
    # the tiled family needs operands below its size limit
    assert tg.tg_gemm_path(tg.TG_PATH_SKINNY, 65, 64, 64, I.F16, PA, PB, None, 0, PC, None) == tg.TG_ERR_UNSUPPORTED
    assert tg.tg_gemm_path(tg.TG_PATH_SKINNY, 16, 64, 60, I.F16, PA, PB, None, 0, PC, None) == tg.TG_ERR_UNSUPPORTED
    assert tg.tg_gemm_path(tg.TG_PATH_SKINNY, 16, 64, 64, I.F16, PA + 4, PB, None, 0, PC, None) \
        == tg.TG_ERR_UNSUPPORTED
    assert tg.tg_gemm_path(tg.TG_PATH_TILED, 130812, 256, 8192, I.F16, PA, PB, None, 0, PC, None) \
        == tg.TG_ERR_UNSUPPORTED


def ew(op=tg.TG_EW_BIAS_ADD, M=4, N=8, dtype=I.F16, bias=PBIAS, X=PA, Y=PC):
    return tg.tg_elementwise(op, M, N, dtype, bias, X, Y, None)


@pytest.mark.parametrize("args,status", [
    (dict(M=-1), tg.TG_ERR_INVALID_ARG),
    (dict(N=-1), tg.TG_ERR_INVALID_ARG),
    (dict(op=2), tg.TG_ERR_INVALID_ARG),
    (dict(dtype=2), tg.TG_ERR_INVALID_ARG),
    (dict(bias=None), tg.TG_ERR_INVALID_ARG),                              # add without bias
    (dict(op=tg.TG_EW_GELU_TANH), tg.TG_ERR_INVALID_ARG),                  # GELU with a bias
    (dict(X=None), tg.TG_ERR_INVALID_ARG),
    (dict(Y=None), tg.TG_ERR_INVALID_ARG),
    (dict(Y=PA + 2), tg.TG_ERR_INVALID_ARG),                                # Y overlaps X, not in place
    (dict(Y=PBIAS + 4), tg.TG_ERR_INVALID_ARG),                             # Y overlaps bias
    (dict(M=1 << 16, N=1 << 15), tg.TG_ERR_UNSUPPORTED),                    # 2^31 elements
    (dict(M=0), tg.TG_OK),                                                  # nothing to do
    (dict(N=0, op=tg.TG_EW_GELU_TANH, bias=None), tg.TG_OK),
])
def test_elementwise_argument_checks(lib, args, status):
    assert ew(**args) == status


def test_unfused_checks_arguments_like_tg_gemm(lib):
    assert tg.tg_gemm_unfused(4, 4, 4, I.F16, PA, PB, None, I.EPI_BIAS, PC, None) == tg.TG_ERR_INVALID_ARG
    assert tg.tg_gemm_unfused(4, 4, 4, I.F16, PA, PB, PBIAS, I.EPI_NONE, PC, None) == tg.TG_ERR_INVALID_ARG
    assert tg.tg_gemm_unfused(4, 4, 4, I.F16, PA, PB, None, I.EPI_NONE, PA, None) == tg.TG_ERR_INVALID_ARG
    assert tg.tg_gemm_unfused(0, 4, 4, I.F16, None, None, PBIAS, I.EPI_BIAS, None, None) == tg.TG_OK


def test_w4_packed_size(lib):
    assert tg.tg_w4_packed_bytes(4096, 11008) == 32 * 4096 * 172
    assert tg.tg_w4_packed_bytes(32, 1) == 32 * 32
    assert tg.tg_w4_packed_bytes(0, 5) == 0
    assert tg.tg_w4_packed_bytes(48, 64) == -1          # K % 32 != 0
    assert tg.tg_w4_packed_bytes(-32, 64) == -1


def w4(M=16, N=64, K=128, dtype=I.F16, A=PA, packed=PB, scales=PBIAS + 4096, group=32, bias=None,
       epi=I.EPI_NONE, C=PC):
    return tg.tg_gemm_w4(M, N, K, dtype, A, packed, scales, group, bias, epi, C, None)


@pytest.mark.parametrize("args,status", [
    (dict(M=-1), tg.TG_ERR_INVALID_ARG),
    (dict(dtype=3), tg.TG_ERR_INVALID_ARG),
    (dict(epi=3), tg.TG_ERR_INVALID_ARG),
    (dict(group=48), tg.TG_ERR_INVALID_ARG),
    (dict(group=256), tg.TG_ERR_INVALID_ARG),             # K % group != 0
    (dict(K=100, group=32), tg.TG_ERR_INVALID_ARG),
    (dict(bias=PBIAS), tg.TG_ERR_INVALID_ARG),             # bias with no epilogue
    (dict(epi=I.EPI_BIAS), tg.TG_ERR_INVALID_ARG),         # epilogue without bias
    (dict(A=None), tg.TG_ERR_INVALID_ARG),
    (dict(packed=None), tg.TG_ERR_INVALID_ARG),
    (dict(scales=None), tg.TG_ERR_INVALID_ARG),
    (dict(C=None), tg.TG_ERR_INVALID_ARG),
    (dict(C=PA + 64), tg.TG_ERR_INVALID_ARG),              # C overlaps A
    (dict(C=PB + 64), tg.TG_ERR_INVALID_ARG),              # C overlaps the packed weights
    (dict(M=16 * 65536), tg.TG_ERR_UNSUPPORTED),
    (dict(M=0), tg.TG_OK),
])
def test_w4_argument_checks(lib, args, status):
    assert w4(**args) == status


def test_w4_pack_argument_checks(lib):
    assert tg.tg_w4_pack(48, 64, PA, PB, None) == tg.TG_ERR_INVALID_ARG       # K % 32
    assert tg.tg_w4_pack(64, 64, None, PB, None) == tg.TG_ERR_INVALID_ARG
    assert tg.tg_w4_pack(64, 64, PA, PB + 8, None) == tg.TG_ERR_INVALID_ARG   # packed misaligned
    assert tg.tg_w4_pack(64, 64, PA, PA + 1024, None) == tg.TG_ERR_INVALID_ARG  # overlap
    assert tg.tg_w4_pack(0, 64, None, None, None) == tg.TG_OK


def attn(Bn=1, Sq=256, Sk=256, H=2, Dh=128, dtype=I.F16, Q=PA, K=PB, V=PBIAS, causal=0, scale=0.0, O=PC):
    return tg.tg_attention_fwd(Bn, Sq, Sk, H, Dh, dtype, Q, K, V, causal, scale, O, None)


@pytest.mark.parametrize("args,status", [
    (dict(Bn=-1), tg.TG_ERR_INVALID_ARG),
    (dict(Sk=-1), tg.TG_ERR_INVALID_ARG),
    (dict(dtype=2), tg.TG_ERR_INVALID_ARG),
    (dict(causal=2), tg.TG_ERR_INVALID_ARG),
    (dict(causal=1, Sk=128), tg.TG_ERR_INVALID_ARG),          # causal needs Sq == Sk
    (dict(scale=-1.0), tg.TG_ERR_INVALID_ARG),
    (dict(scale=float("nan")), tg.TG_ERR_INVALID_ARG),
    (dict(scale=float("inf")), tg.TG_ERR_INVALID_ARG),
    (dict(Q=None), tg.TG_ERR_INVALID_ARG),
    (dict(V=None), tg.TG_ERR_INVALID_ARG),
    (dict(O=None), tg.TG_ERR_INVALID_ARG),
    (dict(O=PA + 256), tg.TG_ERR_INVALID_ARG),                # O overlaps Q
    (dict(O=PBIAS + 64), tg.TG_ERR_INVALID_ARG),              # O overlaps V
    (dict(Dh=64), tg.TG_ERR_UNSUPPORTED),
    (dict(H=65536), tg.TG_ERR_UNSUPPORTED),
    (dict(Sq=1 << 30), tg.TG_ERR_UNSUPPORTED),
    (dict(Bn=0), tg.TG_OK),
    (dict(Sq=0), tg.TG_OK),
])
def test_attention_argument_checks(lib, args, status):
    assert attn(**args) == status


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(tg, "_lib", None)
    monkeypatch.setattr(tg, "LIBRARY", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        tg.load_library()


# ------------------------------------------------------------ tile configurations

def test_tiled_entry_point_checks_arguments(lib):
    for bad in (-1, max(tg.TILES_NAMES) + 1, 99):
        assert tg.tg_gemm_tiled(bad, 64, 64, 64, I.F16, PA, PB, None, I.EPI_NONE, PC, None) == tg.TG_ERR_INVALID_ARG
    # raster groups of 1..64 tile rows (0: the library's choice)
    for bad in (-1, 65):
        assert tg.tg_gemm_tiled_grouped(tg.TG_TILES_256x256, bad, 64, 64, 64, I.F16, PA, PB, None, I.EPI_NONE, PC,
                                        None) == tg.TG_ERR_INVALID_ARG
    for ok in (0, 1, 64):
        assert tg.tg_gemm_tiled_grouped(tg.TG_TILES_256x256, ok, 0, 64, 64, I.F16, None, None, None, I.EPI_NONE,
                                        None, None) == tg.TG_OK
    # the tiled family's size limit applies to every configuration
    for cfg in (tg.TG_TILES_AUTO, tg.TG_TILES_128x128):
        assert tg.tg_gemm_tiled(cfg, 130812, 256, 8192, I.F16, PA, PB, None, I.EPI_NONE, PC, None) \
            == tg.TG_ERR_UNSUPPORTED
    # argument rules are tg_gemm's: bias with no epilogue, C overlapping A
    assert tg.tg_gemm_tiled(tg.TG_TILES_256x128, 64, 64, 64, I.F16, PA, PB, PBIAS, I.EPI_NONE, PC, None) \
        == tg.TG_ERR_INVALID_ARG
    assert tg.tg_gemm_tiled(tg.TG_TILES_128x256, 64, 64, 64, I.F16, PA, PB, None, I.EPI_NONE, PA + 64, None) \
        == tg.TG_ERR_INVALID_ARG
    # nothing to compute: a no-op for every configuration, without a GPU
    for cfg in tg.TILES_NAMES:
        assert tg.tg_gemm_tiled(cfg, 0, 64, 64, I.F16, None, None, None, I.EPI_NONE, None, None) == tg.TG_OK


def test_tiles_plan_checks_arguments(lib):
    assert lib.tg_gemm_tiles_plan(64, 64, 64, 256, None) == tg.TG_ERR_INVALID_ARG
    assert tg.tg_gemm_tiles_plan(-1, 64, 64, 256)[0] == tg.TG_ERR_INVALID_ARG
    assert tg.tg_gemm_tiles_plan(64, 64, -1, 256)[0] == tg.TG_ERR_INVALID_ARG


@pytest.mark.parametrize("M,N,K,cfg", [
    (8192, 8192, 8192, tg.TG_TILES_256x256),    # four 256x256 tiles per CU: the most efficient tile
    (4096, 4096, 4096, tg.TG_TILES_256x256),    # exactly one per CU
    (4000, 4093, 4111, tg.TG_TILES_256x256),
    (2048, 2048, 2048, tg.TG_TILES_128x128),    # 64 tiles of 256x256 would leave 3/4 of the CUs idle
    (1024, 1024, 8192, tg.TG_TILES_128x128),
    (1000, 3000, 6000, tg.TG_TILES_128x128),
    (512, 11008, 4096, tg.TG_TILES_256x128_K64),   # 172 tiles of 256x128 or 128x256; the k64 one is fastest
    (17, 11008, 4096, tg.TG_TILES_128x128),     # one row of tiles: the smallest tile wastes least
])
def test_tiles_plan_on_an_mi355x(lib, M, N, K, cfg):
    """The choice on 256 CUs for the measured shape classes."""
    assert tg.tg_gemm_tiles_plan(M, N, K, 256) == (tg.TG_OK, cfg)
    assert tg.tg_gemm_tiles_plan(M, N, K, 0) == (tg.TG_OK, cfg)       # 0: an MI355X's 256 CUs assumed


def test_tiles_plan_follows_the_cu_count(lib):
    # with 4x the CUs the 4096-cube has too few 256x256 tiles; with 1/4 the 2048-cube has enough
    assert tg.tg_gemm_tiles_plan(4096, 4096, 4096, 1024)[1] != tg.TG_TILES_256x256
    assert tg.TILES_AXES[tg.tg_gemm_tiles_plan(2048, 2048, 2048, 64)[1]][:2] == (256, 256)


def test_smoke_cases_are_planned_as_smoke_expects(lib):
    """smoke() asserts the family tg_gemm picks for each of its cases; the
    plan is host logic, so check it here (allocations are at least 256-byte
    aligned, as the made-up pointers are)."""
    import __graft_entry__
    for name, M, N, K, dtype, epi, want, _ in __graft_entry__.smoke_cases():
        assert plan(M, N, K, dtype=dtype, epi=epi, bias=PBIAS if epi else None) == (tg.TG_OK, want), name


# ------------------------------------------------------------ split-K

def test_split_workspace_bytes(lib):
    # counters (4 bytes per 64-column slab, in a region of at least 64 KiB,
    # so the partials start at the same place for every N up to 2^20), then
    # 4 KiB per slab and split
    assert tg.tg_gemm_split_workspace_bytes(4096, 4) == 65536 + 64 * 4 * 4096
    assert tg.tg_gemm_split_workspace_bytes(11008, 2) == 65536 + 172 * 2 * 4096
    assert tg.tg_gemm_split_workspace_bytes(4100, 3) == 65536 + 65 * 3 * 4096
    assert tg.tg_gemm_split_workspace_bytes(2 ** 20 + 64, 2) == 65792 + 16385 * 2 * 4096
    for splits in (0, 1):
        assert tg.tg_gemm_split_workspace_bytes(4096, splits) == 0
    assert tg.tg_gemm_split_workspace_bytes(0, 8) == 0
    # stream-K: counters, then one partial block per (slab, workgroup) pair,
    # for up to 1024 workgroups
    assert tg.tg_gemm_split_workspace_bytes(11008, tg.TG_SPLIT_STREAM_K) == 65536 + (1024 + 172 - 1) * 4096
    assert tg.tg_gemm_split_workspace_bytes(64, tg.TG_SPLIT_STREAM_K) == 65536 + 1024 * 4096
    for N, splits in ((-1, 2), (4096, -2), (4096, 65), (2 ** 30 + 1, 2), (2 ** 30 + 1, tg.TG_SPLIT_STREAM_K)):
        assert tg.tg_gemm_split_workspace_bytes(N, splits) == -1


def test_split_entry_point_checks_arguments(lib):
    ws = 0x7F4000000000
    need = tg.tg_gemm_split_workspace_bytes(4096, 4)

    def call(splits, M=16, N=4096, K=4096, ws=ws, nbytes=need, C=PC, bias=None, epi=I.EPI_NONE):
        return tg.tg_gemm_split(splits, M, N, K, I.F16, PA, PB, bias, epi, C, ws, nbytes, None)

    for bad in (-2, 65, 1000):
        assert call(bad) == tg.TG_ERR_INVALID_ARG
    assert call(4, nbytes=-1) == tg.TG_ERR_INVALID_ARG
    assert call(4, ws=None) == tg.TG_ERR_INVALID_ARG                      # a split needs a workspace
    assert call(4, nbytes=need - 1) == tg.TG_ERR_INVALID_ARG              # too small
    assert call(4, ws=ws + 8) == tg.TG_ERR_INVALID_ARG                    # not 16-byte aligned
    assert call(4, ws=PC + 1024) == tg.TG_ERR_INVALID_ARG                 # overlaps C
    assert call(4, ws=PA) == tg.TG_ERR_INVALID_ARG                        # overlaps A
    assert call(4, ws=PB + 4096) == tg.TG_ERR_INVALID_ARG                 # overlaps B
    assert call(4, ws=PBIAS, bias=PBIAS, epi=I.EPI_BIAS) == tg.TG_ERR_INVALID_ARG
    # tg_gemm's own rules come first
    assert call(4, bias=PBIAS) == tg.TG_ERR_INVALID_ARG                   # bias with no epilogue
    assert call(4, C=PA + 64) == tg.TG_ERR_INVALID_ARG                    # C overlapping A
    # nothing to compute: a no-op whatever the workspace, without a GPU
    assert tg.tg_gemm_split(4, 0, 4096, 4096, I.F16, None, None, None, I.EPI_NONE, None, None, 0, None) == tg.TG_OK


def test_split_plan_checks_arguments(lib):
    st = ctypes.c_int()
    nb = ctypes.c_int64()
    assert lib.tg_gemm_split_plan(16, 4096, 4096, 256, None, ctypes.byref(nb)) == tg.TG_ERR_INVALID_ARG
    assert lib.tg_gemm_split_plan(16, 4096, 4096, 256, ctypes.byref(st), None) == tg.TG_ERR_INVALID_ARG
    for M, N, K in ((-1, 64, 64), (16, -1, 64), (16, 64, -1), (16, 2 ** 30 + 1, 64)):
        assert tg.tg_gemm_split_plan(M, N, K, 256)[0] == tg.TG_ERR_INVALID_ARG
    # off the skinny path, and empty products, never split
    assert tg.tg_gemm_split_plan(17, 4096, 11008, 256) == (tg.TG_OK, 1, 0)
    assert tg.tg_gemm_split_plan(0, 4096, 11008, 256) == (tg.TG_OK, 1, 0)
    assert tg.tg_gemm_split_plan(16, 0, 11008, 256) == (tg.TG_OK, 1, 0)


def _streamk_groups(N, K, cus):
    """Stream-K workgroups: one per CU (256 if unknown), at most 1024, at
    least 16 32-k steps each, at least one."""
    total = -(-N // 64) * -(-K // 32)
    return max(1, min(cus or 256, 1024, total // 16))


def test_split_plan_workspace_matches_its_split_count(lib):
    for M, N, K in ((16, 4096, 11008), (16, 11008, 4096), (1, 2048, 8192), (16, 4096, 256), (8, 64, 65536),
                    (16, 28672, 4096), (16, 8256, 512)):
        for cus in (0, 64, 256, 1024):
            st, splits, nbytes = tg.tg_gemm_split_plan(M, N, K, cus)
            assert st == tg.TG_OK and (1 <= splits <= 64 or splits == tg.TG_SPLIT_STREAM_K)
            if splits == tg.TG_SPLIT_STREAM_K:
                slabs = -(-N // 64)
                groups = _streamk_groups(N, K, cus)
                assert nbytes == 65536 + (groups + slabs - 1) * 4096
                assert nbytes <= tg.tg_gemm_split_workspace_bytes(N, splits)
            else:
                assert nbytes == tg.tg_gemm_split_workspace_bytes(N, splits)
                assert 32 * 16 * splits <= max(K, 32 * 16) + 31       # at least 16 32-k steps per split


@pytest.mark.parametrize("M,N,K,splits", [
    (16, 4096, 11008, 4),     # 64 slabs: four splits fill 256 CUs
    (16, 4096, 4096, 4),
    (16, 1024, 4096, 8),      # 16 slabs: 16 splits would leave 8 steps each; 8 keeps 16
    # 172 slabs: even splits need a second round of workgroups, and stream-K's
    # 86 steps per CU do not pay for its exchange (measured 23.6 against 19.1 us)
    (16, 11008, 4096, 1),
    # long K: stream-K's 231 steps per CU against 344 (47.5 against 55.0 us)
    (16, 11008, 11008, tg.TG_SPLIT_STREAM_K),
    (8, 28672, 4096, 1),      # 448 slabs: 2 rounds of 128 steps, 46.3 us; stream-K 48.3 us
    (16, 16384, 4096, 1),     # 256 slabs: one per CU, nothing to gain
    (16, 4096, 256, 1),       # 8 steps in all: too few to split
    (1, 64, 65536, 64),       # one slab, deep K: capped at 64 splits
])
def test_split_plan_on_an_mi355x(lib, M, N, K, splits):
    st, got, nbytes = tg.tg_gemm_split_plan(M, N, K, 256)
    assert (st, got) == (tg.TG_OK, splits)
    assert tg.tg_gemm_split_plan(M, N, K, 0)[1] == splits              # 0: 256 CUs assumed
    if splits == tg.TG_SPLIT_STREAM_K:
        slabs = -(-N // 64)
        assert nbytes == 65536 + (256 + slabs - 1) * 4096
    else:
        assert nbytes == tg.tg_gemm_split_workspace_bytes(N, splits)


def test_static_split_checks_arguments_before_any_device_work(lib):
    # Invalid split counts and scratch overflows are refused on the host,
    # before the first HIP call, like every other argument error.
    args = (16, 4096, 4096, I.F16, PA, PB, None, I.EPI_NONE, PC, None)
    assert lib.tg_gemm_split_static(-2, *args) == tg.TG_ERR_INVALID_ARG
    assert lib.tg_gemm_split_static(65, *args) == tg.TG_ERR_INVALID_ARG
    # 64 slabs x 32 splits = 2048 partial blocks of 4 KiB: above the 4 MiB scratch
    assert lib.tg_gemm_split_static(32, *args) == tg.TG_ERR_UNSUPPORTED
    # more than 16384 slabs: more counters than the scratch holds
    wide = (16, 16384 * 64 + 64, 4096, I.F16, PA, PB, None, I.EPI_NONE, PC, None)
    assert lib.tg_gemm_split_static(2, *wide) == tg.TG_ERR_UNSUPPORTED
    # stream-K on 256 CUs (none here: 256 assumed) over 800 slabs: 1055 partial blocks
    many = (16, 800 * 64, 4096, I.F16, PA, PB, None, I.EPI_NONE, PC, None)
    assert lib.tg_gemm_split_static(tg.TG_SPLIT_STREAM_K, *many) == tg.TG_ERR_UNSUPPORTED
    # the tg_gemm rules come first
    assert lib.tg_gemm_split_static(4, -1, 4096, 4096, I.F16, PA, PB, None, I.EPI_NONE, PC, None) == \
        tg.TG_ERR_INVALID_ARG
    assert lib.tg_gemm_split_static(4, 16, 0, 4096, I.F16, PA, PB, None, I.EPI_NONE, PC, None) == tg.TG_OK
