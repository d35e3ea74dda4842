"""Host-side checks of the C-ABI library: it loads, exports every entry point
include/bitlinear.h declares, sizes agree with the layout description, and
every argument error is reported before any device work (so these run on a
machine without a GPU)."""

import ctypes as C
import math
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")
LIB = os.path.join(ROOT, "bitlinear_absmean_ternarise_amd", "lib", "libbitlinear.so")

BL_OK, BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_VALUE = 0, -1, -2, -3, -4
BL_ERR_DEVICE, BL_ERR_ARCH, BL_ERR_WORKSPACE, BL_ERR_SCRATCH = -5, -6, -7, -8
MAX_K = 16909320


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|const char \*)\s*(bitlinear_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "bitlinear_build", os.path.join(ROOT, "bitlinear_absmean_ternarise_amd", "build.py"))
        b = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(b)
        b.build()
    L = C.CDLL(LIB)
    i64, p, sz = C.c_int64, C.c_void_p, C.c_size_t
    L.bitlinear_packed_bytes.argtypes = [i64, i64, C.POINTER(sz)]
    L.bitlinear_pack_workspace_bytes.argtypes = [i64, i64, C.POINTER(sz)]
    L.bitlinear_pack_weights.argtypes = [p, i64, i64, C.c_float, p, sz, p, p, p]
    L.bitlinear_quant_act.argtypes = [p, i64, i64, C.c_float, p, p, p]
    L.bitlinear_forward.argtypes = [p, p, i64, i64, p, p, i64, p, p, p]
    L.bitlinear_flip_update.argtypes = [p, p, i64, C.c_int32, p, p, p]
    L.bitlinear_strerror.restype = C.c_char_p
    return L


def test_every_declared_symbol_is_exported(lib):
    syms = declared_symbols()
    assert set(syms) == {"bitlinear_packed_bytes", "bitlinear_pack_workspace_bytes",
                         "bitlinear_pack_weights", "bitlinear_quant_act", "bitlinear_rmsnorm_quant_act",
                         "bitlinear_forward", "bitlinear_pack_binary", "bitlinear_flip_stats",
                         "bitlinear_adamw_step", "bitlinear_pack_transposed", "bitlinear_backward_input",
                         "bitlinear_pack_weights_grouped",
                         "bitlinear_forward_grouped", "bitlinear_flip_update", "bitlinear_strerror",
                         "bitlinear_forward_workspace_bytes", "bitlinear_forward_grouped_ws",
                         "bitlinear_layout_version", "bitlinear_backward_input_grouped",
                         "bitlinear_forward_grouped_noalloc", "bitlinear_quant_forward_grouped",
                         "bitlinear_quant_forward_workspace_bytes", "bitlinear_packed_bytes_b1",
                         "bitlinear_pack_binary_b1", "bitlinear_forward_b1", "bitlinear_forward_b1_grouped",
                         "bitlinear_forward_grouped_dot4", "bitlinear_quant_forward_b1_grouped"}
    for s in syms:
        assert hasattr(lib, s), s


def test_layout_version_and_strerror(lib):
    assert lib.bitlinear_layout_version() == 1
    for st in range(-8, 1):
        msg = lib.bitlinear_strerror(st).decode()
        assert msg and msg != "unknown status"
    assert lib.bitlinear_strerror(-99).decode() == "unknown status"


@pytest.mark.parametrize("N,K", [(1, 1), (16, 64), (17, 65), (512, 256), (3200, 8640), (28672, 8192), (5, MAX_K)])
def test_packed_bytes_match_layout(lib, N, K):
    out = C.c_size_t()
    assert lib.bitlinear_packed_bytes(N, K, C.byref(out)) == BL_OK
    assert out.value == math.ceil(N / 16) * math.ceil(K / 64) * 256
    assert out.value == oracle.packed_bytes(N, K)
    assert lib.bitlinear_pack_workspace_bytes(N, K, C.byref(out)) == BL_OK
    assert out.value >= 8


def test_size_queries_reject_bad_shapes(lib):
    out = C.c_size_t()
    for (N, K) in [(0, 64), (16, 0), (-1, 64), (16, MAX_K + 1)]:
        assert lib.bitlinear_packed_bytes(N, K, C.byref(out)) == BL_ERR_SHAPE
        assert lib.bitlinear_pack_workspace_bytes(N, K, C.byref(out)) == BL_ERR_SHAPE
    assert lib.bitlinear_packed_bytes(16, 64, None) == BL_ERR_NULL


# Fake device addresses: never dereferenced, because every call below fails
# validation on the host before touching the device.
A = C.c_void_p(1 << 20)          # 16-byte aligned
A2 = C.c_void_p((1 << 20) + 4096)
U = C.c_void_p((1 << 20) + 4)    # misaligned


def test_pack_errors(lib):
    f = lib.bitlinear_pack_weights
    assert f(None, 16, 64, 1e-5, A, 64, A, A, None) == BL_ERR_NULL
    assert f(A, 16, 64, 1e-5, A, 64, None, A, None) == BL_ERR_NULL
    assert f(A, 16, 64, 1e-5, A, 64, A, None, None) == BL_ERR_NULL
    assert f(A, 0, 64, 1e-5, A, 64, A, A, None) == BL_ERR_SHAPE
    assert f(A, 16, MAX_K + 1, 1e-5, A, 64, A, A, None) == BL_ERR_SHAPE
    assert f(A, 16, 64, -1.0, A, 64, A, A, None) == BL_ERR_VALUE
    assert f(A, 16, 64, float("nan"), A, 64, A, A, None) == BL_ERR_VALUE
    assert f(A, 16, 64, float("inf"), A, 64, A, A, None) == BL_ERR_VALUE
    assert f(A, 16, 64, 1e-5, None, 64, A, A, None) == BL_ERR_WORKSPACE
    assert f(A, 16, 64, 1e-5, A, 0, A, A, None) == BL_ERR_WORKSPACE
    assert f(U, 16, 64, 1e-5, A, 64, A, A, None) == BL_ERR_ALIGN
    assert f(A, 16, 64, 1e-5, A, 64, U, A, None) == BL_ERR_ALIGN


def test_quant_errors(lib):
    f = lib.bitlinear_quant_act
    assert f(None, 4, 64, 1e-5, A, A, None) == BL_ERR_NULL
    assert f(A, 4, 64, 1e-5, None, A, None) == BL_ERR_NULL
    assert f(A, -1, 64, 1e-5, A, A, None) == BL_ERR_SHAPE
    assert f(A, 4, 0, 1e-5, A, A, None) == BL_ERR_SHAPE
    assert f(A, 4, 64, 0.0, A, A, None) == BL_ERR_VALUE
    assert f(A, 4, 64, -1e-5, A, A, None) == BL_ERR_VALUE
    assert f(A, 4, 64, float("nan"), A, A, None) == BL_ERR_VALUE
    assert f(U, 4, 64, 1e-5, A, A, None) == BL_ERR_ALIGN
    assert f(A, 4, 64, 1e-5, A, U, None) == BL_ERR_ALIGN
    # no tokens: nothing to do, no pointer needed
    assert f(None, 0, 64, 1e-5, None, None, None) == BL_OK


def test_rmsnorm_quant_errors(lib):
    f = lib.bitlinear_rmsnorm_quant_act
    f.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int64, C.c_float, C.c_float, C.c_void_p, C.c_void_p,
                  C.c_void_p]
    assert f(None, None, 4, 64, 1e-6, 1e-5, A, A2, None) == BL_ERR_NULL
    assert f(A, None, 4, 64, 1e-6, 1e-5, None, A2, None) == BL_ERR_NULL
    assert f(A, None, -1, 64, 1e-6, 1e-5, A, A2, None) == BL_ERR_SHAPE
    assert f(A, None, 4, 0, 1e-6, 1e-5, A, A2, None) == BL_ERR_SHAPE
    assert f(A, None, 4, 64, -1e-6, 1e-5, A, A2, None) == BL_ERR_VALUE
    assert f(A, None, 4, 64, float("nan"), 1e-5, A, A2, None) == BL_ERR_VALUE
    assert f(A, None, 4, 64, 1e-6, 0.0, A, A2, None) == BL_ERR_VALUE
    assert f(U, None, 4, 64, 1e-6, 1e-5, A, A2, None) == BL_ERR_ALIGN
    assert f(A, U, 4, 64, 1e-6, 1e-5, A, A2, None) == BL_ERR_ALIGN  # misaligned gain
    assert f(None, None, 0, 64, 0.0, 1e-5, None, None, None) == BL_OK


def test_forward_errors(lib):
    f = lib.bitlinear_forward
    assert f(None, A, 16, 64, A, A, 4, A, None, None) == BL_ERR_NULL
    assert f(A, A, 16, 64, A, A, 4, None, None, None) == BL_ERR_NULL
    assert f(A, A, 0, 64, A, A, 4, A, None, None) == BL_ERR_SHAPE
    assert f(A, A, 16, MAX_K + 1, A, A, 4, A, None, None) == BL_ERR_SHAPE
    assert f(A, A, 16, 64, A, A, -3, A, None, None) == BL_ERR_SHAPE
    assert f(A, A, 16, 64, U, A, 4, A, None, None) == BL_ERR_ALIGN
    assert f(A, A, 16, 64, A, A, 4, A, U, None) == BL_ERR_ALIGN
    assert f(None, None, 16, 64, None, None, 0, None, None, None) == BL_OK


class FwdArgs(C.Structure):
    _fields_ = [("packed", C.c_void_p), ("gamma", C.c_void_p), ("N", C.c_int64), ("K", C.c_int64),
                ("xq", C.c_void_p), ("x_scale", C.c_void_p), ("M", C.c_int64), ("y", C.c_void_p),
                ("acc", C.c_void_p)]


def test_forward_grouped_errors(lib):
    f = lib.bitlinear_forward_grouped
    f.argtypes = [C.POINTER(FwdArgs), C.c_int, C.c_void_p]
    good = FwdArgs(A.value, A.value, 16, 64, A.value, A.value, 4, A2.value, None)
    arr = (FwdArgs * 9)(*([good] * 9))
    assert f(None, 1, None) == BL_ERR_NULL
    assert f(arr, 0, None) == BL_ERR_SHAPE
    assert f(arr, 9, None) == BL_ERR_SHAPE  # more than BITLINEAR_MAX_GROUP
    bad = (FwdArgs * 2)(good, FwdArgs(A.value, A.value, 16, 64, A.value, A.value, 4, None, None))
    assert f(bad, 2, None) == BL_ERR_NULL   # second entry lacks y
    bad = (FwdArgs * 2)(good, FwdArgs(A.value, A.value, 0, 64, A.value, A.value, 4, A2.value, None))
    assert f(bad, 2, None) == BL_ERR_SHAPE
    bad = (FwdArgs * 2)(good, FwdArgs(A.value, A.value, 16, 64, U.value, A.value, 4, A2.value, None))
    assert f(bad, 2, None) == BL_ERR_ALIGN
    empty = (FwdArgs * 1)(FwdArgs(None, None, 16, 64, None, None, 0, None, None))
    # an entry with no tokens needs no pointers; on a machine without a GPU the
    # device check still comes first
    assert f(empty, 1, None) in (BL_OK, BL_ERR_DEVICE)


def split_bytes(entries):
    """The workspace the decode-batch GEMM needs for entries (M, N, K),
    restated from its rule: by the largest M, 32 x 256 tiles (14..32 tokens)
    or 64 x 128 tiles (33..64); runs S = 256 // tiles over all entries; at
    14..32 tokens the path is taken only with S >= 2 and every entry >= 64
    groups of 256 columns long; per entry at most one run per 4 groups; one
    int32 [M][N] per run of an entry cut into several, each entry's block
    256-byte aligned."""
    max_m = max(M for M, _, _ in entries)
    if max_m < 14 or max_m > 64 or any(K % 16 for _, _, K in entries):
        return 0
    bm, bn = (32, 256) if max_m <= 32 else (64, 128)
    tiles = sum(-(-M // bm) * -(-N // bn) for M, N, _ in entries)
    S = 256 // tiles
    ngs = [-(-K // 256) for _, _, K in entries]
    if bm == 32 and (S < 2 or min(ngs) < 64):
        return 0
    total = 0
    for (M, N, K), NG in zip(entries, ngs):
        si = 1 if S < 1 else min(S, max(1, NG // 4))
        gps = -(-NG // si)
        runs = -(-NG // gps)
        total += 0 if runs == 1 else -(-(runs * M * N * 4) // 256) * 256
    return total


@pytest.mark.parametrize("M,N,K", [(64, 8192, 28672), (64, 8192, 8192), (17, 1024, 8192), (64, 1000, 4160),
                                   (16, 8192, 8192), (65, 8192, 8192), (64, 57344, 8192), (33, 96, 200),
                                   (40, 1536, 512), (32, 8192, 28672), (17, 2100, 16448), (20, 1024, 8192),
                                   (33, 4096, 4104), (16, 8192, 28672), (14, 2100, 16448), (13, 8192, 28672)])
def test_forward_workspace_bytes(lib, M, N, K):
    f = lib.bitlinear_forward_workspace_bytes
    f.argtypes = [C.POINTER(FwdArgs), C.c_int, C.POINTER(C.c_size_t)]
    arr = (FwdArgs * 1)(FwdArgs(A.value, A.value, N, K, A.value, A.value, M, A2.value, None))
    out = C.c_size_t(123)
    assert f(arr, 1, C.byref(out)) == BL_OK
    assert out.value == split_bytes([(M, N, K)])


def test_forward_workspace_threshold():
    # the 70B down projection (8192 x 28672): 32 tiles, 8 runs of 14 groups
    # from 14 tokens up; the decode kernel below that
    assert split_bytes([(16, 8192, 28672)]) == 8 * 16 * 8192 * 4
    assert split_bytes([(14, 8192, 28672)]) == 8 * 14 * 8192 * 4
    assert split_bytes([(13, 8192, 28672)]) == 0


def test_forward_workspace_errors(lib):
    q = lib.bitlinear_forward_workspace_bytes
    q.argtypes = [C.POINTER(FwdArgs), C.c_int, C.POINTER(C.c_size_t)]
    f = lib.bitlinear_forward_grouped_ws
    f.argtypes = [C.POINTER(FwdArgs), C.c_int, C.c_void_p, C.c_size_t, C.c_void_p]
    good = FwdArgs(A.value, A.value, 8192, 28672, A.value, A.value, 64, A2.value, None)
    arr = (FwdArgs * 2)(good, FwdArgs(A.value, A.value, 8192, 28672, A.value, A.value, 64, A.value, None))
    out = C.c_size_t(0)
    assert q(arr, 2, None) == BL_ERR_NULL
    assert q(None, 1, C.byref(out)) == BL_ERR_NULL
    assert q(arr, 0, C.byref(out)) == BL_ERR_SHAPE
    bad = (FwdArgs * 1)(FwdArgs(A.value, A.value, 16, 64, U.value, A.value, 4, A2.value, None))
    assert q(bad, 1, C.byref(out)) == BL_ERR_ALIGN
    assert q(arr, 2, C.byref(out)) == BL_OK
    need = out.value
    assert need == split_bytes([(64, 8192, 28672)] * 2) == 2 * 2 * 64 * 8192 * 4
    # every error comes before any device work
    assert f(arr, 2, A.value, need - 1, None) == BL_ERR_WORKSPACE
    assert f(arr, 2, U.value, need, None) == BL_ERR_ALIGN
    assert f(bad, 1, A.value, need, None) == BL_ERR_ALIGN
    assert f(None, 1, A.value, need, None) == BL_ERR_NULL
    # no workspace needed: a NULL workspace is fine (then it is the plain grouped call)
    small = (FwdArgs * 1)(FwdArgs(A.value, A.value, 16, 64, A.value, A.value, 4, A2.value, None))
    assert q(small, 1, C.byref(out)) == BL_OK and out.value == 0


def test_pack_binary_errors(lib):
    f = lib.bitlinear_pack_binary
    f.argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p, C.c_void_p,
                  C.c_void_p]
    assert f(None, 16, 64, A, 64, A, A2, A2, None) == BL_ERR_NULL
    assert f(A, 16, 64, A, 64, A, A2, None, None) == BL_ERR_NULL  # alpha is an output
    assert f(A, 0, 64, A, 64, A, A2, A2, None) == BL_ERR_SHAPE
    assert f(A, 16, 64, None, 64, A, A2, A2, None) == BL_ERR_WORKSPACE
    assert f(A, 16, 64, A, 0, A, A2, A2, None) == BL_ERR_WORKSPACE
    assert f(A, 16, 64, A, 64, A, A2, U, None) == BL_ERR_ALIGN


B1_MAX_K = 262080


@pytest.mark.parametrize("N,K", [(1, 64), (16, 64), (17, 128), (33, 320), (3200, 8640), (28672, 8192),
                                 (8192, 28672), (5, B1_MAX_K)])
def test_packed_bytes_b1_match_layout(lib, N, K):
    f = lib.bitlinear_packed_bytes_b1
    f.argtypes = [C.c_int64, C.c_int64, C.POINTER(C.c_size_t)]
    out = C.c_size_t()
    assert f(N, K, C.byref(out)) == BL_OK
    assert out.value == math.ceil(N / 16) * math.ceil(K / 128) * 256 == oracle.packed_bytes_b1(N, K)


def test_b1_errors(lib):
    sz = lib.bitlinear_packed_bytes_b1
    sz.argtypes = [C.c_int64, C.c_int64, C.POINTER(C.c_size_t)]
    out = C.c_size_t()
    for (N, K) in [(0, 64), (16, 0), (16, 96), (16, 65), (16, B1_MAX_K + 64), (1 << 20, 1 << 17)]:
        assert sz(N, K, C.byref(out)) == BL_ERR_SHAPE, (N, K)  # K % 64, K limit, 2 GB of codes
    assert sz(16, 64, None) == BL_ERR_NULL
    pk = lib.bitlinear_pack_binary_b1
    pk.argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p, C.c_void_p,
                   C.c_void_p]
    assert pk(None, 16, 64, A, 64, A, A2, A2, None) == BL_ERR_NULL
    assert pk(A, 16, 64, A, 64, A, A2, None, None) == BL_ERR_NULL
    assert pk(A, 16, 96, A, 64, A, A2, A2, None) == BL_ERR_SHAPE
    assert pk(A, 16, 64, None, 64, A, A2, A2, None) == BL_ERR_WORKSPACE
    assert pk(A, 16, 64, A, 0, A, A2, A2, None) == BL_ERR_WORKSPACE
    assert pk(A, 16, 64, A, 64, U, A2, A2, None) == BL_ERR_ALIGN
    fw = lib.bitlinear_forward_b1
    fw.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p,
                   C.c_void_p, C.c_void_p]
    assert fw(None, A, 16, 64, A, A, 4, A, None, None) == BL_ERR_NULL
    assert fw(A, A, 16, 64, A, A, 4, None, None, None) == BL_ERR_NULL
    assert fw(A, A, 16, 80, A, A, 4, A, None, None) == BL_ERR_SHAPE
    assert fw(A, A, 16, B1_MAX_K + 64, A, A, 4, A, None, None) == BL_ERR_SHAPE
    assert fw(A, A, 16, 64, A, A, -1, A, None, None) == BL_ERR_SHAPE
    assert fw(A, A, 16, 64, U, A, 4, A, None, None) == BL_ERR_ALIGN
    assert fw(A, A, 16, 64, A, A, 4, A, U, None) == BL_ERR_ALIGN
    assert fw(None, None, 16, 64, None, None, 0, None, None, None) == BL_OK
    assert fw(None, None, 16, 96, None, None, 0, None, None, None) == BL_ERR_SHAPE
    assert fw(A, A, 1 << 20, 64, A, A, (1 << 31) - 16, A, None, None) == BL_ERR_SHAPE  # grid past 2^31
    g = lib.bitlinear_forward_b1_grouped
    g.argtypes = [C.POINTER(FwdArgs), C.c_int, C.c_void_p]
    ok = FwdArgs(A.value, A.value, 16, 64, A.value, A.value, 4, A2.value, None)
    assert g(None, 1, None) == BL_ERR_NULL
    assert g((FwdArgs * 1)(ok), 0, None) == BL_ERR_SHAPE
    assert g((FwdArgs * 9)(*([ok] * 9)), 9, None) == BL_ERR_SHAPE
    bad_k = FwdArgs(A.value, A.value, 16, 192 + 32, A.value, A.value, 4, A2.value, None)
    assert g((FwdArgs * 2)(ok, bad_k), 2, None) == BL_ERR_SHAPE
    bad_y = FwdArgs(A.value, A.value, 16, 64, A.value, A.value, 4, U.value, None)
    assert g((FwdArgs * 2)(ok, bad_y), 2, None) == BL_ERR_ALIGN
    no_y = FwdArgs(A.value, A.value, 16, 64, A.value, A.value, 4, None, None)
    assert g((FwdArgs * 2)(ok, no_y), 2, None) == BL_ERR_NULL


def test_quant_forward_b1_errors(lib):
    f = lib.bitlinear_quant_forward_b1_grouped
    f.argtypes = [C.POINTER(QFwdArgs), C.c_int, C.c_float, C.c_void_p]
    ok = QFwdArgs(A.value, A.value, 64, 64, A.value, 4, A2.value, A2.value, A2.value, None)
    assert f(None, 1, 1e-5, None) == BL_ERR_NULL
    assert f((QFwdArgs * 1)(ok), 0, 1e-5, None) == BL_ERR_SHAPE
    assert f((QFwdArgs * 1)(ok), 1, 0.0, None) == BL_ERR_VALUE
    assert f((QFwdArgs * 1)(ok), 1, float("nan"), None) == BL_ERR_VALUE
    bad_k = QFwdArgs(A.value, A.value, 64, 96, A.value, 4, A2.value, A2.value, A2.value, None)
    assert f((QFwdArgs * 2)(ok, bad_k), 2, 1e-5, None) == BL_ERR_SHAPE  # K % 64: no b1 layout
    big_k = QFwdArgs(A.value, A.value, 64, 262144, A.value, 1, A2.value, A2.value, A2.value, None)
    assert f((QFwdArgs * 1)(big_k), 1, 1e-5, None) == BL_ERR_SHAPE
    no_y = QFwdArgs(A.value, A.value, 64, 64, A.value, 4, A2.value, A2.value, None, None)
    assert f((QFwdArgs * 2)(ok, no_y), 2, 1e-5, None) == BL_ERR_NULL
    mis = QFwdArgs(A.value, A.value, 64, 64, U.value, 4, A2.value, A2.value, A2.value, None)
    assert f((QFwdArgs * 2)(ok, mis), 2, 1e-5, None) == BL_ERR_ALIGN
    empty = QFwdArgs(None, None, 64, 64, None, 0, None, None, None, None)
    assert f((QFwdArgs * 1)(empty), 1, 1e-5, None) == BL_OK


def test_forward_dot4_errors(lib):
    g = lib.bitlinear_forward_grouped_dot4
    g.argtypes = [C.POINTER(FwdArgs), C.c_int, C.c_void_p]
    ok = FwdArgs(A.value, A.value, 16, 64, A.value, A.value, 4, A2.value, None)
    assert g(None, 1, None) == BL_ERR_NULL
    assert g((FwdArgs * 1)(ok), 0, None) == BL_ERR_SHAPE
    assert g((FwdArgs * 9)(*([ok] * 9)), 9, None) == BL_ERR_SHAPE
    for bad in (FwdArgs(A.value, A.value, 16, 64, A.value, A.value, 5, A2.value, None),  # more than 4 tokens
                FwdArgs(A.value, A.value, 16, 72, A.value, A.value, 1, A2.value, None),  # K % 16
                FwdArgs(A.value, A.value, 16, 262144, A.value, A.value, 1, A2.value, None),  # K above the x64 sums
                FwdArgs(A.value, A.value, 0, 64, A.value, A.value, 1, A2.value, None)):
        assert g((FwdArgs * 2)(ok, bad), 2, None) == BL_ERR_SHAPE
    assert g((FwdArgs * 2)(ok, FwdArgs(A.value, A.value, 16, 64, U.value, A.value, 1, A2.value, None)), 2,
             None) == BL_ERR_ALIGN
    assert g((FwdArgs * 2)(ok, FwdArgs(A.value, None, 16, 64, A.value, A.value, 1, A2.value, None)), 2,
             None) == BL_ERR_NULL


def test_flip_stats_errors(lib):
    f = lib.bitlinear_flip_stats
    f.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p]
    assert f(None, A, 8, 10, A, A2, None) == BL_ERR_NULL
    assert f(A, A, -1, 10, A, A2, None) == BL_ERR_SHAPE
    assert f(A, A, 8, 0, A, A2, None) == BL_ERR_VALUE
    assert f(A, A, 8, 32768, A, A2, None) == BL_ERR_VALUE
    assert f(A, A, 8, 10, U, A2, None) == BL_ERR_ALIGN
    assert f(None, None, 0, 10, None, None, None) == BL_OK


def test_adamw_errors(lib):
    f = lib.bitlinear_adamw_step
    d = C.c_double
    f.argtypes = [C.c_void_p] * 4 + [C.c_int64, C.c_int32, d, d, d, d, d, C.c_void_p, C.c_void_p, C.c_void_p]
    ok = (1e-3, 0.9, 0.999, 1e-8, 0.1)
    assert f(None, A, A, A, 8, 1, *ok, None, None, None) == BL_ERR_NULL
    assert f(A, A, A, A, -1, 1, *ok, None, None, None) == BL_ERR_SHAPE
    assert f(A, A, A, A, 8, 0, *ok, None, None, None) == BL_ERR_VALUE
    assert f(A, A, A, A, 8, 1, 1e-3, 1.0, 0.999, 1e-8, 0.1, None, None, None) == BL_ERR_VALUE
    assert f(A, A, A, A, 8, 1, -1e-3, 0.9, 0.999, 1e-8, 0.1, None, None, None) == BL_ERR_VALUE
    assert f(A, A, A, A, 8, 1, float("nan"), 0.9, 0.999, 1e-8, 0.1, None, None, None) == BL_ERR_VALUE
    assert f(A, A, A, A, 8, 1, *ok, A, None, None) == BL_ERR_NULL        # one counter without the other
    assert f(A, A, A, A, 8, 40000, *ok, A, A2, None) == BL_ERR_VALUE     # step beyond int16 while tracking
    assert f(A, U, A, A, 8, 1, *ok, None, None, None) == BL_ERR_ALIGN
    assert f(None, None, None, None, 0, 1, *ok, None, None, None) == BL_OK


class PackArgs(C.Structure):
    _fields_ = [("W", C.c_void_p), ("N", C.c_int64), ("K", C.c_int64), ("eps", C.c_float),
                ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t), ("packed", C.c_void_p),
                ("gamma", C.c_void_p), ("packed_t", C.c_void_p)]


def test_pack_grouped_errors(lib):
    f = lib.bitlinear_pack_weights_grouped
    f.argtypes = [C.POINTER(PackArgs), C.c_int, C.c_void_p]
    big = 1 << 20

    def args(n, **kw):
        arr = (PackArgs * n)()
        for i in range(n):
            d = dict(W=big, N=16, K=64, eps=1e-5, workspace=big, workspace_bytes=1 << 16, packed=big, gamma=big)
            d.update(kw if i == n - 1 else {})
            arr[i] = PackArgs(**d)
        return arr
    assert f(None, 1, None) == BL_ERR_NULL
    assert f(args(1), 0, None) == BL_ERR_SHAPE
    assert f(args(65), 65, None) == BL_ERR_SHAPE
    assert f(args(3, W=None), 3, None) == BL_ERR_NULL          # the last entry is bad: nothing runs
    assert f(args(2, N=0), 2, None) == BL_ERR_SHAPE
    assert f(args(2, eps=-1.0), 2, None) == BL_ERR_VALUE
    assert f(args(2, workspace_bytes=4), 2, None) == BL_ERR_WORKSPACE
    assert f(args(2, workspace=None), 2, None) == BL_ERR_WORKSPACE
    assert f(args(2, packed=big + 4), 2, None) == BL_ERR_ALIGN
    assert f(args(2, packed_t=big + 8), 2, None) == BL_ERR_ALIGN


def test_backward_errors(lib):
    pt = lib.bitlinear_pack_transposed
    pt.argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_void_p]
    assert pt(None, 16, 64, A, None) == BL_ERR_NULL
    assert pt(A, 0, 64, A, None) == BL_ERR_SHAPE
    assert pt(A, 16, MAX_K + 1, A, None) == BL_ERR_SHAPE
    assert pt(A, 16, 64, U, None) == BL_ERR_ALIGN
    f = lib.bitlinear_backward_input
    f.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_int64, C.c_void_p, C.c_int,
                  C.c_void_p]
    assert f(None, A, 64, 32, A, 4, A, 0, None) == BL_ERR_NULL
    assert f(A, A, 0, 32, A, 4, A, 0, None) == BL_ERR_SHAPE
    assert f(A, A, 60, 32, A, 4, A, 0, None) == BL_ERR_SHAPE        # N % 8 != 0
    assert f(A, A, 64, 32, A, -1, A, 0, None) == BL_ERR_SHAPE
    assert f(A, A, 1 << 20, 32, A, 1 << 10, A, 0, None) == BL_ERR_SHAPE  # dy of 2 GB
    assert f(A, A, 64, 32, U, 4, A, 0, None) == BL_ERR_ALIGN
    assert f(None, None, 64, 32, None, 0, None, 0, None) == BL_OK    # M = 0: nothing to do


class BackwardArgs(C.Structure):
    _fields_ = [("packed_t", C.c_void_p), ("gamma", C.c_void_p), ("N", C.c_int64), ("dy", C.c_void_p)]


def test_backward_input_grouped_errors(lib):
    f = lib.bitlinear_backward_input_grouped
    f.argtypes = [C.POINTER(BackwardArgs), C.c_int, C.c_int64, C.c_int64, C.c_void_p, C.c_int, C.c_void_p]

    def args(*rows):
        arr = (BackwardArgs * max(len(rows), 5))()
        for i, r in enumerate(rows):
            arr[i] = BackwardArgs(*r)
        return arr
    good = (A, A, 64, A)
    assert f(None, 1, 32, 4, A, 0, None) == BL_ERR_NULL
    assert f(args(good), 0, 32, 4, A, 0, None) == BL_ERR_SHAPE
    assert f(args(good, good, good, good, good), 5, 32, 4, A, 0, None) == BL_ERR_SHAPE  # above the entry limit
    assert f(args(good), 1, 0, 4, A, 0, None) == BL_ERR_SHAPE
    assert f(args(good), 1, MAX_K + 1, 4, A, 0, None) == BL_ERR_SHAPE
    assert f(args(good), 1, 32, -1, A, 0, None) == BL_ERR_SHAPE
    assert f(args(good, (A, A, 60, A)), 2, 32, 4, A, 0, None) == BL_ERR_SHAPE      # N % 8 != 0
    assert f(args(good, (A, A, 0, A)), 2, 32, 4, A, 0, None) == BL_ERR_SHAPE
    assert f(args(good, (A, A, 1 << 20, A)), 2, 32, 1 << 10, A, 0, None) == BL_ERR_SHAPE  # dy of 2 GB
    assert f(args(good), 1, 32, 4, None, 0, None) == BL_ERR_NULL
    assert f(args(good, (A, None, 64, A)), 2, 32, 4, A, 0, None) == BL_ERR_NULL
    assert f(args(good), 1, 32, 4, U, 0, None) == BL_ERR_ALIGN
    assert f(args(good, (A, A, 64, U)), 2, 32, 4, A, 0, None) == BL_ERR_ALIGN
    # M = 0: nothing to do, and no pointer is looked at
    assert f(args((None, None, 64, None)), 1, 32, 0, None, 0, None) == BL_OK


def test_flip_errors(lib):
    f = lib.bitlinear_flip_update
    assert f(None, A, 8, 5, A, A, None) == BL_ERR_NULL
    assert f(A, A, -1, 5, A, A, None) == BL_ERR_SHAPE
    assert f(A, A, 8, 0, A, A, None) == BL_ERR_VALUE
    assert f(A, A, 8, 32768, A, A, None) == BL_ERR_VALUE
    assert f(A, A, 8, 5, A, U, None) == BL_ERR_ALIGN
    assert f(None, None, 0, 5, None, None, None) == BL_OK


def _device_may_be_present():
    """True unless the HIP runtime itself says there is no device.  Decided
    without torch (a CPU-only torch on a GPU host would say "no GPU"): the
    kernel driver's node first, then hipGetDeviceCount from the runtime the
    library links."""
    if os.path.exists("/dev/kfd"):
        return True
    try:
        hip = C.CDLL("libamdhip64.so")
    except OSError:
        try:
            hip = C.CDLL("/opt/rocm/lib/libamdhip64.so")
        except OSError:
            return True  # cannot tell: assume a device
    n = C.c_int(0)
    rc = hip.hipGetDeviceCount(C.byref(n))
    return rc == 0 and n.value > 0


SCRATCH_BYTES = 9437184  # BITLINEAR_SCRATCH_BYTES


def test_header_scratch_size():
    assert re.search(r"#define BITLINEAR_SCRATCH_BYTES (\d+)", open(HEADER).read()).group(1) == str(SCRATCH_BYTES)


def test_no_plan_needs_more_than_the_fixed_scratch(lib):
    # The split-K plan (decode batches of 14..64 tokens) sizes its partial
    # sums by tiles x runs <= 256; sweep token counts, widths, depths and
    # group sizes: no plan needs more than 8 MiB + 2 KiB, under the scratch.
    q = lib.bitlinear_forward_workspace_bytes
    q.argtypes = [C.POINTER(FwdArgs), C.c_int, C.POINTER(C.c_size_t)]
    worst = 0
    out = C.c_size_t(0)
    for M in (14, 16, 17, 24, 31, 32, 33, 48, 63, 64):
        for N in (16, 128, 1000, 1024, 4096, 8192, 8200, 28672, 65536):
            for K in (256, 4096, 8192, 16384, 16400, 28672, 65536):
                for count in (1, 2, 3, 8):
                    arr = (FwdArgs * count)(*[FwdArgs(A.value, A.value, N, K, A.value, A.value, M, A2.value, None)
                                              for _ in range(count)])
                    assert q(arr, count, C.byref(out)) == BL_OK
                    worst = max(worst, out.value)
    assert 0 < worst <= 8 * 2 ** 20 + 2048 <= SCRATCH_BYTES


def test_forward_noalloc_errors(lib):
    f = lib.bitlinear_forward_grouped_noalloc
    f.argtypes = [C.POINTER(FwdArgs), C.c_int, C.c_void_p]
    good = FwdArgs(A.value, A.value, 8192, 28672, A.value, A.value, 64, A2.value, None)
    assert f(None, 1, None) == BL_ERR_NULL
    assert f((FwdArgs * 1)(good), 0, None) == BL_ERR_SHAPE
    assert f((FwdArgs * 9)(*([good] * 9)), 9, None) == BL_ERR_SHAPE
    assert f((FwdArgs * 1)(FwdArgs(A.value, A.value, 8192, 0, A.value, A.value, 64, A2.value, None)), 1, None) == \
        BL_ERR_SHAPE
    assert f((FwdArgs * 1)(FwdArgs(A.value, A.value, 16, 64, U.value, A.value, 4, A2.value, None)), 1, None) == \
        BL_ERR_ALIGN
    assert f((FwdArgs * 1)(FwdArgs(A.value, None, 16, 64, A.value, A.value, 4, A2.value, None)), 1, None) == \
        BL_ERR_NULL


class QFwdArgs(C.Structure):
    _fields_ = [("packed", C.c_void_p), ("gamma", C.c_void_p), ("N", C.c_int64), ("K", C.c_int64),
                ("x", C.c_void_p), ("M", C.c_int64), ("xq", C.c_void_p), ("x_scale", C.c_void_p),
                ("y", C.c_void_p), ("acc", C.c_void_p)]


def test_quant_forward_errors(lib):
    g = lib.bitlinear_quant_forward_grouped
    g.argtypes = [C.POINTER(QFwdArgs), C.c_int, C.c_float, C.c_void_p, C.c_size_t, C.c_void_p]

    def f(arr, count, eps, stream, ws=None, wsb=0):
        return g(arr, count, eps, ws, wsb, stream)

    def one(**kw):
        d = dict(packed=A.value, gamma=A.value, N=64, K=64, x=A.value, M=4, xq=A2.value, x_scale=A2.value,
                 y=A2.value, acc=None)
        d.update(kw)
        return (QFwdArgs * 1)(QFwdArgs(**d))

    assert f(None, 1, 1e-5, None) == BL_ERR_NULL
    assert f(one(), 0, 1e-5, None) == BL_ERR_SHAPE
    assert f((QFwdArgs * 9)(*([one()[0]] * 9)), 9, 1e-5, None) == BL_ERR_SHAPE
    assert f(one(), 1, 0.0, None) == BL_ERR_VALUE
    assert f(one(), 1, float("nan"), None) == BL_ERR_VALUE
    assert f(one(K=0), 1, 1e-5, None) == BL_ERR_SHAPE
    assert f(one(K=MAX_K + 1), 1, 1e-5, None) == BL_ERR_SHAPE
    assert f(one(M=-1), 1, 1e-5, None) == BL_ERR_SHAPE
    for k in ("packed", "gamma", "x", "xq", "x_scale", "y"):
        assert f(one(**{k: None}), 1, 1e-5, None) == BL_ERR_NULL, k
        assert f(one(**{k: U.value}), 1, 1e-5, None) == BL_ERR_ALIGN, k
    assert f(one(acc=U.value), 1, 1e-5, None) == BL_ERR_ALIGN
    # M = 0: skipped, no pointer looked at
    assert f(one(M=0, packed=None, x=None, xq=None, y=None), 1, 1e-5, None) == BL_OK
    # the workspace of a decode batch that falls back to the cut forward
    q = lib.bitlinear_quant_forward_workspace_bytes
    q.argtypes = [C.POINTER(QFwdArgs), C.c_int, C.POINTER(C.c_size_t)]
    out = C.c_size_t(7)
    assert q(one(), 1, None) == BL_ERR_NULL
    assert q(one(), 1, C.byref(out)) == BL_OK and out.value == 0  # one launch, no workspace
    big = one(N=8192, K=28672, M=32)
    assert q(big, 1, C.byref(out)) == BL_OK and out.value == 8 * 32 * 8192 * 4
    assert f(big, 1, 1e-5, None, ws=A.value, wsb=out.value - 1) == BL_ERR_WORKSPACE
    assert f(big, 1, 1e-5, None, ws=U.value, wsb=out.value) == BL_ERR_ALIGN


def test_valid_call_without_gpu_reports_device_error(lib):
    # The calls below pass host validation with fake device addresses; they
    # must never reach a real device, so the test runs only where the runtime
    # reports none.
    if _device_may_be_present():
        pytest.skip("a GPU may be present; device calls are covered by the gpu tests")
    assert lib.bitlinear_flip_update(A, A2, 8, 5, A, A2, None) == BL_ERR_DEVICE
    g = lib.bitlinear_forward_b1_grouped
    g.argtypes = [C.POINTER(FwdArgs), C.c_int, C.c_void_p]
    assert g((FwdArgs * 1)(FwdArgs(A.value, A.value, 8192, 28672, A.value, A.value, 16, A2.value, None)), 1,
             None) == BL_ERR_DEVICE
    g = lib.bitlinear_forward_grouped_dot4
    g.argtypes = [C.POINTER(FwdArgs), C.c_int, C.c_void_p]
    assert g((FwdArgs * 1)(FwdArgs(A.value, A.value, 8192, 28672, A.value, A.value, 1, A2.value, None)), 1,
             None) == BL_ERR_DEVICE
    q = lib.bitlinear_quant_forward_b1_grouped
    q.argtypes = [C.POINTER(QFwdArgs), C.c_int, C.c_float, C.c_void_p]
    assert q((QFwdArgs * 1)(QFwdArgs(A.value, A.value, 64, 64, A.value, 1, A2.value, A2.value, A2.value, None)), 1,
             1e-5, None) == BL_ERR_DEVICE
    f = lib.bitlinear_forward_grouped_noalloc
    f.argtypes = [C.POINTER(FwdArgs), C.c_int, C.c_void_p]
    assert f((FwdArgs * 1)(FwdArgs(A.value, A.value, 8192, 28672, A.value, A.value, 64, A2.value, None)), 1,
             None) == BL_ERR_DEVICE
    f = lib.bitlinear_backward_input_grouped
    f.argtypes = [C.POINTER(BackwardArgs), C.c_int, C.c_int64, C.c_int64, C.c_void_p, C.c_int, C.c_void_p]
    arr = (BackwardArgs * 2)(BackwardArgs(A.value, A.value, 64, A.value), BackwardArgs(A.value, A.value, 8, A.value))
    assert f(arr, 2, 32, 4, A2.value, 0, None) == BL_ERR_DEVICE


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    # The Python binding refuses to import when the library is missing (no CPU fallback).
    import importlib.util
    src = os.path.join(ROOT, "bitlinear_absmean_ternarise_amd", "__init__.py")
    pkg = tmp_path / "fakepkg"
    pkg.mkdir()
    (pkg / "__init__.py").write_text(open(src).read())
    spec = importlib.util.spec_from_file_location("fakepkg", pkg / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    with pytest.raises(ImportError):
        spec.loader.exec_module(mod)
