"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, answers size queries, and rejects bad arguments on the host
before any HIP call (no compute call is made here)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from bit_weight_only_amd import nf4
from gpu_helpers import k_parts

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nf4.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nf4_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    declared = header_functions()
    assert set(declared) == set(nf4.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", nf4.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (nf4_\w+)", out))
    assert set(declared) <= exported, set(declared) - exported
    L = nf4.lib()
    for name in declared:
        assert hasattr(L, name)


def test_status_strings():
    for s in range(8):
        assert nf4.nf4_status_string(s).startswith("NF4_")
    assert "unknown" in nf4.nf4_status_string(99)


@pytest.mark.parametrize("N,K", [(16, 64), (48, 192), (4608, 3584), (152064, 3584), (3072, 9216)])
def test_size_queries(N, K):
    KT = -(-K // 128)
    assert nf4.nf4_qweight_bytes(N, K) == (N // 16) * KT * 1024
    assert nf4.nf4_absmax_bytes(N, K) == (N // 16) * KT * 128
    assert nf4.nf4_qweight_bytes(N, K) >= N * K // 2
    assert nf4.nf4_absmax_bytes(N, K) >= 4 * N * K // 64


@pytest.mark.parametrize("N,K", [(0, 64), (8, 64), (24, 64), (16, 0), (16, 32), (16, 100),
                                 (-16, 64), (1 << 31, 64)])
def test_size_queries_reject_bad_shapes(N, K):
    assert nf4.nf4_qweight_bytes(N, K) == 0
    assert nf4.nf4_absmax_bytes(N, K) == 0
    assert nf4.nf4_workspace_bytes(1, N, K) == 0


A = 1 << 20  # a 16-byte aligned stand-in address; never dereferenced
CB = np.linspace(-1, 1, 16, dtype=np.float32)
CB[7] = 0.0


def call(name, *args):
    return getattr(nf4.lib(), name)(*args)


def cbarr(v=CB):
    return (ctypes.c_float * 16)(*np.asarray(v, np.float32).tolist())


def test_linear_validation():
    g = lambda *a: call("nf4_gemv", *a)
    m = lambda *a: call("nf4_gemm", *a)
    ok = (A, 1, A, A, cbarr(), 16, 64, A, None, 0, None)
    for f in (g, m):
        for i in (0, 2, 3, 7):
            bad = list(ok)
            bad[i] = None
            assert f(*bad) == nf4.NF4_ERR_NULL
        assert f(A, 0, A, A, cbarr(), 16, 64, A, None, 0, None) == nf4.NF4_ERR_SHAPE
        assert f(A, 1, A, A, cbarr(), 24, 64, A, None, 0, None) == nf4.NF4_ERR_SHAPE
        assert f(A, 1, A, A, cbarr(), 16, 96, A, None, 0, None) == nf4.NF4_ERR_SHAPE
        assert f(A + 8, 1, A, A, cbarr(), 16, 64, A, None, 0, None) == nf4.NF4_ERR_ALIGN
        assert f(A, 1, A + 4, A, cbarr(), 16, 64, A, None, 0, None) == nf4.NF4_ERR_ALIGN
        assert f(A, 1, A, A + 8, cbarr(), 16, 64, A, None, 0, None) == nf4.NF4_ERR_ALIGN
        assert f(A, 1, A, A, cbarr(), 16, 64, A + 4, None, 0, None) == nf4.NF4_ERR_ALIGN
        bad = CB.copy()
        bad[3] = np.inf
        assert f(A, 1, A, A, cbarr(bad), 16, 64, A, None, 0, None) == nf4.NF4_ERR_CODEBOOK
        bad[3] = np.nan
        assert f(A, 1, A, A, cbarr(bad), 16, 64, A, None, 0, None) == nf4.NF4_ERR_CODEBOOK
        bad[3] = 3.4e38  # rounds past the bf16 range: no exact term split
        assert f(A, 1, A, A, cbarr(bad), 16, 64, A, None, 0, None) == nf4.NF4_ERR_CODEBOOK
    assert g(A, 9, A, A, cbarr(), 16, 64, A, None, 0, None) == nf4.NF4_ERR_SHAPE


def split_bytes(M, N, K):
    """Workspace of the tiled GEMM with K in P > 1 parts: per output tile of
    128 rows x 16 RG columns one 4-byte counter (the counters padded to 256
    bytes) and every part's fp32 sums; the largest of the three workgroup
    widths RG = 16, 14 and 8."""
    P = k_parts(N, K)
    if P == 1:
        return 0
    G, mt = N // 16, -(-M // 128)

    def width(rg):
        tiles = -(-G // rg) * mt
        return -(-tiles * 4 // 256) * 256 + tiles * P * 128 * 16 * rg * 4
    return max(width(16), width(14), width(8))


@pytest.mark.parametrize("M,N,K", [(1, 3584, 18944), (64, 3584, 18944), (65, 3584, 18944),
                                   (1024, 3584, 18944), (1024, 3072, 9216), (300, 256, 8128),
                                   (300, 256, 8192), (1024, 37888, 3584), (14449, 152064, 3584),
                                   (1024, 512, 3584), (1024, 1024, 3072), (1024, 3584, 3584),
                                   (1024, 4608, 3584), (300, 272, 704), (1024, 256, 256)])
def test_gemm_workspace_bytes(M, N, K):
    """Only nf4_gemm past 64 rows with K in more than one part needs a
    workspace (K >= 8192, or narrow N with enough K)."""
    assert nf4.nf4_workspace_bytes(M, N, K) == (0 if M <= 64 else split_bytes(M, N, K))
    if M > 64 and k_parts(N, K) > 1:
        assert nf4.nf4_workspace_bytes(M, N, K) >= 4 * k_parts(N, K) * M * N


def test_k_parts_at_the_model_shapes():
    """The parts the rule gives the Qwen2-7B and Voxtral linears: one for the
    wide fused ones, two for long K, more only for narrow N."""
    assert [k_parts(N, K) for N, K in [(4608, 3584), (3584, 3584), (37888, 3584),
                                       (3584, 18944), (152064, 3584)]] == [1, 1, 1, 2, 1]
    assert [k_parts(N, K) for N, K in [(6144, 3072), (3072, 4096), (18432, 3072),
                                       (3072, 9216)]] == [1, 1, 1, 2]
    assert [k_parts(N, K) for N, K in [(512, 3584), (1024, 3072), (256, 256)]] == [7, 4, 1]


def test_gemm_workspace_validation():
    m = lambda *a: call("nf4_gemm", *a)
    M, N, K = 1024, 3584, 18944
    need = nf4.nf4_workspace_bytes(M, N, K)
    assert m(A, M, A, A, cbarr(), N, K, A, None, 0, None) == nf4.NF4_ERR_NULL
    assert m(A, M, A, A, cbarr(), N, K, A, A, need - 1, None) == nf4.NF4_ERR_WORKSPACE
    assert m(A, M, A, A, cbarr(), N, K, A, A + 8, need, None) == nf4.NF4_ERR_ALIGN


def test_pack_validation():
    p = lambda *a: call("nf4_pack", *a)
    assert p(None, 16, 64, cbarr(), A, A, None) == nf4.NF4_ERR_NULL
    assert p(A, 16, 64, None, A, A, None) == nf4.NF4_ERR_NULL
    assert p(A, 16, 64, cbarr(), None, A, None) == nf4.NF4_ERR_NULL
    assert p(A, 17, 64, cbarr(), A, A, None) == nf4.NF4_ERR_SHAPE
    assert p(A + 4, 16, 64, cbarr(), A, A, None) == nf4.NF4_ERR_ALIGN
    for mutate in ("unsorted", "no_zero", "neg_zero", "dup", "nan"):
        bad = CB.copy()
        if mutate == "unsorted":
            bad[[2, 3]] = bad[[3, 2]]
        elif mutate == "no_zero":
            bad[7] = 0.01
        elif mutate == "neg_zero":
            bad[7] = -0.0
        elif mutate == "dup":
            bad[9] = bad[8]
        else:
            bad[0] = np.nan
        assert p(A, 16, 64, cbarr(bad), A, A, None) == nf4.NF4_ERR_CODEBOOK, mutate


def test_layout_entry_validation():
    for name in ("nf4_repack", "nf4_unpack"):
        f = lambda *a: call(name, *a)
        assert f(None, A, 16, 64, A, A, None) == nf4.NF4_ERR_NULL
        assert f(A, A, 16, 32, A, A, None) == nf4.NF4_ERR_SHAPE
        assert f(A, A + 4, 16, 64, A, A, None) == nf4.NF4_ERR_ALIGN
    d = lambda *a: call("nf4_dequant", *a)
    assert d(A, A, None, 16, 64, A, None) == nf4.NF4_ERR_NULL
    assert d(A, A, cbarr(), 16, 65, A, None) == nf4.NF4_ERR_SHAPE
    bad = CB.copy()
    bad[0] = np.inf
    assert d(A, A, cbarr(bad), 16, 64, A, None) == nf4.NF4_ERR_CODEBOOK


def test_argmax_validation():
    f = lambda *a: call("nf4_gemv_argmax", *a)
    ok = [A, 1, A, A, cbarr(), 16, 64, A, A, A, 1 << 20, None]
    for i, err in ((0, nf4.NF4_ERR_NULL), (2, nf4.NF4_ERR_NULL), (7, nf4.NF4_ERR_NULL),
                   (8, nf4.NF4_ERR_NULL), (9, nf4.NF4_ERR_NULL)):
        bad = list(ok)
        bad[i] = None
        assert f(*bad) == err, i
    for M in (0, 9):
        bad = list(ok)
        bad[1] = M
        assert f(*bad) == nf4.NF4_ERR_SHAPE
    bad = list(ok)
    bad[5] = 24
    assert f(*bad) == nf4.NF4_ERR_SHAPE
    bad = list(ok)
    bad[8] = A + 4
    assert f(*bad) == nf4.NF4_ERR_ALIGN
    for M, N, K in ((0, 16, 64), (9, 16, 64), (1, 24, 64), (1, 16, 96)):
        assert nf4.nf4_gemv_argmax_workspace_bytes(M, N, K) == 0


def test_prefetch_validation():
    """nf4_gemv_prefetch checks its own arguments as nf4_gemv does, and the
    next matrix when one is named; only calls that fail before any HIP call
    are made here."""
    f = lambda *a: call("nf4_gemv_prefetch", *a)
    ok = [A, 1, A, A, cbarr(), 16, 64, A, None, 0, A, A, 32, 128, None]
    for i, err in ((0, nf4.NF4_ERR_NULL), (2, nf4.NF4_ERR_NULL), (7, nf4.NF4_ERR_NULL)):
        bad = list(ok)
        bad[i] = None
        assert f(*bad) == err, i
    bad = list(ok)
    bad[1] = 9
    assert f(*bad) == nf4.NF4_ERR_SHAPE
    bad = list(ok)
    bad[11] = None                      # next qweight without next absmax
    assert f(*bad) == nf4.NF4_ERR_NULL
    for i in (10, 11):
        bad = list(ok)
        bad[i] = A + 8
        assert f(*bad) == nf4.NF4_ERR_ALIGN, i
    for nN, nK in ((24, 128), (32, 96), (0, 64), (16, 0)):
        bad = list(ok)
        bad[12], bad[13] = nN, nK
        assert f(*bad) == nf4.NF4_ERR_SHAPE, (nN, nK)


def test_binding_raises_named_errors():
    with pytest.raises(nf4.NF4Error) as e:
        nf4.nf4_gemv(A, 9, A, A, CB, 16, 64, A, stream=0)
    assert e.value.status == nf4.NF4_ERR_SHAPE and "NF4_ERR_SHAPE" in str(e.value)


@pytest.mark.parametrize("K", [64, 192, 3584])
def test_packed_weight_rows_view(K):
    """A row range of a packed weight is the contiguous run of its 16-row
    groups in both buffers, shared with the whole (no copy)."""
    import torch
    N = 96
    pw = nf4.PackedWeight(N, K, device="cpu")
    pw.qweight.copy_(torch.arange(pw.qweight.numel(), dtype=torch.int64).to(torch.uint8))
    pw.absmax.copy_(torch.arange(pw.absmax.numel(), dtype=torch.float32))
    KT = -(-K // 128)
    v = pw.rows(32, 80)
    assert (v.N, v.K) == (48, K)
    assert v.qweight.numel() == nf4.nf4_qweight_bytes(48, K)
    assert v.absmax.numel() * 4 == nf4.nf4_absmax_bytes(48, K)
    assert v.qweight.data_ptr() == pw.qweight.data_ptr() + 2 * KT * 1024
    assert v.absmax.data_ptr() == pw.absmax.data_ptr() + 2 * KT * 128
    assert torch.equal(v.absmax, pw.absmax[2 * KT * 32:5 * KT * 32])
    for n0, n1 in ((0, 8), (8, 32), (32, 32), (0, 112), (-16, 16)):
        with pytest.raises(nf4.NF4Error):
            pw.rows(n0, n1)


# ----------------------------------------------- asymmetric int4, group 128
@pytest.mark.parametrize("N,K", [(16, 128), (48, 256), (4608, 3584), (3584, 18944)])
def test_awq_size_queries(N, K):
    assert nf4.nf4_awq_params_bytes(N, K) == (N // 16) * (K // 128) * 64 == 4 * N * K // 128
    for M in (1, 8, 64, 65, 127, 128, 129, 14449):
        Mp = -(-M // 128) * 128
        extra = 0 if M <= 64 else split_bytes(M, N, K)
        assert nf4.nf4_awq_workspace_bytes(M, N, K) == (K // 128) * Mp * 4 + extra


@pytest.mark.parametrize("N,K", [(16, 64), (16, 192), (24, 128), (0, 128), (16, 0)])
def test_awq_size_queries_reject_bad_shapes(N, K):
    assert nf4.nf4_awq_params_bytes(N, K) == 0
    assert nf4.nf4_awq_workspace_bytes(1, N, K) == 0


def test_awq_layout_validation():
    p = lambda *a: call("nf4_awq_pack", *a)
    assert p(None, 16, 128, A, A, None) == nf4.NF4_ERR_NULL
    assert p(A, 16, 128, None, A, None) == nf4.NF4_ERR_NULL
    assert p(A, 16, 128, A, None, None) == nf4.NF4_ERR_NULL
    assert p(A, 16, 64, A, A, None) == nf4.NF4_ERR_SHAPE       # K % 128 != 0
    assert p(A, 24, 128, A, A, None) == nf4.NF4_ERR_SHAPE
    assert p(A + 4, 16, 128, A, A, None) == nf4.NF4_ERR_ALIGN
    assert p(A, 16, 128, A, A + 8, None) == nf4.NF4_ERR_ALIGN
    for name in ("nf4_awq_repack", "nf4_awq_unpack"):
        f = lambda *a: call(name, *a)
        ok = [A, A, A, 16, 128, A, A, None] if name == "nf4_awq_repack" else \
             [A, A, 16, 128, A, A, A, None]
        ptrs = [i for i, v in enumerate(ok) if v == A]
        for i in ptrs:
            bad = list(ok)
            bad[i] = None
            assert f(*bad) == nf4.NF4_ERR_NULL, (name, i)
            bad[i] = A + 2
            assert f(*bad) == nf4.NF4_ERR_ALIGN, (name, i)
        bad = list(ok)
        k_at = 4 if name == "nf4_awq_repack" else 3
        bad[k_at] = 192
        assert f(*bad) == nf4.NF4_ERR_SHAPE
    d = lambda *a: call("nf4_awq_dequant", *a)
    assert d(A, None, 16, 128, A, None) == nf4.NF4_ERR_NULL
    assert d(A, A, 16, 320, A, None) == nf4.NF4_ERR_SHAPE
    assert d(A, A, 16, 128, A + 4, None) == nf4.NF4_ERR_ALIGN


def test_awq_linear_validation():
    g = lambda *a: call("nf4_awq_gemv", *a)
    m = lambda *a: call("nf4_awq_gemm", *a)
    ok = [A, 1, A, A, 16, 128, A, A, 1 << 20, None]
    for f in (g, m):
        for i in (0, 2, 3, 6):
            bad = list(ok)
            bad[i] = None
            assert f(*bad) == nf4.NF4_ERR_NULL, i
            bad[i] = A + 8
            assert f(*bad) == nf4.NF4_ERR_ALIGN, i
        for M, N, K in ((0, 16, 128), (1, 24, 128), (1, 16, 64), (1, 16, 192)):
            bad = list(ok)
            bad[1], bad[4], bad[5] = M, N, K
            assert f(*bad) == nf4.NF4_ERR_SHAPE, (M, N, K)
    assert g(*([A, 9] + ok[2:])) == nf4.NF4_ERR_SHAPE
    # the GEMM always needs the x sums in the workspace
    assert m(A, 1, A, A, 16, 128, A, None, 0, None) == nf4.NF4_ERR_NULL
    assert m(A, 1, A, A, 16, 128, A, A, 511, None) == nf4.NF4_ERR_WORKSPACE
    assert m(A, 1, A, A, 16, 128, A, A + 4, 512, None) == nf4.NF4_ERR_ALIGN
    # x of 8 x 18944 bf16 (303 KB) does not fit the GEMV's LDS: it needs the
    # workspace of the GEMM it falls back on
    need = nf4.nf4_awq_workspace_bytes(8, 16, 18944)
    assert need == 148 * 128 * 4
    assert g(A, 8, A, A, 16, 18944, A, None, 0, None) == nf4.NF4_ERR_NULL
    assert g(A, 8, A, A, 16, 18944, A, A, need - 1, None) == nf4.NF4_ERR_WORKSPACE
    # byte offsets past 32 bits
    assert m(A, 1 << 17, A, A, 16, 1 << 14, A, A, 1 << 40, None) == nf4.NF4_ERR_SHAPE


def test_gather_validation():
    f = lambda *a: call("nf4_gather_columns", *a)
    ok = [A, 4, 3584, A, A, None]
    for i in (0, 3, 4):
        bad = list(ok)
        bad[i] = None
        assert f(*bad) == nf4.NF4_ERR_NULL, i
        bad[i] = A + 4
        assert f(*bad) == nf4.NF4_ERR_ALIGN, i
    for M, K in ((0, 128), (1, 0), (1, 4), (1, 100), (1 << 24, 128)):
        assert f(A, M, K, A, A, None) == nf4.NF4_ERR_SHAPE, (M, K)


def test_awq_prefetch_validation():
    f = lambda *a: call("nf4_awq_gemv_prefetch", *a)
    ok = [A, 1, A, A, 16, 128, A, None, 0, A, A, 32, 256, None]
    for i in (0, 2, 3, 6):
        bad = list(ok)
        bad[i] = None
        assert f(*bad) == nf4.NF4_ERR_NULL, i
    bad = list(ok)
    bad[1] = 9
    assert f(*bad) == nf4.NF4_ERR_SHAPE
    bad = list(ok)
    bad[10] = None                      # next qweight without next params
    assert f(*bad) == nf4.NF4_ERR_NULL
    for i in (9, 10):
        bad = list(ok)
        bad[i] = A + 8
        assert f(*bad) == nf4.NF4_ERR_ALIGN, i
    for nN, nK in ((24, 128), (32, 64), (32, 192), (0, 128)):
        bad = list(ok)
        bad[11], bad[12] = nN, nK
        assert f(*bad) == nf4.NF4_ERR_SHAPE, (nN, nK)


# ------------------------------------------------------- the default codebook
def golden_codebook():
    """The 16 hex floats of tests/golden/nf4_codebook.txt (written from the oracle)."""
    path = os.path.join(ROOT, "tests", "golden", "nf4_codebook.txt")
    vals = [float.fromhex(ln.split("#")[0].strip()) for ln in open(path)
            if ln.strip() and not ln.startswith("#")]
    return np.array(vals, np.float32)


def test_library_codebook_equals_the_golden_table():
    """nf4_codebook (host code of the library: Newton's method on erfc, its own
    bf16 rounding) gives the fixture's table bit for bit, and the oracle's."""
    import oracle
    cb = nf4.nf4_codebook()
    gold = golden_codebook()
    assert np.array_equal(cb.view(np.uint32), gold.view(np.uint32))
    assert np.array_equal(cb.view(np.uint32), oracle.codebook()[0].view(np.uint32))


@pytest.mark.parametrize("delta", [0.8, 0.9, 0.95, 0.99, 0.9999])
def test_library_codebook_invariants_and_oracle_agreement(delta):
    """Other tail probabilities: 16 strictly increasing bf16 values, -1, +0.0
    and +1 at indices 0, 7 and 15, equal to the oracle's construction."""
    import oracle
    cb = nf4.nf4_codebook(delta)
    assert np.all(np.diff(cb) > 0)
    assert cb[0] == -1.0 and cb[15] == 1.0
    assert cb[7] == 0.0 and not np.signbit(cb[7])
    assert np.all((cb.view(np.uint32) & 0xFFFF) == 0)  # bf16-exact
    assert np.array_equal(cb.view(np.uint32), oracle.codebook(delta)[0].view(np.uint32))


@pytest.mark.parametrize("delta", [0.5, 0.75, 1.0, float("nan"), -1.0])
def test_library_codebook_rejects_bad_delta(delta):
    with pytest.raises(nf4.NF4Error) as e:
        nf4.nf4_codebook(delta)
    assert e.value.status == nf4.NF4_ERR_CODEBOOK


# ------------------------------------------- GEMV + argmax without allocation
def test_noalloc_rejects_bad_arguments_on_the_host():
    """nf4_gemv_argmax_noalloc validates like nf4_gemv_argmax before any HIP
    call (no compute call is made here)."""
    L, cb = nf4.lib(), (ctypes.c_float * 16)(*nf4.nf4_codebook().tolist())
    f = L.nf4_gemv_argmax_noalloc
    assert f(None, 1, A, A, cb, 256, 256, A, A, None) == nf4.NF4_ERR_NULL
    assert f(A, 1, A, A, cb, 256, 256, A, None, None) == nf4.NF4_ERR_NULL
    assert f(A, 9, A, A, cb, 256, 256, A, A, None) == nf4.NF4_ERR_SHAPE
    assert f(A, 0, A, A, cb, 256, 256, A, A, None) == nf4.NF4_ERR_SHAPE
    assert f(A, 1, A, A, cb, 24, 256, A, A, None) == nf4.NF4_ERR_SHAPE
    assert f(A + 4, 1, A, A, cb, 256, 256, A, A, None) == nf4.NF4_ERR_ALIGN
    assert f(A, 1, A, A, cb, 256, 256, A, A + 4, None) == nf4.NF4_ERR_ALIGN
