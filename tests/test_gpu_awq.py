"""GPU parity of the second weight format, asymmetric int4 in groups of 128
along K (w = (q - z) * s; vibevoice.c README, "Quantization" > "Weights": the
INT4 quantizer option and the AWQ/GPTQ repack paragraph), against the oracle
on the same seeded inputs.

Load-time path (nf4_awq_pack, nf4_awq_repack / nf4_awq_unpack,
nf4_awq_dequant): codes, zero points, binary16 scale bits and dequantized
binary32 values bit for bit, including binary16 rounding ties, subnormal and
overflowing scales, and groups narrower than the 1e-5 floor.

Linear path (nf4_awq_gemv, nf4_awq_gemm): rel-L2 <= 1e-5 per call and every
element within 1e-4 * sum_k |x*w|; exact where the arithmetic is exact
(one-hot x); rows of the GEMM independent of the batch; shapes of Qwen2-7B
(hidden 3584, MLP 18944, head 152064) at decode, M = 1024 prefill and a long
M = 14449 prefill; the Voxtral decoder's fused linears at decode.
"""
import numpy as np
import pytest

import oracle
from bit_weight_only_amd import synth

from gpu_helpers import (QWEN, QWEN_FUSED, VOXTRAL_FUSED, Side, assert_linear_ok,
                         oracle_awq_layer, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def side():
    return Side()


def check_pack(side, W):
    codes, scales, zeros = oracle.awq_quantize(W)
    packed = oracle.pack(codes)
    aw = side.awq_pack(W)
    gc, gs, gz = side.awq_unpack(aw)
    np.testing.assert_array_equal(gc, packed)
    np.testing.assert_array_equal(gz, zeros)
    np.testing.assert_array_equal(gs.view(np.uint32), scales.view(np.uint32))
    return aw, packed, scales, zeros


# ------------------------------------------------------------ load-time path
SHAPES = [(16, 128), (48, 256), (256, 384), (512, 3584), (64, 18944), (4608, 128)]


@pytest.mark.parametrize("N,K", SHAPES)
def test_awq_pack_bit_exact(side, N, K):
    say(f"[awq pack] N={N} K={K}")
    W = synth.weights(0, 2, 11, N, K)
    W[1, :128] = 0.0                 # an all-zero group
    W[2, 128 % K:128 % K + 128] = 0.25  # a constant group (range below the floor)
    aw, packed, scales, zeros = check_pack(side, W)
    deq = side.awq_dequant(aw)
    np.testing.assert_array_equal(deq.view(np.uint32),
                                  oracle.awq_dequant(packed, scales, zeros).view(np.uint32))


def test_awq_pack_scale_rounding_edges(side):
    """Scales on binary16 rounding ties (to even, both directions), subnormal
    binary16 scales, one-sided groups (z = 0 and z = 15) and a scale past the
    binary16 range (+inf: every code and zero point 0)."""
    W = np.zeros((16, 256), np.float32)
    W[0, 0], W[0, 1] = 0.0, 15 * (1 + 2 ** -11)        # range/15 halfway: to 1.0
    W[1, 0], W[1, 1] = 0.0, 15 * (1 + 3 * 2 ** -11)    # halfway: to 1 + 2^-9
    W[2, 0], W[2, 1] = -7.5, 7.5 + 15 * 2 ** -11        # tie with a negative minimum
    W[3, :128] = np.linspace(1e-6, 8e-5, 128, dtype=np.float32)   # subnormal binary16 scale
    W[4, :128] = np.linspace(-3e-4, -1e-6, 128, dtype=np.float32)  # all negative: z = 15
    W[5, :128] = np.linspace(0.5, 2.0, 128, dtype=np.float32)     # all positive: z = 0
    W[6, 0], W[6, 1] = -6e5, 6e5                       # s overflows binary16
    W[7, 128:256] = np.float32(3e-7)                    # constant: the 1e-5 floor
    W[8, 128:256] = synth.weights(0, 3, 0, 1, 128)[0] * 1e-3
    codes, scales, zeros = oracle.awq_quantize(W)
    assert scales[0, 0] == 1.0 and scales[1, 0] == np.float32(1 + 2 ** -9)
    assert np.isinf(scales[6, 0]) and zeros[4, 0] == 15 and zeros[5, 0] == 0
    assert 0 < scales[3, 0] < 2 ** -14
    check_pack(side, W)


def test_awq_repack_unpack_roundtrip(side):
    rng = np.random.default_rng(5)
    N, K = 48, 384
    packed = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = rng.uniform(1e-4, 2.0, (N, K // 128)).astype(np.float16).astype(np.float32)
    zeros = rng.integers(0, 16, (N, K // 128), dtype=np.uint8)
    aw = side.awq_repack(packed, scales, zeros)
    gc, gs, gz = side.awq_unpack(aw)
    np.testing.assert_array_equal(gc, packed)
    np.testing.assert_array_equal(gs, scales)
    np.testing.assert_array_equal(gz, zeros)
    np.testing.assert_array_equal(side.awq_dequant(aw).view(np.uint32),
                                  oracle.awq_dequant(packed, scales, zeros).view(np.uint32))


# ------------------------------------------------------------ linear path
def awq_case(side, N, K, mid=30, cfg=0, layer=0):
    W, packed, scales, zeros = oracle_awq_layer(cfg, layer, mid, N, K)
    return packed, scales, zeros, side.awq_repack(packed, scales, zeros)


@pytest.mark.parametrize("kind,M", [("gemv", 1), ("gemv", 4), ("gemm", 1), ("gemm", 4)])
def test_awq_tiny_config(side, kind, M):
    """256 x 256 layer packed on the GPU from the seeded W."""
    say(f"[awq {kind}] tiny M={M}")
    W = synth.weights(0, 0, 0, 256, 256)
    aw, packed, scales, zeros = check_pack(side, W)
    x = synth.activations(0, M, 256)
    y = side.awq_run(kind, x, aw)
    yr, b = oracle.awq_linear(x, packed, scales, zeros)
    assert_linear_ok(y, yr, b, f"awq {kind} tiny M={M}")


# (8, 64, 18944): x of 303 KB does not fit the GEMV's LDS, so nf4_awq_gemv
# runs the tiled GEMM
GEMV_EDGES = [(M, N, K) for M in (1, 2, 3, 5, 8) for (N, K) in
              [(16, 128), (48, 256), (512, 384), (16, 3584), (64, 18944), (4608, 128)]]


@pytest.mark.parametrize("M,N,K", GEMV_EDGES)
def test_awq_gemv_edges(side, M, N, K):
    say(f"[awq gemv] M={M} N={N} K={K}")
    packed, scales, zeros, aw = awq_case(side, N, K, mid=31)
    x = synth.activations(0, M, K, stream=M)
    yr, b = oracle.awq_linear(x, packed, scales, zeros)
    assert_linear_ok(side.awq_run("gemv", x, aw), yr, b, f"awq gemv M={M} N={N} K={K}")


GEMM_EDGES = [(1, 48, 128), (9, 272, 256), (100, 16, 384), (128, 512, 3584), (129, 160, 1024),
              (300, 272, 640), (257, 2048, 256), (64, 64, 18944), (300, 272, 8320),
              (129, 512, 8192), (29, 512, 3584), (32, 64, 18944)]


@pytest.mark.parametrize("M,N,K", GEMM_EDGES)
def test_awq_gemm_edges(side, M, N, K):
    say(f"[awq gemm] M={M} N={N} K={K}")
    packed, scales, zeros, aw = awq_case(side, N, K, mid=32)
    x = synth.activations(0, M, K, stream=7)
    yr, b = oracle.awq_linear(x, packed, scales, zeros)
    assert_linear_ok(side.awq_run("gemm", x, aw), yr, b, f"awq gemm M={M} N={N} K={K}")


@pytest.mark.parametrize("kind", ["gemv", "gemm"])
def test_awq_one_hot_rows_are_dequantized_weights(side, kind):
    """x = e_k: the group of k sums to 1 and every other group to 0, so the
    output is (q - z) * s exactly: the dequantized weight column."""
    N, K = 64, 384
    packed, scales, zeros, aw = awq_case(side, N, K, mid=33)
    ks = [0, 1, 127, 128, 200, 383] if kind == "gemm" else [5, 130, 383]
    x = np.zeros((len(ks), K), np.uint16)
    for m, k in enumerate(ks):
        x[m, k] = 0x3F80  # bf16 1.0
    y = side.awq_run(kind, x, aw)
    deq = oracle.awq_dequant(packed, scales, zeros)
    np.testing.assert_array_equal(y.view(np.uint32), deq[:, ks].T.copy().view(np.uint32))


@pytest.mark.parametrize("kind", ["gemv", "gemm"])
def test_awq_zero_point_cancellation(side, kind):
    """The hardest case for folding z into the product: almost every code
    equals its zero point, so sum x q and z X nearly cancel; two codes per
    group (0 and 15) carry the whole output."""
    N, K, M = 32, 3584, 3 if kind == "gemv" else 40
    rng = np.random.default_rng(9)
    zeros = rng.integers(6, 10, (N, K // 128), dtype=np.uint8)
    codes = np.repeat(zeros, 128, axis=1).astype(np.uint8)
    n = np.arange(N)
    for g in range(K // 128):
        codes[n, 128 * g + rng.integers(0, 64, N)] = 0
        codes[n, 128 * g + rng.integers(64, 128, N)] = 15
    scales = rng.uniform(0.01, 0.1, (N, K // 128)).astype(np.float16).astype(np.float32)
    packed = oracle.pack(codes)
    aw = side.awq_repack(packed, scales, zeros)
    x = synth.activations(0, M, K, stream=11)
    yr, b = oracle.awq_linear(x, packed, scales, zeros)
    rel, worst = assert_linear_ok(side.awq_run(kind, x, aw), yr, b, f"awq {kind} cancellation")
    say(f"  rel-L2 {rel:.2e}, worst element {worst:.3f} x bar")


@pytest.mark.parametrize("N,K", [(272, 1024), (272, 8320), (4608, 3584), (4608, 8192)])
def test_awq_gemm_deterministic_and_batch_independent(side, N, K):
    """Rows do not depend on the batch: 300 rows take the tiled path, up to
    32 rows the narrow path, 33 the skinny path (K = 8320, N = 272: summed
    in 10 parts on every path; N = 4608: the narrow form with two
    workgroups per CU, K in one part and, at K = 8192, in two), and a reused
    workspace full of stale bytes gives the same bits (every call sets what
    it reads)."""
    packed, scales, zeros, aw = awq_case(side, N, K, mid=34)
    x = synth.activations(0, 300, K, stream=12)
    y1 = side.awq_run("gemm", x, aw)
    y2 = side.awq_run("gemm", x, aw)
    np.testing.assert_array_equal(y1, y2)
    for lo, hi in ((0, 1), (5, 13), (17, 46), (40, 73), (128, 300), (290, 300)):
        np.testing.assert_array_equal(side.awq_run("gemm", x[lo:hi], aw), y1[lo:hi])
    t = side.torch
    ws = t.full((side.nf4.nf4_awq_workspace_bytes(300, N, K),), 0xFF, dtype=t.uint8,
                device="cuda")
    for _ in range(2):
        y3 = side.awq_linear("gemm", side.x_dev(x), 300, aw, ws=ws).cpu().numpy()
        np.testing.assert_array_equal(y3, y1)


def test_awq_gemv_deterministic_and_agrees_with_gemm(side):
    N, K = 4608, 3584
    packed, scales, zeros, aw = awq_case(side, N, K, mid=35)
    x = synth.activations(0, 2, K, stream=13)
    yv = side.awq_run("gemv", x, aw)
    np.testing.assert_array_equal(yv, side.awq_run("gemv", x, aw))
    ym = side.awq_run("gemm", x, aw)
    yr, b = oracle.awq_linear(x, packed, scales, zeros)
    assert_linear_ok(yv, yr, b, "awq gemv")
    assert_linear_ok(ym, yr, b, "awq gemm")


# ------------------------------------------------------------ full sizes
_FULL = {}


def full_awq_case(side, cfg, mid, N, K, rows):
    """Pack the full seeded weight on the GPU; the oracle quantizes only the
    sampled output rows."""
    key = (cfg, mid, N, K, tuple(rows))
    if key in _FULL:
        return _FULL[key]
    _FULL.clear()
    W = synth.weights(cfg, 0, mid, N, K)
    aw = side.awq_pack(W)
    del W
    Wr = synth.weights(cfg, 0, mid, N, K, rows=rows)
    codes, scales, zeros = oracle.awq_quantize(Wr)
    _FULL[key] = (aw, oracle.pack(codes), scales, zeros)
    return _FULL[key]


def sample_rows(N, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 15, 16, N // 2, N - 16, N - 1],
                                     rng.integers(0, N, 250)]))


@pytest.mark.parametrize("M", [1, 2])
@pytest.mark.parametrize("name", list(QWEN_FUSED) + ["lm_head"])
def test_awq_qwen_decode_full_size(side, name, M):
    N, K = QWEN_FUSED.get(name) or QWEN[name]
    say(f"[awq gemv] qwen {name} M={M} N={N} K={K}")
    rows = sample_rows(N, 21)
    aw, packed, scales, zeros = full_awq_case(
        side, 2, 80 + (list(QWEN_FUSED) + ["lm_head"]).index(name), N, K, rows)
    x = synth.activations(2, M, K)
    y = side.awq_run("gemv", x, aw)
    yr, b = oracle.awq_linear(x, packed, scales, zeros)
    assert_linear_ok(y[:, rows], yr, b, f"awq qwen {name} M={M}")
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("name", list(VOXTRAL_FUSED))
def test_awq_voxtral_decode_full_size(side, name):
    N, K = VOXTRAL_FUSED[name]
    say(f"[awq gemv] voxtral {name} N={N} K={K}")
    rows = sample_rows(N, 24)
    aw, packed, scales, zeros = full_awq_case(side, 1, 110 + list(VOXTRAL_FUSED).index(name),
                                              N, K, rows)
    x = synth.activations(1, 1, K)
    y = side.awq_run("gemv", x, aw)
    yr, b = oracle.awq_linear(x, packed, scales, zeros)
    assert_linear_ok(y[:, rows], yr, b, f"awq voxtral {name}")
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("name", list(QWEN_FUSED))
def test_awq_qwen_prefill_full_size(side, name):
    """M = 1024; sampled columns on token rows {0, 1023, 6 seeded}."""
    N, K = QWEN_FUSED[name]
    say(f"[awq gemm] qwen prefill {name} M=1024 N={N} K={K}")
    rows = sample_rows(N, 22)
    aw, packed, scales, zeros = full_awq_case(side, 3, 90 + list(QWEN_FUSED).index(name), N, K,
                                              rows)
    x = synth.activations(3, 1024, K)
    y = side.awq_run("gemm", x, aw)
    toks = np.unique(np.concatenate([[0, 1023], np.random.default_rng(4).integers(0, 1024, 6)]))
    yr, b = oracle.awq_linear(x[toks], packed, scales, zeros)
    assert_linear_ok(y[toks][:, rows], yr, b, f"awq prefill {name}")
    assert np.all(np.isfinite(y))
    np.testing.assert_array_equal(side.awq_run("gemm", x, aw), y)
    for m in (0, 1023):
        np.testing.assert_array_equal(side.awq_run("gemm", x[m:m + 1], aw), y[m:m + 1])


def test_awq_long_prefill_one_call(side):
    """M = 14449 = 14 x 1024 + 113 through the o projection in one call (113
    rows in the last 128-row tile): every row of the ragged tail and two rows
    per 1024-row span against the oracle on sampled columns."""
    N, K = QWEN_FUSED["o"]
    M = 14449
    rows = sample_rows(N, 23)
    aw, packed, scales, zeros = full_awq_case(side, 4, 99, N, K, rows)
    x = synth.activations(4, M, K)
    say(f"[awq gemm] long prefill M={M} N={N} K={K}")
    y = side.awq_run("gemm", x, aw)
    assert np.all(np.isfinite(y))
    picks = np.concatenate([np.arange(14336, M)] + [[c, c + 1023] for c in range(0, 14336, 1024)])
    yr, b = oracle.awq_linear(x[picks], packed, scales, zeros)
    assert_linear_ok(y[picks][:, rows], yr, b, "awq long prefill")


# ------------------------------------------------------------ act-order gather
def gather_dev(side, x_bits, perm):
    t = side.torch
    M, K = x_bits.shape
    xd = side.x_dev(x_bits)
    pd = side.to_dev(np.ascontiguousarray(perm, np.int32))
    out = t.empty((M, K), dtype=t.int16, device="cuda")
    side.stream.wait_stream(t.cuda.current_stream())
    side.nf4.nf4_gather_columns(xd, M, K, pd, out, stream=side.stream)
    side.sync()
    return out


@pytest.mark.parametrize("M,K", [(1, 8), (3, 128), (1, 3584), (5, 18944), (1024, 3584)])
def test_gather_columns_bit_exact(side, M, K):
    say(f"[gather] M={M} K={K}")
    rng = np.random.default_rng(K + M)
    perm = rng.permutation(K).astype(np.int32)
    x = synth.activations(0, M, K, stream=21)
    got = gather_dev(side, x, perm).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, oracle.gather_columns(x, perm))


def test_gather_columns_clamps_out_of_range(side):
    K = 256
    perm = np.arange(K, dtype=np.int32)[::-1].copy()
    perm[[0, 7, 100]] = [-5, K, 1 << 30]
    x = synth.activations(0, 2, K, stream=22)
    got = gather_dev(side, x, perm).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, oracle.gather_columns(x, np.clip(perm, 0, K - 1)))


@pytest.mark.parametrize("kind,M", [("gemv", 1), ("gemv", 2), ("gemm", 64), ("gemm", 300)])
def test_act_order_pipeline(side, kind, M):
    """Scattered groups: the channel order sorted by group on the host (the
    loader's step), the sorted weight packed on the GPU, x gathered on the GPU
    through the same order, then the int4 linear; against the oracle's
    pipeline on the same seeded inputs."""
    N, K = 512, 3584
    say(f"[act-order {kind}] M={M} N={N} K={K}")
    rng = np.random.default_rng(31)
    g_idx = rng.permutation(np.repeat(np.arange(K // 128), 128))
    perm = oracle.act_order_perm(g_idx)
    W = synth.weights(0, 5, 2, N, K)
    Ws = oracle.gather_columns(W, perm)
    aw, packed, scales, zeros = check_pack(side, Ws)
    x = synth.activations(0, M, K, stream=23)
    xg = gather_dev(side, x, perm)
    y = side.awq_linear(kind, xg, M, aw).cpu().numpy()
    yr, b = oracle.awq_linear(oracle.gather_columns(x, perm), packed, scales, zeros)
    assert_linear_ok(y, yr, b, f"act-order {kind} M={M}")


# ------------------------------------------------------------ read-ahead hint
@pytest.mark.parametrize("M", [1, 2, 8])
def test_awq_prefetch_hint_keeps_results_bitwise(side, M):
    """A decode chain over the fused Qwen2-7B linears, each launch naming the
    next one's matrix (and the last naming the first): y equals the plain
    nf4_awq_gemv bit for bit, and the oracle's within the bar."""
    t = side.torch
    names = list(QWEN_FUSED)
    rows = {n: sample_rows(QWEN_FUSED[n][0], 40 + i) for i, n in enumerate(names)}
    aws, refs = {}, {}
    for i, n in enumerate(names):
        N, K = QWEN_FUSED[n]
        W = synth.weights(2, 1, 70 + i, N, K)
        aws[n] = side.awq_pack(W)
        codes, scales, zeros = oracle.awq_quantize(W[rows[n]])
        refs[n] = (oracle.pack(codes), scales, zeros)
        del W
    for i, n in enumerate(names):
        N, K = QWEN_FUSED[n]
        say(f"[awq prefetch] M={M} {n}")
        aw, nx = aws[n], aws[names[(i + 1) % len(names)]]
        x = synth.activations(2, M, K, stream=30 + i)
        xd = side.x_dev(x)
        ws_bytes = side.nf4.nf4_awq_workspace_bytes(M, N, K)
        ws = t.empty(max(ws_bytes, 16), dtype=t.uint8, device="cuda")
        y0 = t.empty((M, N), dtype=t.float32, device="cuda")
        y1 = t.empty((M, N), dtype=t.float32, device="cuda")
        side.stream.wait_stream(t.cuda.current_stream())
        side.nf4.nf4_awq_gemv(xd, M, aw.qweight, aw.params, N, K, y0, ws, ws_bytes,
                              stream=side.stream)
        side.nf4.nf4_awq_gemv_prefetch(xd, M, aw.qweight, aw.params, N, K, y1, ws, ws_bytes,
                                       nx.qweight, nx.params, nx.N, nx.K, stream=side.stream)
        side.sync()
        a, b = y0.cpu().numpy(), y1.cpu().numpy()
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
        packed, scales, zeros = refs[n]
        yr, bd = oracle.awq_linear(x, packed, scales, zeros)
        assert_linear_ok(b[:, rows[n]], yr, bd, f"awq prefetch {n} M={M}")


def test_awq_gemm_k_parts_in_a_replayed_graph(side):
    """The int4 GEMM with K in parts (pre-pass, which zeroes the counters
    with ordinary stores, then the tiled kernel) captured in a HIP graph:
    every replay equals the eager call bit for bit, with an eager call on
    the same workspace between replays."""
    t = side.torch
    N, K, M = 512, 8192, 300
    packed, scales, zeros, aw = awq_case(side, N, K, mid=36)
    xd = side.x_dev(synth.activations(0, M, K, stream=13))
    wsb = side.nf4.nf4_awq_workspace_bytes(M, N, K)
    ws = t.full((wsb,), 0x5A, dtype=t.uint8, device="cuda")
    y0 = side.awq_linear("gemm", xd, M, aw, ws=ws).clone()
    y = t.empty((M, N), dtype=t.float32, device="cuda")
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g, stream=side.stream):
        side.nf4.nf4_awq_gemm(xd, M, aw.qweight, aw.params, N, K, y, ws, wsb, stream=side.stream)
    side.sync()
    for rep in range(3):
        with t.cuda.stream(side.stream):
            y.fill_(float("nan"))
            g.replay()
        side.sync()
        assert t.equal(y.view(t.int32), y0.view(t.int32)), f"replay {rep}"
        assert t.equal(side.awq_linear("gemm", xd, M, aw, ws=ws).view(t.int32), y0.view(t.int32))
    yr, b = oracle.awq_linear(synth.activations(0, M, K, stream=13)[[0, 299]], packed, scales, zeros)
    assert_linear_ok(y0.cpu().numpy()[[0, 299]], yr, b, "awq gemm K in parts")


@pytest.mark.parametrize("N,K", [(33024, 1024), (16512, 8192)])
def test_awq_gemm_skinny_three_per_cu_rows_identical(side, N, K):
    """Int4 skinny grids of more than two rounds of two workgroups per CU at
    17-64 rows (the 32-row instance) run three per CU: rows agree bit for bit
    with the tiled path (K in one part, and in two at K = 8192), and sampled
    outputs match the oracle."""
    say(f"[awq gemm] skinny, three per CU: N={N} K={K}")
    rows = sample_rows(N, 8)
    aw, packed, scales, zeros = full_awq_case(side, 4, 72 + (K > 4096), N, K, rows)
    x = synth.activations(4, 300, K, stream=10)
    yt = side.awq_run("gemm", x, aw)
    for lo, hi in ((3, 4), (10, 26), (40, 69), (100, 164)):
        np.testing.assert_array_equal(side.awq_run("gemm", x[lo:hi], aw), yt[lo:hi],
                                      err_msg=f"rows {lo}..{hi}")
    picks = [3, 40, 163, 299]
    yr, b = oracle.awq_linear(x[picks], packed, scales, zeros)
    assert_linear_ok(yt[picks][:, rows], yr, b, f"awq three per CU N={N} K={K}")
