"""GPU parity of the hot path: nf4_gemv (decode) and nf4_gemm (prefill)
against the oracle on the same seeded inputs.

Bar (floating point): rel-L2 <= 1e-5 per call and every element within
1e-4 * sum_k |x*w|.  Closed forms that must hold bit for bit: one-hot x,
all-zero-code weights, the dyadic exactly-representable case, doubling the
scales, determinism, and rows computed alone vs inside a batch.

Dequantization is fused into the multiply and the decode GEMV is bandwidth
bound (vibevoice.c README, "The kernels that matter"); prefill runs on the
matrix cores ("Quantization" > "Weights", M > 1 bullet).  Shapes: Qwen2-7B
(hidden 3584, MLP 18944, k/v 512, head 152064) and the Voxtral/Mistral
decoder of the ExecuTorch notes ("Model Parameters": dim 3072, 32 q / 8 kv
heads of 128, FFN 9216).
"""
import numpy as np
import pytest

import oracle
from bit_weight_only_amd import synth

from gpu_helpers import (QWEN, QWEN_FUSED, VOXTRAL_FUSED, Side, assert_linear_ok, k_parts,
                         oracle_layer, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def side():
    return Side()


@pytest.fixture(scope="module")
def cb():
    return oracle.codebook()[0]


def case(side, cb, N, K, mid=20, cfg=0, layer=0):
    W, packed, absmax = oracle_layer(cfg, layer, mid, N, K, cb)
    return packed, absmax, side.repack(packed, absmax)


# --------------------------------------------------------------- tiny config
@pytest.mark.parametrize("kind,M", [("gemv", 1), ("gemv", 4), ("gemm", 1), ("gemm", 4)])
def test_tiny_config(side, cb, kind, M):
    """256 x 256 layer, M = 1 and 4, weights packed on the GPU from the seeded W."""
    say(f"[{kind}] tiny M={M}")
    W = synth.weights(0, 0, 0, 256, 256)
    codes, absmax = oracle.quantize(W, cb)
    packed = oracle.pack(codes)
    pw = side.pack(W, cb)
    x = synth.activations(0, M, 256)
    y = side.run(kind, x, pw, cb)
    yr, b = oracle.linear(x, packed, absmax, cb)
    assert_linear_ok(y, yr, b, f"{kind} tiny M={M}")


# --------------------------------------------------------------- edge sweeps
GEMV_EDGES = [(M, N, K) for M in (1, 2, 3, 5, 8) for (N, K) in
              [(16, 64), (48, 192), (512, 256), (16, 3584), (64, 18944), (4608, 128)]]


@pytest.mark.parametrize("M,N,K", GEMV_EDGES)
def test_gemv_edges(side, cb, M, N, K):
    say(f"[gemv] M={M} N={N} K={K}")
    packed, absmax, pw = case(side, cb, N, K, mid=21)
    x = synth.activations(0, M, K, stream=1)
    yr, b = oracle.linear(x, packed, absmax, cb)
    assert_linear_ok(side.run("gemv", x, pw, cb), yr, b, f"gemv M={M} N={N} K={K}")


GEMM_EDGES = [(1, 48, 192), (2, 16, 64), (3, 512, 256), (5, 48, 128), (8, 4608, 256),
              (9, 16, 3584), (16, 256, 192), (113, 512, 3584), (127, 144, 256),
              (128, 128, 128), (129, 400, 320), (256, 64, 18944), (1024, 48, 64),
              (300, 1024, 1024), (17, 512, 18944), (32, 272, 704)]


@pytest.mark.parametrize("M,N,K", GEMM_EDGES)
def test_gemm_edges(side, cb, M, N, K):
    say(f"[gemm] M={M} N={N} K={K}")
    packed, absmax, pw = case(side, cb, N, K, mid=22)
    x = synth.activations(0, M, K, stream=2)
    yr, b = oracle.linear(x, packed, absmax, cb)
    assert_linear_ok(side.run("gemm", x, pw, cb), yr, b, f"gemm M={M} N={N} K={K}")


# --------------------------------------------------------------- closed forms
@pytest.mark.parametrize("kind", ["gemv", "gemm"])
def test_one_hot_rows_are_dequantized_weights(side, cb, kind):
    N, K = 64, 320
    packed, absmax, pw = case(side, cb, N, K, mid=23)
    Wd = oracle.dequant(packed, absmax, cb)
    ks = [0, 1, 63, 64, 127, 128, 200, 319]
    x = np.zeros((len(ks), K), np.uint16)
    x[np.arange(len(ks)), ks] = 0x3F80  # bf16 1.0
    for lo in range(0, len(ks), 8 if kind == "gemv" else len(ks)):
        xs = x[lo:lo + 8]
        y = side.run(kind, xs, pw, cb)
        np.testing.assert_array_equal(y, Wd[:, ks[lo:lo + 8]].T)


@pytest.mark.parametrize("kind", ["gemv", "gemm"])
def test_zero_codes_give_zero(side, cb, kind):
    N, K = 48, 256
    codes = np.full((N, K), 7, np.uint8)
    pw = side.repack(oracle.pack(codes), np.ones((N, K // 64), np.float32))
    y = side.run(kind, synth.activations(0, 4, K), pw, cb)
    assert np.all(y == 0)


@pytest.mark.parametrize("kind,M,N,K", [("gemv", 3, 96, 4096), ("gemm", 37, 160, 4096),
                                        ("gemm", 130, 48, 1024)])
def test_dyadic_exact(side, kind, M, N, K):
    """Codebook (i-7)/8, scales 2^[-4,0], integer x in [-2, 2]: every partial
    sum is exact in fp32, so y equals the integer result in any order."""
    rng = np.random.default_rng(5)
    dy = ((np.arange(16) - 7) / 8).astype(np.float32)
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    e = rng.integers(-4, 1, size=(N, K // 64))
    absmax = np.ldexp(np.float32(1), e).astype(np.float32)
    xi = rng.integers(-2, 3, size=(M, K))
    x = synth.fp32_to_bf16_bits(xi.astype(np.float32))
    pw = side.repack(oracle.pack(codes), absmax)
    W = (codes.astype(np.int64) - 7) * np.repeat(np.left_shift(1, e + 4), 64, axis=1)  # 2^-7 units
    exact = (xi @ W.T).astype(np.float64) / 128.0
    np.testing.assert_array_equal(side.run(kind, x, pw, dy).astype(np.float64), exact)


@pytest.mark.parametrize("kind", ["gemv", "gemm"])
def test_doubling_scales_doubles_output(side, cb, kind):
    N, K, M = 128, 512, 2
    packed, absmax, pw = case(side, cb, N, K, mid=24)
    pw2 = side.repack(packed, absmax * 2)
    x = synth.activations(0, M, K)
    np.testing.assert_array_equal(side.run(kind, x, pw2, cb), 2 * side.run(kind, x, pw, cb))


@pytest.mark.parametrize("kind", ["gemv", "gemm"])
def test_deterministic_and_batch_independent(side, cb, kind):
    N, K = 512, 3584
    packed, absmax, pw = case(side, cb, N, K, mid=25)
    M = 8 if kind == "gemv" else 200
    x = synth.activations(0, M, K)
    y1 = side.run(kind, x, pw, cb)
    y2 = side.run(kind, x, pw, cb)
    np.testing.assert_array_equal(y1, y2)
    for m in (0, M - 1):
        np.testing.assert_array_equal(side.run(kind, x[m:m + 1], pw, cb), y1[m:m + 1])


@pytest.mark.parametrize("N,K", [(512, 3584), (256, 18944), (272, 704), (272, 8256),
                                 (512, 8192), (4608, 3584), (4608, 8192), (16, 18944)])
def test_gemm_skinny_and_tiled_rows_identical(side, cb, N, K):
    """nf4_gemm runs a batch of up to 32 rows on the narrow path (these
    matrices have at most 1024 row groups: the four waves of a workgroup
    take turns over one row group's tiles and fold in K order), up to 64
    rows on the skinny path (one wave per row group streaming all of K) and
    a wide batch on the tiled path; all perform the same operations per
    output, so rows agree bit for bit whichever path the batch size selects
    (K = 704 and 8256 end in a half tile).  K is summed in the same parts on
    every path (k_parts: 1 to 32 here), on separate workgroups of the tiled
    path and one after the other in the other two.  Narrow grids of more
    workgroups than CUs (N = 4608: 288 row groups per 16-row block) take
    the form with two workgroups per CU, K in one part (K = 3584) and in two
    (K = 8192); smaller grids the form with one."""
    packed, absmax, pw = case(side, cb, N, K, mid=27)
    x = synth.activations(0, 300, K, stream=3)
    yt = side.run("gemm", x, pw, cb)            # 300 rows: tiled
    for M, m0 in ((1, 0), (1, 299), (16, 3), (29, 17), (32, 100), (33, 150), (64, 200),
                  (256, 40)):
        np.testing.assert_array_equal(side.run("gemm", x[m0:m0 + M], pw, cb), yt[m0:m0 + M],
                                      err_msg=f"M={M} rows {m0}..")
    yr, b = oracle.linear(x[[0, 17, 299]], packed, absmax, cb)
    assert_linear_ok(yt[[0, 17, 299]], yr, b, f"tiled N={N} K={K}")


@pytest.mark.parametrize("N,K", [(3584, 18944), (3584, 8256), (3072, 9216), (2048, 8256),
                                 (3584, 3584), (2048, 704)])
def test_gemm_stream_rows_identical(side, cb, N, K):
    """Up to 16 rows on a matrix whose row groups fit the CUs once, with K
    in one or two parts, run the stream path (x and code words loaded
    straight into registers; with two parts, two groups of four waves fold
    part 0 and part 1 side by side and add them in part order).  Its rows
    equal the tiled path's bit for bit and sampled rows meet the bar against
    the oracle.  Shapes: down (K in halves of 74 tiles), K = 8256 (halves of
    33 and 32 tiles, the last one half: part 1's group runs one window with
    no tile of its own), Voxtral's w2, o (one part, 28 tiles) and a 6-tile K
    whose last tile is half (no steady loop)."""
    assert k_parts(N, K) <= 2 and N // 16 <= 256
    packed, absmax, pw = case(side, cb, N, K, mid=29)
    x = synth.activations(0, 300, K, stream=4)
    yt = side.run("gemm", x, pw, cb)            # 300 rows: tiled
    for M, m0 in ((1, 0), (1, 299), (3, 7), (8, 100), (13, 31), (16, 284)):
        say(f"[gemm] stream N={N} K={K} M={M} rows {m0}..")
        np.testing.assert_array_equal(side.run("gemm", x[m0:m0 + M], pw, cb), yt[m0:m0 + M],
                                      err_msg=f"N={N} K={K} M={M} rows {m0}..")
    picks = [0, 31, 299]
    yr, b = oracle.linear(x[picks], packed, absmax, cb)
    assert_linear_ok(yt[picks], yr, b, f"stream shapes N={N} K={K}")


def test_gemm_k_halves_repeat(side, cb):
    """K = 8320 (65 device tiles) at N = 1024 is summed in halves of 33 and 32
    tiles that meet through the workspace: calls with other inputs in
    between leave nothing behind (the arrival counters return to zero), and
    sampled rows match the oracle."""
    N, K, M = 1024, 8320, 520
    assert k_parts(N, K) == 2
    packed, absmax, pw = case(side, cb, N, K, mid=28)
    x1 = synth.activations(0, M, K, stream=5)
    x2 = synth.activations(0, M, K, stream=6)
    t = side.torch
    ws = t.zeros(side.nf4.nf4_workspace_bytes(M, N, K), dtype=t.uint8, device="cuda")
    assert ws.numel() > 0
    run = lambda x: side.linear("gemm", side.x_dev(x), M, pw, cb, ws=ws).cpu().numpy()
    y1 = run(x1)
    y2 = run(x2)
    np.testing.assert_array_equal(run(x1), y1)
    np.testing.assert_array_equal(side.run("gemm", x2, pw, cb), y2)  # a fresh workspace
    picks = np.array([0, 127, 128, 300, 519])
    for x, y in ((x1, y1), (x2, y2)):
        yr, b = oracle.linear(x[picks], packed, absmax, cb)
        assert_linear_ok(y[picks], yr, b, "K halves")


def test_gemm_workspace_shared_by_shapes_and_garbage(side, cb):
    """One workspace serves GEMMs with K in parts of different shapes: the
    arrival counters of a call with more output tiles lie where a call with
    fewer kept part sums, so every call clears its counters first.  Calls on
    a workspace full of 0xFF bytes, and alternating between M = 520 and
    M = 1040 (twice the tiles), give the bits of a fresh workspace."""
    N, K = 1024, 8320
    assert k_parts(N, K) == 2
    packed, absmax, pw = case(side, cb, N, K, mid=29)
    t = side.torch
    xs = {M: side.x_dev(synth.activations(0, M, K, stream=M)) for M in (520, 1040)}
    fresh = {M: side.linear("gemm", xs[M], M, pw, cb).cpu().numpy() for M in xs}
    wsb = max(side.nf4.nf4_workspace_bytes(M, N, K) for M in xs)
    ws = t.full((wsb,), 255, dtype=t.uint8, device="cuda")
    for M in (1040, 520, 1040, 520, 520, 1040):
        y = side.linear("gemm", xs[M], M, pw, cb, ws=ws).cpu().numpy()
        np.testing.assert_array_equal(y, fresh[M])
    picks = np.array([0, 519, 1039])
    x = synth.activations(0, 1040, K, stream=1040)
    yr, b = oracle.linear(x[picks], packed, absmax, cb)
    assert_linear_ok(fresh[1040][picks], yr, b, "shared workspace")


def test_gemv_and_gemm_agree(side, cb):
    N, K = 1024, 3584
    packed, absmax, pw = case(side, cb, N, K, mid=26)
    x = synth.activations(0, 8, K)
    yv, ym = side.run("gemv", x, pw, cb), side.run("gemm", x, pw, cb)
    yr, b = oracle.linear(x, packed, absmax, cb)
    assert_linear_ok(yv, yr, b, "gemv")
    assert_linear_ok(ym, yr, b, "gemm")


@pytest.mark.parametrize("kind,N,K", [("gemv", 256, 256), ("gemm", 256, 256),
                                      ("gemm", 64, 3584), ("gemm", 32, 8256)])
def test_codebook_needing_three_bf16_terms(side, kind, N, K):
    """A codebook that is not bf16-exact (the unrounded quantiles as fp32)
    runs as three exact bf16 terms (the generic kernels; the GEMM with K in
    1, 7 and 16 parts here)."""
    _, unr = oracle.codebook()
    cb32 = unr.astype(np.float32)
    W = synth.weights(0, 0, 30, N, K)
    codes, absmax = oracle.quantize(W, cb32)
    packed = oracle.pack(codes)
    pw = side.pack(W, cb32)
    gc, gs = side.unpack(pw)
    np.testing.assert_array_equal(gc, packed)
    x = synth.activations(0, 4, K)
    yr, b = oracle.linear(x, packed, absmax, cb32)
    assert_linear_ok(side.run(kind, x, pw, cb32), yr, b, f"{kind} 3-term codebook")
    if kind == "gemm":
        assert k_parts(N, K) == {256: 1, 3584: 7, 8256: 16}[K]


def test_fused_projection_slices_equal_separate_calls(side, cb):
    """q|k|v concatenated along N at pack time: each column slice of one call
    matches the separate projection (vibevoice.c README, decode GEMV bullet:
    same-input projections share one launch).  The GEMM computes each output
    from the same operations when both matrices sum K in the same parts, so
    those slices are bit-identical (q and q|k|v; two 4096-row halves of an
    8192-row matrix: one part each); k and v alone are narrow enough to take
    more parts of K, and the GEMV splits the fused matrix's tiles over waves
    differently from the separate ones: those slices agree to the oracle's
    bar."""
    K = 3584
    parts = [oracle_layer(2, 0, mid, n, K, cb) for mid, n in
             [(synth.Q, 3584), (synth.K_, 512), (synth.V, 512)]]
    fused = side.repack(np.vstack([p[1] for p in parts]), np.vstack([p[2] for p in parts]))
    x = synth.activations(2, 2, K)
    yf = side.run("gemv", x, fused, cb)
    yg = side.run("gemm", x, fused, cb)
    col = 0
    for W, packed, absmax in parts:
        n = packed.shape[0]
        pw = side.repack(packed, absmax)
        yr, b = oracle.linear(x, packed, absmax, cb)
        assert_linear_ok(yf[:, col:col + n], yr, b, "fused gemv slice")
        assert_linear_ok(side.run("gemv", x, pw, cb), yr, b, "separate gemv")
        ys = side.run("gemm", x, pw, cb)
        if k_parts(n, K) == k_parts(fused.N, K):
            np.testing.assert_array_equal(yg[:, col:col + n], ys)
        else:
            assert_linear_ok(yg[:, col:col + n], yr, b, "fused gemm slice")
            assert_linear_ok(ys, yr, b, "separate gemm")
        col += n
    assert [k_parts(p[1].shape[0], K) for p in parts] == [1, 7, 7]
    # two halves with the fused matrix's parts: bit-identical GEMM slices
    halves = [oracle_layer(2, 1, mid, 4096, K, cb) for mid in (synth.Q, synth.O)]
    assert k_parts(8192, K) == k_parts(4096, K) == 1
    fused = side.repack(np.vstack([p[1] for p in halves]), np.vstack([p[2] for p in halves]))
    yg = side.run("gemm", x, fused, cb)
    for i, (W, packed, absmax) in enumerate(halves):
        np.testing.assert_array_equal(yg[:, 4096 * i:4096 * (i + 1)],
                                      side.run("gemm", x, side.repack(packed, absmax), cb))


# --------------------------------------------------------------- full sizes
_FULL = {}


def full_case(side, cb, cfg, mid, N, K, sample_rows):
    """Pack the full seeded weight on the GPU; the oracle quantizes only the
    sampled output rows (regenerated from the same counter-based stream)."""
    key = (cfg, mid, N, K, tuple(sample_rows))
    if key in _FULL:
        return _FULL[key]
    _FULL.clear()
    W = synth.weights(cfg, 0, mid, N, K)
    pw = side.pack(W, cb)
    del W
    Wr = synth.weights(cfg, 0, mid, N, K, rows=sample_rows)
    codes, absmax = oracle.quantize(Wr, cb)
    _FULL[key] = (pw, oracle.pack(codes), absmax)
    return _FULL[key]


def sample_rows(N, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 15, 16, N // 2, N - 16, N - 1],
                                     rng.integers(0, N, 250)]))


@pytest.mark.parametrize("name", list(VOXTRAL_FUSED))
def test_voxtral_decode_full_size(side, cb, name):
    N, K = VOXTRAL_FUSED[name]
    say(f"[gemv] voxtral {name} N={N} K={K}")
    rows = sample_rows(N, 1)
    pw, packed, absmax = full_case(side, cb, 1, 40 + list(VOXTRAL_FUSED).index(name), N, K, rows)
    x = synth.activations(1, 1, K)
    y = side.run("gemv", x, pw, cb)
    yr, b = oracle.linear(x, packed, absmax, cb)
    assert_linear_ok(y[:, rows], yr, b, f"voxtral {name}")
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("M", [1, 2])
@pytest.mark.parametrize("name", list(QWEN_FUSED) + ["lm_head"])
def test_qwen_decode_full_size(side, cb, name, M):
    N, K = QWEN_FUSED.get(name) or QWEN[name]
    say(f"[gemv] qwen {name} M={M} N={N} K={K}")
    rows = sample_rows(N, 2)
    pw, packed, absmax = full_case(side, cb, 2, 50 + (list(QWEN_FUSED) + ["lm_head"]).index(name),
                                   N, K, rows)
    x = synth.activations(2, M, K)
    y = side.run("gemv", x, pw, cb)
    yr, b = oracle.linear(x, packed, absmax, cb)
    assert_linear_ok(y[:, rows], yr, b, f"qwen {name} M={M}")
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("M", [3, 8])
def test_qwen_down_decode_batch(side, cb, M):
    """A decode batch of 3 to 8 slots through down (K = 18944): x is too long
    for the fast GEMV's LDS, so nf4_gemv takes the stream path (two groups
    of four waves fold the two halves of K side by side).  Sampled columns
    meet the bar against the oracle, and the rows equal nf4_gemm's."""
    N, K = QWEN_FUSED["down"]
    say(f"[gemv] qwen down batch M={M}")
    rows = sample_rows(N, 2)
    pw, packed, absmax = full_case(side, cb, 2, 61, N, K, rows)
    x = synth.activations(2, M, K, stream=M)
    y = side.run("gemv", x, pw, cb)
    yr, b = oracle.linear(x, packed, absmax, cb)
    assert_linear_ok(y[:, rows], yr, b, f"qwen down M={M}")
    np.testing.assert_array_equal(side.run("gemm", x, pw, cb), y)


@pytest.mark.parametrize("name", list(QWEN_FUSED))
def test_qwen_prefill_full_size(side, cb, name):
    """M = 1024 prefill chunk; all N columns on token rows {0, 1023, 6 seeded}."""
    N, K = QWEN_FUSED[name]
    say(f"[gemm] qwen prefill {name} M=1024 N={N} K={K}")
    rows = sample_rows(N, 3)
    pw, packed, absmax = full_case(side, cb, 3, 60 + list(QWEN_FUSED).index(name), N, K, rows)
    x = synth.activations(3, 1024, K)
    y = side.run("gemm", x, pw, cb)
    toks = np.unique(np.concatenate([[0, 1023], np.random.default_rng(4).integers(0, 1024, 6)]))
    yr, b = oracle.linear(x[toks], packed, absmax, cb)
    assert_linear_ok(y[toks][:, rows], yr, b, f"prefill {name}")
    assert np.all(np.isfinite(y))
    # the same bits again (down: the halves' counters are back at zero), and
    # single rows on the skinny path equal the rows of the tiled launch
    np.testing.assert_array_equal(side.run("gemm", x, pw, cb), y)
    for m in (0, 1023):
        np.testing.assert_array_equal(side.run("gemm", x[m:m + 1], pw, cb), y[m:m + 1])


def test_long_audio_prefill_chunks_and_tail(side, cb):
    """M = 14449 = 14 x 1024 + 113 through the o projection in chunks; every
    row of the 113-row tail and sampled rows of each chunk against the oracle,
    and the tail equals the same rows computed inside a full chunk."""
    N, K = QWEN_FUSED["o"]
    M = 14449
    packed, absmax, pw = case(side, cb, N, K, mid=70, cfg=4)
    x = synth.activations(4, M, K)
    xd = side.x_dev(x)
    y = side.torch.empty((M, N), dtype=side.torch.float32, device="cuda")
    for c0 in range(0, M, 1024):
        rows = min(1024, M - c0)
        say(f"[gemm] long-audio chunk rows {c0}..{c0 + rows}")
        side.linear("gemm", xd[c0:c0 + rows], rows, pw, cb, y=y[c0:c0 + rows])
    y = y.cpu().numpy()
    tail = np.arange(14336, M)
    yr, b = oracle.linear(x[tail], packed, absmax, cb)
    assert_linear_ok(y[tail], yr, b, "long-audio tail")
    picks = np.concatenate([[c, c + 1023] for c in range(0, 14336, 1024)])
    yr, b = oracle.linear(x[picks], packed, absmax, cb)
    assert_linear_ok(y[picks], yr, b, "long-audio chunk rows")
    # the ragged tail inside a full 1024-row chunk
    xin = side.x_dev(x[M - 1024:])
    yin = side.linear("gemm", xin, 1024, pw, cb).cpu().numpy()
    np.testing.assert_array_equal(yin[1024 - 113:], y[tail])


def test_gemm_k_parts_in_a_replayed_graph(side, cb):
    """The parts of K meet through counters that each call sets back to zero
    itself (no memset anywhere): a HIP graph holding two GEMMs with K in parts
    (N = 512, K = 3584: 7 parts; N = 256, K = 18944: 16 parts) replays with
    the eager results bit for bit, with eager calls on the same workspace and
    fills of y between the replays."""
    t = side.torch
    M = 300
    shapes = [(512, 3584, 41), (256, 18944, 42)]
    assert [k_parts(N, K) for N, K, _ in shapes] == [7, 16]
    wsb = max(side.nf4.nf4_workspace_bytes(M, N, K) for N, K, _ in shapes)
    ws = t.zeros(wsb, dtype=t.uint8, device="cuda")
    cases, eager = [], []
    for N, K, mid in shapes:
        packed, absmax, pw = case(side, cb, N, K, mid=mid)
        xd = side.x_dev(synth.activations(0, M, K, stream=mid))
        eager.append(side.linear("gemm", xd, M, pw, cb, ws=ws).clone())
        cases.append((pw, xd, t.empty((M, N), dtype=t.float32, device="cuda")))
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g, stream=side.stream):
        for pw, xd, y in cases:
            side.nf4.nf4_gemm(xd, M, pw.qweight, pw.absmax, cb, pw.N, pw.K, y, ws, wsb,
                              stream=side.stream)
    side.sync()
    for rep in range(3):
        with t.cuda.stream(side.stream):
            for _, _, y in cases:
                y.fill_(float("nan"))
            g.replay()
        side.sync()
        for (pw, xd, y), y0 in zip(cases, eager):
            assert t.equal(y.view(t.int32), y0.view(t.int32)), f"replay {rep} N={pw.N} K={pw.K}"
        # an eager call on the shared workspace between replays
        pw, xd, _ = cases[rep % 2]
        assert t.equal(side.linear("gemm", xd, M, pw, cb, ws=ws).view(t.int32),
                       eager[rep % 2].view(t.int32))


@pytest.mark.parametrize("N,K", [(37888, 3584), (33024, 8192), (33040, 1088)])
def test_gemm_skinny_three_per_cu_rows_identical(side, cb, N, K):
    """Skinny grids of more than two rounds of two workgroups per CU (more
    than 2048 row groups up to 32 rows, 1024 from 33 to 64 rows: gate|up
    shapes) run three workgroups per CU with half the tiles in flight and a
    16-copy pair table.  Rows agree bit for bit with the tiled path, with K
    in one part and in two, and with a row-group count that leaves the last
    workgroup partly empty and a K that ends in a half tile (N = 33040,
    K = 1088); sampled outputs match the oracle."""
    say(f"[gemm] skinny, three per CU: N={N} K={K}")
    rows = sample_rows(N, 7)
    pw, packed, absmax = full_case(side, cb, 4, 70 + (K > 4096) + 2 * (K % 128 != 0), N, K,
                                   rows)
    x = synth.activations(4, 300, K, stream=9)
    yt = side.run("gemm", x, pw, cb)
    for M, m0 in ((1, 5), (16, 20), (29, 40), (64, 100)):
        np.testing.assert_array_equal(side.run("gemm", x[m0:m0 + M], pw, cb), yt[m0:m0 + M],
                                      err_msg=f"M={M} rows {m0}..")
    picks = [5, 40, 163, 299]
    yr, b = oracle.linear(x[picks], packed, absmax, cb)
    assert_linear_ok(yt[picks][:, rows], yr, b, f"three per CU N={N} K={K}")


@pytest.mark.parametrize("N", [3584, 3328])
def test_gemm_fourteen_row_group_tiles(side, cb, N):
    """A tiled grid with K in parts that would leave CUs idle at 16 row
    groups per workgroup (K = 8192 in two parts, 600 rows; N = 3584: 140
    workgroups, N = 3328: 130) runs 14 row groups per workgroup (160 and
    150; at N = 3328 the last tile holds 12 row groups): rows equal the
    skinny path's bit for bit (the ragged last row tile included), a reused
    workspace full of stale bytes gives the same bits, and sampled outputs
    match the oracle."""
    K, M = 8192, 600
    assert k_parts(N, K) == 2
    packed, absmax, pw = case(side, cb, N, K, mid=43 + (N != 3584))
    x = synth.activations(0, M, K, stream=14)
    t = side.torch
    ws = t.full((side.nf4.nf4_workspace_bytes(M, N, K),), 0xFF, dtype=t.uint8, device="cuda")
    xd = side.x_dev(x)
    y1 = side.linear("gemm", xd, M, pw, cb, ws=ws).cpu().numpy()
    np.testing.assert_array_equal(side.linear("gemm", xd, M, pw, cb, ws=ws).cpu().numpy(), y1)
    for m0 in (0, 536):
        np.testing.assert_array_equal(side.run("gemm", x[m0:m0 + 64], pw, cb), y1[m0:m0 + 64],
                                      err_msg=f"rows {m0}..")
    picks = [0, 127, 128, 511, 599]
    yr, b = oracle.linear(x[picks], packed, absmax, cb)
    assert_linear_ok(y1[picks], yr, b, f"14 row groups per workgroup, N={N}")
