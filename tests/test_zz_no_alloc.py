"""nf4_gemv_argmax_noalloc (scratch in a static device array of the library)
against nf4_gemv_argmax (scratch in a caller workspace): the same y and index
bit for bit, on consecutive calls that share the static array, the later
ones smaller, on the fast GEMV path and on the generic one (a codebook that
needs three bf16 terms), and inside a replayed HIP graph."""
import numpy as np
import pytest

import oracle
from bit_weight_only_amd import synth

from gpu_helpers import Side, oracle_layer, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def side():
    return Side()


def with_workspace(side, xd, M, pw, cb):
    t = side.torch
    y = t.empty((M, pw.N), dtype=t.float32, device="cuda")
    idx = t.full((8,), -7, dtype=t.int32, device="cuda")
    wsb = side.nf4.nf4_gemv_argmax_workspace_bytes(M, pw.N, pw.K)
    ws = t.zeros(wsb, dtype=t.uint8, device="cuda")
    side.stream.wait_stream(t.cuda.current_stream())
    side.nf4.nf4_gemv_argmax(xd, M, pw.qweight, pw.absmax, cb, pw.N, pw.K, y, idx, ws, wsb,
                             stream=side.stream)
    side.sync()
    return y.cpu().numpy(), idx.cpu().numpy()[:M]


def without_workspace(side, xd, M, pw, cb):
    t = side.torch
    y = t.empty((M, pw.N), dtype=t.float32, device="cuda")
    idx = t.full((8,), -7, dtype=t.int32, device="cuda")
    side.stream.wait_stream(t.cuda.current_stream())
    side.nf4.nf4_gemv_argmax_noalloc(xd, M, pw.qweight, pw.absmax, cb, pw.N, pw.K, y, idx,
                                     stream=side.stream)
    side.sync()
    return y.cpu().numpy(), idx.cpu().numpy()[:M]


def three_term_codebook():
    cb = oracle.codebook()[0].astype(np.float64)
    return (cb + np.where(cb != 0, 2.0 ** -12, 0.0)).astype(np.float32)


def test_noalloc_equals_workspace_entry_point(side):
    cb = oracle.codebook()[0]
    # (M, N, K, codebook): decreasing sizes; the last runs the generic path
    calls = [(8, 65536, 3584, cb), (2, 4096, 1024, cb), (1, 512, 256, three_term_codebook())]
    for i, (M, N, K, c) in enumerate(calls):
        say(f"[noalloc] call {i}: M={M} N={N} K={K}")
        _, packed, absmax = oracle_layer(0, 0, 90 + i, N, K, oracle.codebook()[0])
        pw = side.repack(packed, absmax)
        xd = side.x_dev(synth.activations(0, M, K, stream=90 + i))
        y0, i0 = with_workspace(side, xd, M, pw, c)
        y1, i1 = without_workspace(side, xd, M, pw, c)
        assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32)), f"call {i}: y differs"
        assert np.array_equal(i0, i1), f"call {i}: index {i1} != {i0}"
        # the index is the first maximum of the kernel's own y
        assert np.array_equal(i1, np.argmax(y1, axis=1))


def test_noalloc_in_a_replayed_graph(side):
    """Captured once, replayed three times with eager calls of both entry
    points on the same device in between: every replay gives the eager bits."""
    t = side.torch
    cb = oracle.codebook()[0]
    M, N, K = 2, 8192, 3584
    _, packed, absmax = oracle_layer(0, 0, 95, N, K, cb)
    pw = side.repack(packed, absmax)
    xd = side.x_dev(synth.activations(0, M, K, stream=95))
    y_ref, i_ref = with_workspace(side, xd, M, pw, cb)
    y = t.empty((M, N), dtype=t.float32, device="cuda")
    idx = t.full((8,), -7, dtype=t.int32, device="cuda")
    side.sync()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g, stream=side.stream):
        side.nf4.nf4_gemv_argmax_noalloc(xd, M, pw.qweight, pw.absmax, cb, N, K, y, idx,
                                         stream=side.stream)
    side.sync()
    for rep in range(3):
        say(f"[noalloc] graph replay {rep}")
        with t.cuda.stream(side.stream):
            y.fill_(float("nan"))
            idx.fill_(-7)
            g.replay()
        side.sync()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32))
        assert np.array_equal(idx.cpu().numpy()[:M], i_ref)
        y1, i1 = without_workspace(side, xd, M, pw, cb)
        assert np.array_equal(i1, i_ref)
