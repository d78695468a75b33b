"""Helpers for the GPU parity tests: oracle-side reference data and HIP-side
calls through the C ABI on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from bit_weight_only_amd import synth

# decoder shapes (N = out features, K = in features)
QWEN = {"q": (3584, 3584), "k": (512, 3584), "v": (512, 3584), "o": (3584, 3584),
        "gate": (18944, 3584), "up": (18944, 3584), "down": (3584, 18944),
        "lm_head": (152064, 3584)}
QWEN_FUSED = {"qkv": (4608, 3584), "o": (3584, 3584), "gate_up": (37888, 3584),
              "down": (3584, 18944)}
VOXTRAL_FUSED = {"qkv": (6144, 3072), "wo": (3072, 4096), "w13": (18432, 3072),
                 "w2": (3072, 9216)}


def k_parts(N, K):
    """Parts of K as nf4.h documents them: 2 from K = 8192 on; for narrow N
    (fewer than 128 output tiles of 128 x 128 at 1024 rows, counted after
    the first rule) as many as fill 256 CUs once, of at least 4 device tiles
    each."""
    KT = -(-K // 128)
    P = 2 if K >= 8192 else 1
    tiles = -(-(N // 16) // 8) * 8
    if tiles * P < 128:
        P = max(P, min(256 // tiles, KT // 4))
    return P


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def say(*a):
    print(*a, file=sys.stderr, flush=True)


class Side:
    """Torch device memory and a non-default stream for one test module."""

    def __init__(self):
        self.torch = torch_cuda()
        from bit_weight_only_amd import nf4
        self.nf4 = nf4
        nf4.lib()
        self.stream = self.torch.cuda.Stream()

    def to_dev(self, a: np.ndarray):
        t = self.torch.from_numpy(np.ascontiguousarray(a))
        return t.to("cuda", non_blocking=False)

    def sync(self):
        self.stream.synchronize()

    def pack(self, W: np.ndarray, cb):
        N, K = W.shape
        Wd = self.to_dev(W.astype(np.float32))
        pw = self.nf4.PackedWeight(N, K)
        self.nf4.nf4_pack(Wd, N, K, cb, pw.qweight, pw.absmax, stream=self.stream)
        self.sync()
        del Wd
        return pw

    def repack(self, packed: np.ndarray, absmax: np.ndarray):
        N, K2 = packed.shape
        K = 2 * K2
        pw = self.nf4.PackedWeight(N, K)
        c, s = self.to_dev(packed), self.to_dev(absmax.astype(np.float32))
        self.nf4.nf4_repack(c, s, N, K, pw.qweight, pw.absmax, stream=self.stream)
        self.sync()
        return pw

    def unpack(self, pw):
        t = self.torch
        codes = t.empty((pw.N, pw.K // 2), dtype=t.uint8, device="cuda")
        scales = t.empty((pw.N, pw.K // 64), dtype=t.float32, device="cuda")
        self.nf4.nf4_unpack(pw.qweight, pw.absmax, pw.N, pw.K, codes, scales, stream=self.stream)
        self.sync()
        return codes.cpu().numpy(), scales.cpu().numpy()

    def dequant(self, pw, cb):
        t = self.torch
        out = t.empty((pw.N, pw.K), dtype=t.float32, device="cuda")
        self.nf4.nf4_dequant(pw.qweight, pw.absmax, cb, pw.N, pw.K, out, stream=self.stream)
        self.sync()
        return out.cpu().numpy()

    def x_dev(self, x_bits: np.ndarray):
        return self.to_dev(x_bits.astype(np.uint16).view(np.int16))

    def linear(self, kind: str, xd, M: int, pw, cb, y=None, ws=None):
        """ws: a workspace to reuse (zero-filled once by the caller), else a
        fresh zero-filled one of nf4_workspace_bytes."""
        t = self.torch
        if y is None:
            y = t.empty((M, pw.N), dtype=t.float32, device="cuda")
        fn = self.nf4.nf4_gemv if kind == "gemv" else self.nf4.nf4_gemm
        ws_bytes = self.nf4.nf4_workspace_bytes(M, pw.N, pw.K)
        if ws is not None:
            assert ws.numel() >= ws_bytes
        elif ws_bytes:
            ws = t.zeros(max(ws_bytes, 16), dtype=t.uint8, device="cuda")
        self.stream.wait_stream(t.cuda.current_stream())  # the zero fill ran on torch's stream
        fn(xd, M, pw.qweight, pw.absmax, cb, pw.N, pw.K, y, ws, ws_bytes, stream=self.stream)
        self.sync()
        return y

    def run(self, kind: str, x_bits: np.ndarray, pw, cb) -> np.ndarray:
        M = x_bits.shape[0]
        return self.linear(kind, self.x_dev(x_bits), M, pw, cb).cpu().numpy()


    # ---- asymmetric int4, groups of 128
    def awq_pack(self, W: np.ndarray):
        N, K = W.shape
        Wd = self.to_dev(W.astype(np.float32))
        aw = self.nf4.AwqWeight(N, K)
        self.nf4.nf4_awq_pack(Wd, N, K, aw.qweight, aw.params, stream=self.stream)
        self.sync()
        del Wd
        return aw

    def awq_repack(self, packed: np.ndarray, scales: np.ndarray, zeros: np.ndarray):
        """Canonical codes, fp32 scales (binary16 values) and zero points."""
        N, K2 = packed.shape
        K = 2 * K2
        aw = self.nf4.AwqWeight(N, K)
        s16 = np.ascontiguousarray(scales, np.float32).astype(np.float16)
        assert np.array_equal(s16.astype(np.float32), scales), "scales must be binary16 values"
        c, s, z = self.to_dev(packed), self.to_dev(s16.view(np.int16)), self.to_dev(zeros)
        self.nf4.nf4_awq_repack(c, s, z, N, K, aw.qweight, aw.params, stream=self.stream)
        self.sync()
        return aw

    def awq_unpack(self, aw):
        """-> (canonical codes [N, K/2], scales float32 [N, K/128], zeros [N, K/128])."""
        t = self.torch
        G = aw.K // 128
        codes = t.empty((aw.N, aw.K // 2), dtype=t.uint8, device="cuda")
        scales = t.empty((aw.N, G), dtype=t.int16, device="cuda")
        zeros = t.empty((aw.N, G), dtype=t.uint8, device="cuda")
        self.nf4.nf4_awq_unpack(aw.qweight, aw.params, aw.N, aw.K, codes, scales, zeros,
                                stream=self.stream)
        self.sync()
        s16 = scales.cpu().numpy().view(np.float16)
        return codes.cpu().numpy(), s16.astype(np.float32), zeros.cpu().numpy()

    def awq_dequant(self, aw):
        t = self.torch
        out = t.empty((aw.N, aw.K), dtype=t.float32, device="cuda")
        self.nf4.nf4_awq_dequant(aw.qweight, aw.params, aw.N, aw.K, out, stream=self.stream)
        self.sync()
        return out.cpu().numpy()

    def awq_linear(self, kind: str, xd, M: int, aw, y=None, ws=None):
        """ws: a workspace to reuse (any contents), else a fresh one."""
        t = self.torch
        if y is None:
            y = t.empty((M, aw.N), dtype=t.float32, device="cuda")
        fn = self.nf4.nf4_awq_gemv if kind == "gemv" else self.nf4.nf4_awq_gemm
        ws_bytes = self.nf4.nf4_awq_workspace_bytes(M, aw.N, aw.K)
        if ws is None:
            ws = t.empty(max(ws_bytes, 16), dtype=t.uint8, device="cuda")
        assert ws.numel() >= ws_bytes
        self.stream.wait_stream(t.cuda.current_stream())
        fn(xd, M, aw.qweight, aw.params, aw.N, aw.K, y, ws, ws_bytes, stream=self.stream)
        self.sync()
        return y

    def awq_run(self, kind: str, x_bits: np.ndarray, aw) -> np.ndarray:
        M = x_bits.shape[0]
        return self.awq_linear(kind, self.x_dev(x_bits), M, aw).cpu().numpy()


def oracle_awq_layer(cfg, layer, mid, N, K, rows=None):
    """Oracle int4 quantization of the seeded weight (all rows or selected rows):
    (W, canonical codes, scales, zeros)."""
    W = synth.weights(cfg, layer, mid, N, K, rows=rows)
    codes, scales, zeros = oracle.awq_quantize(W)
    return W, oracle.pack(codes), scales, zeros


def oracle_layer(cfg, layer, mid, N, K, cb, rows=None):
    """Oracle quantization of the seeded weight (all rows or selected rows)."""
    W = synth.weights(cfg, layer, mid, N, K, rows=rows)
    codes, absmax = oracle.quantize(W, cb)
    return W, oracle.pack(codes), absmax


def assert_linear_ok(y_test, y_ref, bound, what=""):
    ok, rel, worst = oracle.check_linear(y_test, y_ref, bound)
    assert ok, f"{what}: rel-L2 {rel:.3e} (bar 1e-5), worst element {worst:.3f} x bar"
    return rel, worst
