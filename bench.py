"""Throughput of the NF4 4-bit weight-only linear layer on one MI355X.

One step = one pass of the hot path over one batch of synthetic input on the
Qwen2-7B-shaped decoder (hidden 3584, MLP 18944, k/v 512, head 152064):
  decode : M = 1, 28 layers x {q|k|v, o, gate|up, down} + lm_head = 113
           nf4_gemv launches reading 3.977 GB of packed weights;
  prefill: M = 1024, 28 layers x the same 4 fused linears = 112 nf4_gemm
           launches, 13.364 TFLOP.
Weights are seeded N(0, 0.02^2) fp32 drawn on the GPU and quantized there by
nf4_pack (load time, untimed); activations are seeded N(0, 1) in bf16.  Each
sequence is captured once in a HIP graph and replayed.  Every decode launch
names the next one's matrix as its read-ahead hint (nf4_gemv_prefetch):
a decoder knows its weights ahead of the activations.  The JSON line's
`value` is decode packed-weight GB/s over the whole step (launch gaps
included); prefill TFLOP/s sits beside it.

`int4_group128` repeats decode, prefill and both rooflines with the same
seeded weights quantized to the second format, asymmetric int4 in groups of
128 (nf4_awq_pack; nf4_awq_gemv_prefetch with the same read-ahead hints /
nf4_awq_gemm; algorithmic bytes N K / 2 + 4 N K / 128: codes and one 4-byte
(s, z) per group).

`roofline` covers the dominant decode kernel (the gate|up GEMV, 28 launches
per step): its 28 launches on distinct weights are replayed back to back in
one graph, each naming the next as its hint as in the step, each replay
timed with events on the launch stream; the median
replay / 28 is the launch duration.  `roofline_prefill`
does the same for the gate|up GEMM.  `traffic` is the HBM bytes per launch
from rocprofv3 counters (FETCH_SIZE + WRITE_SIZE, each scaled by what the
counter reads for a plain 1 GiB copy), recorded below together with a hash of
the kernel source they were taken on; it is null when the source differs.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu] [--no-int4]
    python bench.py --pmc-pass          # workload for rocprofv3 --pmc runs
    python bench.py --summarize DIR --launch-log FILE --title T --command C
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
CSRC = os.path.join(ROOT, "bit_weight_only_amd", "csrc")

METRIC = "decode GEMV packed-weight GB/s (M=1) + prefill GEMM TFLOP/s (M=1024), Qwen2-7B"
HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (published)

LAYERS = 28
HIDDEN, MLP, KV, VOCAB = 3584, 18944, 512, 152064
LINEARS = [("qkv", HIDDEN + 2 * KV, HIDDEN), ("o", HIDDEN, HIDDEN),
           ("gate_up", 2 * MLP, HIDDEN), ("down", HIDDEN, MLP)]
PREFILL_M = 1024
TAIL_M = 113  # last chunk of the 14449-row long-audio prompt
CHUNK_M = 29  # rows of one chunk of streamed input
DOMINANT = ("gate_up", 2 * MLP, HIDDEN)
# the unfused 7-linear sequence: (linear, fused matrix, first row, end row)
UNFUSED = [("q", "qkv", 0, HIDDEN), ("k", "qkv", HIDDEN, HIDDEN + KV),
           ("v", "qkv", HIDDEN + KV, HIDDEN + 2 * KV), ("o", "o", 0, HIDDEN),
           ("gate", "gate_up", 0, MLP), ("up", "gate_up", MLP, 2 * MLP), ("down", "down", 0, HIDDEN)]
# Voxtral/Mistral-shaped decoder (hidden 3072, q 4096, k and v 1024 each, FFN 9216)
VOXTRAL_LAYERS = 26
VOXTRAL = [("qkv", 6144, 3072), ("wo", 3072, 4096), ("w13", 18432, 3072), ("w2", 3072, 9216)]
LONG_M, LONG_CHUNKS = 14449, 14  # the long-audio prompt: 14 x 1024 rows + the 113-row tail

# HBM traffic per launch of the dominant kernels, from rocprofv3 --pmc runs of
# `python bench.py --pmc-pass` (profiles/hbm_traffic_gate_up.md): counter KiB
# per dispatch and the calibration of each counter on a plain 1 GiB copy.
TRAFFIC = {
    "gemv": {"source": "gemv.hip", "fetch_kib": 42713, "write_kib": 148,
             "sha256": "06d88eadf44e341f16f0ed60b6f9b9a215b0837c03260c23416ab488040e22aa"},
    "gemm": {"source": "gemm.hip", "fetch_kib": 180759, "write_kib": 151961,
             "sha256": "48ca7077af481c8e09889f6509177380f245e767fa71cb5cbf878ecfb837e4f2"},
    "awq_gemv": {"source": "gemv.hip", "fetch_kib": 40355, "write_kib": 148,
                 "sha256": "06d88eadf44e341f16f0ed60b6f9b9a215b0837c03260c23416ab488040e22aa"},
    "awq_gemm": {"source": "gemm.hip", "fetch_kib": 180913, "write_kib": 151929,
                 "sha256": "48ca7077af481c8e09889f6509177380f245e767fa71cb5cbf878ecfb837e4f2"},
}
COPY_CALIBRATION = {"fetch_kib_per_gib": 524308, "write_kib_per_gib": 1048576}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def awq_packed_bytes(N, K):
    """Algorithmic bytes of an int4 (group 128) matrix: codes + 4 B per group."""
    return N * K // 2 + 4 * N * (K // 128)


def packed_bytes(N, K):
    return N * K // 2 + 4 * N * (K // 64)


def cpu_threads():
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return n


def source_sha256(name):
    with open(os.path.join(CSRC, name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_bytes(kind):
    """HBM bytes per launch from the recorded counters, or None when they
    were not taken or the kernel source changed since."""
    t, cal = TRAFFIC[kind], COPY_CALIBRATION
    if t is None:
        return None
    if None in (t["sha256"], t["fetch_kib"], t["write_kib"], cal["fetch_kib_per_gib"],
                cal["write_kib_per_gib"]):
        return None
    if source_sha256(t["source"]) != t["sha256"]:
        return None
    gib = float(1 << 30)
    return int(t["fetch_kib"] / cal["fetch_kib_per_gib"] * gib +
               t["write_kib"] / cal["write_kib_per_gib"] * gib)


def cpu_baseline(target_s: float):
    """The oracle (scalar dequant + fp64 dot, threads over rows) on a bounded
    sample of the decode workload: 2048 output rows of each fused linear of
    layer 0 at M = 1, repeated until about `target_s` seconds elapse."""
    import numpy as np

    import oracle
    from bit_weight_only_amd import synth

    cb, _ = oracle.codebook()
    threads = cpu_threads()
    rows = 2048
    mats = []
    for i, (name, N, K) in enumerate(LINEARS):
        sel = np.arange(rows) * (N // rows)
        W = synth.weights(2, 0, 50 + i, N, K, rows=sel)
        codes, absmax = oracle.quantize(W, cb, threads=threads)
        mats.append((oracle.pack(codes), absmax, synth.activations(2, 1, K), K))
    per_pass = sum(packed_bytes(rows, K) for _, _, _, K in mats)
    done, t0 = 0, time.perf_counter()
    while True:
        for packed, absmax, x, K in mats:
            oracle.linear(x, packed, absmax, cb, threads=threads)
        done += 1
        el = time.perf_counter() - t0
        if el >= target_s:
            break
    return {"value": round(done * per_pass / el / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{rows} output rows of each of the 4 fused layer linears (layer 0), M=1, "
                      f"{done} passes of {per_pass / 1e6:.1f} MB packed weight in {el:.1f} s"}


class Model:
    """Packed weights of the 28 layers + lm_head and the activation buffers."""

    def __init__(self, torch, nf4, cb, seed, stream, layers=LAYERS, with_head=True,
                 only=None):
        dev = "cuda"
        self.torch, self.nf4, self.cb, self.s = torch, nf4, cb, stream
        gen = torch.Generator(device=dev)
        self.weights = []
        with torch.cuda.stream(stream):
            for layer in range(layers):
                lw = {}
                for i, (name, N, K) in enumerate(LINEARS):
                    if only is not None and name not in only:
                        continue
                    gen.manual_seed(seed + 16 * layer + i)
                    W = torch.randn((N, K), generator=gen, device=dev, dtype=torch.float32) * 0.02
                    lw[name] = nf4.pack_weight(W, cb, stream=stream)
                    del W
                self.weights.append(lw)
            self.lm_head = None
            if with_head:
                gen.manual_seed(seed + 16 * LAYERS)
                W = torch.randn((VOCAB, HIDDEN), generator=gen, device=dev,
                                dtype=torch.float32) * 0.02
                self.lm_head = nf4.pack_weight(W, cb, stream=stream)
                del W
        stream.synchronize()
        torch.cuda.empty_cache()

        def bf16_randn(M, K, s):
            gen.manual_seed(s)
            return torch.randn((M, K), generator=gen, device=dev).to(torch.bfloat16).view(
                torch.int16)

        self.x1 = {K: bf16_randn(1, K, seed + 1000 + K) for K in (HIDDEN, MLP)}
        # two decode slots (M = 2)
        self.x2 = {K: bf16_randn(2, K, seed + 3000 + K) for K in (HIDDEN, MLP)}
        self.y2 = {name: torch.empty((2, N), dtype=torch.float32, device=dev)
                   for name, N, _ in LINEARS}
        self.y2["lm_head"] = torch.empty((2, VOCAB), dtype=torch.float32, device=dev)
        self.xp = {K: bf16_randn(PREFILL_M, K, seed + 2000 + K) for K in (HIDDEN, MLP)}
        self.y1 = {name: torch.empty((1, N), dtype=torch.float32, device=dev)
                   for name, N, _ in LINEARS}
        self.y1["lm_head"] = torch.empty((1, VOCAB), dtype=torch.float32, device=dev)
        self.yp = {name: torch.empty((PREFILL_M, N), dtype=torch.float32, device=dev)
                   for name, N, _ in LINEARS}
        self.ws_bytes = max([nf4.nf4_workspace_bytes(M, N, K) for M in (1, CHUNK_M, TAIL_M, PREFILL_M)
                             for _, N, K in LINEARS] + [nf4.nf4_workspace_bytes(1, VOCAB, HIDDEN)])
        self.ws = torch.zeros(max(self.ws_bytes, 16), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()  # inputs and the zeroed workspace are ready before stream s runs

    def packed(self, name, layer):
        return self.lm_head if name == "lm_head" else self.weights[layer][name]

    def gemv(self, name, layer, nxt=None, M=1):
        """One decode GEMV (M = 1 or 2 rows); nxt = (name, layer) of the next
        launch on the stream, named as a read-ahead hint (nf4_gemv_prefetch)."""
        pw = self.packed(name, layer)
        x, y = (self.x1[pw.K], self.y1[name]) if M == 1 else (self.x2[pw.K], self.y2[name])
        if nxt is None:
            self.nf4.nf4_gemv(x, M, pw.qweight, pw.absmax, self.cb, pw.N, pw.K, y, self.ws,
                              self.ws_bytes)
        else:
            npw = self.packed(*nxt)
            self.nf4.nf4_gemv_prefetch(x, M, pw.qweight, pw.absmax, self.cb, pw.N, pw.K, y,
                                       self.ws, self.ws_bytes, npw.qweight, npw.absmax, npw.N,
                                       npw.K)

    def gemm(self, name, layer):
        pw = self.weights[layer][name]
        K = pw.K
        self.nf4.nf4_gemm(self.xp[K], PREFILL_M, pw.qweight, pw.absmax, self.cb, pw.N, K,
                          self.yp[name], self.ws, self.ws_bytes)


class AwqModel:
    """The same seeded weights quantized to the int4 group-128 format; shares
    the activation and output buffers of `base`."""

    def __init__(self, torch, nf4, seed, stream, base, layers=LAYERS, with_head=True, only=None):
        dev = "cuda"
        self.torch, self.nf4, self.s, self.base = torch, nf4, stream, base
        gen = torch.Generator(device=dev)
        self.weights = []
        with torch.cuda.stream(stream):
            for layer in range(layers):
                lw = {}
                for i, (name, N, K) in enumerate(LINEARS):
                    if only is not None and name not in only:
                        continue
                    gen.manual_seed(seed + 16 * layer + i)
                    W = torch.randn((N, K), generator=gen, device=dev, dtype=torch.float32) * 0.02
                    lw[name] = nf4.awq_pack_weight(W, stream=stream)
                    del W
                self.weights.append(lw)
            self.lm_head = None
            if with_head:
                gen.manual_seed(seed + 16 * LAYERS)
                W = torch.randn((VOCAB, HIDDEN), generator=gen, device=dev,
                                dtype=torch.float32) * 0.02
                self.lm_head = nf4.awq_pack_weight(W, stream=stream)
                del W
        stream.synchronize()
        torch.cuda.empty_cache()
        self.ws_bytes = max(nf4.nf4_awq_workspace_bytes(M, N, K)
                            for M in (1, CHUNK_M, TAIL_M, PREFILL_M) for _, N, K in LINEARS)
        self.ws = torch.zeros(max(self.ws_bytes, 16), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    def packed(self, name, layer):
        return self.lm_head if name == "lm_head" else self.weights[layer][name]

    def gemv(self, name, layer, nxt=None):
        """One decode GEMV; nxt = (name, layer) of the next launch, named as
        a read-ahead hint (nf4_awq_gemv_prefetch)."""
        aw, b = self.packed(name, layer), self.base
        if nxt is None:
            self.nf4.nf4_awq_gemv(b.x1[aw.K], 1, aw.qweight, aw.params, aw.N, aw.K, b.y1[name],
                                  self.ws, self.ws_bytes)
        else:
            na = self.packed(*nxt)
            self.nf4.nf4_awq_gemv_prefetch(b.x1[aw.K], 1, aw.qweight, aw.params, aw.N, aw.K,
                                           b.y1[name], self.ws, self.ws_bytes, na.qweight,
                                           na.params, na.N, na.K)

    def gemm(self, name, layer, M=PREFILL_M):
        aw, b = self.weights[layer][name], self.base
        self.nf4.nf4_awq_gemm(b.xp[aw.K], M, aw.qweight, aw.params, aw.N, aw.K, b.yp[name],
                              self.ws, self.ws_bytes)


def decode_labels():
    return [name for _ in range(LAYERS) for name, _, _ in LINEARS] + ["lm_head"]


def prefill_labels():
    return [name for _ in range(LAYERS) for name, _, _ in LINEARS]


def graph_ms(torch, stream, fn, replays, warm=1):
    """Capture fn once on `stream`, replay it, return the median ms per
    replay (a pair of events on the launch stream around each replay)."""
    import statistics
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    stream.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(warm):
            g.replay()
    stream.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(replays)]
    with torch.cuda.stream(stream):
        for e0, e1 in ev:
            e0.record(stream)
            g.replay()
            e1.record(stream)
    stream.synchronize()
    return statistics.median(e0.elapsed_time(e1) for e0, e1 in ev)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-int4", action="store_true",
                    help="skip the int4 group-128 format's decode and prefill measurements")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--seed", type=int, default=0x4E4634)
    ap.add_argument("--dominant-replays", type=int, default=9)
    ap.add_argument("--launch-log", default=None,
                    help="write the label of every nf4_gemv/nf4_gemm launch, in order, to FILE")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="run only the counter workload: a 1 GiB copy, 3 gate|up GEMVs, 1 GEMM "
                         "(both formats), and down at M=29")
    ap.add_argument("--summarize", default=None, metavar="DIR",
                    help="print a markdown summary of rocprofv3 CSV output under DIR")
    ap.add_argument("--title", default="")
    ap.add_argument("--command", default="")
    args = ap.parse_args()
    if args.summarize:
        summarize(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from bit_weight_only_amd import nf4

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    nf4.lib()
    cb = nf4.nf4_codebook()  # the library's default table (host computation)
    s = torch.cuda.Stream()
    if args.pmc_pass:
        pmc_pass(torch, nf4, cb, args.seed, s)
        return

    t0 = time.perf_counter()
    mdl = Model(torch, nf4, cb, args.seed, s)
    log(f"[bench] packed {LAYERS} layers + lm_head in {time.perf_counter() - t0:.1f} s")
    launches = []

    decode_bytes = sum(packed_bytes(N, K) for _, N, K in LINEARS) * LAYERS \
        + packed_bytes(VOCAB, HIDDEN)
    prefill_flop = 2 * PREFILL_M * sum(N * K for _, N, K in LINEARS) * LAYERS

    # a decode step's launches in order; each names the next one as its
    # read-ahead hint (the weights are known ahead, the activations are not)
    decode_order = [(name, layer) for layer in range(LAYERS) for name, _, _ in LINEARS] + \
        [("lm_head", 0)]

    def decode_step():
        for i, (name, layer) in enumerate(decode_order):
            mdl.gemv(name, layer, decode_order[i + 1] if i + 1 < len(decode_order) else None)

    def prefill_step():
        for layer in range(LAYERS):
            for name, _, _ in LINEARS:
                mdl.gemm(name, layer)

    # ---- capture each sequence once; replay it per step
    with torch.cuda.stream(s):
        decode_step()
        prefill_step()
    s.synchronize()
    launches += [("gemv", n) for n in decode_labels()] + [("gemm", n) for n in prefill_labels()]
    g_dec, g_pre = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_dec, stream=s):
        decode_step()
    with torch.cuda.graph(g_pre, stream=s):
        prefill_step()
    s.synchronize()
    log("[bench] graphs captured")

    with torch.cuda.stream(s):
        for _ in range(args.warmup):
            g_dec.replay()
            g_pre.replay()
    s.synchronize()
    log(f"[bench] {args.warmup} warmup steps done")
    for _ in range(args.warmup):
        launches += [("gemv", n) for n in decode_labels()] + \
                    [("gemm", n) for n in prefill_labels()]

    # ---- dominant kernels, timed alone before the steps: the 28 gate|up
    # launches back to back
    name, N, K = DOMINANT
    reps = args.dominant_replays
    # (each launch hints the next layer's gate|up, as the launch before a
    # gate|up in a decode step hints it)
    gemv_ms = graph_ms(torch, s, lambda: [mdl.gemv(name, l, (name, (l + 1) % LAYERS))
                                          for l in range(LAYERS)], reps)
    gemv_us = gemv_ms * 1e3 / LAYERS
    launches += [("gemv", name)] * (LAYERS * (reps + 1))
    gemm_ms = graph_ms(torch, s, lambda: [mdl.gemm(name, l) for l in range(LAYERS)], reps)
    gemm_us = gemm_ms * 1e3 / LAYERS
    launches += [("gemm", name)] * (LAYERS * (reps + 1))
    log(f"[bench] dominant {name}: gemv {gemv_us:.2f} us, gemm {gemm_us:.2f} us per launch")
    # ---- the decode step with two slots (M = 2), same read-ahead hints
    def decode_step_m2():
        for i, (nm, layer) in enumerate(decode_order):
            mdl.gemv(nm, layer, decode_order[i + 1] if i + 1 < len(decode_order) else None, M=2)

    dec2_ms = graph_ms(torch, s, decode_step_m2, max(args.steps, 5))
    launches += [("gemv", "m2:" + n) for n in decode_labels()] * (max(args.steps, 5) + 1)
    log(f"[bench] decode M=2: {dec2_ms:.3f} ms per step")
    # ---- lm_head: plain GEMV vs GEMV + on-device argmax (4 launches per replay)
    amx_ws_bytes = nf4.nf4_gemv_argmax_workspace_bytes(1, VOCAB, HIDDEN)
    amx_ws = torch.zeros(max(amx_ws_bytes, 16), dtype=torch.uint8, device="cuda")
    amx_idx = torch.zeros(8, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()

    def lm_head_argmax():
        pw = mdl.lm_head
        nf4.nf4_gemv_argmax(mdl.x1[HIDDEN], 1, pw.qweight, pw.absmax, cb, VOCAB, HIDDEN,
                            mdl.y1["lm_head"], amx_idx, amx_ws, amx_ws_bytes)

    head_us = graph_ms(torch, s, lambda: [mdl.gemv("lm_head", 0) for _ in range(4)],
                       reps) * 1e3 / 4
    launches += [("gemv", "lm_head")] * (4 * (reps + 1))
    head_amx_us = graph_ms(torch, s, lambda: [lm_head_argmax() for _ in range(4)], reps) * 1e3 / 4
    launches += [("gemv", "lm_head_argmax")] * (4 * (reps + 1))
    log(f"[bench] lm_head: gemv {head_us:.2f} us, gemv + argmax {head_amx_us:.2f} us")
    # ---- the 113-row tail of the 14449-row long-audio prefill (14 x 1024 + 113)
    def tail_step():
        for layer in range(LAYERS):
            for lname, _, _ in LINEARS:
                pw = mdl.weights[layer][lname]
                nf4.nf4_gemm(mdl.xp[pw.K], TAIL_M, pw.qweight, pw.absmax, cb, pw.N, pw.K,
                             mdl.yp[lname], mdl.ws, mdl.ws_bytes)
    tail_ms = graph_ms(torch, s, tail_step, reps)
    launches += [("gemm", n) for _ in range(reps + 1) for n in prefill_labels()]
    tail_flop = 2 * TAIL_M * sum(N_ * K_ for _, N_, K_ in LINEARS) * LAYERS
    log(f"[bench] prefill tail M={TAIL_M}: {tail_ms:.3f} ms")
    # ---- one 29-row chunk of streamed input through the same linears
    def chunk_step():
        for layer in range(LAYERS):
            for lname, _, _ in LINEARS:
                pw = mdl.weights[layer][lname]
                nf4.nf4_gemm(mdl.xp[pw.K], CHUNK_M, pw.qweight, pw.absmax, cb, pw.N, pw.K,
                             mdl.yp[lname], mdl.ws, mdl.ws_bytes)
    chunk_ms = graph_ms(torch, s, chunk_step, reps)
    launches += [("gemm", n) for _ in range(reps + 1) for n in prefill_labels()]
    chunk_flop = 2 * CHUNK_M * sum(N_ * K_ for _, N_, K_ in LINEARS) * LAYERS
    chunk_bytes = sum(packed_bytes(N_, K_) for _, N_, K_ in LINEARS) * LAYERS
    log(f"[bench] prefill chunk M={CHUNK_M}: {chunk_ms:.3f} ms")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    with torch.cuda.stream(s):
        for e0, e1, e2 in ev:
            e0.record(s)
            g_dec.replay()
            e1.record(s)
            g_pre.replay()
            e2.record(s)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - w0) * 1e3 / args.steps
    for _ in range(args.steps):
        launches += [("gemv", n) for n in decode_labels()] + \
                    [("gemm", n) for n in prefill_labels()]
    dec_all = [e0.elapsed_time(e1) for e0, e1, _ in ev]
    pre_all = [e1.elapsed_time(e2) for _, e1, e2 in ev]
    dec_ms, pre_ms = float(np.mean(dec_all)), float(np.mean(pre_all))
    log(f"[bench] {args.steps} timed steps: decode {dec_ms:.3f} ms, prefill {pre_ms:.3f} ms")

    # ---- the unfused 7-linear sequence, on row views of the fused weights
    # (the parts of a fused matrix are weights in the device layout)
    views = [{u: mdl.weights[l][f].rows(n0, n1) for u, f, n0, n1 in UNFUSED}
             for l in range(LAYERS)]
    yu1 = {u: torch.empty((1, n1 - n0), dtype=torch.float32, device="cuda")
           for u, _, n0, n1 in UNFUSED}
    yup = {u: torch.empty((PREFILL_M, n1 - n0), dtype=torch.float32, device="cuda")
           for u, _, n0, n1 in UNFUSED}
    uorder = [(u, l) for l in range(LAYERS) for u, _, _, _ in UNFUSED]
    ulabels = ["u:" + u for u, _ in uorder]

    def decode_unfused():
        for i, (u, l) in enumerate(uorder):
            pw = views[l][u]
            nx = views[uorder[i + 1][1]][uorder[i + 1][0]] if i + 1 < len(uorder) else mdl.lm_head
            nf4.nf4_gemv_prefetch(mdl.x1[pw.K], 1, pw.qweight, pw.absmax, cb, pw.N, pw.K, yu1[u],
                                  mdl.ws, mdl.ws_bytes, nx.qweight, nx.absmax, nx.N, nx.K)
        mdl.gemv("lm_head", 0)

    def prefill_unfused():
        for u, l in uorder:
            pw = views[l][u]
            nf4.nf4_gemm(mdl.xp[pw.K], PREFILL_M, pw.qweight, pw.absmax, cb, pw.N, pw.K, yup[u],
                         mdl.ws, mdl.ws_bytes)

    decu_ms = graph_ms(torch, s, decode_unfused, reps)
    launches += [("gemv", n) for _ in range(reps + 1) for n in ulabels + ["lm_head"]]
    preu_ms = graph_ms(torch, s, prefill_unfused, reps)
    launches += [("gemm", n) for _ in range(reps + 1) for n in ulabels]
    log(f"[bench] unfused: decode {decu_ms:.3f} ms, prefill {preu_ms:.3f} ms")

    # ---- Voxtral-shaped decode: 26 layers x 4 fused linears at M = 1
    t1 = time.perf_counter()
    vgen = torch.Generator(device="cuda")
    vw = []
    with torch.cuda.stream(s):
        for l in range(VOXTRAL_LAYERS):
            lw = {}
            for i, (vn, N_, K_) in enumerate(VOXTRAL):
                vgen.manual_seed(args.seed + 0x10000 + 16 * l + i)
                W = torch.randn((N_, K_), generator=vgen, device="cuda") * 0.02
                lw[vn] = nf4.pack_weight(W, cb, stream=s)
                del W
            vw.append(lw)
    s.synchronize()
    torch.cuda.empty_cache()
    vx = {}
    for K_ in sorted({K_ for _, _, K_ in VOXTRAL}):
        vgen.manual_seed(args.seed + 0x20000 + K_)
        vx[K_] = torch.randn((1, K_), generator=vgen, device="cuda").to(torch.bfloat16).view(
            torch.int16)
    vy = {vn: torch.empty((1, N_), dtype=torch.float32, device="cuda") for vn, N_, _ in VOXTRAL}
    torch.cuda.synchronize()
    log(f"[bench] Voxtral: packed {VOXTRAL_LAYERS} layers in {time.perf_counter() - t1:.1f} s")
    vorder = [(vn, l) for l in range(VOXTRAL_LAYERS) for vn, _, _ in VOXTRAL]
    vbytes = sum(packed_bytes(N_, K_) for _, N_, K_ in VOXTRAL) * VOXTRAL_LAYERS

    def voxtral_decode():
        for i, (vn, l) in enumerate(vorder):
            pw = vw[l][vn]
            if i + 1 < len(vorder):
                nx = vw[vorder[i + 1][1]][vorder[i + 1][0]]
                nf4.nf4_gemv_prefetch(vx[pw.K], 1, pw.qweight, pw.absmax, cb, pw.N, pw.K,
                                      vy[vn], mdl.ws, mdl.ws_bytes, nx.qweight, nx.absmax, nx.N,
                                      nx.K)
            else:
                nf4.nf4_gemv(vx[pw.K], 1, pw.qweight, pw.absmax, cb, pw.N, pw.K, vy[vn], mdl.ws,
                             mdl.ws_bytes)

    vdec_ms = graph_ms(torch, s, voxtral_decode, max(args.steps, 5))
    launches += [("gemv", "vx:" + vn) for _ in range(max(args.steps, 5) + 1) for vn, _ in vorder]
    log(f"[bench] Voxtral decode: {vdec_ms:.3f} ms per step")
    del vw
    torch.cuda.empty_cache()

    # ---- what one launch moving the same bytes reaches on this machine: device
    # copies (torch's copy kernel) of a gate|up GEMV's bytes (half read, half
    # written) rotated over 8 buffer pairs (beyond the memory-side cache), and
    # of 1 GiB
    def copy_rate(total, pairs):
        n = total // 8  # floats per side: total/2 bytes read, total/2 written
        bufs = [(torch.empty(n, device="cuda"), torch.empty(n, device="cuda"))
                for _ in range(pairs)]
        for a, b in bufs:
            a.fill_(1.0)
        torch.cuda.synchronize()
        ms = graph_ms(torch, s, lambda: [b.copy_(a) for a, b in bufs], reps) / pairs
        del bufs
        torch.cuda.empty_cache()
        return 8 * n / (ms * 1e-3) / 1e9, ms * 1e3
    ref_small = copy_rate(packed_bytes(N, K), 8)
    ref_big = copy_rate(1 << 30, 2)
    log(f"[bench] copies: {ref_small[0]:.0f} GB/s at {packed_bytes(N, K) / 1e6:.1f} MB, "
        f"{ref_big[0]:.0f} GB/s at 1 GiB")

    # ---- the floor of one launch inside a replayed graph: a graph of as many
    # one-element kernels as the decode step has launches
    one = torch.zeros(1, device="cuda")
    nlaunch = len(decode_order)
    floor_us = graph_ms(torch, s, lambda: [one.add_(1.0) for _ in range(nlaunch)], reps) \
        * 1e3 / nlaunch

    if args.launch_log:
        with open(args.launch_log, "w") as f:
            json.dump(launches, f)

    dec_gbps = decode_bytes / (dec_ms * 1e-3) / 1e9
    pre_tflops = prefill_flop / (pre_ms * 1e-3) / 1e12
    gv_bytes = packed_bytes(N, K)
    gv_gbps = gv_bytes / (gemv_us * 1e-6) / 1e9
    gm_flop = 2 * PREFILL_M * N * K
    gm_tflops = gm_flop / (gemm_us * 1e-6) / 1e12
    out = {
        "metric": METRIC, "value": round(dec_gbps, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Qwen2-7B-shaped decoder layer linears (28 layers, fused q|k|v "
                               "and gate|up) + lm_head: decode M=1 then prefill M=1024",
                   "decode_M": 1, "prefill_M": PREFILL_M, "layers": LAYERS,
                   "decode_read_ahead": "each nf4_gemv names the next launch's matrix",
                   "decode_packed_bytes": decode_bytes, "prefill_flop": prefill_flop,
                   "block": 64, "scale_dtype": "fp32", "out_dtype": "fp32"},
        "decode_ms": round(dec_ms, 4),
        "decode_ms_median": round(float(np.median(dec_all)), 4),
        "decode_ms_min": round(float(np.min(dec_all)), 4),
        "decode_m2": {"value": round(decode_bytes / (dec2_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                      "ms": round(dec2_ms, 4),
                      "note": "the same 113 launches with two activation rows (two server slots)"},
        "prefill": {"value": round(pre_tflops, 2), "unit": "TFLOP/s", "ms": round(pre_ms, 3),
                    "ms_median": round(float(np.median(pre_all)), 3),
                    "ms_min": round(float(np.min(pre_all)), 3)},
        "roofline": {"bound": "hbm", "achieved": round(gv_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gv_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_bytes("gemv"),
                     "kernel": f"nf4_gemv gate|up N={N} K={K} M=1",
                     "algorithmic_bytes": gv_bytes, "launch_us": round(gemv_us, 2)},
        "prefill_tail": {"M": TAIL_M, "ms": round(tail_ms, 3),
                         "value": round(tail_flop / (tail_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                         "note": "28 layers x 4 fused linears at M=113 (skinny path for narrow N)"},
        "prefill_chunk": {"M": CHUNK_M, "ms": round(chunk_ms, 3),
                          "value": round(chunk_flop / (chunk_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                          "weight_gbps": round(chunk_bytes / (chunk_ms * 1e-3) / 1e9, 1),
                          "note": "28 layers x 4 fused linears at M=29 (narrow kernel on q|k|v, o "
                                  "and down, skinny kernel on gate|up)"},
        "decode_unfused": {"value": round(decode_bytes / (decu_ms * 1e-3) / 1e9, 1),
                           "unit": "GB/s", "ms": round(decu_ms, 4),
                           "note": "28 x {q, k, v, o, gate, up, down} + lm_head = 197 launches "
                                   "on row views of the fused weights, read-ahead hints"},
        "prefill_unfused": {"value": round(prefill_flop / (preu_ms * 1e-3) / 1e12, 2),
                            "unit": "TFLOP/s", "ms": round(preu_ms, 3),
                            "note": "28 x 7 nf4_gemm calls at M=1024"},
        "voxtral_decode": {"value": round(vbytes / (vdec_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                           "ms": round(vdec_ms, 4), "packed_bytes": vbytes,
                           "note": f"{VOXTRAL_LAYERS} layers x {{q|k|v 6144x3072, wo 3072x4096, "
                                   "w1|w3 18432x3072, w2 3072x9216}, M=1, read-ahead hints"},
        "long_audio": {"M": LONG_M,
                       "value": round(2 * LONG_M * sum(N_ * K_ for _, N_, K_ in LINEARS) * LAYERS
                                      / ((LONG_CHUNKS * pre_ms + tail_ms) * 1e-3) / 1e12, 2),
                       "unit": "TFLOP/s", "ms": round(LONG_CHUNKS * pre_ms + tail_ms, 2),
                       "note": "14 prefill steps at M=1024 and the 113-row tail step, as timed "
                               "above (1680 nf4_gemm calls)"},
        "hbm_reference": {"copy_gbps_gate_up_bytes": round(ref_small[0], 1),
                          "copy_us_gate_up_bytes": round(ref_small[1], 2),
                          "copy_gbps_1gib": round(ref_big[0], 1), "unit": "GB/s",
                          "note": "torch device copies moving the bytes of one gate|up GEMV "
                                  "launch (half read, half written; 8 buffer pairs rotated) "
                                  "and 1 GiB, one copy per launch, in a replayed graph"},
        "launch_floor_us": {"value": round(floor_us, 2),
                            "note": f"a replayed graph of {nlaunch} one-element torch kernels, "
                                    "per launch"},
        "lm_head_argmax": {"gemv_us": round(head_us, 2), "gemv_argmax_us": round(head_amx_us, 2),
                           "host_copy_bytes": {"logits": 4 * VOCAB, "index": 4},
                           "kernel": f"nf4_gemv_argmax N={VOCAB} K={HIDDEN} M=1"},
        "roofline_prefill": {"bound": "mfma", "achieved": round(gm_tflops, 2),
                             "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(gm_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                             "traffic": traffic_bytes("gemm"),
                             "kernel": f"nf4_gemm gate|up N={N} K={K} M={PREFILL_M}",
                             "algorithmic_flop": gm_flop, "launch_us": round(gemm_us, 2)},
    }
    if not args.no_int4:
        del g_dec, g_pre
        out["int4_group128"] = int4_leg(torch, nf4, args, s, mdl, launches)
        if args.launch_log:
            with open(args.launch_log, "w") as f:
                json.dump(launches, f)
    if not args.no_cpu:
        log("[bench] timing the CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


def int4_leg(torch, nf4, args, s, mdl, launches):
    """Decode (M=1) and prefill (M=1024) steps and the gate|up rooflines for
    the int4 group-128 format; launch labels go to `launches` as int4:<linear>."""
    import numpy as np
    t0 = time.perf_counter()
    amdl = AwqModel(torch, nf4, args.seed, s, mdl)
    log(f"[bench] int4: packed {LAYERS} layers + lm_head in {time.perf_counter() - t0:.1f} s")
    dec_labels = ["int4:" + n for n in decode_labels()]
    pre_labels = ["int4:" + n for n in prefill_labels()]
    decode_bytes = sum(awq_packed_bytes(N, K) for _, N, K in LINEARS) * LAYERS \
        + awq_packed_bytes(VOCAB, HIDDEN)
    prefill_flop = 2 * PREFILL_M * sum(N * K for _, N, K in LINEARS) * LAYERS

    order = [(name, layer) for layer in range(LAYERS) for name, _, _ in LINEARS] + \
        [("lm_head", 0)]

    def decode_step():
        for i, (name, layer) in enumerate(order):
            amdl.gemv(name, layer, order[i + 1] if i + 1 < len(order) else None)

    def prefill_step():
        for layer in range(LAYERS):
            for name, _, _ in LINEARS:
                amdl.gemm(name, layer)

    with torch.cuda.stream(s):
        decode_step()
        prefill_step()
    s.synchronize()
    launches += [("gemv", n) for n in dec_labels] + [("gemm", n) for n in pre_labels]
    g_dec, g_pre = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_dec, stream=s):
        decode_step()
    with torch.cuda.graph(g_pre, stream=s):
        prefill_step()
    s.synchronize()
    with torch.cuda.stream(s):
        for _ in range(args.warmup):
            g_dec.replay()
            g_pre.replay()
    s.synchronize()
    launches += ([("gemv", n) for n in dec_labels] + [("gemm", n) for n in pre_labels]) \
        * args.warmup
    name, N, K = DOMINANT
    reps = args.dominant_replays
    gemv_us = graph_ms(torch, s, lambda: [amdl.gemv(name, l, (name, (l + 1) % LAYERS))
                                          for l in range(LAYERS)], reps) * 1e3 / LAYERS
    launches += [("gemv", "int4:" + name)] * (LAYERS * (reps + 1))
    gemm_us = graph_ms(torch, s, lambda: [amdl.gemm(name, l) for l in range(LAYERS)],
                       reps) * 1e3 / LAYERS
    launches += [("gemm", "int4:" + name)] * (LAYERS * (reps + 1))
    log(f"[bench] int4 dominant {name}: gemv {gemv_us:.2f} us, gemm {gemm_us:.2f} us per launch")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        for e0, e1, e2 in ev:
            e0.record(s)
            g_dec.replay()
            e1.record(s)
            g_pre.replay()
            e2.record(s)
    torch.cuda.synchronize()
    launches += ([("gemv", n) for n in dec_labels] + [("gemm", n) for n in pre_labels]) \
        * args.steps
    dec_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1, _ in ev]))
    pre_ms = float(np.mean([e1.elapsed_time(e2) for _, e1, e2 in ev]))
    log(f"[bench] int4 {args.steps} timed steps: decode {dec_ms:.3f} ms, prefill {pre_ms:.3f} ms")
    gv_bytes = awq_packed_bytes(N, K)
    gv_gbps = gv_bytes / (gemv_us * 1e-6) / 1e9
    gm_flop = 2 * PREFILL_M * N * K
    gm_tflops = gm_flop / (gemm_us * 1e-6) / 1e12
    del g_dec, g_pre, amdl
    torch.cuda.empty_cache()
    return {
        "format": "asymmetric int4, groups of 128 along K, w = (q - z) * s, fp16 s",
        "decode": {"value": round(decode_bytes / (dec_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                   "ms": round(dec_ms, 4), "packed_bytes": decode_bytes},
        "prefill": {"value": round(prefill_flop / (pre_ms * 1e-3) / 1e12, 2),
                    "unit": "TFLOP/s", "ms": round(pre_ms, 3),
                    "note": "each nf4_awq_gemm = x-sum pre-pass + GEMM kernel"},
        "roofline": {"bound": "hbm", "achieved": round(gv_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gv_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_bytes("awq_gemv"),
                     "kernel": f"nf4_awq_gemv gate|up N={N} K={K} M=1",
                     "algorithmic_bytes": gv_bytes, "launch_us": round(gemv_us, 2)},
        "roofline_prefill": {"bound": "mfma", "achieved": round(gm_tflops, 2),
                             "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(gm_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                             "traffic": traffic_bytes("awq_gemm"),
                             "kernel": f"nf4_awq_gemm gate|up N={N} K={K} M={PREFILL_M}",
                             "algorithmic_flop": gm_flop, "launch_us": round(gemm_us, 2)},
    }


def pmc_pass(torch, nf4, cb, seed, s):
    """Counter workload, each step synchronized: a plain copy of 1 GiB
    (counter calibration), then three gate|up GEMVs on distinct weights and
    one gate|up GEMM, and down at M=29 (the narrow kernel, K in two parts)."""
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    mdl = Model(torch, nf4, cb, seed, s, layers=3, with_head=False, only=("gate_up",))
    with torch.cuda.stream(s):
        for layer in range(3):
            mdl.gemv("gate_up", layer, ("gate_up", (layer + 1) % 3))
            s.synchronize()
        mdl.gemm("gate_up", 0)
        s.synchronize()
    dmdl = Model(torch, nf4, cb, seed, s, layers=1, with_head=False, only=("down",))
    pw = dmdl.weights[0]["down"]
    with torch.cuda.stream(s):
        nf4.nf4_gemm(dmdl.xp[pw.K], CHUNK_M, pw.qweight, pw.absmax, cb, pw.N, pw.K,
                     dmdl.yp["down"], dmdl.ws, dmdl.ws_bytes)
        s.synchronize()
    del dmdl
    torch.cuda.empty_cache()
    amdl = AwqModel(torch, nf4, seed, s, mdl, layers=3, with_head=False, only=("gate_up",))
    with torch.cuda.stream(s):
        for layer in range(3):
            amdl.gemv("gate_up", layer, ("gate_up", (layer + 1) % 3))
            s.synchronize()
        amdl.gemm("gate_up", 0)
        s.synchronize()
    log("[bench] pmc pass: copy 1 GiB, 3 x gate|up gemv, 1 x gate|up gemm, both formats; "
        "down at M=29")


def _kernel_short(name):
    name = name.replace("void ", "").replace("nf4::(anonymous namespace)::", "")
    return name.split("(")[0]


def summarize(args):
    """Markdown summary of rocprofv3 CSV output: kernel trace (per kernel and
    linear, using the launch log to label nf4 launches in dispatch order) and
    counter collection (per kernel, KiB per dispatch)."""
    print(f"# {args.title}\n\nCommand (from the repository root, on one MI355X):\n\n```\n"
          f"{args.command}\n```\n")
    stats = glob.glob(os.path.join(args.summarize, "**", "*kernel_stats.csv"), recursive=True)
    for st in stats:
        print("rocprofv3 --stats, per kernel:\n")
        print("| kernel | calls | total ms | mean us | min us | max us | % of GPU time |")
        print("|---|---|---|---|---|---|---|")
        for r in csv.DictReader(open(st)):
            print(f"| `{_kernel_short(r['Name'])[:60]}` | {r['Calls']} | "
                  f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['AverageNs']) / 1e3:.2f} | "
                  f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                  f"{float(r['Percentage']):.2f} |")
        print()
    traces = glob.glob(os.path.join(args.summarize, "**", "*kernel_trace.csv"), recursive=True)
    if traces:
        rows = []
        for t in traces:
            rows += list(csv.DictReader(open(t)))
        rows.sort(key=lambda r: int(r["Start_Timestamp"]))
        labels = json.load(open(args.launch_log)) if args.launch_log else None
        nf4_rows = [r for r in rows if "nf4::" in r["Kernel_Name"] and
                    ("gemv" in r["Kernel_Name"] or "gemm" in r["Kernel_Name"])]
        if labels is not None:
            assert len(labels) == len(nf4_rows), (len(labels), len(nf4_rows))
        d = collections.defaultdict(list)
        for i, r in enumerate(nf4_rows):
            lab = labels[i][1] if labels else ""
            d[(_kernel_short(r["Kernel_Name"]), lab)].append(
                int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        print("Per kernel and linear (nf4 launches labelled in dispatch order from the "
              "launch log):\n")
        print("| kernel | linear | calls | mean us | median us | min us | total ms |")
        print("|---|---|---|---|---|---|---|")
        for (k, lab), v in sorted(d.items(), key=lambda kv: -sum(kv[1])):
            v.sort()
            print(f"| `{k}` | {lab} | {len(v)} | {sum(v) / len(v) / 1e3:.2f} | "
                  f"{v[len(v) // 2] / 1e3:.2f} | {v[0] / 1e3:.2f} | {sum(v) / 1e6:.3f} |")
        print()
    counters = glob.glob(os.path.join(args.summarize, "**", "*counter_collection.csv"),
                         recursive=True)
    if counters:
        d = collections.defaultdict(list)
        for c in counters:
            for r in csv.DictReader(open(c)):
                kn = r["Kernel_Name"]
                if not ("copy" in kn.lower() or ("nf4::" in kn and ("gemv" in kn or "gemm" in kn))):
                    continue
                d[(_kernel_short(kn)[:60], r["Counter_Name"])].append(
                    float(r["Counter_Value"]))
        print("| kernel | counter | dispatches | values per dispatch |")
        print("|---|---|---|---|")
        for (k, cn), v in d.items():
            print(f"| `{k}` | {cn} | {len(v)} | {', '.join(f'{x:.0f}' for x in v)} |")
        print()


if __name__ == "__main__":
    main()
