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
per step) and `roofline_prefill` the gate|up GEMM: 28 launches on the 28
layers' distinct matrices, replayed back to back in one graph (each GEMV
naming the next as its hint, as in the step).  Before this process touches
the GPU it runs rocprofv3 on child runs of itself: a kernel trace of
`--kernel-pass` (the same replays), whose mean dispatch duration is the
launch duration `achieved` is computed from (`rocprof_mean_us`; the event
time per launch of this run's own replays is `event_us`), and two counter
runs of `--pmc-pass` (FETCH_SIZE, then WRITE_SIZE) whose readings, each
scaled by what the counter reads for a plain 1 GiB copy, give `traffic`, the
HBM bytes per launch.  Without rocprofv3 (or with --no-rocprof) `achieved`
falls back to the event time and `traffic` is null; `timed_on` says which.

`cpu_baseline` times the CPU oracle on this host (see cpu_baseline()).

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu] [--no-int4]
                    [--no-rocprof] [--profile-out DIR]
    python bench.py --kernel-pass --launch-log FILE   # rocprofv3 kernel-trace workload
    python bench.py --pmc-pass --launch-log FILE      # rocprofv3 --pmc workload
    python bench.py --summarize DIR --launch-log FILE --title T --command C
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import shutil
import subprocess
import tempfile
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


def pin_cpus(n):
    """Restrict this process (and the oracle threads it starts) to the first
    n CPUs of its allowed set, one oracle thread per CPU; returns them."""
    use = sorted(os.sched_getaffinity(0))[:n]
    os.sched_setaffinity(0, use)
    return use


# The unfused linears of the two decoder shapes, (N, K) = (out, in)
VOXTRAL_UNFUSED = [(4096, 3072), (1024, 3072), (1024, 3072), (3072, 4096), (9216, 3072),
                   (9216, 3072), (3072, 9216)]
QWEN_UNFUSED = [(HIDDEN, HIDDEN), (KV, HIDDEN), (KV, HIDDEN), (HIDDEN, HIDDEN), (MLP, HIDDEN),
                (MLP, HIDDEN), (HIDDEN, MLP)]


def cpu_baseline():
    """The CPU oracle (scalar dequant + fp64 dot, its own threads over output
    rows) timed on this host, pinned one thread per CPU:
      C0  the tiny layer (N = K = 256) at M = 1 and 4, repeated for 0.3 s;
      C1  the full Voxtral decode at M = 1: 26 layers x 7 linears;
      C2  the full Qwen2-7B decode at M = 1 and M = 2: 28 layers x 7 linears
          + lm_head;
      C3  one 1024-row prefill chunk, sampled: rows {0, 1023} and 6 seeded
          random rows through layer 0's 7 linears;
      C4  the 14449-row prompt, sampled: C3's rows plus the 113 tail rows
          through layer 0's 7 linears.
    C3 and C4 are extrapolated (labelled so) from the two samples: per
    layer a + b M seconds for M rows (every layer has the same shapes), a and
    b fitted to the 8-row and 113-row samples.  Each layer of C1 and C2 is
    a distinct copy in memory of one generated layer (the oracle's time does
    not depend on the values; distinct copies keep a layer from being served
    by the caches the previous one filled); inputs are the seeded synthetic
    ones (SplitMix64 + Box-Muller), quantized by the oracle's quantizer."""
    import numpy as np

    import oracle
    from bit_weight_only_amd import synth

    threads = cpu_threads()
    cpus = pin_cpus(threads)
    cb, _ = oracle.codebook()
    t_start = time.perf_counter()

    def make(cfg, shapes, base_id):
        mats = []
        for i, (N, K) in enumerate(shapes):
            W = synth.weights(cfg, 0, base_id + i, N, K)
            codes, absmax = oracle.quantize(W, cb, threads=threads)
            del W
            mats.append((oracle.pack(codes), absmax))
        return mats

    def copies(mats, n):
        return [[(p.copy(), a.copy()) for p, a in mats] for _ in range(n)]

    def run(layers, xs):
        t0 = time.perf_counter()
        for mats in layers:
            for p, a in mats:
                oracle.linear(xs[p.shape[1] * 2], p, a, cb, threads=threads)
        return time.perf_counter() - t0

    def nbytes(mats):
        return sum(packed_bytes(p.shape[0], p.shape[1] * 2) for p, _ in mats)

    out = {}
    # C0
    c0 = make(0, [(256, 256)], 0)
    for M in (1, 4):
        xs = {256: synth.activations(0, M, 256)}
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 0.3:
            run([c0], xs)
            n += 1
        el = time.perf_counter() - t0
        out[f"C0_m{M}"] = {"ms": round(el / n * 1e3, 4),
                           "gbps": round(nbytes(c0) * n / el / 1e9, 3)}
    # C1: Voxtral decode, M = 1
    layer = make(1, VOXTRAL_UNFUSED, 0)
    layers = copies(layer, VOXTRAL_LAYERS)
    xs = {K: synth.activations(1, 1, K) for K in (3072, 4096, 9216)}
    el = run(layers, xs)
    b1 = nbytes(layer) * VOXTRAL_LAYERS
    out["C1_m1"] = {"ms": round(el * 1e3, 1), "gbps": round(b1 / el / 1e9, 3),
                    "packed_bytes": b1}
    del layers, layer
    # C2: Qwen2-7B decode, M = 1 and 2 (lm_head: 8 distinct copies of a
    # generated 1/8 of its rows)
    layer = make(2, QWEN_UNFUSED, 0)
    layers = copies(layer, LAYERS)
    hp, ha = make(2, [(VOCAB // 8, HIDDEN)], 100)[0]
    head = [(np.concatenate([hp] * 8), np.concatenate([ha] * 8))]
    b2 = nbytes(layer) * LAYERS + nbytes(head)
    for M in (1, 2):
        xs = {K: synth.activations(2, M, K, stream=M) for K in (HIDDEN, MLP)}
        el = run(layers + [head], xs)
        out[f"C2_m{M}"] = {"ms": round(el * 1e3, 1), "gbps": round(b2 / el / 1e9, 3),
                           "packed_bytes": b2}
    del layers, head
    # C3 / C4 samples through layer 0
    rng = np.random.default_rng(0xC3)
    rows8 = np.concatenate([[0, 1023], np.sort(rng.choice(np.arange(1, 1023), 6, replace=False))])
    x8 = {K: synth.activations(3, PREFILL_M, K, rows=rows8) for K in (HIDDEN, MLP)}
    t8 = run([layer], x8)
    x113 = {K: synth.activations(4, LONG_M, K, rows=np.arange(LONG_CHUNKS * PREFILL_M, LONG_M))
            for K in (HIDDEN, MLP)}
    t113 = run([layer], x113)
    b = max((t113 - t8) / (TAIL_M - 8), 0.0)
    a = max(t8 - 8 * b, 0.0)
    layer_flop = 2 * sum(N * K for N, K in QWEN_UNFUSED)
    c3_s = LAYERS * (a + b * PREFILL_M)
    c4_s = LAYERS * (LONG_CHUNKS * (a + b * PREFILL_M) + a + b * TAIL_M)
    out["C3_m1024"] = {"extrapolated_s": round(c3_s, 1),
                       "gflops": round(LAYERS * PREFILL_M * layer_flop / c3_s / 1e9, 2),
                       "sample": "rows 0, 1023 and 6 seeded random rows of the chunk through "
                                 f"layer 0's 7 linears: {t8:.2f} s"}
    out["C4_m14449"] = {"extrapolated_s": round(c4_s, 1),
                        "gflops": round(LAYERS * LONG_M * layer_flop / c4_s / 1e9, 2),
                        "sample": f"the 113 tail rows through layer 0's 7 linears: {t113:.2f} s, "
                                  "with the 8-row sample above"}
    total = time.perf_counter() - t_start
    return {"value": out["C2_m1"]["gbps"], "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "value: the full Qwen2-7B decode step at M=1 (28 layers x 7 linears + "
                      "lm_head, 3.977 GB packed) through the oracle; C0-C2 full runs, C3/C4 "
                      "extrapolated from row samples (per layer a + b M, fitted to 8 and 113 "
                      f"rows); {total:.0f} s in all including input generation",
            "pinned_cpus": cpus, "configs": out}


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
    ap.add_argument("--seed", type=int, default=0x4E4634)
    ap.add_argument("--dominant-replays", type=int, default=9)
    ap.add_argument("--launch-log", default=None,
                    help="write the label of every nf4_gemv/nf4_gemm launch, in order, to FILE")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="run only the counter workload: a 1 GiB copy, 3 gate|up GEMVs and "
                         "1 GEMM in both formats (labels to --launch-log)")
    ap.add_argument("--kernel-pass", action="store_true",
                    help="run only the dominant kernels' timing workload (labels to --launch-log)")
    ap.add_argument("--no-rocprof", action="store_true",
                    help="do not run the live rocprofv3 passes (rooflines from events only)")
    ap.add_argument("--profile-out", default=None, metavar="DIR",
                    help="write markdown summaries of the live rocprofv3 passes to DIR")
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

    child = args.pmc_pass or args.kernel_pass
    if child:
        prof = {}
    elif args.no_rocprof:
        prof = {"error": "not run (--no-rocprof)"}
    else:
        # before this process touches the GPU: the children are profiled
        # processes of their own
        prof = run_profiler(args)
        if "error" in prof:
            log(f"[bench] rocprofv3 passes: {prof['error']}")
        elif args.profile_out:
            write_profiles(prof, args.profile_out)

    import numpy as np
    import torch

    from bit_weight_only_amd import nf4

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    nf4.lib()
    cb = nf4.nf4_codebook()  # the library's default table (host computation)
    s = torch.cuda.Stream()
    if args.pmc_pass:
        pmc_pass(torch, nf4, cb, args, s)
        return
    if args.kernel_pass:
        kernel_pass(torch, nf4, cb, args, s)
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

    # ---- dominant kernels, timed alone before the steps (the same
    # sequence the live rocprofv3 kernel trace times)
    name, N, K = DOMINANT
    reps = args.dominant_replays
    dom = dominant(torch, s, mdl, None, reps, launches)
    gemv_us, gemm_us = dom["nf4_gemv_us"], dom["nf4_gemm_us"]
    log(f"[bench] dominant {name}: gemv {gemv_us:.2f} us, gemm {gemm_us:.2f} us per launch "
        "(events)")
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
    launches += [("gemm", "t113:" + n) for _ in range(reps + 1) for n in prefill_labels()]
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
    launches += [("gemm", "c29:" + n) for _ in range(reps + 1) for n in prefill_labels()]
    chunk_flop = 2 * CHUNK_M * sum(N_ * K_ for _, N_, K_ in LINEARS) * LAYERS
    chunk_bytes = sum(packed_bytes(N_, K_) for _, N_, K_ in LINEARS) * LAYERS
    log(f"[bench] prefill chunk M={CHUNK_M}: {chunk_ms:.3f} ms")
    # ---- the 14449-row long-audio prompt as one timed sequence: 14 chunks of
    # 1024 rows and the 113-row tail through the 28 layers' linears, 1680
    # nf4_gemm calls in one graph, on x rows of their own
    lgen = torch.Generator(device="cuda")
    xl = {}
    for K_ in (HIDDEN, MLP):
        lgen.manual_seed(args.seed + 0x30000 + K_)
        xl[K_] = torch.randn((LONG_M, K_), generator=lgen, device="cuda").to(torch.bfloat16).view(
            torch.int16)
    torch.cuda.synchronize()

    def long_seq():
        for c in range(LONG_CHUNKS + 1):
            m0 = c * PREFILL_M
            rows = PREFILL_M if c < LONG_CHUNKS else LONG_M - m0
            for layer in range(LAYERS):
                for lname, _, _ in LINEARS:
                    pw = mdl.weights[layer][lname]
                    nf4.nf4_gemm(xl[pw.K][m0:m0 + rows], rows, pw.qweight, pw.absmax, cb, pw.N,
                                 pw.K, mdl.yp[lname], mdl.ws, mdl.ws_bytes)
    long_reps = 2
    long_ms = graph_ms(torch, s, long_seq, long_reps)
    launches += [("gemm", ("c4:" if c < LONG_CHUNKS else "c4t:") + n)
                 for _ in range(long_reps + 1) for c in range(LONG_CHUNKS + 1)
                 for n in prefill_labels()]
    del xl
    torch.cuda.empty_cache()
    log(f"[bench] long audio M={LONG_M}: {long_ms:.2f} ms in one sequence")
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
    gm_flop = 2 * PREFILL_M * N * K
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
        "roofline": roofline_entry(prof, "dom:" + name, gemv_us, gv_bytes, HBM_PEAK_GBPS, "GB/s",
                                   "hbm", f"nf4_gemv gate|up N={N} K={K} M=1",
                                   "algorithmic_bytes"),
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
                                      / (long_ms * 1e-3) / 1e12, 2),
                       "unit": "TFLOP/s", "ms": round(long_ms, 2),
                       "stitched_ms": round(LONG_CHUNKS * pre_ms + tail_ms, 2),
                       "note": "one timed sequence of 1680 nf4_gemm calls in a replayed graph: "
                               "14 chunks of 1024 rows and the 113-row tail of a 14449-row x, "
                               "28 layers x 4 fused linears each (median of 2 replays); "
                               "stitched_ms: 14 prefill steps plus the tail step as timed above"},
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
        "roofline_prefill": roofline_entry(prof, "dom:" + name, gemm_us, gm_flop,
                                           MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", "mfma",
                                           f"nf4_gemm gate|up N={N} K={K} M={PREFILL_M}",
                                           "algorithmic_flop"),
    }
    if not args.no_int4:
        del g_dec, g_pre
        out["int4_group128"] = int4_leg(torch, nf4, args, s, mdl, launches, prof)
        if args.launch_log:
            with open(args.launch_log, "w") as f:
                json.dump(launches, f)
    if not args.no_cpu:
        log("[bench] timing the CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


def int4_leg(torch, nf4, args, s, mdl, launches, prof):
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
    dom = dominant(torch, s, None, amdl, args.dominant_replays, launches)
    gemv_us, gemm_us = dom["int4_gemv_us"], dom["int4_gemm_us"]
    log(f"[bench] int4 dominant {name}: gemv {gemv_us:.2f} us, gemm {gemm_us:.2f} us per launch "
        "(events)")
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
    gm_flop = 2 * PREFILL_M * N * K
    del g_dec, g_pre, amdl
    torch.cuda.empty_cache()
    return {
        "format": "asymmetric int4, groups of 128 along K, w = (q - z) * s, fp16 s",
        "decode": {"value": round(decode_bytes / (dec_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                   "ms": round(dec_ms, 4), "packed_bytes": decode_bytes},
        "prefill": {"value": round(prefill_flop / (pre_ms * 1e-3) / 1e12, 2),
                    "unit": "TFLOP/s", "ms": round(pre_ms, 3),
                    "note": "each nf4_awq_gemm = x-sum pre-pass + GEMM kernel"},
        "roofline": roofline_entry(prof, "dom:int4:" + name, gemv_us, gv_bytes, HBM_PEAK_GBPS,
                                   "GB/s", "hbm", f"nf4_awq_gemv gate|up N={N} K={K} M=1",
                                   "algorithmic_bytes"),
        "roofline_prefill": roofline_entry(prof, "dom:int4:" + name, gemm_us, gm_flop,
                                           MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", "mfma",
                                           f"nf4_awq_gemm gate|up N={N} K={K} M={PREFILL_M}",
                                           "algorithmic_flop"),
    }


# warm-up replays before the dominant kernels are timed: in a fresh process
# the gate|up GEMV's duration drifts over its first replays (a kernel trace
# of 63 back-to-back replays of the 28 launches: 16.7 us per launch over
# replays 0-3, 18-20 us over replays 4-21, 16.5-16.7 us from replay 22 on),
# so the timed replays start after 30
DOMINANT_WARM = 30


def dominant(torch, s, mdl, amdl, reps, launches):
    """The dominant kernels timed alone, at a fixed point of a run (after the
    weights are packed and DOMINANT_WARM warm-up replays): 28 gate|up GEMV
    launches on the 28 layers' distinct matrices replayed back to back in one
    graph, each naming the next as its read-ahead hint as in a decode step,
    then the 28 gate|up GEMMs (M = 1024) the same way; `reps` timed replays
    each, events on the launch stream around each replay, the median replay
    / 28 per launch.  The warm-up launches carry labels of their own
    ("warm:..."), so a kernel trace's mean covers the timed replays only.
    amdl: the same for the int4 group-128 format (or None)."""
    name = DOMINANT[0]
    res = {}
    for fmt, m in (("nf4", mdl), ("int4", amdl)):
        if m is None:
            continue
        tag = "dom:" if fmt == "nf4" else "dom:int4:"
        res[fmt + "_gemv_us"] = graph_ms(
            torch, s, lambda: [m.gemv(name, l, (name, (l + 1) % LAYERS)) for l in range(LAYERS)],
            reps, warm=DOMINANT_WARM) * 1e3 / LAYERS
        launches += [("gemv", "warm:" + tag + name)] * (LAYERS * DOMINANT_WARM) + \
            [("gemv", tag + name)] * (LAYERS * reps)
        res[fmt + "_gemm_us"] = graph_ms(torch, s, lambda: [m.gemm(name, l) for l in range(LAYERS)],
                                         reps, warm=DOMINANT_WARM) * 1e3 / LAYERS
        launches += [("gemm", "warm:" + tag + name)] * (LAYERS * DOMINANT_WARM) + \
            [("gemm", tag + name)] * (LAYERS * reps)
    return res


def kernel_pass(torch, nf4, cb, args, s):
    """Workload of the live rocprofv3 kernel-trace run: the dominant kernels
    of both formats exactly as the main run times them (dominant())."""
    mdl = Model(torch, nf4, cb, args.seed, s, with_head=False, only=("gate_up",))
    amdl = AwqModel(torch, nf4, args.seed, s, mdl, with_head=False, only=("gate_up",))
    launches = []
    res = dominant(torch, s, mdl, amdl, args.dominant_replays, launches)
    with open(args.launch_log, "w") as f:
        json.dump(launches, f)
    log(f"[bench] kernel pass: {res}")


def pmc_pass(torch, nf4, cb, args, s):
    """Counter workload, each step synchronized: a plain device copy of 1 GiB
    (counter calibration), then three gate|up GEMVs on distinct weights, each
    naming the next as its hint, and one gate|up GEMM, in both formats; then
    down and gate|up at M = 29."""
    launches = []
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    mdl = Model(torch, nf4, cb, args.seed, s, layers=3, with_head=False, only=("gate_up",))
    amdl = AwqModel(torch, nf4, args.seed, s, mdl, layers=3, with_head=False, only=("gate_up",))
    for tag, m in (("pmc:", mdl), ("pmc:int4:", amdl)):
        with torch.cuda.stream(s):
            for layer in range(3):
                m.gemv("gate_up", layer, ("gate_up", (layer + 1) % 3))
                s.synchronize()
                launches.append(("gemv", tag + "gate_up"))
            m.gemm("gate_up", 0)
            s.synchronize()
            launches.append(("gemm", tag + "gate_up"))
    # the 29-row chunk through down (the narrow kernel, K in two parts)
    dmdl = Model(torch, nf4, cb, args.seed, s, layers=1, with_head=False, only=("down",))
    pw = dmdl.weights[0]["down"]
    with torch.cuda.stream(s):
        nf4.nf4_gemm(dmdl.xp[pw.K], CHUNK_M, pw.qweight, pw.absmax, cb, pw.N, pw.K,
                     dmdl.yp["down"], dmdl.ws, dmdl.ws_bytes)
        s.synchronize()
    launches.append(("gemm", "pmc:c29:down"))
    # and through gate|up (the skinny kernel, three workgroups per CU)
    with torch.cuda.stream(s):
        pw = mdl.weights[0]["gate_up"]
        nf4.nf4_gemm(mdl.xp[pw.K], CHUNK_M, pw.qweight, pw.absmax, cb, pw.N, pw.K,
                     mdl.yp["gate_up"], mdl.ws, mdl.ws_bytes)
        s.synchronize()
    launches.append(("gemm", "pmc:c29:gate_up"))
    with open(args.launch_log, "w") as f:
        json.dump(launches, f)
    log("[bench] pmc pass: copy 1 GiB, 3 x gate|up gemv, 1 x gate|up gemm, both formats; "
        "down and gate|up at M=29")


def _kernel_short(name):
    name = name.replace("void ", "").replace("nf4::(anonymous namespace)::", "")
    return name.split("(")[0]


_K_OF = {n: K for n, _, K in LINEARS}
SHAPES = {**{n: (N, K) for n, N, K in LINEARS}, "lm_head": (VOCAB, HIDDEN),
          **{"vx:" + n: (N, K) for n, N, K in VOXTRAL},
          **{"u:" + u: (n1 - n0, _K_OF[f]) for u, f, n0, n1 in UNFUSED}}
GEMM_ROWS = {"": PREFILL_M, "t113:": TAIL_M, "c29:": CHUNK_M, "c4:": PREFILL_M, "c4t:": TAIL_M}


def label_work(kind, label):
    """(work per launch, unit, peak) of a launch-log label: packed bytes for a
    GEMV (GB/s against HBM), flop for a GEMM (TFLOP/s against bf16 MFMA)."""
    lab = label
    for p in ("dom:", "pmc:"):
        lab = lab[len(p):] if lab.startswith(p) else lab
    awq = lab.startswith("int4:")
    lab = lab[5:] if awq else lab
    rows = 1
    if kind == "gemv" and lab.startswith("m2:"):
        lab = lab[3:]
    if kind == "gemm":
        rows = PREFILL_M
        for p, m in GEMM_ROWS.items():
            if p and lab.startswith(p):
                lab, rows = lab[len(p):], m
    if lab == "lm_head_argmax":
        lab = "lm_head"
    if lab not in SHAPES:
        return None
    N, K = SHAPES[lab]
    if kind == "gemv":
        return (awq_packed_bytes(N, K) if awq else packed_bytes(N, K)), "GB/s", HBM_PEAK_GBPS
    return 2 * rows * N * K, "TFLOP/s", MFMA_BF16_PEAK_TFLOPS


def summarize(args):
    """Markdown summary of rocprofv3 CSV output under args.summarize: the
    per-kernel statistics, the nf4 dispatches per launch-log label (mean
    duration and the rate it gives against the peak), and counter values."""
    print(f"# {args.title}\n\nCommand (from the repository root, on one MI355X):\n\n```\n"
          f"{args.command}\n```\n")
    for r0 in [_csvs(args.summarize, "kernel_stats.csv")]:
        if not r0:
            continue
        print("rocprofv3 --stats, per kernel:\n")
        print("| kernel | calls | total ms | mean us | min us | max us | % of GPU time |")
        print("|---|---|---|---|---|---|---|")
        for r in r0:
            print(f"| `{_kernel_short(r['Name'])[:60]}` | {r['Calls']} | "
                  f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['AverageNs']) / 1e3:.2f} | "
                  f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                  f"{float(r['Percentage']):.2f} |")
        print()
    if args.launch_log and _csvs(args.summarize, "kernel_trace.csv"):
        d = labelled_durations(args.summarize, args.launch_log)
        print("nf4 launches per label (dispatch order matched to the launch log); rate = "
              "algorithmic work per launch / mean duration:\n")
        print("| entry | label | kernel | calls | mean us | median us | min us | rate | of peak |")
        print("|---|---|---|---|---|---|---|---|---|")
        for (kind, lab), (names, v) in sorted(d.items(), key=lambda kv: -sum(kv[1][1])):
            v = sorted(v)
            mean = sum(v) / len(v) / 1e3
            w = label_work(kind, lab)
            rate = frac = ""
            if w:
                scale = 1e9 if w[1] == "GB/s" else 1e12
                r = w[0] / (mean * 1e-6) / scale
                rate, frac = f"{r:.1f} {w[1]}", f"{r / w[2]:.3f}"
            print(f"| {kind} | {lab} | `{', '.join(sorted(names))[:48]}` | {len(v)} | {mean:.2f} | "
                  f"{v[len(v) // 2] / 1e3:.2f} | {v[0] / 1e3:.2f} | {rate} | {frac} |")
        print()
    counters = _csvs(args.summarize, "counter_collection.csv")
    if counters:
        d = collections.defaultdict(list)
        for r in counters:
            kn = r["Kernel_Name"]
            if COPY_KERNEL in kn or _nf4_launch(kn):
                d[(_kernel_short(kn)[:60], r["Counter_Name"])].append(float(r["Counter_Value"]))
        print("| kernel | counter | dispatches | values per dispatch (KiB for FETCH_SIZE and "
              "WRITE_SIZE) |")
        print("|---|---|---|---|")
        for (k, cn), v in d.items():
            print(f"| `{k}` | {cn} | {len(v)} | {', '.join(f'{x:.0f}' for x in v)} |")
        print()
        mfma_summary(d)


def mfma_summary(d):
    """Derived matrix-core figures per kernel from the SQ counters, when the
    run took them: MFMA work (MOPS_BF16 x 512 flop), busy cycles per MFMA,
    MFMA busy (busy cycles over 1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs: the
    GRBM count is summed over the XCDs), VALU and LDS instructions per MFMA
    (VALU counts include the MFMAs) and the share of wave cycles in
    s_waitcnt."""
    need = ("SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
            "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_INSTS_LDS",
            "SQ_INSTS_VALU", "GRBM_GUI_ACTIVE")
    kernels = sorted({k for k, _ in d})
    rows = []
    for k in kernels:
        if not all((k, c) in d for c in need):
            continue
        m = {c: sum(d[(k, c)]) / len(d[(k, c)]) for c in need}
        if not m["SQ_INSTS_MFMA"]:
            continue
        rows.append(
            f"| `{k}` | {len(d[(k, need[0])])} | {m['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512 / 1e9:.1f} "
            f"GFLOP | {m['SQ_VALU_MFMA_BUSY_CYCLES'] / m['SQ_INSTS_MFMA']:.1f} | "
            f"{100 * m['SQ_VALU_MFMA_BUSY_CYCLES'] / (1024 * m['GRBM_GUI_ACTIVE'] / 8):.1f} % | "
            f"{m['SQ_INSTS_VALU'] / m['SQ_INSTS_MFMA']:.2f} | "
            f"{m['SQ_INSTS_LDS'] / m['SQ_INSTS_MFMA']:.2f} | "
            f"{100 * m['SQ_WAIT_INST_ANY'] / m['SQ_WAVE_CYCLES']:.0f} % "
            f"({100 * m['SQ_WAIT_INST_LDS'] / m['SQ_WAVE_CYCLES']:.0f} % on LDS) |")
    if rows:
        print("Derived, mean per dispatch:\n")
        print("| kernel | dispatches | MFMA work | busy cycles per MFMA | MFMA busy | "
              "VALU instr. per MFMA | LDS instr. per MFMA | wave cycles in s_waitcnt |")
        print("|---|---|---|---|---|---|---|---|")
        print("\n".join(rows))
        print()


# ---------------------------------------------------------------- rocprofv3
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 30


def _nf4_launch(kernel_name):
    """Is this dispatch an nf4_gemv / nf4_gemm main kernel (the ones the
    launch logs label)?"""
    return "nf4::" in kernel_name and ("gemv" in kernel_name or "gemm" in kernel_name)


def _csvs(d, suffix):
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True):
        rows += list(csv.DictReader(open(f)))
    return rows


def labelled_durations(d, launch_log):
    """{(kind, label): (kernel names, [ns per dispatch])} from a kernel trace
    under d, its nf4 dispatches labelled in dispatch order by the launch log
    (kind: gemv or gemm, the entry point the label belongs to)."""
    rows = sorted(_csvs(d, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))
    rows = [r for r in rows if _nf4_launch(r["Kernel_Name"])]
    labels = json.load(open(launch_log))
    if len(labels) != len(rows):
        raise RuntimeError(f"{len(rows)} nf4 dispatches in the trace, {len(labels)} in the log")
    out = collections.defaultdict(lambda: (set(), []))
    for (kind, lab), r in zip(labels, rows):
        out[(kind, lab)][0].add(_kernel_short(r["Kernel_Name"]))
        out[(kind, lab)][1].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return dict(out)


def labelled_counters(d, launch_log, counter):
    """({(kind, label): [KiB per dispatch]}, copy kernel KiB) from a counter
    run."""
    rows = [r for r in _csvs(d, "counter_collection.csv") if r["Counter_Name"] == counter]
    key = "Dispatch_Id" if rows and "Dispatch_Id" in rows[0] else "Correlation_Id"
    rows.sort(key=lambda r: int(r[key]))
    copy = [float(r["Counter_Value"]) for r in rows if COPY_KERNEL in r["Kernel_Name"]]
    rows = [r for r in rows if _nf4_launch(r["Kernel_Name"])]
    labels = json.load(open(launch_log))
    if len(labels) != len(rows):
        raise RuntimeError(f"{len(rows)} nf4 dispatches counted, {len(labels)} in the log")
    out = collections.defaultdict(list)
    for (kind, lab), r in zip(labels, rows):
        out[(kind, lab)].append(float(r["Counter_Value"]))
    return dict(out), (copy[0] if copy else None)


def run_profiler(args):
    """rocprofv3 on child runs of this script, started before this process
    touches the GPU: a kernel trace of --kernel-pass (the dominant kernels'
    mean durations) and two counter runs of --pmc-pass (FETCH_SIZE, then
    WRITE_SIZE, each calibrated on a plain 1 GiB copy: counter KiB per byte
    read or written).  Returns the parsed results, or {"error": ...}."""
    exe = shutil.which("rocprofv3") or "/opt/rocm/bin/rocprofv3"
    if not os.path.exists(exe):
        return {"error": "rocprofv3 not found"}
    base = tempfile.mkdtemp(prefix="nf4_bench_rocprof_", dir="/tmp")
    env = dict(os.environ, TMPDIR="/tmp")
    me = os.path.abspath(__file__)
    runs = {
        "trace": (["--kernel-trace", "--stats"], "--kernel-pass", 900),
        "fetch": (["--pmc", "FETCH_SIZE"], "--pmc-pass", 600),
        "write": (["--pmc", "WRITE_SIZE"], "--pmc-pass", 600),
    }
    res = {"dir": base, "commands": {}}
    for key, (opts, mode, limit) in runs.items():
        d = os.path.join(base, key)
        lg = os.path.join(base, key + "_launches.json")
        cmd = [exe, *opts, "--output-format", "csv", "-d", d, "-o", "run", "--", sys.executable,
               me, mode, "--launch-log", lg, "--seed", str(args.seed),
               "--dominant-replays", str(args.dominant_replays)]
        res["commands"][key] = "cd /tmp && " + " ".join(cmd)
        log(f"[bench] rocprofv3 {key}: {' '.join(opts)} on {mode}")
        t0 = time.perf_counter()
        try:
            p = subprocess.run(cmd, cwd="/tmp", env=env, timeout=limit, capture_output=True,
                               text=True)
            rc = p.returncode
        except subprocess.TimeoutExpired:
            return {"error": f"rocprofv3 {key} run timed out after {limit} s"}
        log(f"[bench] rocprofv3 {key}: exit {rc} in {time.perf_counter() - t0:.0f} s")
        # rocprofv3 may end with a fault of its own after the program's last
        # line; the results are used whenever the program's log is complete
        if not os.path.exists(lg):
            tail = (p.stderr or "")[-800:]
            return {"error": f"rocprofv3 {key} run failed (exit {rc}): {tail}"}
        try:
            if key == "trace":
                res["trace"] = labelled_durations(d, lg)
            else:
                res[key] = labelled_counters(d, lg, "FETCH_SIZE" if key == "fetch" else
                                             "WRITE_SIZE")
        except (RuntimeError, KeyError, ValueError) as e:
            return {"error": f"rocprofv3 {key}: {e}"}
    return res


def write_profiles(prof, outdir):
    """Markdown summary of the live rocprofv3 passes (kernel trace and the two
    counter runs, with the traffic derived from them) into outdir."""
    import contextlib
    import io
    import types
    os.makedirs(outdir, exist_ok=True)
    buf = io.StringIO()
    with contextlib.redirect_stdout(buf):
        for key, title in (("trace", "kernel trace of the dominant kernels (--kernel-pass)"),
                           ("fetch", "FETCH_SIZE per dispatch (--pmc-pass)"),
                           ("write", "WRITE_SIZE per dispatch (--pmc-pass)")):
            ns = types.SimpleNamespace(
                summarize=os.path.join(prof["dir"], key),
                launch_log=os.path.join(prof["dir"], key + "_launches.json") if key == "trace"
                else None,
                title=title, command=prof["commands"][key])
            summarize(ns)
        (fd, fcopy), (wd, wcopy) = prof["fetch"], prof["write"]
        print("# HBM traffic per launch\n")
        print(f"Calibration on the plain 1 GiB device copy ({COPY_KERNEL}, reads and writes "
              f"1 GiB): FETCH_SIZE {fcopy:.0f} KiB, WRITE_SIZE {wcopy:.0f} KiB; each counter is "
              "scaled by 1 GiB over its reading.\n")
        print("| entry | label | FETCH_SIZE KiB (mean) | WRITE_SIZE KiB (mean) | traffic MB | "
              "algorithmic | traffic / algorithmic |")
        print("|---|---|---|---|---|---|---|")
        for key in sorted(fd):
            f, w = fd[key], wd.get(key, [0.0])
            t = traffic_bytes(prof, key)
            work = label_work(*key)
            alg = ""
            ratio = ""
            if work and work[1] == "GB/s":
                alg, ratio = f"{work[0] / 1e6:.2f} MB packed weight", f"{t / work[0]:.3f}"
            elif work:
                # weight + x + y bytes of an M = 1024 (or labelled M) GEMM
                rows = work[0] // (2 * SHAPES[key[1].split(":")[-1]][0] *
                                   SHAPES[key[1].split(":")[-1]][1])
                N, K = SHAPES[key[1].split(":")[-1]]
                bts = (awq_packed_bytes(N, K) if "int4:" in key[1] else packed_bytes(N, K)) \
                    + rows * K * 2 + rows * N * 4
                alg, ratio = f"{bts / 1e6:.2f} MB (weight + x + y)", f"{t / bts:.3f}"
            print(f"| {key[0]} | {key[1]} | {sum(f) / len(f):.0f} | {sum(w) / len(w):.0f} | "
                  f"{t / 1e6:.2f} | {alg} | {ratio} |")
        print()
    text = buf.getvalue().replace(prof["dir"], "<tmp>").replace(ROOT, "<repo>").replace(
        sys.executable, "python3")
    path = os.path.join(outdir, "dominant_kernels_gate_up.md")
    with open(path, "w") as fh:
        fh.write(f"Made by `python bench.py --profile-out {outdir}` on one MI355X, which runs "
                 "the three rocprofv3 commands below as child processes before it touches the "
                 "GPU itself (<tmp>: a fresh temporary directory).\n\n" + text)
    log(f"[bench] wrote {path}")


def rocprof_mean_us(prof, key):
    """(mean us, kernel names) of the dispatches of key = (kind, label), or
    (None, None)."""
    if "trace" not in prof or key not in prof["trace"]:
        return None, None
    names, v = prof["trace"][key]
    return sum(v) / len(v) / 1e3, sorted(names)


def traffic_bytes(prof, key):
    """HBM bytes per launch of the labelled pmc dispatches: mean FETCH_SIZE
    and WRITE_SIZE, each scaled by the counter's reading on the 1 GiB copy
    (which reads 1 GiB and writes 1 GiB)."""
    try:
        (fd, fcopy), (wd, wcopy) = prof["fetch"], prof["write"]
        f, w = fd[key], wd[key]
    except (KeyError, TypeError):
        return None
    if not fcopy or not wcopy:
        return None
    return int(sum(f) / len(f) * COPY_BYTES / fcopy + sum(w) / len(w) * COPY_BYTES / wcopy)


def roofline_entry(prof, label, event_us, work, peak, unit, bound, kernel, work_key):
    """The roofline object: `achieved` is the algorithmic work per launch over
    the rocprofv3 mean duration of the labelled dispatches (events beside)."""
    kind = "gemv" if unit == "GB/s" else "gemm"
    mean_us, names = rocprof_mean_us(prof, (kind, label))
    t_us = mean_us if mean_us else event_us
    scale = 1e9 if unit == "GB/s" else 1e12
    ach = work / (t_us * 1e-6) / scale
    return {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
            "frac": round(ach / peak, 4),
            "traffic": traffic_bytes(prof, (kind, label.replace("dom:", "pmc:"))), "kernel": kernel,
            work_key: work, "rocprof_mean_us": round(mean_us, 3) if mean_us else None,
            "rocprof_kernels": names, "event_us": round(event_us, 3),
            "timed_on": ("rocprofv3 kernel trace of `bench.py --kernel-pass` (the same 28-launch "
                         "graph replays as the event timing)") if mean_us else
                        "events only (" + prof.get("error", "no rocprofv3 run") + ")"}


if __name__ == "__main__":
    main()
