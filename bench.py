"""Throughput of the NF4 4-bit weight-only linear layer on one MI355X.

One step = one pass of the hot path over one batch of synthetic input on the
Qwen2-7B-shaped decoder (hidden 3584, MLP 18944, k/v 512, head 152064):
  decode : M = 1, 28 layers x {q|k|v, o, gate|up, down} + lm_head = 113
           nf4_gemv launches reading 3.977 GB of packed weights;
  prefill: M = 1024, 28 layers x the same 4 fused linears = 112 nf4_gemm
           launches, 13.364 TFLOP.
Weights are seeded N(0, 0.02^2) fp32 drawn on the GPU and quantized there by
nf4_pack (load time, untimed); activations are seeded N(0, 1) in bf16.  Each
sequence is captured once in a HIP graph and replayed.  The JSON line's
`value` is decode packed-weight GB/s; prefill TFLOP/s sits beside it.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode GEMV packed-weight GB/s (M=1) + prefill GEMM TFLOP/s (M=1024), Qwen2-7B"
HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (published)

LAYERS = 28
HIDDEN, MLP, KV, VOCAB = 3584, 18944, 512, 152064
LINEARS = [("qkv", HIDDEN + 2 * KV, HIDDEN), ("o", HIDDEN, HIDDEN),
           ("gate_up", 2 * MLP, HIDDEN), ("down", HIDDEN, MLP)]
PREFILL_M = 1024


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def packed_bytes(N, K):
    return N * K // 2 + 4 * N * (K // 64)


def cpu_threads():
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return n


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--seed", type=int, default=0x4E4634)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import oracle
    from bit_weight_only_amd import nf4

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    nf4.lib()
    cb, _ = oracle.codebook()
    dev = "cuda"
    s = torch.cuda.Stream()

    # ---- weights: seeded fp32 on the GPU, quantized by nf4_pack (untimed)
    gen = torch.Generator(device=dev)
    weights = []
    t0 = time.perf_counter()
    with torch.cuda.stream(s):
        for layer in range(LAYERS):
            lw = {}
            for i, (name, N, K) in enumerate(LINEARS):
                gen.manual_seed(args.seed + 16 * layer + i)
                W = torch.randn((N, K), generator=gen, device=dev, dtype=torch.float32) * 0.02
                lw[name] = nf4.pack_weight(W, cb, stream=s)
                del W
            weights.append(lw)
        gen.manual_seed(args.seed + 16 * LAYERS)
        W = torch.randn((VOCAB, HIDDEN), generator=gen, device=dev, dtype=torch.float32) * 0.02
        lm_head = nf4.pack_weight(W, cb, stream=s)
        del W
    s.synchronize()
    torch.cuda.empty_cache()
    log(f"[bench] packed {LAYERS} layers + lm_head in {time.perf_counter() - t0:.1f} s")

    def bf16_randn(M, K, seed):
        gen.manual_seed(seed)
        return torch.randn((M, K), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)

    x1 = {K: bf16_randn(1, K, args.seed + 1000 + K) for K in (HIDDEN, MLP)}
    xp = {K: bf16_randn(PREFILL_M, K, args.seed + 2000 + K) for K in (HIDDEN, MLP)}
    y1 = {name: torch.empty((1, N), dtype=torch.float32, device=dev) for name, N, _ in LINEARS}
    y1["lm_head"] = torch.empty((1, VOCAB), dtype=torch.float32, device=dev)
    yp = {name: torch.empty((PREFILL_M, N), dtype=torch.float32, device=dev)
          for name, N, _ in LINEARS}
    ws_bytes = max([nf4.nf4_workspace_bytes(M, N, K) for M in (1, PREFILL_M)
                    for _, N, K in LINEARS] + [nf4.nf4_workspace_bytes(1, VOCAB, HIDDEN)])
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()  # inputs and the zeroed workspace are ready before stream s runs

    decode_bytes = sum(packed_bytes(N, K) for _, N, K in LINEARS) * LAYERS \
        + packed_bytes(VOCAB, HIDDEN)
    prefill_flop = 2 * PREFILL_M * sum(N * K for _, N, K in LINEARS) * LAYERS

    def decode_step():
        for lw in weights:
            for name, N, K in LINEARS:
                pw = lw[name]
                nf4.nf4_gemv(x1[K], 1, pw.qweight, pw.absmax, cb, N, K, y1[name], ws, ws_bytes)
        nf4.nf4_gemv(x1[HIDDEN], 1, lm_head.qweight, lm_head.absmax, cb, VOCAB, HIDDEN,
                     y1["lm_head"], ws, ws_bytes)

    def prefill_step():
        for lw in weights:
            for name, N, K in LINEARS:
                pw = lw[name]
                nf4.nf4_gemm(xp[K], PREFILL_M, pw.qweight, pw.absmax, cb, N, K, yp[name],
                             ws, ws_bytes)

    # ---- capture each sequence once; replay it per step
    with torch.cuda.stream(s):
        decode_step()
        prefill_step()
    s.synchronize()
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
    dec_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1, _ in ev]))
    pre_ms = float(np.mean([e1.elapsed_time(e2) for _, e1, e2 in ev]))
    log(f"[bench] {args.steps} timed steps: decode {dec_ms:.3f} ms, prefill {pre_ms:.3f} ms")

    dec_gbps = decode_bytes / (dec_ms * 1e-3) / 1e9
    pre_tflops = prefill_flop / (pre_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(dec_gbps, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Qwen2-7B-shaped decoder layer linears (28 layers, fused q|k|v "
                               "and gate|up) + lm_head: decode M=1 then prefill M=1024",
                   "decode_M": 1, "prefill_M": PREFILL_M, "layers": LAYERS,
                   "decode_packed_bytes": decode_bytes, "prefill_flop": prefill_flop,
                   "block": 64, "scale_dtype": "fp32", "out_dtype": "fp32"},
        "decode_ms": round(dec_ms, 4),
        "prefill": {"value": round(pre_tflops, 2), "unit": "TFLOP/s", "ms": round(pre_ms, 3)},
        "roofline": {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": None, "kernel": "nf4_gemv (113 launches per decode step)"},
        "roofline_prefill": {"bound": "mfma", "achieved": round(pre_tflops, 2),
                             "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(pre_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                             "traffic": None, "kernel": "nf4_gemm (112 launches per prefill step)"},
    }
    if not args.no_cpu:
        log("[bench] timing the CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
