"""Benchmark of the MoE block on one MI355X.

    python bench.py [--gpus 1] [--steps 1000] [--warmup 50] [--stack]

Headline: decode of the 35B-shaped block (hidden 2048, 256 routed experts,
top-4, intermediate 512, one shared expert, LoRA rank 16, int8 router), batch
1, fresh seeded x every step, weights resident in HBM.  One step = one call
of moe_block_decode (router, top-K, four routed experts + the shared expert
with their LoRA deltas, weighted combine: one kernel launch).  Steps are
captured in HIP graphs of up to 100 steps (each step reads its own x and
writes its own output) and replayed; the timed region is bracketed by
torch.cuda.synchronize(), and HIP events on the launch stream around it give
the kernel's average launch duration for the roofline figure.

Also reported: prefill of 3300 tokens through the same block with a Zipf(1.1)
rank bias on the router logits (tokens/s and the grouped GEMMs' MFMA
utilisation), and with --stack the 24-layer stack (hidden 2048, 128 experts,
top-8, no shared expert; residual + RMSNorm between layers).  Prints one JSON
line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-block decode tokens/s + achieved HBM GB/s; prefill tokens/s + MFMA util"
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense bf16 / fp16


def blob_bytes(w) -> int:
    H, I, r = w["H"], w["I"], w["r"]
    return (2 * I * H // 2 + 2 * I * (H // 64) * 4 + H * I // 2 + H * (I // 64) * 4 +
            2 * r * H * 2 + 2 * I * r * 2 + r * I * 2 + H * r * 2)


def decode_bytes(w) -> dict:
    """Bytes the method must read per decode token (weights only)."""
    H, E, K, S = w["H"], w["E"], w["K"], w["n_shared"]
    router = E * H + E * (H // 64) * 4 + S * (H + (H // 64) * 4)
    experts = (K + S) * blob_bytes(w)
    return {"experts": experts, "router": router, "total": experts + router}


def prefill_flops(w, T) -> dict:
    H, I, r, K, S = w["H"], w["I"], w["r"], w["K"], w["n_shared"]
    per_row = 2 * (2 * I * H + H * I) + 2 * (2 * r * H + 2 * I * r + r * I + H * r)
    return {"expert_gemm": per_row * T * (K + S), "router": 2 * T * (w["E"] + S) * H}


def cores_used() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(w, budget_s: float = 12.0, max_steps: int = 200) -> dict:
    """The fp64 oracle on a bounded sample of the same decode workload."""
    import oracle as O
    import synth
    router = synth.router_tensors(w, 0)
    shared = synth.expert_tensors(w, 0, w["E"])
    experts = {}

    def expert_of(e):
        if e not in experts:
            experts[e] = synth.expert_tensors(w, 0, e)
        return experts[e]

    xs = [synth.tokens(w, s) for s in range(max_steps)]
    # generate the touched experts outside the timed region
    n_pre = 40
    for s in range(n_pre):
        l = O.router_logits(router["router_q"], router["router_s"], xs[s])[0]
        for e in O.select_topk(l, w["K"]):
            expert_of(int(e))
    n = 0
    t0 = time.perf_counter()
    while n < n_pre and time.perf_counter() - t0 < budget_s:
        O.moe_block(w, router, expert_of, xs[n], shared=shared)
        n += 1
    dt = time.perf_counter() - t0
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": cores_used(),
            "kind": "oracle",
            "sample": f"{n} decode steps (batch 1, fresh x) of the same block, numpy float64 "
                      f"oracle, {dt:.1f} s of CPU time"}


def make_layer(w, layer=0, threads=8):
    import synth
    from int4_expert_ffn_int8_amd.layer import MoeLayer, pack_experts
    router = synth.router_tensors(w, layer)
    blobs = pack_experts(w["H"], w["I"], w["r"], lambda e: synth.expert_tensors(w, layer, e),
                         n=w["E"], threads=threads)
    shared = synth.expert_tensors(w, layer, w["E"]) if w["n_shared"] else None
    return MoeLayer(w["H"], w["I"], w["E"], w["K"], w["r"], w["n_shared"], w["lora_scale"],
                    router, None, shared, blobs=blobs)


def bench_decode(steps, warm, torch):
    import synth
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(1)
    L = make_layer(w)
    H = w["H"]
    x_all = dev(np.stack([synth.tokens(w, s) for s in range(steps + warm)]))  # [n, 1, H]
    out_all = torch.empty((steps + warm, 1, H), dtype=torch.int16, device="cuda")
    fb = L.fused_buffers(1)
    for s in range(min(warm, 5)):  # eager: loads the kernels
        L.decode_fused(x_all[s], fb, out=out_all[s])
    torch.cuda.synchronize()

    CH = 100

    def capture(first, count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in range(first, first + count):
                L.decode_fused(x_all[s], fb, out=out_all[s])
        return g

    graphs_w = [capture(s, min(CH, warm - s)) for s in range(0, warm, CH)]
    graphs_t = [capture(warm + s, min(CH, steps - s)) for s in range(0, steps, CH)]
    for g in graphs_w:
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for g in graphs_t:
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    assert L.fused_error_word(fb) == 0
    gpu_ms = e0.elapsed_time(e1)
    nbytes = decode_bytes(w)
    avg_us = gpu_ms * 1e3 / steps
    ach = nbytes["total"] / (avg_us * 1e-6) / 1e9
    return dict(w=w, steps=steps, warm=warm, wall_s=t1 - t0, gpu_ms=gpu_ms, avg_us=avg_us,
                achieved=ach, nbytes=nbytes)


def bench_prefill(torch, reps=20):
    import synth
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(4)
    T = w["T"]
    L = make_layer(w)
    x = dev(synth.tokens(w, 0))
    bias = dev(synth.zipf_bias(w))
    b = L.buffers(T, prefill=True)
    L.forward(x, b, bias=bias)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.forward(x, b, bias=bias)
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    block_ms = e0.elapsed_time(e1) / reps
    # the grouped GEMMs alone (moe_expert_forward), back to back
    e0.record()
    for _ in range(reps):
        L.experts_forward(x, b)
    e1.record()
    torch.cuda.synchronize()
    gemm_ms = e0.elapsed_time(e1) / reps
    counts = b["counts"].cpu().numpy()
    fl = prefill_flops(w, T)
    tflops = fl["expert_gemm"] / (gemm_ms * 1e-3) / 1e12
    return {
        "workload": w["name"], "tokens": T, "value": round(T / (block_ms * 1e-3), 1),
        "unit": "tokens/s", "block_ms": round(block_ms, 4),
        "experts_used": int((counts > 0).sum()), "largest_group": int(counts.max()),
        "roofline": {"bound": "mfma", "kernel": "moe_expert_forward (grouped GEMMs)",
                     "achieved": round(tflops, 1), "peak": MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_PEAK_TFLOPS, 4),
                     "flops_per_launch": fl["expert_gemm"], "avg_ms": round(gemm_ms, 4),
                     "traffic": None},
    }


def bench_stack(torch, tokens=200, warm=10):
    import synth
    from int4_expert_ffn_int8_amd import binding as B
    from int4_expert_ffn_int8_amd.layer import dev
    w = synth.workload(2)
    layers = [make_layer(w, l, threads=16) for l in range(w["layers"])]
    fbs = [Lr.fused_buffers(1) for Lr in layers]
    n = tokens + warm
    x_all = dev(np.stack([synth.tokens(w, s) for s in range(n)]))
    hbuf = torch.empty((w["layers"] + 1, 1, w["H"]), dtype=torch.int16, device="cuda")
    flags = B.DECODE_NORM_INPUT | B.DECODE_RESIDUAL

    def token(s):
        hbuf[0].copy_(x_all[s])
        for l, (Lr, fb) in enumerate(zip(layers, fbs)):
            Lr.decode_fused(hbuf[l], fb, flags=flags, eps=w["rms_eps"], out=hbuf[l + 1])

    token(0)
    torch.cuda.synchronize()
    CH = 10

    def capture(first, count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in range(first, first + count):
                token(s)
        return g

    gw = [capture(s, min(CH, warm - s)) for s in range(0, warm, CH)]
    gt = [capture(warm + s, min(CH, tokens - s)) for s in range(0, tokens, CH)]
    for g in gw:
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for g in gt:
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    per_token = decode_bytes(w)["total"] * w["layers"]
    return {"workload": w["name"], "value": round(tokens / (ms * 1e-3), 1), "unit": "tokens/s",
            "tokens": tokens, "warmup": warm, "ms_per_token": round(ms / tokens, 4),
            "hbm_gbps": round(per_token / (ms / tokens * 1e-3) / 1e9, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--stack", action="store_true", help="also time the 24-layer stack")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    d = bench_decode(args.steps, args.warmup, torch)
    w = d["w"]
    res = {
        "metric": METRIC,
        "value": round(d["steps"] * w["T"] / d["wall_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": d["steps"],
        "warmup": d["warm"],
        "ms_per_step": round(d["wall_s"] * 1e3 / d["steps"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random int4/int8 weights, bf16 activations)",
        "config": {"workload": w["name"], "tokens_per_step": w["T"], "hidden": w["H"],
                   "experts": w["E"], "top_k": w["K"], "intermediate": w["I"],
                   "shared_experts": w["n_shared"], "lora_rank": w["r"],
                   "path": "moe_block_decode (one kernel per step), HIP graphs of 100 steps"},
        "roofline": {"bound": "hbm", "kernel": "k_fused_decode<2048,512>",
                     "achieved": round(d["achieved"], 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(d["achieved"] / HBM_PEAK_GBPS, 4),
                     "traffic": None, "bytes_per_launch": d["nbytes"]["total"],
                     "avg_us": round(d["avg_us"], 3)},
    }
    if not args.no_prefill:
        res["prefill"] = bench_prefill(torch)
    if args.stack:
        res["stack24"] = bench_stack(torch)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
