#!/usr/bin/env python3
"""Benchmark of the gfx950 QLoRA adapted linear (libqlora).

One step = one forward (saving T = X A^T) plus one backward (dX, dA, dB) of a
single QLoRA linear, d = k = 4096, r = 16, alpha = 32, M = 4096 tokens
(batch 4 x sequence 1024), on seeded synthetic inputs already resident in
HBM; W0 ~ N(0, 0.02^2) quantised once to NF4 with double-quantised absmax
before timing.  The headline value is whole-step throughput in TFLOP/s of
algorithmic work F = 4 M d k + 6 M r (d + k) (T reused, no dW0).

Also reported on the same JSON line:
  * the same step captured in a HIP graph and replayed (hip_graph_step);
  * the same step at r = 8, alpha = 16;
  * decode-shaped forwards (M = 16, r = 16) on 4096x4096, 11008x4096 and
    4096x11008, rotating over 64 copies of the weight (past the 256 MB
    last-level cache), as NF4 weight GB/s: per call issued eagerly, and the
    same 64 calls captured once in a HIP graph and replayed;
  * the 256 x 256 layer (r = 8, alpha = 16, 32 tokens): microseconds per
    quantise, forward, backward, merge and unmerge call;
  * a dense bf16 yardstick: torch.matmul (the vendor GEMM) of X w~^T and
    dY w~ at 4096^3 on the dequantised weight, beside the fused kernels;
  * fwd+bwd of the three projection shapes of a 7B-shaped layer (4096 x
    4096, 11008 x 4096, 4096 x 11008, r = 16, M = 2048) and of a 65B-shaped
    layer (8192 x 8192, 22016 x 8192, 8192 x 22016, r = 64, alpha = 16,
    M = 4096), and the merge of each shape as GB/s;
  * the two stacks as configured, all NF4 weights resident in HBM at once:
    32 layers x 7 projections of the 7B shapes (r = 16, M = 2048), fwd+bwd
    of every projection; 80 layers x 7 projections of the 65B shapes (r =
    64, M = 4096, 33.4 GB of NF4), fwd+bwd of every projection and the merge
    of every projection (skipped with --no-65b);
  * roofline of the dominant kernel from HIP-event brackets recorded by the
    library on its own stream during a timed pass;
  * cpu_baseline: the CPU oracle (numpy float64) timed on this host: the
    headline step, plus quantise / forward / backward / merge of the 256^2
    layer, of the 4096^2 layer and the M = 16 decode forwards;
  * memory_context: NF4 storage of the 7B- and 65B-shaped linear weights
    from the library's size query, beside the pages' memory figures.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-65b]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "QLoRA linear fwd+bwd TFLOP/s + NF4 weight GB/s (% roofline), 4096²,r=16"
TRAIN_KEY = "d4096_k4096_M4096_r16"      # workload key of the stored HBM counters
DECODE_KEY = "d4096_k4096_M16_r16"

# Kernel -> source file whose hash gates the stored HBM-traffic counters.
KERNEL_SRC = {"fwd_rich": "gemm_fwd.hip", "fwd_decode": "gemm_fwd.hip", "dx": "gemm_dx.hip",
              "token_reduce": "lora.hip", "lora_proj": "lora.hip", "merge": "merge.hip"}


def nf4_bytes(d: int, k: int) -> int:
    nb = d * k // 64
    return d * k // 2 + nb + 4 * ((nb + 255) // 256) + 4


def step_flops(M, d, k, r):
    return 4 * M * d * k + 6 * M * r * (d + k)


def kernel_flops(name, M, d, k, r):
    """Algorithmic flops of one launch of the named kernel in a step."""
    if name == "fwd_rich":
        return 2 * M * d * k + 2 * M * d * r
    if name == "dx":
        return 2 * M * d * k + 2 * M * k * r
    return None


def src_sha(kernel: str) -> str | None:
    f = KERNEL_SRC.get(kernel)
    if f is None:
        return None
    p = os.path.join(ROOT, "parameter_efficient_fine_nf4_amd", "csrc", f)
    with open(p, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if absent or taken on a different kernel source."""
    p = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        rec = json.load(fh).get(f"{kernel}@{workload}")
    if not rec or rec.get("src_sha") != src_sha(kernel):
        return None
    return rec.get("bytes_per_launch")


class Layer:
    def __init__(self, q, d, k, r, M, cfg, dev, alpha):
        import numpy as np
        import torch
        import workloads as WL
        self.d, self.k, self.r, self.M, self.alpha = d, k, r, M, float(alpha)
        self.inp = WL.layer_inputs(d, k, r, M, cfg=cfg)

        def up(bits):
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

        self.W0 = torch.from_numpy(self.inp["W0"]).to(dev)
        self.w = q.quantize(self.W0)
        self.A, self.B = up(self.inp["A"]), up(self.inp["B"])
        self.X, self.dY = up(self.inp["X"]), up(self.inp["dY"])
        self.Y = torch.empty((M, d), dtype=torch.bfloat16, device=dev)


def progress(msg):
    """One line on stderr per finished leg (stdout carries only the JSON line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def time_steps(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def bench_train_step(q, L, steps, warmup):
    def step():
        _, T = q.forward(L.X, L.w, L.A, L.B, L.alpha, save_t=True, out=L.Y)
        q.backward(L.dY, L.X, L.w, L.A, L.B, L.alpha, T_saved=T)

    sec = time_steps(step, steps, warmup)
    # second pass of the same steps with per-kernel HIP-event brackets
    with q.kernel_timing():
        t_k = time_steps(step, steps, 0)
    kt = q.kernel_timing.totals()
    return sec, t_k, kt


def graph_step_time(q, L, steps, warmup):
    """The same training step captured once in a HIP graph and replayed:
    the launch gaps between its five kernels shrink to the graph's."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _, T = q.forward(L.X, L.w, L.A, L.B, L.alpha, save_t=True, out=L.Y)
        q.backward(L.dY, L.X, L.w, L.A, L.B, L.alpha, T_saved=T)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _, T = q.forward(L.X, L.w, L.A, L.B, L.alpha, save_t=True, out=L.Y)
        q.backward(L.dY, L.X, L.w, L.A, L.B, L.alpha, T_saved=T)
    sec = time_steps(g.replay, steps, warmup)
    del g
    return sec


def bench_decode(q, dev, shapes, r, alpha, copies, reps):
    import torch
    import workloads as WL
    import numpy as np
    out = {}
    for (d, k) in shapes:
        inp = WL.layer_inputs(d, k, r, 16, cfg=2)
        w0 = q.quantize(torch.from_numpy(inp["W0"]).to(dev))
        ws = [w0]
        for _ in range(copies - 1):
            ws.append(q.NF4Weight(d, k, w0.codes.clone(), w0.absmax_q.clone(),
                                  w0.absmax_scale.clone(), w0.absmax_mean.clone()))

        def up(bits):
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

        X, A, B = up(inp["X"]), up(inp["A"]), up(inp["B"])
        Y = torch.empty((16, d), dtype=torch.bfloat16, device=dev)

        def run():
            for w in ws:
                q.forward(X, w, A, B, alpha, out=Y)

        sec = time_steps(run, reps, 2) / copies
        # the same calls captured once in a HIP graph (as a serving loop
        # would), replayed: the host's per-call launch cost drops out
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        gsec = time_steps(graph.replay, reps, 2) / copies
        del graph
        # (no per-kernel HIP-event times here: eager calls of a few
        # microseconds are issued more slowly than the GPU runs them, and the
        # event pairs would hold that wait; the rocprofv3 trace has the
        # kernels' own durations)
        nb = nf4_bytes(d, k)
        total = nb + 2 * 16 * k + 2 * 16 * d + 2 * r * k + 2 * d * r
        out[f"{d}x{k}"] = {
            "us_per_call_wall": round(sec * 1e6, 2),
            "us_per_call_graph": round(gsec * 1e6, 2),
            "nf4_bytes": nb,
            "nf4_GBps_graph": round(nb / gsec / 1e9, 1),
            "frac_hbm_graph": round(nb / gsec / 1e9 / PEAK_HBM_GBS, 4),
            "total_GBps_graph": round(total / gsec / 1e9, 1),
        }
        del ws
        torch.cuda.empty_cache()
    return out


def bench_decode_multi(q, dev, shapes, r, alpha, nad, copies, reps):
    """Decode-shaped forward (M = 16) with a per-token adapter: nad adapters
    over one NF4 base, the tokens' adapter indices drawn uniformly (seeded).
    Rotates over ``copies`` weight copies like the single-adapter leg."""
    import torch
    import workloads as WL
    import numpy as np
    out = {}
    for (d, k) in shapes:
        inp = WL.layer_inputs(d, k, r, 16, cfg=2)
        w0 = q.quantize(torch.from_numpy(inp["W0"]).to(dev))
        ws = [w0] + [q.NF4Weight(d, k, w0.codes.clone(), w0.absmax_q.clone(), w0.absmax_scale.clone(),
                                 w0.absmax_mean.clone()) for _ in range(copies - 1)]
        g = torch.Generator(device=dev)
        g.manual_seed(6000)
        A = (torch.randn(nad * r, k, generator=g, device=dev) * k ** -0.5).to(torch.bfloat16)
        B = (torch.randn(nad * d, r, generator=g, device=dev) * 0.01).to(torch.bfloat16)
        idx = torch.from_numpy(np.random.default_rng(6001).integers(0, nad, 16).astype(np.int32)).to(dev)
        X = torch.from_numpy(inp["X"].view(np.int16)).view(torch.bfloat16).to(dev)
        Y = torch.empty((16, d), dtype=torch.bfloat16, device=dev)

        def run():
            for w in ws:
                q.forward_multi(X, w, A, B, idx, alpha, out=Y)

        sec = time_steps(run, reps, 2) / copies
        # replayed from a HIP graph, as in the single-adapter leg
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        gsec = time_steps(graph.replay, reps, 2) / copies
        del graph
        nb = nf4_bytes(d, k)
        stream = nb + 2 * nad * r * k  # the NF4 weight and every adapter's A go through the decode kernel
        out[f"{d}x{k}"] = {
            "adapters": nad,
            "us_per_call_wall": round(sec * 1e6, 2),
            "us_per_call_graph": round(gsec * 1e6, 2),
            "nf4_plus_A_bytes": stream,
            "GBps_graph": round(stream / gsec / 1e9, 1),
        }
        del ws, A, B
        torch.cuda.empty_cache()
    return out


def memory_context(q):
    """Weight-storage figures of the shaped stacks from the library's own
    size query (bytes it needs per NF4 weight), next to the pages' memory
    figures, which are quoted as context (other models and hardware)."""
    def stack(layers, hidden, ffn, r):
        shapes = [(hidden, hidden)] * 4 + [(ffn, hidden)] * 2 + [(hidden, ffn)]
        nf4 = sum(sum(q.nf4_sizes(d, k).values()) for d, k in shapes)
        params = sum(d * k for d, k in shapes)
        adapters = sum(r * (d + k) for d, k in shapes)
        return {"layers": layers, "nf4_GB": round(layers * nf4 / 1e9, 2),
                "bf16_GB": round(layers * 2 * params / 1e9, 2),
                "adapters_bf16_GB": round(layers * 2 * adapters / 1e9, 2),
                "nf4_bits_per_param": round(8 * nf4 / params, 4)}
    return {
        "linear_weights_65b_shaped": stack(80, 8192, 22016, 64),
        "linear_weights_7b_shaped": stack(32, 4096, 11008, 16),
        "pages_context": {"65b_qlora_finetune_GB": "< 48 (one 48 GB GPU)",
                          "65b_16bit_full_finetune_GB": "> 780",
                          "gpt3_175b_full_finetune_TB": 1.2, "gpt3_175b_lora_GB": 350},
    }


def bench_dropout_step(q, L, p, steps, warmup):
    """The training step of layer L with LoRA dropout p on the adapter input
    (a seeded mask drawn on the device once; same flops as without)."""
    import torch
    g = torch.Generator(device=L.X.device)
    g.manual_seed(8000)
    keep = (torch.rand(L.X.shape, generator=g, device=L.X.device) >= p).to(torch.uint8)

    Xd = torch.empty_like(L.X)

    def step():
        _, T = q.forward_dropout(L.X, L.w, L.A, L.B, L.alpha, keep, p, save_t=True, out=L.Y, xd_out=Xd)
        q.backward_dropout(L.dY, L.X, L.w, L.A, L.B, L.alpha, keep, p, T_saved=T, Xd_saved=Xd)

    sec = time_steps(step, steps, warmup)
    with q.kernel_timing():
        time_steps(step, steps, 0)
    kt = q.kernel_timing.totals()
    fl = step_flops(L.M, L.d, L.k, L.r)
    return {"p": p, "ms_per_step": round(sec * 1e3, 4), "TFLOPs": round(fl / sec / 1e12, 2),
            "kernels_us_per_launch": {n: round(ms / c * 1e3, 2) for n, (ms, c) in sorted(kt.items())}}


def bench_adam(q, dev, steps):
    """One Adam step over the adapter parameters of a 65B-shaped layer (r =
    64 on all seven projections, 9.99 M parameters, 24 bytes each), with the
    fp32 state in device memory and in pinned host memory (paged state)."""
    import torch
    r = 64
    n = sum(cnt * r * (d + k) for d, k, cnt in [(8192, 8192, 4), (22016, 8192, 2), (8192, 22016, 1)])
    g = torch.Generator(device=dev)
    g.manual_seed(9000)
    G = (torch.randn(n, generator=g, device=dev) * 1e-3).to(torch.bfloat16)
    P = torch.empty(n, dtype=torch.bfloat16, device=dev)
    out = {"params": n, "bytes_per_step": 24 * n}
    for where in ("device", "pinned_host"):
        W = torch.randn(n, generator=g, device=dev) * 0.02
        m = torch.zeros(n, device=dev)
        v = torch.zeros(n, device=dev)
        if where == "pinned_host":
            W, m, v = (t.cpu().pin_memory() for t in (W, m, v))
        it = [0]

        def step():
            it[0] += 1
            q.adam_step(P, W, G, m, v, 1e-4, it[0])

        sec = time_steps(step, steps, 3)
        out[where] = {"us": round(sec * 1e6, 2), "GBps": round(24 * n / sec / 1e9, 1)}
        if where == "device":
            out[where]["frac_hbm"] = round(24 * n / sec / 1e9 / PEAK_HBM_GBS, 4)
        del W, m, v
    return out


def sections_step_time(q, dev, nsec, d, k, r, M, alpha, steps, seed):
    """Seconds per fwd+bwd of nsec d x k projections sharing one input,
    stacked by rows and run through forward_sections / backward_sections.
    Weights and activations drawn on the device (seeded torch generator,
    the distributions of the other workloads)."""
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    Ws = [torch.randn(d, k, generator=g, device=dev, dtype=torch.float32) * 0.02 for _ in range(nsec)]
    w = q.quantize_sections(Ws)
    del Ws
    A = (torch.randn(nsec * r, k, generator=g, device=dev) * k ** -0.5).to(torch.bfloat16)
    B = (torch.randn(nsec * d, r, generator=g, device=dev) * 0.01).to(torch.bfloat16)
    X = torch.randn(M, k, generator=g, device=dev).to(torch.bfloat16)
    dY = torch.randn(M, nsec * d, generator=g, device=dev).to(torch.bfloat16)
    Y = torch.empty((M, nsec * d), dtype=torch.bfloat16, device=dev)

    def step():
        _, T = q.forward_sections(X, w, A, B, alpha, save_t=True, out=Y)
        q.backward_sections(dY, X, w, A, B, alpha, T_saved=T)

    sec = time_steps(step, steps, 5)
    del w, A, B, X, dY, Y
    torch.cuda.empty_cache()
    return sec


def merge_bytes(d, k, r):
    return nf4_bytes(d, k) + 2 * d * k + 2 * r * (d + k)


def bench_7b_layer(q, dev, steps):
    """fwd+bwd of the three projection shapes of a 7B-shaped layer (hidden
    4096, FFN 11008, r = 16, alpha = 32, M = 2048 tokens); seeded inputs as
    in the other workloads.  The same shapes again with q, k, v as one
    three-section call and gate, up as one two-section call (each
    projection keeps its own weight, mean and adapter; same flops)."""
    M, r, alpha = 2048, 16, 32.0
    out = {}
    for i, (d, k) in enumerate([(4096, 4096), (11008, 4096), (4096, 11008)]):
        L = Layer(q, d, k, r, M, 3, dev, alpha)
        sec, _, _ = bench_train_step(q, L, steps, 5)
        fl = step_flops(M, d, k, r)
        out[f"{d}x{k}"] = {"ms_per_step": round(sec * 1e3, 4), "TFLOPs": round(fl / sec / 1e12, 2),
                           "frac_of_bf16_peak": round(fl / sec / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del L
    t_qkv = sections_step_time(q, dev, 3, 4096, 4096, r, M, alpha, steps, 7001)
    t_gu = sections_step_time(q, dev, 2, 11008, 4096, r, M, alpha, steps, 7002)
    for name, t, fl in (("qkv_sections_3x4096x4096", t_qkv, 3 * step_flops(M, 4096, 4096, r)),
                        ("gate_up_sections_2x11008x4096", t_gu, 2 * step_flops(M, 11008, 4096, r))):
        out[name] = {"ms_per_step": round(t * 1e3, 4), "TFLOPs": round(fl / t / 1e12, 2),
                     "frac_of_bf16_peak": round(fl / t / 1e12 / PEAK_BF16_TFLOPS, 4)}
    return out


def bench_65b_layer(q, dev, steps):
    """fwd+bwd of the three projection shapes of a 65B-shaped layer (hidden
    8192, FFN 22016, r = 64, alpha = 16, M = 4096 tokens), and the merge of
    each shape; then q, k, v as one three-section call (192 adapter ranks in
    all) and gate, up as one two-section call.  Weights and activations are
    drawn on the device (seeded torch generator; same distributions as the
    other workloads)."""
    import torch
    M, r, alpha = 4096, 64, 16.0
    g = torch.Generator(device=dev)
    out = {}
    for i, (d, k) in enumerate([(8192, 8192), (22016, 8192), (8192, 22016)]):
        g.manual_seed(5000 + i)
        W0 = torch.randn(d, k, generator=g, device=dev, dtype=torch.float32) * 0.02
        w = q.quantize(W0)
        del W0
        A = (torch.randn(r, k, generator=g, device=dev) * k ** -0.5).to(torch.bfloat16)
        B = (torch.randn(d, r, generator=g, device=dev) * 0.01).to(torch.bfloat16)
        X = torch.randn(M, k, generator=g, device=dev).to(torch.bfloat16)
        dY = torch.randn(M, d, generator=g, device=dev).to(torch.bfloat16)
        Y = torch.empty((M, d), dtype=torch.bfloat16, device=dev)

        def step():
            _, T = q.forward(X, w, A, B, alpha, save_t=True, out=Y)
            q.backward(dY, X, w, A, B, alpha, T_saved=T)

        sec = time_steps(step, steps, 5)
        fl = step_flops(M, d, k, r)
        Wm = torch.empty((d, k), dtype=torch.bfloat16, device=dev)
        msec = time_steps(lambda: q.merge(w, A, B, alpha, out=Wm), steps, 5)
        mb = merge_bytes(d, k, r)
        out[f"{d}x{k}"] = {"ms_per_step": round(sec * 1e3, 4), "TFLOPs": round(fl / sec / 1e12, 2),
                           "frac_of_bf16_peak": round(fl / sec / 1e12 / PEAK_BF16_TFLOPS, 4),
                           "merge_us": round(msec * 1e6, 2), "merge_GBps": round(mb / msec / 1e9, 1),
                           "merge_frac_hbm": round(mb / msec / 1e9 / PEAK_HBM_GBS, 4)}
        del w, A, B, X, dY, Y, Wm
        torch.cuda.empty_cache()
    t_qkv = sections_step_time(q, dev, 3, 8192, 8192, r, M, alpha, steps, 7003)
    t_gu = sections_step_time(q, dev, 2, 22016, 8192, r, M, alpha, steps, 7004)
    for name, t, fl in (("qkv_sections_3x8192x8192", t_qkv, 3 * step_flops(M, 8192, 8192, r)),
                        ("gate_up_sections_2x22016x8192", t_gu, 2 * step_flops(M, 22016, 8192, r))):
        out[name] = {"ms_per_step": round(t * 1e3, 4), "TFLOPs": round(fl / t / 1e12, 2),
                     "frac_of_bf16_peak": round(fl / t / 1e12 / PEAK_BF16_TFLOPS, 4)}
    return out


def bench_stack(q, dev, layers, hidden, ffn, r, alpha, M, seed, merge, passes=2, sections=False):
    """A whole stack as configured: ``layers`` layers of seven projections
    (q, k, v, o: hidden x hidden; gate, up: ffn x hidden; down: hidden x
    ffn), every NF4 weight and adapter resident in HBM at once (drawn per
    projection on the device with a seeded torch generator: W0 ~ N(0,
    0.02^2) fp32, quantised, then freed; A ~ N(0, 1/k), B ~ N(0, 0.01^2)).
    One pass runs forward (saving T) and backward of every projection of
    every layer, each on the activation pool of its shape (X, dY ~ N(0, 1)
    bf16, one pool per shape: the linear parts only, no chaining).  With
    ``merge``, a second pass merges every projection of every layer into a
    dense bf16 buffer of its shape.  With ``sections`` the projections that
    share their input in a layer run as one call each: q, k, v as a
    three-section weight and gate, up as a two-section one (the same
    weights, adapters and products; o and down alone)."""
    import torch
    shapes = [(hidden, hidden)] * 4 + [(ffn, hidden)] * 2 + [(hidden, ffn)]
    # calls of a layer: (first projection, number of sections)
    groups = [(0, 3), (3, 1), (4, 2), (6, 1)] if sections else [(p, 1) for p in range(7)]
    g = torch.Generator(device=dev)
    t0 = time.perf_counter()
    stack = []
    for l in range(layers):
        drawn = []
        for p, (d, k) in enumerate(shapes):
            g.manual_seed(seed * 1000003 + l * 8 + p)
            W0 = torch.randn(d, k, generator=g, device=dev, dtype=torch.float32) * 0.02
            w = None if sections else q.quantize(W0)
            A = (torch.randn(r, k, generator=g, device=dev) * k ** -0.5).to(torch.bfloat16)
            B = (torch.randn(d, r, generator=g, device=dev) * 0.01).to(torch.bfloat16)
            drawn.append((W0 if sections else None, w, A, B))
            del W0
        calls = []
        for p0, ns in groups:
            part = drawn[p0:p0 + ns]
            if ns == 1 and not sections:
                calls.append((part[0][1], part[0][2], part[0][3], 1))
            elif ns == 1:
                calls.append((q.quantize(part[0][0]), part[0][2], part[0][3], 1))
            else:
                calls.append((q.quantize_sections([e[0] for e in part]), torch.cat([e[2] for e in part]),
                              torch.cat([e[3] for e in part]), ns))
        del drawn
        stack.append(calls)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t0
    g.manual_seed(seed * 1000003 + 999)
    pools = {}
    for d, k in set(shapes):
        pools[(d, k)] = (torch.randn(M, k, generator=g, device=dev).to(torch.bfloat16),
                         torch.randn(M, d, generator=g, device=dev).to(torch.bfloat16),
                         torch.empty((M, d), dtype=torch.bfloat16, device=dev))
    for p0, ns in groups:  # output-gradient pools of the section calls (inputs shared)
        d, k = shapes[p0]
        if ns > 1:
            pools[(ns * d, k)] = (pools[(d, k)][0],
                                  torch.randn(M, ns * d, generator=g, device=dev).to(torch.bfloat16),
                                  torch.empty((M, ns * d), dtype=torch.bfloat16, device=dev))
    nf4_total = sum(sum(q.nf4_sizes(d, k).values()) for d, k in shapes) * layers

    def fwd_bwd():
        for calls in stack:
            for (w, A, B, ns), (p0, _) in zip(calls, groups):
                d, k = shapes[p0]
                X, dY, Y = pools[(ns * d, k)]
                if ns == 1:
                    _, T = q.forward(X, w, A, B, alpha, save_t=True, out=Y)
                    q.backward(dY, X, w, A, B, alpha, T_saved=T)
                else:
                    _, T = q.forward_sections(X, w, A, B, alpha, save_t=True, out=Y)
                    q.backward_sections(dY, X, w, A, B, alpha, T_saved=T)

    sec = time_steps(fwd_bwd, passes, 1)
    flops = layers * sum(step_flops(M, d, k, r) for d, k in shapes)
    out = {"layers": layers, "projections": layers * len(shapes), "calls_per_layer": len(groups), "r": r,
           "alpha": alpha, "tokens": M,
           "nf4_resident_GB": round(nf4_total / 1e9, 3), "setup_s": round(setup_s, 2),
           "fwd_bwd_ms": round(sec * 1e3, 3), "fwd_bwd_TFLOPs": round(flops / sec / 1e12, 2),
           "frac_of_bf16_peak": round(flops / sec / 1e12 / PEAK_BF16_TFLOPS, 4)}
    if merge:
        outs = {dk: torch.empty(dk, dtype=torch.bfloat16, device=dev) for dk in set(shapes)}

        def merge_all():
            for calls in stack:
                for (w, A, B, _), (d, k) in zip(calls, shapes):
                    q.merge(w, A, B, alpha, out=outs[(d, k)])

        msec = time_steps(merge_all, passes, 1)
        mb = layers * sum(merge_bytes(d, k, r) for d, k in shapes)
        out.update({"merge_all_ms": round(msec * 1e3, 3), "merge_GB_moved": round(mb / 1e9, 2),
                    "merge_GBps": round(mb / msec / 1e9, 1),
                    "merge_frac_hbm": round(mb / msec / 1e9 / PEAK_HBM_GBS, 4)})
        del outs
    del stack, pools
    torch.cuda.empty_cache()
    return out


def bench_small_layer(q, dev, reps=200):
    """The 256 x 256 layer (r = 8, alpha = 16, 32 tokens, seeded inputs):
    microseconds per call of quantise, forward, backward, merge and unmerge
    (latency-bound: the work is a few MFLOP), and the B = 0 forward."""
    import numpy as np
    import torch
    import workloads as WL
    d = k = 256
    r, alpha, M = 8, 16.0, 32
    inp = WL.layer_inputs(d, k, r, M, cfg=0)

    def up(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    W0 = torch.from_numpy(inp["W0"]).to(dev)
    w = q.quantize(W0)
    A, B, X, dY = up(inp["A"]), up(inp["B"]), up(inp["X"]), up(inp["dY"])
    B0 = torch.zeros_like(B)
    Y = torch.empty((M, d), dtype=torch.bfloat16, device=dev)
    _, T = q.forward(X, w, A, B, alpha, save_t=True)
    Wm = q.merge(w, A, B, alpha)
    Wu = torch.empty_like(Wm)
    legs = {
        "quantize": lambda: q.quantize(W0, out=w),
        "forward": lambda: q.forward(X, w, A, B, alpha, out=Y),
        "forward_b_zero": lambda: q.forward(X, w, A, B0, alpha, out=Y),
        "backward": lambda: q.backward(dY, X, w, A, B, alpha, T_saved=T),
        "merge": lambda: q.merge(w, A, B, alpha, out=Wm),
        "unmerge": lambda: q.unmerge(Wm, A, B, alpha, out=Wu),
    }
    out = {"workload": f"d={d} k={k} r={r} alpha={alpha:g} M={M}"}
    for name, fn in legs.items():
        out[f"{name}_us"] = round(time_steps(fn, reps, 10) * 1e6, 2)
    return out


def bench_dense_yardstick(q, L, steps):
    """The vendor library's dense bf16 GEMM (torch.matmul) on the same shapes
    as the step's two big products, with the dequantised weight w~ (from
    lora_merge with r = 0) stored dense: X w~^T and dY w~.  A yardstick for
    the fused NF4 kernels, which read a quarter of the weight bytes but
    decode every weight in registers."""
    import torch
    Wt = q.merge(L.w)                                    # d x k bf16, w~ itself
    M, d, k = L.M, L.d, L.k
    out = {}
    for name, fn, fl in (("x_wT", lambda: torch.matmul(L.X, Wt.t()), 2 * M * d * k),
                         ("dy_w", lambda: torch.matmul(L.dY, Wt), 2 * M * d * k)):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / steps * 1e3
        out[name] = {"us": round(us, 2), "TFLOPs": round(fl / us / 1e6, 2),
                     "frac_of_bf16_peak": round(fl / us / 1e6 / PEAK_BF16_TFLOPS, 4)}
    del Wt
    return out


def _cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model


def cpu_baseline(L, budget_s=12.0):
    """The oracle timed on this host, BLAS on every core available to the
    process (set with threadpoolctl and recorded): its forward + backward
    on the timed workload (the headline comparison), then its quantise,
    forward, backward and merge on the 256^2 layer, its quantise and merge
    on the 4096^2 layer, and its quantise + M = 16 forward on the three
    decode shapes (single runs; about 15-30 s in all)."""
    import numpy as np
    import oracle as O
    import workloads as WL
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=cores, user_api="blas")
        threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"),
                      default=cores)
    except Exception:  # pragma: no cover
        limiter, threads = None, cores
    q = O.quantize(L.inp["W0"])
    Wt = O.dequantize(q)
    n = 0
    t0 = time.perf_counter()
    while True:
        O.forward(L.inp["X"], Wt, L.inp["A"], L.inp["B"], L.alpha)
        O.backward(L.inp["dY"], L.inp["X"], Wt, L.inp["A"], L.inp["B"], L.alpha)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 5:
            break
    sec = el / n

    def timed(fn):
        t = time.perf_counter()
        r = fn()
        return r, time.perf_counter() - t

    legs = {}
    s_in = WL.layer_inputs(256, 256, 8, 32, cfg=0)
    qs, t_q = timed(lambda: O.quantize(s_in["W0"]))
    Ws, t_d = timed(lambda: O.dequantize(qs))
    _, t_f = timed(lambda: O.forward(s_in["X"], Ws, s_in["A"], s_in["B"], 16.0))
    _, t_b = timed(lambda: O.backward(s_in["dY"], s_in["X"], Ws, s_in["A"], s_in["B"], 16.0))
    _, t_m = timed(lambda: O.merge(Ws, s_in["A"], s_in["B"], 16.0))
    legs["d256_k256_r8_M32"] = {"quantize_ms": round(t_q * 1e3, 2), "dequantize_ms": round(t_d * 1e3, 2),
                                "forward_ms": round(t_f * 1e3, 2), "backward_ms": round(t_b * 1e3, 2),
                                "merge_ms": round(t_m * 1e3, 2)}
    _, t_q = timed(lambda: O.quantize(L.inp["W0"]))
    _, t_m = timed(lambda: O.merge(Wt, L.inp["A"], L.inp["B"], L.alpha))
    legs[f"d{L.d}_k{L.k}_r{L.r}"] = {"quantize_ms": round(t_q * 1e3, 1), "merge_ms": round(t_m * 1e3, 1),
                                     "fwd_bwd_ms": round(sec * 1e3, 1)}
    for (d, k) in [(4096, 4096), (11008, 4096), (4096, 11008)]:
        di = WL.layer_inputs(d, k, 16, 16, cfg=2)
        qd, t_q = timed(lambda: O.quantize(di["W0"]))
        Wd, t_d = timed(lambda: O.dequantize(qd))
        _, t_f = timed(lambda: O.forward(di["X"], Wd, di["A"], di["B"], 32.0))
        legs[f"decode_d{d}_k{k}_M16_r16"] = {"quantize_ms": round(t_q * 1e3, 1),
                                             "dequantize_ms": round(t_d * 1e3, 1),
                                             "forward_ms": round(t_f * 1e3, 2),
                                             "nf4_GBps_forward": round(nf4_bytes(d, k) / t_f / 1e9, 3)}
        del di, qd, Wd
    if limiter is not None:
        limiter.restore_original_limits()
    return {"value": round(step_flops(L.M, L.d, L.k, L.r) / sec / 1e12, 4), "unit": "TFLOP/s",
            "cores": int(threads), "kind": "oracle",
            "sample": f"{n} full oracle fwd+bwd step(s) of the timed workload "
                      f"(float64 numpy, w~ precomputed), {sec:.2f} s/step",
            "cpu_model": _cpu_info(), "cpus_available": cores, "blas_threads": int(threads),
            "legs": legs}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-reps", type=int, default=8)
    ap.add_argument("--no-65b", action="store_true", help="skip the 65B-shaped layer leg")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import parameter_efficient_fine_nf4_amd as q

    dev = "cuda:0"
    d = k = 4096
    M = 4096
    L16 = Layer(q, d, k, 16, M, 1, dev, 32.0)
    sec16, sec16_k, kt16 = bench_train_step(q, L16, args.steps, args.warmup)
    F16 = step_flops(M, d, k, 16)
    value = F16 / sec16 / 1e12
    sec16_g = graph_step_time(q, L16, args.steps, args.warmup)

    # dominant kernel of the step and its roofline
    per_launch = {n: (ms / c) for n, (ms, c) in kt16.items()}
    dom = max(kt16, key=lambda n: kt16[n][0])
    dom_fl = kernel_flops(dom, M, d, k, 16)
    dom_s = per_launch[dom] * 1e-3
    workload = f"qlora_linear d={d} k={k} r=16 alpha=32 M={M} fwd+bwd"
    roof = {"bound": "mfma", "kernel": dom,
            "achieved": round(dom_fl / dom_s / 1e12, 2) if dom_fl else None,
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(dom_fl / dom_s / 1e12 / PEAK_BF16_TFLOPS, 4) if dom_fl else None,
            "traffic": stored_traffic(dom, TRAIN_KEY),
            "us_per_launch": round(per_launch[dom] * 1e3, 2)}

    L8 = Layer(q, d, k, 8, M, 1, dev, 16.0)
    sec8, _, kt8 = bench_train_step(q, L8, max(5, args.steps // 2), 3)

    decode = bench_decode(q, dev, [(4096, 4096), (11008, 4096), (4096, 11008)], 16, 32.0,
                          copies=64, reps=args.decode_reps)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(sec16 * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "global_batch": 4, "seq_len": 1024, "tokens": M,
                   "d": d, "k": k, "r": 16, "alpha": 32, "parallelism": "none (1 GPU)"},
        "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": roof,
        "kernels_us_per_launch": {n: round(v * 1e3, 2) for n, v in sorted(per_launch.items())},
        "ms_per_step_kernel_timing_pass": round(sec16_k * 1e3, 4),
        "hip_graph_step": {"ms_per_step": round(sec16_g * 1e3, 4), "TFLOPs": round(F16 / sec16_g / 1e12, 2)},
        "r8_alpha16": {"ms_per_step": round(sec8 * 1e3, 4),
                       "TFLOPs": round(step_flops(M, d, k, 8) / sec8 / 1e12, 2),
                       "kernels_us_per_launch": {n: round(ms / c * 1e3, 2)
                                                 for n, (ms, c) in sorted(kt8.items())}},
        "lora_dropout_step": bench_dropout_step(q, L16, 0.1, max(5, args.steps // 2), args.warmup),
        "adam_step_65b_layer_adapters": bench_adam(q, dev, max(5, args.steps // 2)),
        "nf4_decode_m16_r16": decode,
        "nf4_decode_m16_r16_8_adapters": bench_decode_multi(q, dev, [(4096, 4096), (11008, 4096)], 16, 32.0, 8,
                                                            64, args.decode_reps),
    }
    progress("headline, graph, r=8, dropout, adam and decode legs done")
    line["layer_256_r8_M32"] = bench_small_layer(q, dev)
    line["dense_bf16_yardstick_4096"] = bench_dense_yardstick(q, L16, args.steps)
    line["dense_bf16_yardstick_4096"]["fused_fwd_rich_us"] = round(per_launch.get("fwd_rich", 0.0) * 1e3, 2)
    line["dense_bf16_yardstick_4096"]["fused_dx_us"] = round(per_launch.get("dx", 0.0) * 1e3, 2)
    progress("256^2 layer and dense yardstick done")
    if not args.no_65b:
        line["layer_7b_r16_M2048"] = bench_7b_layer(q, dev, max(5, args.steps // 5))
        line["layer_65b_r64_M4096"] = bench_65b_layer(q, dev, max(5, args.steps // 5))
        progress("7B- and 65B-shaped layer legs done")
        line["stack_7b_32_layers_r16_M2048"] = bench_stack(q, dev, 32, 4096, 11008, 16, 32.0, 2048, 31,
                                                           merge=False)
        line["stack_7b_32_layers_r16_M2048_section_calls"] = bench_stack(q, dev, 32, 4096, 11008, 16, 32.0, 2048,
                                                                         31, merge=False, sections=True)
        progress("32-layer stack done")
        line["stack_65b_80_layers_r64_M4096"] = bench_stack(q, dev, 80, 8192, 22016, 64, 16.0, 4096, 79,
                                                            merge=True)
        line["stack_65b_80_layers_r64_M4096_section_calls"] = bench_stack(q, dev, 80, 8192, 22016, 64, 16.0, 4096,
                                                                          79, merge=False, sections=True)
        progress("80-layer stack done")
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(L16)
        progress("cpu baseline done")
    line["memory_context"] = memory_context(q)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
