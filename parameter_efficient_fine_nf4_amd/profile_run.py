"""Fixed workloads of libqlora for profiler runs (rocprofv3 counters).

Usage:  python parameter_efficient_fine_nf4_amd/profile_run.py
            [--what train,decode,copy] [--steps N]

train   N x (forward saving T + backward), d = k = 4096, r = 16, alpha = 32,
        M = 4096 tokens: the benchmark's training step.
decode  N x forward at M = 16 tokens on the same 4096 x 4096 weight.
decode_rot
        N passes of forwards at M = 16 over 64 copies of that weight in turn
        (551 MB of NF4, past the 256 MB last-level cache: every call reads
        its weight from HBM, as in the benchmark's decode legs).
copy    3 x a plain streaming kernel over 256 MiB (torch.neg into a second
        buffer: an elementwise kernel, unlike copy_, which may become a DMA
        transfer), the reference of known traffic (256 MiB read, 256 MiB
        written per launch) used to scale the HBM byte counters.
merge   after the others: quantise an 8192 x 8192 weight, then N x the
        merge W = w~ + s B A with r = 64, alpha = 16 (the 65B-shaped
        layer's square projection).

Inputs are the seeded synthetic tensors of the benchmark.  Each workload
prints one line when it is done.
"""

from __future__ import annotations

import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

COPY_BYTES = 256 << 20


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--what", default="train,decode,copy")
    ap.add_argument("--steps", type=int, default=3)
    args = ap.parse_args()
    what = set(args.what.split(","))

    import numpy as np
    import torch

    import parameter_efficient_fine_nf4_amd as q
    import workloads as WL

    dev = "cuda:0"

    def up(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    d = k = 4096
    if "train" in what or "decode" in what or "decode_rot" in what:
        inp = WL.layer_inputs(d, k, 16, 4096, cfg=1)
        w = q.quantize(torch.from_numpy(inp["W0"]).to(dev))
        A, B, X, dY = up(inp["A"]), up(inp["B"]), up(inp["X"]), up(inp["dY"])
        torch.cuda.synchronize()
    if "train" in what:
        for _ in range(args.steps):
            _, T = q.forward(X, w, A, B, 32.0, save_t=True)
            q.backward(dY, X, w, A, B, 32.0, T_saved=T)
        torch.cuda.synchronize()
        print(f"train: {args.steps} step(s) done", flush=True)
    if "decode" in what:
        Xd = X[:16].contiguous()
        for _ in range(args.steps):
            q.forward(Xd, w, A, B, 32.0)
        torch.cuda.synchronize()
        print(f"decode: {args.steps} forward(s) done", flush=True)
    if "decode_rot" in what:
        Xd = X[:16].contiguous()
        ws = [w] + [q.NF4Weight(d, k, w.codes.clone(), w.absmax_q.clone(), w.absmax_scale.clone(),
                                w.absmax_mean.clone()) for _ in range(63)]
        Yd = torch.empty((16, d), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            for wc in ws:
                q.forward(Xd, wc, A, B, 32.0, out=Yd)
        torch.cuda.synchronize()
        print(f"decode_rot: {args.steps} pass(es) over 64 weight copies done", flush=True)
        del ws
    if "copy" in what:
        src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(f"copy: 3 x {COPY_BYTES >> 20} MiB done", flush=True)
        del src, dst
    if "merge" in what:
        dm = km = 8192
        inp = WL.layer_inputs(dm, km, 64, 1, cfg=5)
        wm = q.quantize(torch.from_numpy(inp["W0"]).to(dev))
        Am, Bm = up(inp["A"]), up(inp["B"])
        Wm = torch.empty((dm, km), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            q.merge(wm, Am, Bm, 16.0, out=Wm)
        torch.cuda.synchronize()
        print(f"merge: {args.steps} merge(s) of {dm} x {km}, r = 64 done", flush=True)


if __name__ == "__main__":
    main()
