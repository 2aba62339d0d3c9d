"""Per-kernel timing (qlora_timing_*) on the GPU: while it is on, launches
carry events stamped by the dispatch.  The results must not change, every
launch must be counted once, and each kernel's time must fit inside the wall
time of the block that ran it."""

import time

import numpy as np
import pytest
import torch

import workloads as WL
from gpu_util import Layer, bits_host, f32_dev

pytestmark = pytest.mark.gpu


def _step(lib, L):
    Y, T = lib.forward(L.X, L.w, L.A, L.B, L.alpha, save_t=True)
    dX, dA, dB = lib.backward(L.dY, L.X, L.w, L.A, L.B, L.alpha, T_saved=T)
    W = lib.merge(L.w, L.A, L.B, L.alpha)
    return [bits_host(t) for t in (Y, dX, dA, dB, W)]


@pytest.mark.parametrize("d,k,r,M", [(512, 512, 16, 300), (1024, 768, 64, 1024)])
def test_timing_same_results_and_counts(lib, d, k, r, M):
    print("case: timing", d, k, r, M, flush=True)
    L = Layer(lib, d, k, r, M, oracle_quant=False)
    ref = _step(lib, L)
    torch.cuda.synchronize()
    steps = 3
    t0 = time.perf_counter()
    with lib.kernel_timing():
        got = [_step(lib, L) for _ in range(steps)]
        torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    tot = lib.kernel_timing.totals()
    for g in got:
        for a, b in zip(g, ref):
            assert np.array_equal(a, b)
    assert tot["fwd_rich"][1] == steps
    assert tot["dx"][1] == steps
    assert tot["merge"][1] == steps
    assert tot["lora_proj"][1] >= 2 * steps
    assert tot["token_reduce"][1] >= steps
    for name, (ms, n) in tot.items():
        assert 0.0 < ms < wall_ms, (name, ms, wall_ms)
    # nothing is counted once timing is off again
    _step(lib, L)
    torch.cuda.synchronize()
    assert lib.kernel_timing.totals() == tot


def test_timing_quantize_counts(lib):
    print("case: timing quantize", flush=True)
    W0 = f32_dev(WL.normal_f32((256, 1024), 0.02, (0, 21, 256, 1024, 0)))
    ref = lib.quantize(W0)
    with lib.kernel_timing():
        w = lib.quantize(W0)
        torch.cuda.synchronize()
    tot = lib.kernel_timing.totals()
    for n in ("quant_blocks", "quant_group_sums", "quant_mean", "quant_dq"):
        assert tot[n][1] == 1 and tot[n][0] > 0.0
    assert torch.equal(w.codes, ref.codes)
    assert torch.equal(w.absmax_q, ref.absmax_q)
