"""GPU check of qlora_backward_noalloc, the backward for callers that cannot
allocate: two calls in a row on one GPU, the second with a smaller input,
each compared with qlora_backward (caller workspace) on the same inputs --
bit-identical, since both run the same kernels on the same data -- and with
the oracle at the usual bars (dX within 1e-2, dA and dB within 2e-2 of
max|ref|).  The first call is a split-K shape that fills several MiB of the
scratch array; the second reads a smaller part of the array that still
holds the first call's data.
"""

import numpy as np
import pytest
import torch

from gpu_util import Layer, bits_host, rel

pytestmark = pytest.mark.gpu


def _check(lib, L, save_t):
    T = None
    if save_t:
        _, T = lib.forward(L.X, L.w, L.A, L.B, L.alpha, save_t=True)
    ref = lib.backward(L.dY, L.X, L.w, L.A, L.B, L.alpha, T_saved=T)
    got = lib.backward_noalloc(L.dY, L.X, L.w, L.A, L.B, L.alpha, T_saved=T)
    torch.cuda.synchronize()
    for g, r in zip(got, ref):
        assert np.array_equal(bits_host(g), bits_host(r))
    dXr, dAr, dBr = L.oracle_bwd()
    eX, eA, eB = rel(bits_host(got[0]), dXr), rel(bits_host(got[1]), dAr), rel(bits_host(got[2]), dBr)
    print(f"  rel errors dX {eX:.2e} dA {eA:.2e} dB {eB:.2e}", flush=True)
    assert eX <= 1e-2 and eA <= 2e-2 and eB <= 2e-2


def test_noalloc_backward_two_calls(lib):
    print("case: noalloc backward d=768 k=1024 r=16 M=300 (split-K dX), then d=256 k=256 r=8 M=64", flush=True)
    big = Layer(lib, 768, 1024, 16, 300, cfg=61)
    assert lib.lib().qlora_backward_workspace_bytes(300, 768, 1024, 16) > 1 << 20
    _check(lib, big, save_t=False)
    small = Layer(lib, 256, 256, 8, 64, cfg=62)
    _check(lib, small, save_t=True)


def test_noalloc_backward_training_shape(lib):
    # the benchmark's layer: 4096 x 4096, r = 16, 4096 tokens, T saved by
    # the forward; compared bit for bit with the workspace call
    print("case: noalloc backward d=k=4096 r=16 M=4096", flush=True)
    L = Layer(lib, 4096, 4096, 16, 4096, cfg=63, oracle_quant=False)
    _, T = lib.forward(L.X, L.w, L.A, L.B, L.alpha, save_t=True)
    ref = lib.backward(L.dY, L.X, L.w, L.A, L.B, L.alpha, T_saved=T)
    got = lib.backward_noalloc(L.dY, L.X, L.w, L.A, L.B, L.alpha, T_saved=T)
    torch.cuda.synchronize()
    for g, r in zip(got, ref):
        assert np.array_equal(bits_host(g), bits_host(r))


def test_noalloc_rejects_oversized_shape(lib):
    # more workspace than the scratch array holds: QLORA_ERR_WORKSPACE,
    # nothing launched
    print("case: noalloc backward oversized d=4096 k=16384 r=16 M=128", flush=True)
    L = Layer(lib, 4096, 16384, 16, 128, cfg=64, oracle_quant=False)
    with pytest.raises(lib.QloraError) as e:
        lib.backward_noalloc(L.dY, L.X, L.w, L.A, L.B, L.alpha)
    assert e.value.status == 5
