"""GPU parity of the per-token adapter forward (qlora_forward_multi)
against the oracle's forward_multi: one frozen NF4 base, nad adapters, an
adapter index per token (indices outside [0, nad) mean no adapter).

Bars: Y within max|err|/max|ref| <= 1e-2; bit-exact against qlora_forward
when one adapter serves every token (M <= 64), and against the base-only
call when no token has an adapter.
"""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from gpu_util import DEV, bf16_dev, bits_host, f32_dev, rel

pytestmark = pytest.mark.gpu

TOL_Y = 1e-2


def _print_case(*args):
    print("case:", *args, flush=True)


class Multi:
    def __init__(self, lib, d, k, r, nad, M, idx=None):
        inp = WL.layer_inputs(d, k, r, M, cfg=95)
        self.Xb = inp["X"]
        self.q_ref = O.quantize(inp["W0"])
        self.Wt = O.dequantize(self.q_ref)
        ads = [WL.layer_inputs(d, k, r, 1, cfg=95, proj=1 + a) for a in range(nad)]
        self.As = [a["A"] for a in ads]
        self.Bs = [a["B"] for a in ads]
        if idx is None:
            idx = np.array([(7 * m + 3) % (nad + 2) - 1 for m in range(M)], np.int32)
        self.idx = idx
        self.w = lib.quantize(f32_dev(inp["W0"]))
        self.X = bf16_dev(self.Xb)
        self.A = bf16_dev(np.concatenate(self.As, axis=0))
        self.B = bf16_dev(np.concatenate(self.Bs, axis=0))
        self.I = torch.from_numpy(idx).to(DEV)
        self.alpha = 2.0 * r


# (d, k, r, nad, M): chunked decode kernel (k % 256 == 0), split-K decode
# kernel (k % 256 != 0), many adapters (512 ranks in the weight stream),
# more than one group of tokens, the 11008-row decode shape
CASES = [
    (256, 256, 8, 4, 16),
    (512, 320, 16, 3, 40),
    (1024, 512, 16, 32, 64),
    (256, 512, 64, 2, 150),     # groups of 128 and 22 tokens
    (256, 320, 16, 3, 150),     # k % 256 != 0: groups of 64, 64 and 22
    (11008, 4096, 16, 8, 16),
]


@pytest.mark.parametrize("d,k,r,nad,M", CASES)
def test_multi_adapter_forward_parity(lib, d, k, r, nad, M):
    _print_case("multi", d, k, r, nad, M)
    S = Multi(lib, d, k, r, nad, M)
    Y = lib.forward_multi(S.X, S.w, S.A, S.B, S.I, S.alpha)
    ref = O.forward_multi(S.Xb, S.Wt, S.As, S.Bs, S.idx, S.alpha)
    assert rel(bits_host(Y), ref) <= TOL_Y


@pytest.mark.parametrize("M", [1, 16, 64])
def test_one_adapter_for_every_token_is_qlora_forward(lib, monkeypatch, M):
    # per-token adapters run the split-K decode kernels; the plain call is
    # held to the same kernels (up to 16 tokens it could also take the
    # single launch, whose sums run in another order)
    _print_case("multi one adapter", M)
    monkeypatch.setenv("QLORA_DECODE", "split")
    S = Multi(lib, 512, 512, 16, 1, M, idx=np.zeros(M, np.int32))
    Y = bits_host(lib.forward_multi(S.X, S.w, S.A, S.B, S.I, S.alpha))
    Y1 = bits_host(lib.forward(S.X, S.w, S.A, S.B, S.alpha))
    assert np.array_equal(Y, Y1)


def test_tokens_without_adapter_get_the_base_output(lib):
    _print_case("multi no adapter")
    M = 40
    S = Multi(lib, 512, 320, 16, 3, M, idx=np.array([-1, 3] * (M // 2), np.int32))
    Y = bits_host(lib.forward_multi(S.X, S.w, S.A, S.B, S.I, S.alpha))
    Y0 = bits_host(lib.forward(S.X, S.w))
    assert np.array_equal(Y, Y0)


def test_multi_adapter_graph_replays_match_eager(lib):
    # a serving loop captures its decode calls once and replays them: every
    # replay must give the eager bits (eager work in between)
    _print_case("multi graph", 1024, 512, 16, 8, 16)
    S = Multi(lib, 1024, 512, 16, 8, 16)
    ref = bits_host(lib.forward_multi(S.X, S.w, S.A, S.B, S.I, S.alpha))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lib.forward_multi(S.X, S.w, S.A, S.B, S.I, S.alpha)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        Y = lib.forward_multi(S.X, S.w, S.A, S.B, S.I, S.alpha)
    for rep in range(3):
        Y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_host(Y), ref), rep
        lib.forward(S.X, S.w, S.A[:16], S.B[:1024], S.alpha)
        torch.cuda.synchronize()
