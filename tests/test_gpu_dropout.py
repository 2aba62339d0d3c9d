"""GPU parity of the adapted linear with LoRA dropout on the adapter input
(qlora_forward_dropout / qlora_backward_dropout) against the oracle's
forward_dropout / backward_dropout, on the same seeded mask.

Bars: Y and dX within max|err|/max|ref| <= 1e-2, dA and dB within 2e-2, the
saved T within 1e-2; bit-exact against the plain calls when p = 0 and
nothing is dropped (eight-wave dX path); the base output and zero adapter
gradients when everything is dropped.
"""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from gpu_util import DEV, Layer, bits_host, rel

pytestmark = pytest.mark.gpu

TOL_Y = 1e-2
TOL_G = 2e-2


def _print_case(*args):
    print("case:", *args, flush=True)


def _mask(M, k, p, seed):
    return (np.random.default_rng(seed).random((M, k)) >= p).astype(np.uint8)


# (d, k, r, M, p): eight-wave GEMMs (256- and 128-row tiles), the four-wave
# dX (k % 256 != 0), the decode forwards (both kernels), a ragged rank
CASES = [
    (512, 512, 16, 300, 0.1),
    (1024, 1024, 16, 1024, 0.5),
    (256, 320, 8, 200, 0.1),
    (256, 256, 16, 40, 0.1),
    (512, 320, 5, 16, 0.2),
    (512, 512, 8, 16, 0.1),     # the chunked split-K decode (dropout always takes it)
    (256, 768, 16, 7, 0.3),
]


@pytest.mark.parametrize("d,k,r,M,p", CASES)
def test_dropout_parity(lib, d, k, r, M, p):
    _print_case("dropout", d, k, r, M, p)
    L = Layer(lib, d, k, r, M)
    keep_h = _mask(M, k, p, 100 + M)
    keep = torch.from_numpy(keep_h).to(DEV)
    Xd = torch.empty((M, k), dtype=torch.bfloat16, device=DEV)
    Y, T = lib.forward_dropout(L.X, L.w, L.A, L.B, L.alpha, keep, p, save_t=True, xd_out=Xd)
    if r:
        assert np.array_equal(bits_host(Xd), O.dropout_input(L.inp["X"], keep_h, p))  # one rounding, bit-exact
    Yref, Tref = O.forward_dropout(L.inp["X"], L.Wt, L.inp["A"], L.inp["B"], L.alpha, keep_h, p)
    assert rel(bits_host(Y), Yref) <= TOL_Y
    ldt = (M + 63) // 64 * 64
    assert rel(bits_host(T)[: r * ldt].reshape(r, ldt)[:, :M], Tref.T) <= TOL_Y
    rX, rA, rB = O.backward_dropout(L.inp["dY"], L.inp["X"], L.Wt, L.inp["A"], L.inp["B"], L.alpha, keep_h, p)
    for Ts, Xs in ((T, Xd), (T, None), (None, None)):
        dX, dA, dB = lib.backward_dropout(L.dY, L.X, L.w, L.A, L.B, L.alpha, keep, p, T_saved=Ts, Xd_saved=Xs)
        assert rel(bits_host(dX), rX) <= TOL_Y
        assert rel(bits_host(dA), rA) <= TOL_G
        assert rel(bits_host(dB), rB) <= TOL_G


@pytest.mark.parametrize("tile", ["128", "256"])
def test_dropout_tiled_variants(lib, monkeypatch, tile):
    _print_case("dropout tile", tile)
    monkeypatch.setenv("QLORA_TILE", tile)
    d, k, r, M, p = 512, 512, 16, 300, 0.3
    L = Layer(lib, d, k, r, M)
    keep_h = _mask(M, k, p, 7)
    keep = torch.from_numpy(keep_h).to(DEV)
    Y = lib.forward_dropout(L.X, L.w, L.A, L.B, L.alpha, keep, p)
    dX, dA, dB = lib.backward_dropout(L.dY, L.X, L.w, L.A, L.B, L.alpha, keep, p)
    Yref, _ = O.forward_dropout(L.inp["X"], L.Wt, L.inp["A"], L.inp["B"], L.alpha, keep_h, p)
    rX, rA, rB = O.backward_dropout(L.inp["dY"], L.inp["X"], L.Wt, L.inp["A"], L.inp["B"], L.alpha, keep_h, p)
    assert rel(bits_host(Y), Yref) <= TOL_Y
    assert rel(bits_host(dX), rX) <= TOL_Y
    assert rel(bits_host(dA), rA) <= TOL_G and rel(bits_host(dB), rB) <= TOL_G


@pytest.mark.parametrize("M", [40, 300])
def test_no_dropout_is_the_plain_call(lib, M):
    _print_case("dropout none", M)
    L = Layer(lib, 512, 512, 16, M)
    keep = torch.ones((M, 512), dtype=torch.uint8, device=DEV)
    Y = bits_host(lib.forward_dropout(L.X, L.w, L.A, L.B, L.alpha, keep, 0.0))
    assert np.array_equal(Y, bits_host(lib.forward(L.X, L.w, L.A, L.B, L.alpha)))
    g = lib.backward_dropout(L.dY, L.X, L.w, L.A, L.B, L.alpha, keep, 0.0)
    g0 = lib.backward(L.dY, L.X, L.w, L.A, L.B, L.alpha)
    for a, b in zip(g, g0):
        assert np.array_equal(bits_host(a), bits_host(b))


@pytest.mark.parametrize("M", [16, 300])
def test_everything_dropped_is_the_base(lib, monkeypatch, M):
    # LoRA dropout runs the split-K decode kernels up to 128 tokens; the
    # base call is held to the same kernels
    _print_case("dropout all", M)
    monkeypatch.setenv("QLORA_DECODE", "split")
    L = Layer(lib, 512, 512, 16, M)
    keep = torch.zeros((M, 512), dtype=torch.uint8, device=DEV)
    Y = bits_host(lib.forward_dropout(L.X, L.w, L.A, L.B, L.alpha, keep, 0.5))
    assert np.array_equal(Y, bits_host(lib.forward(L.X, L.w)))
    dX, dA, dB = lib.backward_dropout(L.dY, L.X, L.w, L.A, L.B, L.alpha, keep, 0.5)
    assert not np.any(bits_host(dA) & 0x7FFF) and not np.any(bits_host(dB) & 0x7FFF)
    dX0, _, _ = lib.backward(L.dY, L.X, L.w)
    assert rel(bits_host(dX), O.bf16_bits_to_f64(bits_host(dX0))) <= 2.0 ** -7
