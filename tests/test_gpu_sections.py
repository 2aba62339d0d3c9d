"""GPU parity of the shared-input projections (qlora_forward_sections and
qlora_backward_sections) against the oracle's forward_sections and
backward_sections: nsec projections of one input stacked by rows, each
quantised on its own with its own mean, each with its own adapter.

Bars as for one projection: Y and dX within max|err|/max|ref| <= 1e-2, dA
and dB within 2e-2; the in-GEMM dequantisation (per-section means) bit-exact
through one-hot inputs; the stacked storage bit-identical to the sections
quantised one by one.
"""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from gpu_util import bf16_dev, bits_host, f32_dev, quant_host, rel

pytestmark = pytest.mark.gpu

TOL_Y = 1e-2
TOL_G = 2e-2


def _print_case(*args):
    print("case:", *args, flush=True)


class Stack:
    """nsec projections dsec x k of one input, rank r each, on host and device."""

    def __init__(self, lib, nsec, dsec, k, r, M, *, b_zero=False, cfg=97):
        self.nsec, self.r = nsec, r
        self.secs = [WL.layer_inputs(dsec, k, r, M, cfg=cfg, proj=p, b_zero=b_zero) for p in range(nsec)]
        self.Xb = self.secs[0]["X"]
        self.dYb = np.concatenate([s["dY"] for s in self.secs], axis=1)
        self.w = lib.quantize_sections([f32_dev(s["W0"]) for s in self.secs])
        self.q_ref = [O.quantize(s["W0"]) for s in self.secs]
        self.Wt = [O.dequantize(q) for q in self.q_ref]
        self.X, self.dY = bf16_dev(self.Xb), bf16_dev(self.dYb)
        self.A = bf16_dev(np.concatenate([s["A"] for s in self.secs], axis=0)) if r else None
        self.B = bf16_dev(np.concatenate([s["B"] for s in self.secs], axis=0)) if r else None
        self.alpha = 2.0 * r

    def args(self):
        return ([s["A"] for s in self.secs], [s["B"] for s in self.secs])

    def oracle_fwd(self):
        As, Bs = self.args()
        return O.forward_sections(self.Xb, self.Wt, As, Bs, self.alpha)

    def oracle_bwd(self):
        As, Bs = self.args()
        return O.backward_sections(self.dYb, self.Xb, self.Wt, As, Bs, self.alpha)


def test_stacked_storage_is_sections_quantised_one_by_one(lib):
    _print_case("sections storage")
    S = Stack(lib, 3, 256, 512, 16, 1)
    for p in range(3):
        got = quant_host(S.w.section(p))
        ref = S.q_ref[p]
        assert np.array_equal(got["codes"], ref["codes"])
        assert np.array_equal(got["absmax_q"], ref["absmax_q"])
        assert np.array_equal(got["absmax_scale"].view(np.uint32), ref["absmax_scale"].view(np.uint32))
        assert np.array_equal(got["absmax_mean"].view(np.uint32), ref["absmax_mean"].view(np.uint32))
        assert np.array_equal(bits_host(lib.merge(S.w.section(p))), S.Wt[p])


# (nsec, dsec, k, r, M): decode kernels (chunked, k % 256 == 0, and the
# split-K one), eight-wave 128-row tiles, 256-row tiles with the tail
# columns in a second launch (288 tiles of 256 x 256), and the token-rich
# forward split over K ranges (a few hundred tokens, k >= 1024: two and
# four splits, the LoRA term and the sections' means in split 0 only)
FWD_CASES = [
    (2, 256, 512, 32, 16),
    (3, 256, 320, 16, 40),
    (3, 256, 256, 16, 300),
    (4, 512, 512, 16, 64),
    (3, 4096, 256, 16, 1536),
    (3, 256, 1024, 16, 300),
    (2, 512, 2048, 16, 200),
    (3, 256, 512, 16, 16),
    (2, 8192, 256, 16, 3),
    # more than 64 ranks in all: T = X A^T in 64-rank launches (token-rich),
    # or 12 and 16 rank tiles of the decode kernels and all of T in the
    # finishing kernel (token-poor)
    (3, 256, 512, 64, 300),
    (3, 256, 512, 32, 200),
    (4, 256, 256, 64, 40),
    (2, 256, 1024, 64, 16),
    (3, 256, 320, 64, 20),
]
# up to 16 tokens both token-poor forms apply (single launch, split-K pair),
# each forced here: each section's own T and mean; with 8192-row sections
# two row blocks per work-group, with 3072-row sections three
SMALL_M_CASES = [(3, 256, 512, 16, 16), (2, 8192, 256, 16, 3), (3, 3072, 256, 16, 16)]


@pytest.mark.parametrize("form", ["single", "split"])
@pytest.mark.parametrize("nsec,dsec,k,r,M", SMALL_M_CASES)
def test_sections_forward_small_m_both_forms(lib, monkeypatch, form, nsec, dsec, k, r, M):
    monkeypatch.setenv("QLORA_DECODE", form)
    test_sections_forward_parity(lib, nsec, dsec, k, r, M)


@pytest.mark.parametrize("nsec,dsec,k,r,M", FWD_CASES)
def test_sections_forward_parity(lib, nsec, dsec, k, r, M):
    _print_case("sections forward", nsec, dsec, k, r, M)
    S = Stack(lib, nsec, dsec, k, r, M)
    Y, T = lib.forward_sections(S.X, S.w, S.A, S.B, S.alpha, save_t=True)
    Yref, Tref = S.oracle_fwd()
    assert rel(bits_host(Y), Yref) <= TOL_Y
    ldt = (M + 63) // 64 * 64
    Tt = bits_host(T)[: nsec * r * ldt].reshape(nsec * r, ldt)[:, :M]
    assert rel(Tt, Tref.T) <= TOL_Y


BWD_CASES = [
    (3, 256, 256, 16, 300),
    (2, 512, 384, 32, 100),
    (4, 256, 512, 16, 20),
    (3, 256, 320, 16, 129),
    (3, 256, 1024, 16, 300),
    (2, 512, 2048, 16, 200),
    # more than 64 ranks in all: U = dY B and the token reductions in
    # launches of whole sections (one section of 64 ranks, or two of 32 then
    # one), T recomputed in 64-rank launches, the dX epilogue over every
    # rank; 40 and 100 tokens split the projections over K ranges
    (3, 256, 512, 64, 300),
    (4, 256, 256, 64, 100),
    (3, 256, 320, 32, 129),
    (2, 512, 1024, 64, 40),
]


@pytest.mark.parametrize("nsec,dsec,k,r,M", BWD_CASES)
def test_sections_backward_parity(lib, nsec, dsec, k, r, M):
    _print_case("sections backward", nsec, dsec, k, r, M)
    S = Stack(lib, nsec, dsec, k, r, M)
    rX, rA, rB = S.oracle_bwd()
    _, T = lib.forward_sections(S.X, S.w, S.A, S.B, S.alpha, save_t=True)
    for Ts in (T, None):  # saved T, then T recomputed from X
        dX, dA, dB = lib.backward_sections(S.dY, S.X, S.w, S.A, S.B, S.alpha, T_saved=Ts)
        assert rel(bits_host(dX), rX) <= TOL_Y
        assert rel(bits_host(dA), rA) <= TOL_G
        assert rel(bits_host(dB), rB) <= TOL_G


@pytest.mark.parametrize("tile", ["128", "256"])
def test_sections_tiled_variants_parity(lib, monkeypatch, tile):
    _print_case("sections tile", tile)
    monkeypatch.setenv("QLORA_TILE", tile)
    S = Stack(lib, 2, 256, 384, 16, 200)
    Y = lib.forward_sections(S.X, S.w, S.A, S.B, S.alpha)
    dX, dA, dB = lib.backward_sections(S.dY, S.X, S.w, S.A, S.B, S.alpha)
    Yref, _ = S.oracle_fwd()
    rX, rA, rB = S.oracle_bwd()
    assert rel(bits_host(Y), Yref) <= TOL_Y
    assert rel(bits_host(dX), rX) <= TOL_Y
    assert rel(bits_host(dA), rA) <= TOL_G and rel(bits_host(dB), rB) <= TOL_G


@pytest.mark.parametrize("M,k", [(16, 256), (16, 320), (256, 256)])
def test_sections_one_hot_exact(lib, M, k):
    # zero adapters and one-hot tokens: Y[c, :] is column c of the stacked
    # dequantised weight, each section decoded with its own mean
    _print_case("sections one-hot", M, k)
    S = Stack(lib, 3, 256, k, 16, M, b_zero=True)
    Xh = np.zeros((M, k), np.float32)
    Xh[np.arange(M), np.arange(M) % k] = 1.0
    Y = bits_host(lib.forward_sections(bf16_dev(WL.to_bf16_bits(Xh)), S.w, S.A, S.B, S.alpha))
    Wcat = np.concatenate(S.Wt, axis=0)
    assert np.array_equal(Y, Wcat[:, np.arange(M) % k].T)


@pytest.mark.parametrize("k", [256, 320])
def test_sections_one_hot_output_gradient_returns_weight(lib, k):
    # dY = I over the stacked outputs: dX is the stacked dequantised weight,
    # the contraction crossing from one section's mean to the next
    _print_case("sections one-hot dY", k)
    S = Stack(lib, 3, 256, k, 16, 768, b_zero=True)
    dY = bf16_dev(WL.to_bf16_bits(np.eye(768, dtype=np.float32)))
    dX, _, _ = lib.backward_sections(dY, S.X, S.w, S.A, S.B, S.alpha)
    assert np.array_equal(bits_host(dX), np.concatenate(S.Wt, axis=0))


def test_sections_match_separate_calls(lib):
    # the stacked call and nsec separate calls agree to the forward bar
    _print_case("sections vs separate")
    S = Stack(lib, 3, 256, 512, 16, 200)
    Y = bits_host(lib.forward_sections(S.X, S.w, S.A, S.B, S.alpha))
    r, d = S.r, 256
    for p in range(3):
        Ap = S.A[p * r:(p + 1) * r].contiguous()
        Bp = S.B[p * d:(p + 1) * d].contiguous()
        Yp = lib.forward(S.X, S.w.section(p), Ap, Bp, S.alpha)
        ref = O.bf16_bits_to_f64(bits_host(Yp))
        assert rel(Y[:, p * d:(p + 1) * d], ref) <= TOL_Y


@pytest.mark.parametrize("M", [16, 300])
def test_sections_without_adapters_use_each_sections_mean(lib, M):
    # r = 0: the base GEMM alone, each section decoded with its own mean
    # (bit-identical to zero adapters)
    _print_case("sections r=0", M)
    S = Stack(lib, 3, 256, 256, 16, M, b_zero=True)
    Y0 = bits_host(lib.forward_sections(S.X, S.w))
    Yb = bits_host(lib.forward_sections(S.X, S.w, S.A, S.B, S.alpha))
    assert np.array_equal(Y0, Yb)
    dX0, _, _ = lib.backward_sections(S.dY, S.X, S.w)
    rX, _, _ = S.oracle_bwd()
    assert rel(bits_host(dX0), rX) <= TOL_Y
