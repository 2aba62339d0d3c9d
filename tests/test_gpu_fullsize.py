"""GPU parity at the workloads' full sizes, on sampled outputs.

Every shape of the benchmark configurations runs through the C ABI in the
launch configuration the benchmark times (the same tile choice follows from
the same M, d, k).  The NF4 storage is compared bit for bit in full.  The
float outputs are compared on sampled rows and columns that the oracle can
compute on its own, each sample through the oracle's plain definitions:

  Y[:, n]  for sampled output features n   (needs w~[n, :] only)
  dX[:, c] and dA[:, c] for sampled input features c   (needs w~[:, c])
  dB[n, :] for sampled output features n   (needs T = X A^T in full)
  merge(W)[n, :] for sampled rows n

The samples hold one index in every 256-wide slice of the output features
and of the input features (so every work-group column of every launch is
looked at), the first and last index and the edges of the first tiles; all
M token rows are compared.  Bars as everywhere: Y and dX max|err|/max|ref| <= 1e-2,
dA and dB <= 2e-2, merge within the fp32-accumulation bound.
"""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from gpu_util import bf16_dev, bits_host, f32_dev, quant_host, rel
from test_gpu_parity import _merge_ok

pytestmark = pytest.mark.gpu

TOL_Y = 1e-2
TOL_G = 2e-2


def _sample(n, count, seed, tile=256):
    """Indices to check along a dimension of size n: one random index in
    every tile-wide slice (every work-group column of the forward, the
    token-rich dX kernel and the decode kernels, tail launches included),
    both ends of the first two slices, the middle and the last index, plus
    ``count`` further random indices."""
    rng = np.random.default_rng(seed)
    edges = [0, n - 1, min(n - 1, tile - 1), min(n - 1, tile), n // 2]
    strata = [rng.integers(t0, min(t0 + tile, n)) for t0 in range(0, n, tile)]
    pick = rng.choice(n, size=min(n, count), replace=False)
    return np.unique(np.concatenate([edges, strata, pick])).astype(np.int64)


def _run_layer(lib, d, k, r, alpha, M, cfg, layer=0, proj=0, nsamp=48, merge=False):
    print(f"case: full-size d={d} k={k} r={r} alpha={alpha} M={M}", flush=True)
    inp = WL.layer_inputs(d, k, r, M, cfg=cfg, layer=layer, proj=proj)
    w = lib.quantize(f32_dev(inp["W0"]))
    q = O.quantize(inp["W0"])
    got = quant_host(w)
    assert np.array_equal(got["codes"], q["codes"])
    assert np.array_equal(got["absmax_q"], q["absmax_q"])
    assert np.array_equal(got["absmax_scale"].view(np.uint32), q["absmax_scale"].view(np.uint32))
    assert np.array_equal(got["absmax_mean"].view(np.uint32), q["absmax_mean"].view(np.uint32))

    A, B = bf16_dev(inp["A"]), bf16_dev(inp["B"])
    X, dY = bf16_dev(inp["X"]), bf16_dev(inp["dY"])
    Y, T = lib.forward(X, w, A, B, alpha, save_t=True)
    dX, dA, dB = lib.backward(dY, X, w, A, B, alpha, T_saved=T)
    Wm = lib.merge(w, A, B, alpha) if merge else None
    torch.cuda.synchronize()

    ns = _sample(d, nsamp, 1 + cfg)
    cs = _sample(k, nsamp, 2 + cfg)
    W_rows = O.dequantize_region(q, ns, np.arange(k))    # w~[ns, :]
    W_cols = O.dequantize_region(q, np.arange(d), cs)    # w~[:, cs]

    Yh = bits_host(Y)
    Yr, _ = O.forward(inp["X"], W_rows, inp["A"], np.ascontiguousarray(inp["B"][ns]), alpha)
    eY = rel(Yh[:, ns], Yr)

    Xc = np.ascontiguousarray(inp["X"][:, cs])
    dXr, dAr, _ = O.backward(inp["dY"], Xc, W_cols, np.ascontiguousarray(inp["A"][:, cs]),
                             inp["B"], alpha)
    eX = rel(bits_host(dX)[:, cs], dXr)
    eA = rel(bits_host(dA)[:, cs], dAr)

    dYn = np.ascontiguousarray(inp["dY"][:, ns])
    _, _, dBr = O.backward(dYn, inp["X"], W_rows, inp["A"], np.ascontiguousarray(inp["B"][ns]), alpha)
    eB = rel(bits_host(dB)[ns], dBr)
    print(f"  rel errors: Y {eY:.2e} dX {eX:.2e} dA {eA:.2e} dB {eB:.2e}", flush=True)
    assert eY <= TOL_Y and eX <= TOL_Y, (eY, eX)
    assert eA <= TOL_G and eB <= TOL_G, (eA, eB)

    if merge:
        # the merge kernel's tiles are 128 rows high: one row in each
        nm = _sample(d, nsamp, 5 + cfg, tile=128)
        Wm_rows = O.dequantize_region(q, nm, np.arange(k))
        Bn = np.ascontiguousarray(inp["B"][nm])
        ref = O.merge(Wm_rows, inp["A"], Bn, alpha)
        _merge_ok(bits_host(Wm)[nm], Wm_rows, inp["A"], Bn, alpha, 1.0, ref)


# Attention projection, 4096 x 4096, M = 4096 (batch 4 x 1024): r = 8,
# alpha = 16, and the benchmark's own r = 16, alpha = 32 (same seeds as the
# benchmark).
@pytest.mark.parametrize("r,alpha,cfg", [(8, 16.0, 1), (16, 32.0, 1)])
def test_attention_projection_4096(lib, r, alpha, cfg):
    _run_layer(lib, 4096, 4096, r, alpha, 4096, cfg)


# Decode-shaped forward, 16 tokens, r = 16, alpha = 32.
@pytest.mark.parametrize("d,k", [(4096, 4096), (11008, 4096), (4096, 11008)])
def test_decode_shapes_forward(lib, d, k):
    print(f"case: decode d={d} k={k}", flush=True)
    inp = WL.layer_inputs(d, k, 16, 16, cfg=2)
    w = lib.quantize(f32_dev(inp["W0"]))
    q = O.quantize(inp["W0"])
    assert np.array_equal(quant_host(w)["codes"], q["codes"])
    Y = lib.forward(bf16_dev(inp["X"]), w, bf16_dev(inp["A"]), bf16_dev(inp["B"]), 32.0)
    ns = _sample(d, 512, 7)
    Yr, _ = O.forward(inp["X"], O.dequantize_region(q, ns, np.arange(k)), inp["A"], inp["B"][ns], 32.0)
    e = rel(bits_host(Y)[:, ns], Yr)
    print(f"  rel error Y {e:.2e}", flush=True)
    assert e <= TOL_Y


# 7B-shaped stack, one layer of each projection shape, r = 16, alpha = 32,
# M = 2048.
@pytest.mark.parametrize("d,k,proj", [(4096, 4096, 0), (11008, 4096, 4), (4096, 11008, 6)])
def test_7b_shapes(lib, d, k, proj):
    _run_layer(lib, d, k, 16, 32.0, 2048, 3, layer=0, proj=proj)


# 65B-shaped stack, one layer of each projection shape, r = 64, alpha = 16,
# M = 4096, with the merge.
@pytest.mark.parametrize("d,k,proj", [(8192, 8192, 0), (22016, 8192, 4), (8192, 22016, 6)])
def test_65b_shapes(lib, d, k, proj):
    _run_layer(lib, d, k, 64, 16.0, 4096, 4, layer=79, proj=proj, nsamp=32, merge=True)


# Eight-wave GEMM paths with a ragged token count (the last 256-row tile is
# partly empty) and ranks that take the three adapter paths of the backward:
# r = 24 (B read as stored, two 16-rank blocks), r = 8 (one block, half
# padding) and r = 12 (not a multiple of 8: B transposed first).
@pytest.mark.parametrize("r,alpha", [(24, 48.0), (8, 16.0), (12, 24.0)])
def test_eight_wave_ragged_tokens(lib, r, alpha):
    _run_layer(lib, 4096, 4096, r, alpha, 3985, 1, layer=2, proj=1)


# 128-row forward tiles with two NF4 blocks per K step (chosen when 256-row
# tiles would not cover the CUs): 1900 tokens, the last tile row partly
# empty; r = 12 takes the scalar B path of the LoRA prologue.
@pytest.mark.parametrize("r,alpha", [(16, 32.0), (12, 24.0)])
def test_short_tile_two_block_steps(lib, r, alpha):
    _run_layer(lib, 4096, 4096, r, alpha, 1900, 1, layer=4, proj=6)


# Token reduction with 64-column strips (chosen when they still give at
# least one work-group per CU): r = 16 and r = 40 on a 16384 x 4096 weight.
@pytest.mark.parametrize("r,alpha", [(16, 32.0), (40, 80.0)])
def test_wide_strip_token_reduction(lib, r, alpha):
    _run_layer(lib, 16384, 4096, r, alpha, 1000, 1, layer=3, proj=5)


# Shared-input sections at full size, the benchmark's section legs: q, k, v
# of the 7B-shaped layer (3 x 4096 x 4096, r = 16, 48 ranks in all), and of
# the 65B-shaped layer (3 x 8192 x 8192, r = 64: 192 ranks, the adapter
# kernels in three section groups) and its gate, up (2 x 22016 x 8192, r =
# 64), M = 4096.
SECTION_LAYERS = [
    (3, 4096, 4096, 16, 32.0, 2048, 3),
    (3, 8192, 8192, 64, 16.0, 4096, 4),
    (2, 22016, 8192, 64, 16.0, 4096, 4),
]


@pytest.mark.parametrize("n,d,k,r,alpha,M,cfg", SECTION_LAYERS)
def test_sections_full_size(lib, n, d, k, r, alpha, M, cfg):
    print(f"case: full-size sections {n} x {d} x {k} r={r} M={M}", flush=True)
    secs = [WL.layer_inputs(d, k, r, M, cfg=cfg, proj=p) for p in range(n)]
    w = lib.quantize_sections([f32_dev(s["W0"]) for s in secs])
    qs = [O.quantize(s["W0"]) for s in secs]
    for s in secs:
        del s["W0"]
    Xb = secs[0]["X"]
    dYb = np.concatenate([s["dY"] for s in secs], axis=1)
    A = bf16_dev(np.concatenate([s["A"] for s in secs], axis=0))
    B = bf16_dev(np.concatenate([s["B"] for s in secs], axis=0))
    X, dY = bf16_dev(Xb), bf16_dev(dYb)
    Y, T = lib.forward_sections(X, w, A, B, alpha, save_t=True)
    dX, dA, dB = lib.backward_sections(dY, X, w, A, B, alpha, T_saved=T)
    torch.cuda.synchronize()
    Yh, dXh, dAh, dBh = (bits_host(t) for t in (Y, dX, dA, dB))
    ns = _sample(d, 24, 31)
    cs = _sample(k, 24, 32)
    dX_ref = 0.0
    for p, (s, q) in enumerate(zip(secs, qs)):
        W_rows = O.dequantize_region(q, ns, np.arange(k))
        W_cols = O.dequantize_region(q, np.arange(d), cs)
        Bn = np.ascontiguousarray(s["B"][ns])
        Yr, _ = O.forward(Xb, W_rows, s["A"], Bn, alpha)
        eY = rel(Yh[:, p * d + ns], Yr)
        dYp = np.ascontiguousarray(dYb[:, p * d:(p + 1) * d])
        gX, gA, _ = O.backward(dYp, np.ascontiguousarray(Xb[:, cs]), W_cols,
                               np.ascontiguousarray(s["A"][:, cs]), s["B"], alpha)
        dX_ref = dX_ref + gX
        eA = rel(dAh[p * r:(p + 1) * r][:, cs], gA)
        _, _, gB = O.backward(np.ascontiguousarray(dYp[:, ns]), Xb, W_rows, s["A"], Bn, alpha)
        eB = rel(dBh[p * d + ns], gB)
        print(f"  section {p}: rel errors Y {eY:.2e} dA {eA:.2e} dB {eB:.2e}", flush=True)
        assert eY <= TOL_Y and eA <= TOL_G and eB <= TOL_G, (eY, eA, eB)
    eX = rel(dXh[:, cs], dX_ref)
    print(f"  rel error dX {eX:.2e}", flush=True)
    assert eX <= TOL_Y


def test_multi_adapter_decode_full_size(lib):
    # the 11008 x 4096 decode shape with 8 adapters and a seeded index per
    # token, the benchmark's multi-adapter leg
    d, k, r, alpha, M, nad = 11008, 4096, 16, 32.0, 16, 8
    print(f"case: full-size multi-adapter {d} x {k} r={r} M={M} adapters={nad}", flush=True)
    inp = WL.layer_inputs(d, k, r, M, cfg=2)
    w = lib.quantize(f32_dev(inp["W0"]))
    q = O.quantize(inp["W0"])
    ads = [WL.layer_inputs(d, k, r, 1, cfg=2, proj=1 + a) for a in range(nad)]
    idx = np.random.default_rng(6001).integers(-1, nad, M).astype(np.int32)
    Y = lib.forward_multi(bf16_dev(inp["X"]), w, bf16_dev(np.concatenate([a["A"] for a in ads], axis=0)),
                          bf16_dev(np.concatenate([a["B"] for a in ads], axis=0)),
                          torch.from_numpy(idx).to("cuda:0"), alpha)
    ns = _sample(d, 64, 33)
    W_rows = O.dequantize_region(q, ns, np.arange(k))
    ref = O.forward_multi(inp["X"], W_rows, [a["A"] for a in ads],
                          [np.ascontiguousarray(a["B"][ns]) for a in ads], idx, alpha)
    assert rel(bits_host(Y)[:, ns], ref) <= TOL_Y
