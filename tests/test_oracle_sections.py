"""Pins of the oracle's shared-input projections (forward_sections,
backward_sections): several adapted projections that read one input, each
with its own frozen weight and adapter.

Facts used: the stack of projections is one linear layer whose weight is the
row-stack of the frozen weights and whose adapter is the row-stack of the
A_p with the B_p on a block diagonal (the LoRA update of each projection is
its own B_p A_p, "The update LoRA is allowed to learn"); the single-layer
forward and backward are already pinned by closed forms and central finite
differences.  So the sectioned results must equal the single-layer ones on
that block-diagonal layer, the block-diagonal dB's off-diagonal blocks being
gradients of entries that the sectioned layer does not have.
"""

import numpy as np

import oracle as O
import workloads as WL


def _sections(n=3, d=16, k=128, r=4, M=6, b_zero=False):
    secs = []
    for p in range(n):
        inp = WL.layer_inputs(d, k, r, M, seed=p, cfg=98, proj=p, b_zero=b_zero)
        inp["Wt"] = O.dequantize(O.quantize(inp["W0"]))
        secs.append(inp)
    X = secs[0]["X"]
    dY = np.concatenate([s["dY"] for s in secs], axis=1)
    return secs, X, dY


def _block_diagonal(secs):
    d, r = secs[0]["B"].shape
    n = len(secs)
    Bbd = np.zeros((n * d, n * r))
    for p, s in enumerate(secs):
        Bbd[p * d:(p + 1) * d, p * r:(p + 1) * r] = O.bf16_bits_to_f64(s["B"])
    W = np.concatenate([O.bf16_bits_to_f64(s["Wt"]) for s in secs], axis=0)
    A = np.concatenate([O.bf16_bits_to_f64(s["A"]) for s in secs], axis=0)
    return W, A, Bbd


def test_forward_is_one_layer_with_block_diagonal_adapter():
    secs, X, _ = _sections()
    alpha = 8.0
    Y, T = O.forward_sections(X, [s["Wt"] for s in secs], [s["A"] for s in secs],
                              [s["B"] for s in secs], alpha)
    W, A, Bbd = _block_diagonal(secs)
    s = O.lora_scale(alpha, secs[0]["A"].shape[0])
    Yr, Tr = O.forward_f64(O.bf16_bits_to_f64(X), W, A, Bbd, s)
    assert np.allclose(Y, Yr, rtol=0, atol=1e-12 * np.max(np.abs(Yr)))
    assert np.allclose(T, Tr, rtol=0, atol=1e-12 * np.max(np.abs(Tr)))


def test_backward_is_one_layer_with_block_diagonal_adapter():
    secs, X, dY = _sections()
    alpha = 8.0
    dX, dA, dB = O.backward_sections(dY, X, [s["Wt"] for s in secs], [s["A"] for s in secs],
                                     [s["B"] for s in secs], alpha)
    W, A, Bbd = _block_diagonal(secs)
    s = O.lora_scale(alpha, secs[0]["A"].shape[0])
    gX, gA, gB = O.backward_f64(O.bf16_bits_to_f64(dY), O.bf16_bits_to_f64(X), W, A, Bbd, s)
    tol = lambda ref: 1e-12 * np.max(np.abs(ref))
    assert np.max(np.abs(dX - gX)) <= tol(gX)
    assert np.max(np.abs(dA - gA)) <= tol(gA)
    d, r = secs[0]["B"].shape
    for p in range(len(secs)):
        blk = gB[p * d:(p + 1) * d, p * r:(p + 1) * r]
        assert np.max(np.abs(dB[p * d:(p + 1) * d] - blk)) <= tol(gB)


def test_one_section_is_the_plain_layer():
    secs, X, _ = _sections(n=1)
    s0 = secs[0]
    Y, T = O.forward_sections(X, [s0["Wt"]], [s0["A"]], [s0["B"]], 8.0)
    Yr, Tr = O.forward(X, s0["Wt"], s0["A"], s0["B"], 8.0)
    assert np.array_equal(Y, Yr) and np.array_equal(T, Tr)
    g = O.backward_sections(s0["dY"], X, [s0["Wt"]], [s0["A"]], [s0["B"]], 8.0)
    gr = O.backward(s0["dY"], X, s0["Wt"], s0["A"], s0["B"], 8.0)
    assert all(np.array_equal(a, b) for a, b in zip(g, gr))


def test_sections_do_not_mix():
    # Changing the adapter of section 1 leaves the outputs of sections 0 and
    # 2, and the adapter gradients of sections 0 and 2, unchanged.
    secs, X, dY = _sections()
    Ws, As, Bs = [s["Wt"] for s in secs], [s["A"] for s in secs], [s["B"] for s in secs]
    Y0, _ = O.forward_sections(X, Ws, As, Bs, 8.0)
    g0 = O.backward_sections(dY, X, Ws, As, Bs, 8.0)
    Bs2 = list(Bs)
    Bs2[1] = WL.to_bf16_bits(O.bf16_bits_to_f64(Bs[1]) * 3.0 + 0.01)
    As2 = list(As)
    As2[1] = WL.to_bf16_bits(O.bf16_bits_to_f64(As[1]) * -2.0)
    Y1, _ = O.forward_sections(X, Ws, As2, Bs2, 8.0)
    g1 = O.backward_sections(dY, X, Ws, As2, Bs2, 8.0)
    d, r = secs[0]["B"].shape
    keep = np.r_[0:d, 2 * d:3 * d]
    assert np.array_equal(Y0[:, keep], Y1[:, keep])
    assert not np.array_equal(Y0[:, d:2 * d], Y1[:, d:2 * d])
    rk = np.r_[0:r, 2 * r:3 * r]
    assert np.array_equal(g0[1][rk], g1[1][rk])
    assert np.array_equal(g0[2][keep], g1[2][keep])


def test_zero_adapters_give_the_stacked_base_output():
    secs, X, _ = _sections(b_zero=True)
    Y, _ = O.forward_sections(X, [s["Wt"] for s in secs], [s["A"] for s in secs],
                              [s["B"] for s in secs], 8.0)
    W = np.concatenate([O.bf16_bits_to_f64(s["Wt"]) for s in secs], axis=0)
    assert np.array_equal(Y, O.bf16_bits_to_f64(X) @ W.T)
