"""Pins of the oracle's per-token adapter forward (forward_multi).

Facts used: a token served by adapter a is the adapted layer with that
adapter ("What to choose and why": unmerged adapters picked per example),
whose batched forward is pinned elsewhere; a token with no adapter gets the
frozen base output, which B = 0 pins exactly.
"""

import numpy as np

import oracle as O
import workloads as WL


def _setup(nad=4, d=24, k=128, r=4, M=11):
    inp = WL.layer_inputs(d, k, r, M, cfg=96)
    Wt = O.dequantize(O.quantize(inp["W0"]))
    As = [WL.layer_inputs(d, k, r, 1, cfg=96, proj=1 + a)["A"] for a in range(nad)]
    Bs = [WL.layer_inputs(d, k, r, 1, cfg=96, proj=1 + a)["B"] for a in range(nad)]
    idx = np.array([(5 * m) % (nad + 2) - 1 for m in range(M)], np.int32)  # -1 .. nad: some without adapter
    return inp["X"], Wt, As, Bs, idx


def test_each_token_is_the_layer_with_its_adapter():
    X, Wt, As, Bs, idx = _setup()
    Y = O.forward_multi(X, Wt, As, Bs, idx, 8.0)
    for a in range(len(As)):
        rows = np.nonzero(idx == a)[0]
        assert rows.size
        Ya, _ = O.forward(X[rows], Wt, As[a], Bs[a], 8.0)
        assert np.max(np.abs(Y[rows] - Ya)) <= 1e-12 * np.max(np.abs(Ya))


def test_tokens_without_adapter_get_the_base_output():
    X, Wt, As, Bs, idx = _setup()
    Y = O.forward_multi(X, Wt, As, Bs, idx, 8.0)
    rows = np.nonzero((idx < 0) | (idx >= len(As)))[0]
    assert rows.size
    Yb, _ = O.forward(X[rows], Wt, As[0], np.zeros_like(Bs[0]), 8.0)  # B = 0: exactly the base
    assert np.array_equal(Y[rows], Yb)


def test_one_adapter_for_all_tokens_is_the_plain_layer():
    X, Wt, As, Bs, _ = _setup(nad=1)
    idx = np.zeros(X.shape[0], np.int32)
    Y = O.forward_multi(X, Wt, As, Bs, idx, 8.0)
    Yr, _ = O.forward(X, Wt, As[0], Bs[0], 8.0)
    assert np.max(np.abs(Y - Yr)) <= 1e-12 * np.max(np.abs(Yr))
