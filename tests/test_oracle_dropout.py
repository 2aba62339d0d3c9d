"""Pins of the oracle's LoRA dropout (dropout on the adapter path's input,
the mask passed in).

Facts used: with nothing dropped and p = 0 the layer is the plain adapted
linear; with everything dropped the adapter path is off (the base output
exactly, zero adapter gradients); the gradients of L = sum(dY * Y) follow
from central finite differences (exact for a loss linear in each argument);
inverted dropout scales kept inputs by 1/(1-p).
"""

import numpy as np
import pytest

import oracle as O
import workloads as WL


def _setup(d=24, k=128, r=4, M=7):
    inp = WL.layer_inputs(d, k, r, M, cfg=94)
    inp["Wt"] = O.dequantize(O.quantize(inp["W0"]))
    keep = (np.random.default_rng(5).random((M, k)) >= 0.25).astype(np.uint8)
    return inp, keep


def test_no_dropout_is_the_plain_layer():
    inp, _ = _setup()
    ones = np.ones_like(inp["X"], dtype=np.uint8)
    args = (inp["Wt"], inp["A"], inp["B"], 8.0)
    Y, T = O.forward_dropout(inp["X"], *args, ones, 0.0)
    Yr, Tr = O.forward(inp["X"], *args)
    assert np.array_equal(Y, Yr) and np.array_equal(T, Tr)
    g = O.backward_dropout(inp["dY"], inp["X"], *args, ones, 0.0)
    gr = O.backward(inp["dY"], inp["X"], *args)
    assert all(np.array_equal(a, b) for a, b in zip(g, gr))


def test_everything_dropped_turns_the_adapter_off():
    inp, _ = _setup()
    zeros = np.zeros_like(inp["X"], dtype=np.uint8)
    args = (inp["Wt"], inp["A"], inp["B"], 8.0)
    Y, T = O.forward_dropout(inp["X"], *args, zeros, 0.3)
    assert not np.any(T)
    assert np.array_equal(Y, O.bf16_bits_to_f64(inp["X"]) @ O.bf16_bits_to_f64(inp["Wt"]).T)
    dX, dA, dB = O.backward_dropout(inp["dY"], inp["X"], *args, zeros, 0.3)
    assert not np.any(dA) and not np.any(dB)
    assert np.array_equal(dX, O.bf16_bits_to_f64(inp["dY"]) @ O.bf16_bits_to_f64(inp["Wt"]))


def test_kept_inputs_are_scaled_by_inverse_keep_probability():
    inp, keep = _setup()
    Xd = O.bf16_bits_to_f64(O.dropout_input(inp["X"], keep, 0.2))
    X = O.bf16_bits_to_f64(inp["X"])
    assert np.all(Xd[keep == 0] == 0)
    kept = keep != 0
    # one bf16 rounding of x * 1.25
    assert np.all(np.abs(Xd[kept] - 1.25 * X[kept]) <= 2.0 ** -8 * np.abs(1.25 * X[kept]))


@pytest.mark.parametrize("which", ["X", "A", "B"])
def test_dropout_gradients_match_central_differences(which):
    rng = np.random.default_rng(13)
    d, k, r, M = 8, 64, 2, 3
    X = rng.standard_normal((M, k))
    W = rng.standard_normal((d, k)) * 0.02
    A = rng.standard_normal((r, k)) / 8
    B = rng.standard_normal((d, r)) * 0.3
    dY = rng.standard_normal((M, d))
    D = (rng.random((M, k)) >= 0.3) / 0.7
    s = 2.0

    def loss():
        Y = X @ W.T + s * ((X * D) @ A.T) @ B.T
        return float(np.sum(dY * Y))

    dX, dA, dB = O.backward_dropout_f64(dY, X, W, A, B, s, D)
    P = {"X": X, "A": A, "B": B}[which]
    grad = {"X": dX, "A": dA, "B": dB}[which]
    fd = np.zeros_like(P)
    h = 0.5
    for idx in np.ndindex(P.shape):
        old = P[idx]
        P[idx] = old + h
        lp = loss()
        P[idx] = old - h
        lm = loss()
        P[idx] = old
        fd[idx] = (lp - lm) / (2 * h)
    assert np.max(np.abs(fd - grad)) <= 1e-9 * np.max(np.abs(grad))


def test_bits_backward_agrees_with_float_core():
    inp, keep = _setup()
    p = 0.25
    dX, dA, dB = O.backward_dropout(inp["dY"], inp["X"], inp["Wt"], inp["A"], inp["B"], 8.0, keep, p)
    D = (keep != 0) / (1 - p)
    f = O.bf16_bits_to_f64
    gX, gA, gB = O.backward_dropout_f64(f(inp["dY"]), f(inp["X"]), f(inp["Wt"]), f(inp["A"]), f(inp["B"]),
                                        O.lora_scale(8.0, 4), D)
    # the bits path scales by fl32(1/(1-p)), the float core by 1/(1-p)
    assert np.max(np.abs(dX - gX)) <= 2.0 ** -23 * np.max(np.abs(gX))
    # dA, dB: the bits path uses the bf16-rounded dropped input (one rounding)
    assert np.max(np.abs(dA - gA)) <= 2.0 ** -8 * np.max(np.abs(gA))
    assert np.max(np.abs(dB - gB)) <= 2.0 ** -8 * np.max(np.abs(gB))
