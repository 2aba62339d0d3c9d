"""Pins of the oracle's Adam step for the adapter parameters.

Facts used (properties of Adam as published by Kingma and Ba): the first
step from zero moments moves every parameter by lr in the direction against
its gradient (the bias corrections make m^ = g and v^ = g^2); a constant
gradient keeps m^ = g and v^ = g^2 exactly at every step, so t steps move a
parameter by t lr |g| / (|g| + eps); a zero gradient leaves the parameter to
the decoupled weight decay alone.
"""

import numpy as np

import oracle as O
import workloads as WL


def _grad(n, seed):
    return WL.normal_bf16((n,), 1e-3, (seed, 93, 0, 0, 4))


def test_first_step_moves_by_lr_against_the_gradient():
    n = 257
    G = _grad(n, 1)
    W = np.linspace(-1, 1, n).astype(np.float32)
    z = np.zeros(n, np.float32)
    W1, m, v, _ = O.adam_step(W, G, z, z, 1e-3, 1, eps=1e-30)
    g = O.bf16_bits_to_f64(G)
    nz = g != 0
    assert np.allclose(W1[nz] - W[nz], -1e-3 * np.sign(g[nz]), rtol=0, atol=1e-7)
    assert np.array_equal(W1[~nz], W[~nz])
    assert np.allclose(m, 0.1 * g, rtol=1e-6) and np.allclose(v, 0.001 * g * g, rtol=1e-6)


def test_constant_gradient_closed_form():
    n, t, lr, eps = 64, 25, 1e-3, 1e-8
    G = _grad(n, 2)
    g = O.bf16_bits_to_f64(G)
    W0 = np.zeros(n, np.float64)
    W, m, v = W0.astype(np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for step in range(1, t + 1):
        W, m, v, _ = O.adam_step(W, G, m, v, lr, step, eps=eps)
    lr32, eps32 = float(np.float32(lr)), float(np.float32(eps))
    ref = W0 - t * lr32 * g / (np.abs(g) + eps32)
    assert np.max(np.abs(W - ref)) <= 1e-6 * np.max(np.abs(ref))


def test_zero_gradient_only_decays():
    n = 40
    G = np.zeros(n, np.uint16)
    W = np.linspace(-2, 2, n).astype(np.float32)
    z = np.zeros(n, np.float32)
    W1, m, v, Pb = O.adam_step(W, G, z, z, 0.01, 3, weight_decay=0.1)
    assert not np.any(m) and not np.any(v)
    assert np.allclose(W1, W * (1 - 0.01 * 0.1), rtol=1e-7)
    assert np.array_equal(Pb, O.bf16_rne_bits_from_f32(W1))
