"""Pins of the oracle's forward, backward and merge/unmerge.

Facts used: h = W0 x + s B A x (a single token is a column; a one-hot token
picks one column of W0), B = 0 at initialisation gives exactly the base
model, the merged layer W0 + s B A gives the same output as the unmerged
one, switching tasks is subtract / add, W0 gets no gradient, and the
adapter parameter count r (d + k) the pages print for 4096 x 4096.
Gradients are checked by central finite differences, which are exact for a
loss that is linear in each argument.
"""

import numpy as np
import pytest

import oracle as O
import workloads as WL

GOLD = {}
with open(__file__.rsplit("/", 1)[0] + "/golden/pages_numbers.txt") as fh:
    for line in fh:
        if line.strip() and not line.startswith("#"):
            key, rest = line.split("=", 1)
            GOLD[key.strip()] = float(rest.split("|")[0])


def small(d=24, k=128, r=4, M=5, seed=0, b_zero=False):
    inp = WL.layer_inputs(d, k, r, M, seed=seed, cfg=99, b_zero=b_zero)
    wq = O.quantize(inp["W0"])
    inp["Wt"] = O.dequantize(wq)
    return inp


def test_single_token_is_column_form():
    # h = W0 x for a one-hot x = e_c is column c of W0 (B = 0).
    inp = small(b_zero=True)
    k = inp["Wt"].shape[1]
    X = WL.to_bf16_bits(np.eye(k, dtype=np.float32))
    Y, _ = O.forward(X, inp["Wt"], inp["A"], inp["B"], 16.0)
    assert np.array_equal(Y, O.bf16_bits_to_f64(inp["Wt"]).T)


def test_b_zero_gives_exact_base_output():
    inp = small(b_zero=True)
    Y, _ = O.forward(inp["X"], inp["Wt"], inp["A"], inp["B"], 8.0)
    r0 = np.zeros((0, inp["Wt"].shape[1]), np.uint16)
    Yb, _ = O.forward(inp["X"], inp["Wt"], r0, np.zeros((inp["Wt"].shape[0], 0), np.uint16), 8.0)
    assert np.array_equal(Y, Yb)


def test_merged_equals_unmerged():
    inp = small()
    Y, _ = O.forward(inp["X"], inp["Wt"], inp["A"], inp["B"], 8.0)
    Wm = O.bf16_bits_to_f64(inp["Wt"]) + O.delta_w(inp["A"], inp["B"], 8.0)
    Ym = O.bf16_bits_to_f64(inp["X"]) @ Wm.T
    assert np.max(np.abs(Y - Ym)) <= 1e-12 * np.max(np.abs(Y))


def test_lora_term_is_rank_r():
    inp = small(d=40, k=128, r=3)
    dw = O.delta_w(inp["A"], inp["B"], 6.0)
    sv = np.linalg.svd(dw, compute_uv=False)
    assert np.sum(sv > 1e-12 * sv[0]) == 3


def _loss(X, W, A, B, s, dY):
    Y, _ = O.forward_f64(X, W, A, B, s)
    return float(np.sum(dY * Y))


@pytest.mark.parametrize("which", ["X", "A", "B"])
def test_backward_matches_central_differences(which):
    rng = np.random.default_rng(11)
    d, k, r, M = 8, 64, 2, 3
    X = rng.standard_normal((M, k))
    W = rng.standard_normal((d, k)) * 0.02
    A = rng.standard_normal((r, k)) / 8
    B = rng.standard_normal((d, r)) * 0.3
    dY = rng.standard_normal((M, d))
    s = 2.0
    dX, dA, dB = O.backward_f64(dY, X, W, A, B, s)
    args = {"X": X, "A": A, "B": B}
    grad = {"X": dX, "A": dA, "B": dB}[which]
    P = args[which]
    h = 0.5
    fd = np.zeros_like(P)
    for idx in np.ndindex(P.shape):
        old = P[idx]
        P[idx] = old + h
        lp = _loss(X, W, A, B, s, dY)
        P[idx] = old - h
        lm = _loss(X, W, A, B, s, dY)
        P[idx] = old
        fd[idx] = (lp - lm) / (2 * h)
    assert np.max(np.abs(fd - grad)) <= 1e-9 * np.max(np.abs(grad))


def test_base_weight_has_no_gradient_path():
    # Perturbing W changes the loss, but the oracle's backward returns no W
    # gradient at all: only dX, dA and dB.
    inp = small()
    out = O.backward(inp["dY"], inp["X"], inp["Wt"], inp["A"], inp["B"], 8.0)
    assert len(out) == 3
    M, k = inp["X"].shape
    d, r = inp["B"].shape
    assert out[0].shape == (M, k) and out[1].shape == (r, k) and out[2].shape == (d, r)


def test_b_zero_backward():
    inp = small(b_zero=True)
    dX, dA, dB = O.backward(inp["dY"], inp["X"], inp["Wt"], inp["A"], inp["B"], 8.0)
    assert np.all(dA == 0)
    assert np.array_equal(dX, O.bf16_bits_to_f64(inp["dY"]) @ O.bf16_bits_to_f64(inp["Wt"]))
    assert np.any(dB != 0)


def test_one_hot_output_gradient_returns_weight():
    inp = small(b_zero=True)
    d = inp["Wt"].shape[0]
    dY = WL.to_bf16_bits(np.eye(d, dtype=np.float32))
    X = inp["X"][:1].repeat(d, axis=0)
    dX, _, _ = O.backward(dY, X, inp["Wt"], inp["A"], inp["B"], 8.0)
    assert np.array_equal(dX, O.bf16_bits_to_f64(inp["Wt"]))


def test_adapter_parameter_count_printed_on_pages():
    inp = WL.layer_inputs(4096, 4096, 8, 1, cfg=98)
    n = inp["A"].size + inp["B"].size
    assert n == GOLD["rank8_adapter_params_4096"]
    assert round(4096 * 4096 / 1e6, 1) == GOLD["attn_params_4096"] / 1e6
    assert round(100 * n / (4096 * 4096), 1) == GOLD["rank8_adapter_fraction_pct"]


def _ulps(a_bits, b_bits):
    a = a_bits.astype(np.int32)
    b = b_bits.astype(np.int32)
    # same-sign bf16 patterns: distance in representable steps
    sa = np.where(a & 0x8000, -(a & 0x7FFF), a)
    sb = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(sa - sb)


def test_merge_b_zero_is_dequantised_base():
    inp = small(b_zero=True)
    assert np.array_equal(O.merge(inp["Wt"], inp["A"], inp["B"], 8.0), inp["Wt"])


def test_merge_is_nearest_bf16_of_exact_sum():
    inp = small()
    Wm = O.merge(inp["Wt"], inp["A"], inp["B"], 8.0)
    exact = O.bf16_bits_to_f64(inp["Wt"]) + O.delta_w(inp["A"], inp["B"], 8.0)
    got = O.bf16_bits_to_f64(Wm)
    # half a bf16 ulp (2^-8 relative to the binade) bounds the error
    _, e = np.frexp(np.abs(exact))
    assert np.all(np.abs(got - exact) <= np.ldexp(1.0, e - 9) + 1e-300)


def _half_ulp(v):
    """Half a bf16 ulp at |v| (2^-134 at zero)."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(v)
    return np.where(v == 0, 2.0 ** -134, np.ldexp(1.0, np.maximum(e - 9, -134)))


def test_unmerge_roundtrip_and_task_switch():
    # Two roundings separate W0 from unmerge(merge(W0)): one when merging,
    # one when unmerging, each at most half a bf16 ulp of the value stored.
    inp = small()
    Wt = inp["Wt"]
    Wm = O.merge(Wt, inp["A"], inp["B"], 8.0)
    back = O.unmerge(Wm, inp["A"], inp["B"], 8.0)
    w0 = O.bf16_bits_to_f64(Wt)
    wm = O.bf16_bits_to_f64(Wm)
    wb = O.bf16_bits_to_f64(back)
    assert np.all(np.abs(wb - w0) <= _half_ulp(wm) + _half_ulp(wb))
    # task switch: subtract B A, add B' A'  vs  merging B' A' directly
    other = small(seed=1)
    switched = O.merge(back, other["A"], other["B"], 8.0)
    direct = O.merge(Wt, other["A"], other["B"], 8.0)
    ws = O.bf16_bits_to_f64(switched)
    wd = O.bf16_bits_to_f64(direct)
    bound = _half_ulp(wm) + _half_ulp(wb) + _half_ulp(ws) + _half_ulp(wd)
    assert np.all(np.abs(ws - wd) <= bound)
    # the difference is a rounding effect, never a wrong term
    assert np.mean(switched == direct) > 0.9
