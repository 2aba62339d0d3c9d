"""Pin of the LoRA scale s = alpha / r in the oracle.

Page "LoRA and QLoRA Explained", section "How LoRA reduces the number of
trainable parameters", writes the adapted weight as W' = W + (alpha/r) B A;
page "Fine-Tuning on a Budget", section "The LoRA hypothesis", puts the same
alpha/r factor on the low-rank branch of the forward pass.  The worked example
below was computed by hand from that formula (no call into the oracle's
lora_scale produces the expected numbers), at alpha = 16 with r = 8
(s = 2) and with r = 64 (s = 1/4): a scale of r/alpha, alpha, or 1 gives
different numbers in every output, so any of those mistakes fails here.

Example (one token, k = 4 input features, d = 3 output features; only ranks
0 and 1 of the adapter are nonzero, the others are zero rows / columns):

  x  = [1, 2, 0, -1]
  W  = [[1,0,0,0], [0,1,0,0], [0,0,0,1]]            x W^T   = [1, 2, -1]
  A0 = [1, 1, 0, 0],  A1 = [0, 0, 1, 1]             T = x A^T = [3, -1, 0...]
  B[:, 0] = [1, 0, 1],  B[:, 1] = [0, 2, 1]         T B^T   = [3, -2, 2]
  Y = x W^T + s T B^T
      s = 2   -> [7, -2, 3]
      s = 1/4 -> [1.75, 1.5, -0.5]

  dy = [1, 0, 2]                                    U = dy B = [3, 2, 0...]
  dX = dy W + s U A,  dy W = [1, 0, 0, 2],  U A = [3, 3, 2, 2]
      s = 2   -> [7, 6, 4, 6]
      s = 1/4 -> [1.75, 0.75, 0.5, 2.5]
  dA = s U^T x:  row 0 = 3 s x, row 1 = 2 s x, other rows 0
  dB = s dy^T T: row n = s dy[n] [3, -1, 0...]
  W' = W + s B A,  B A = [[1,1,0,0], [0,0,2,2], [1,1,1,1]]
"""

import numpy as np
import pytest

import oracle as O
import workloads as WL

X = np.array([[1, 2, 0, -1]], np.float32)
W = np.array([[1, 0, 0, 0], [0, 1, 0, 0], [0, 0, 0, 1]], np.float32)
DY = np.array([[1, 0, 2]], np.float32)

# hand-worked results per scale (see the module docstring)
EXPECTED = {
    2.0: {
        "Y": [[7, -2, 3]],
        "dX": [[7, 6, 4, 6]],
        "dA01": [[6, 12, 0, -6], [4, 8, 0, -4]],
        "dB01": [[6, -2], [0, 0], [12, -4]],
        "Wm": [[3, 2, 0, 0], [0, 1, 4, 4], [2, 2, 2, 3]],
    },
    0.25: {
        "Y": [[1.75, 1.5, -0.5]],
        "dX": [[1.75, 0.75, 0.5, 2.5]],
        "dA01": [[0.75, 1.5, 0, -0.75], [0.5, 1, 0, -0.5]],
        "dB01": [[0.75, -0.25], [0, 0], [1.5, -0.5]],
        "Wm": [[1.25, 0.25, 0, 0], [0, 1, 0.5, 0.5], [0.25, 0.25, 0.25, 1.25]],
    },
}


def _adapter(r):
    A = np.zeros((r, 4), np.float32)
    A[0] = [1, 1, 0, 0]
    A[1] = [0, 0, 1, 1]
    B = np.zeros((3, r), np.float32)
    B[:, 0] = [1, 0, 1]
    B[:, 1] = [0, 2, 1]
    return WL.to_bf16_bits(A), WL.to_bf16_bits(B)


# (alpha, r) -> s = alpha / r as the pages print it
@pytest.mark.parametrize("alpha,r,s", [(16.0, 8, 2.0), (16.0, 64, 0.25)])
def test_worked_example_forward_backward_merge(alpha, r, s):
    Ab, Bb = _adapter(r)
    Xb, Wb, dYb = WL.to_bf16_bits(X), WL.to_bf16_bits(W), WL.to_bf16_bits(DY)
    ex = EXPECTED[s]

    Y, T = O.forward(Xb, Wb, Ab, Bb, alpha)
    assert np.array_equal(Y, np.array(ex["Y"], np.float64))
    assert np.array_equal(T[0, :2], [3.0, -1.0]) and not np.any(T[0, 2:])

    dX, dA, dB = O.backward(dYb, Xb, Wb, Ab, Bb, alpha)
    assert np.array_equal(dX, np.array(ex["dX"], np.float64))
    assert np.array_equal(dA[:2], np.array(ex["dA01"], np.float64)) and not np.any(dA[2:])
    assert np.array_equal(dB[:, :2], np.array(ex["dB01"], np.float64)) and not np.any(dB[:, 2:])

    Wm = O.merge(Wb, Ab, Bb, alpha)
    assert np.array_equal(O.bf16_bits_to_f64(Wm), np.array(ex["Wm"], np.float64))
    # unmerge subtracts the same (alpha/r) B A and recovers W exactly here
    assert np.array_equal(O.unmerge(Wm, Ab, Bb, alpha), Wb)


def test_scale_value_is_alpha_over_r():
    # the configurations' (alpha, r) pairs: (16, 8), (32, 16), (16, 64)
    assert O.lora_scale(16.0, 8) == 2.0
    assert O.lora_scale(32.0, 16) == 2.0
    assert O.lora_scale(16.0, 64) == 0.25
    # not a power of two: alpha / r rounded once to fp32
    assert O.lora_scale(16.0, 3) == float(np.float32(16.0 / 3.0))
    assert O.lora_scale(16.0, 0) == 0.0
