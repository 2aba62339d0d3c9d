"""Pins of the oracle's number formats: bf16 rounding and OCP FP8 E4M3FN.

Each expected value below follows from the format definitions (sign,
exponent bias, fraction width, round-to-nearest-even), worked out by hand,
or from a brute-force search over every representable value.
"""

import numpy as np
import pytest

import oracle as O


def f32(x):
    return np.array(x, dtype=np.float32)


# --- bf16 -----------------------------------------------------------------

@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3F80),
    (1.0 + 2 ** -8, 0x3F80),            # tie between 1 and 1+2^-7 -> even (1)
    (1.0 + 3 * 2 ** -8, 0x3F82),        # tie between 1+2^-7 and 1+2^-6 -> even
    (1.0 + 2 ** -8 + 2 ** -20, 0x3F81),  # just above the tie -> up
    (-2.0, 0xC000),
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (3.0e38, 0x7F62),                   # 3e38 = 1.7633... * 2^127
    (2 ** -130, 0x0008),                # bf16 subnormal: 2^-130 = 8 * 2^-133
])
def test_bf16_rne_hand_table(value, bits):
    assert int(O.bf16_rne_bits_from_f32(f32([value]))[0]) == bits
    assert int(O.bf16_rne_bits_from_f64(np.array([value]))[0]) == bits


def test_bf16_integer_and_grid_methods_agree():
    # Two independent routes to the same rounding: integer bit arithmetic on
    # the fp32 word and exact rounding on the float64 grid.
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, size=400_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 3.3e38)]
    a = O.bf16_rne_bits_from_f32(x)
    b = O.bf16_rne_bits_from_f64(x.astype(np.float64))
    assert np.array_equal(a, b)


def test_bf16_roundtrip_is_identity_on_bf16_values():
    rng = np.random.default_rng(2)
    b = rng.integers(0, 2 ** 16, size=100_000, dtype=np.uint32).astype(np.uint16)
    v = O.bf16_bits_to_f64(b)
    ok = np.isfinite(v)
    assert np.array_equal(O.bf16_rne_bits_from_f64(v[ok]), b[ok])


# --- E4M3FN ----------------------------------------------------------------

@pytest.mark.parametrize("byte,value", [
    (0x00, 0.0), (0x80, -0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),
    (0x08, 2.0 ** -6), (0x38, 1.0), (0x39, 1.125), (0x3F, 1.875),
    (0x40, 2.0), (0x7E, 448.0), (0xFE, -448.0), (0xB8, -1.0), (0x77, 240.0),
])
def test_e4m3_decode_known(byte, value):
    t = O.e4m3_decode_table()
    assert t[byte] == value
    assert np.signbit(t[byte]) == np.signbit(value)


def test_e4m3_nan_patterns():
    t = O.e4m3_decode_table()
    nans = [b for b in range(256) if np.isnan(t[b])]
    assert nans == [0x7F, 0xFF]


def test_e4m3_roundtrip_exhaustive():
    t = O.e4m3_decode_table()
    finite = [b for b in range(256) if np.isfinite(t[b])]
    enc = O.e4m3_encode(t[finite].astype(np.float32))
    assert list(enc) == finite


@pytest.mark.parametrize("x,byte", [
    (1.0625, 0x38),      # midway 1.0 / 1.125 -> even mantissa 0
    (1.1875, 0x3A),      # midway 1.125 / 1.25 -> even mantissa 2
    (2.0 ** -10, 0x00),  # midway 0 / 2^-9 -> 0
    (3 * 2.0 ** -10, 0x02),  # midway 2^-9 / 2^-8 -> even (2 * 2^-9)
    (-3 * 2.0 ** -10, 0x82),
    (464.0, 0x7E),       # midway 448 / (480): saturates to 448
    (1e6, 0x7E), (-1e6, 0xFE), (449.0, 0x7E),
    (15.5 * 2.0 ** -10, 0x08),  # rounds up out of the subnormal range
    (-1e-30, 0x80),
])
def test_e4m3_encode_ties_and_saturation(x, byte):
    assert int(O.e4m3_encode(f32([x]))[0]) == byte


def test_e4m3_encode_is_nearest_bruteforce():
    t = O.e4m3_decode_table()
    finite = np.array([b for b in range(256) if np.isfinite(t[b]) and b != 0x80])
    vals = t[finite]
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.uniform(-460, 460, 20000),
                        rng.uniform(-0.02, 0.02, 20000),
                        rng.standard_normal(20000) * 4]).astype(np.float32)
    enc = O.e4m3_encode(x)
    got = t[enc]
    xc = np.clip(x.astype(np.float64), -448, 448)
    dist = np.abs(xc[:, None] - vals[None, :])
    best = dist.min(axis=1)
    assert np.all(np.abs(np.abs(got - xc) - best) == 0)
    # ties: among equally near candidates the even mantissa is chosen
    nt = np.sum(dist == best[:, None], axis=1)
    for i in np.nonzero(nt > 1)[0]:
        assert enc[i] & 1 == 0
