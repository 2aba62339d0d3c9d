"""Pins of the oracle's NF4 code and blockwise double quantisation.

What the pages fix about the code: 16 levels at standard-normal quantiles
with equal expected count per bin, asymmetric (2^(k-1) negative-side and
2^(k-1)+1 positive-side quantiles, one zero dropped), an exact zero, all 16
codes used, blocks of 64 with their own constant, constants re-quantised to
8 bits in blocks of 256 after subtracting their mean, and the bits/param
arithmetic.  Each test checks one of those facts, a closed form, an error
bound, or a brute-force search.
"""

import math

import mpmath
import numpy as np
import pytest
from scipy.special import ndtr

import oracle as O

GOLD = {}
with open(__file__.rsplit("/", 1)[0] + "/golden/pages_numbers.txt") as fh:
    for line in fh:
        if line.strip() and not line.startswith("#"):
            key, rest = line.split("=", 1)
            GOLD[key.strip()] = float(rest.split("|")[0])


# --- the code ---------------------------------------------------------------

def test_levels_shape_sorted_zero_span():
    q = O.nf4_levels()
    assert q.dtype == np.float32 and q.shape == (int(GOLD["nf4_levels"]),)
    assert np.all(np.diff(q) > 0)
    assert q[0] == -1.0 and q[15] == 1.0
    assert q[7] == 0.0 and not np.signbit(q[7])
    assert np.sum(q < 0) == GOLD["nf4_negative_sets"] - 1
    assert np.sum(q > 0) == GOLD["nf4_positive_sets"] - 1


def test_levels_equal_mass_per_side():
    # Closed form: mapped back through the normal CDF (scipy's ndtr, not the
    # inverse used to build them) the levels sit on two evenly spaced
    # probability grids, 8 steps above 1/2 and 7 steps below.
    q = O.nf4_levels().astype(np.float64)
    z = -math.sqrt(2) * float(mpmath.erfinv(2 * (1 - O.DELTA) - 1))
    p = ndtr(q * z)
    up = p[7:]
    dn = p[:8][::-1]
    step_up = (O.DELTA - 0.5) / 8
    step_dn = (O.DELTA - 0.5) / 7
    assert np.allclose(up, 0.5 + step_up * np.arange(9), atol=1e-7, rtol=0)
    assert np.allclose(dn, 0.5 - step_dn * np.arange(8), atol=1e-7, rtol=0)


def test_levels_cross_implementation_mpmath():
    # Same construction through a different inverse normal (mpmath erfinv at
    # 50 digits) must give the identical fp32 table.
    mpmath.mp.dps = 50
    delta = mpmath.mpf(1) - (mpmath.mpf(1) / 32 + mpmath.mpf(1) / 30) / 2

    def ppf(p):
        return mpmath.sqrt(2) * mpmath.erfinv(2 * p - 1)

    z = ppf(delta)
    half = mpmath.mpf(1) / 2
    pos = [ppf(half + j * (delta - half) / 8) / z for j in range(9)]
    neg = [-ppf(half + j * (delta - half) / 7) / z for j in range(1, 8)]
    ref = np.array(sorted(float(v) for v in pos + neg), dtype=np.float64)
    assert np.array_equal(ref.astype(np.float32), O.nf4_levels())


def test_midpoint_rule_is_nearest_level():
    q = O.nf4_levels().astype(np.float64)
    m = O.nf4_midpoints().astype(np.float64)
    rng = np.random.default_rng(4)
    n = rng.uniform(-1, 1, 200_000)
    code = np.sum(n[:, None] > m[None, :], axis=1)
    near = np.argmin(np.abs(n[:, None] - q[None, :]), axis=1)
    far_from_mid = np.min(np.abs(n[:, None] - m[None, :]), axis=1) > 1e-6
    assert np.array_equal(code[far_from_mid], near[far_from_mid])


# --- blockwise quantisation --------------------------------------------------

def _one_block_matrix(values):
    """A 1 x 64 matrix (one block) padded with zeros."""
    w = np.zeros((1, 64), dtype=np.float32)
    w[0, :len(values)] = values
    return w


def test_codes_of_exact_levels():
    q = O.nf4_levels()
    a = np.float32(2.0 ** -5)
    vals = np.concatenate([q, q[::-1], q]).astype(np.float32) * a  # exact
    w = _one_block_matrix(vals[:64])
    res = O.quantize(w)
    codes = O.unpack_codes(res)[0, :48]
    expect = np.concatenate([np.arange(16), np.arange(16)[::-1], np.arange(16)])
    assert np.array_equal(codes, expect)
    assert res["absmax"][0] == a


def test_zero_block_codes_to_zero_level():
    w = np.zeros((2, 128), dtype=np.float32)
    w[1, 64:] = np.linspace(-1, 1, 64, dtype=np.float32)
    codes = O.unpack_codes(O.quantize(w))
    assert np.all(codes[0] == 7) and np.all(codes[1, :64] == 7)
    assert codes[1, 64] == 0 and codes[1, 127] == 15


def test_ties_go_to_lower_code():
    m = O.nf4_midpoints()
    vals = np.concatenate([[1.0], m]).astype(np.float32)  # absmax exactly 1
    codes = O.unpack_codes(O.quantize(_one_block_matrix(vals)))[0]
    assert np.array_equal(codes[1:16], np.arange(15))
    # one fp32 ulp above each threshold takes the upper code
    up = np.nextafter(m, np.float32(2))
    codes = O.unpack_codes(O.quantize(_one_block_matrix(np.concatenate([[1.0], up]))))[0]
    assert np.array_equal(codes[1:16], np.arange(1, 16))


def test_pack_order_split_nibbles_per_group_of_8():
    # byte j of each 8-element group: element j (low nibble), j+4 (high)
    q = O.nf4_levels()
    vals = np.array([q[0], q[15], q[7], q[3], q[12], q[1], q[9], q[14],
                     q[2], q[5]], dtype=np.float32)
    res = O.quantize(_one_block_matrix(vals))
    assert list(res["codes"][:4]) == [0xC0, 0x1F, 0x97, 0xE3]
    # second group: elements 8, 9 = codes 2, 5; elements 10..15 = 0.0 -> 7
    assert list(res["codes"][4:8]) == [0x72, 0x75, 0x77, 0x77]


def test_codes_bruteforce_against_exact_absmax():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((6, 256)) * 0.02).astype(np.float32)
    w[2, 5] = 0.9                                     # an outlier block
    res = O.quantize(w)
    codes = O.unpack_codes(res).reshape(-1, 64)
    blocks = w.reshape(-1, 64).astype(np.float64)
    a = np.max(np.abs(blocks), axis=1)
    n = blocks / a[:, None]
    q = O.nf4_levels().astype(np.float64)
    near = np.argmin(np.abs(n[..., None] - q), axis=-1)
    mids = O.nf4_midpoints().astype(np.float64)
    safe = np.min(np.abs(n[..., None] - mids), axis=-1) > 1e-6
    assert np.array_equal(codes[safe], near[safe])
    assert np.array_equal(res["absmax"], a.astype(np.float32))


def test_mean_is_sequential_groupwise_sum():
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((40, 1024)) * 0.02).astype(np.float32)  # 640 blocks
    res = O.quantize(w)
    a = res["absmax"]
    total = 0.0
    for g0 in range(0, a.size, 256):
        part = 0.0
        for v in a[g0:g0 + 256]:
            part += float(v)
        total += part
    assert res["absmax_mean"][0] == np.float32(total / a.size)
    assert abs(float(res["absmax_mean"][0]) - math.fsum(map(float, a)) / a.size) \
        <= 2 ** -23 * float(res["absmax_mean"][0])


def test_second_level_scale_maps_group_max_to_fp8_max():
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((64, 512)) * 0.02).astype(np.float32)  # 512 blocks
    res = O.quantize(w)
    dec = O.e4m3_decode_table()[res["absmax_q"]]
    for g in range(res["absmax_scale"].size):
        assert np.max(np.abs(dec[g * 256:(g + 1) * 256])) == 448.0


def test_double_dequant_error_bound():
    # E4M3 with 3 fraction bits: relative rounding error <= 2^-4 in the normal
    # range, absolute <= 2^-10 * c1 in the subnormal range; plus two fp32
    # roundings in the decode.
    rng = np.random.default_rng(8)
    w = (rng.standard_normal((128, 1024)) * 0.02).astype(np.float32)
    w[3, 17] = 0.5
    res = O.quantize(w)
    a = res["absmax"].astype(np.float64)
    ah = O.block_scales(res).astype(np.float64)
    mu = float(res["absmax_mean"][0])
    c1 = np.repeat(res["absmax_scale"], 256)[:a.size].astype(np.float64)
    bound = (2.0 ** -4 * np.abs(a - mu) + 2.0 ** -10 * c1
             + 2.0 ** -23 * (np.abs(ah) + np.abs(a - mu)) * 2)
    assert np.all(np.abs(a - ah) <= bound)


def test_dequant_error_bound():
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((64, 512)) * 0.02).astype(np.float32)
    res = O.quantize(w)
    wt = O.bf16_bits_to_f64(O.dequantize(res))
    q = O.nf4_levels().astype(np.float64)
    gap = np.max(np.diff(q))
    a = np.repeat(res["absmax"].astype(np.float64), 64).reshape(w.shape)
    ah = np.repeat(O.block_scales(res).astype(np.float64), 64).reshape(w.shape)
    bound = 0.5 * gap * a + np.abs(a - ah) + 2.0 ** -8 * np.abs(wt) + 1e-12
    assert np.all(np.abs(w - wt) <= bound)


def test_dequant_of_exact_levels_is_level_times_scale():
    q = O.nf4_levels()
    w = np.tile(np.concatenate([q, q, q, q]), (4, 1)).astype(np.float32) * np.float32(0.25)
    res = O.quantize(w)
    ah = O.block_scales(res)
    wt = O.bf16_bits_to_f64(O.dequantize(res))
    ref = O.bf16_bits_to_f64(O.bf16_rne_bits_from_f32(
        (np.tile(np.concatenate([q, q, q, q]), (4, 1)) * ah[0]).astype(np.float32)))
    assert np.array_equal(wt, ref)


# --- storage arithmetic printed on the pages --------------------------------

def test_storage_bits_per_param():
    d = k = 4096
    sz = O.nf4_storage_bytes(d, k)
    n = d * k
    res_bits = (sz["absmax_q"] * 8 + sz["absmax_scale"] * 8) / n
    assert res_bits == 8 / 64 + 32 / (64 * 256)
    assert round(res_bits, 3) == GOLD["dq_overhead_bits"]
    assert 32 / GOLD["nf4_block"] == GOLD["dq_fp32_overhead_bits"]
    saving = GOLD["dq_fp32_overhead_bits"] - res_bits
    assert round(saving, 3) == GOLD["dq_saving_bits"]
    assert round(saving, 2) == GOLD["dq_saving_rounded_bits"]
    assert round(saving * 65e9 / 8 / 1e9) == GOLD["dq_saving_65b_gb"]
    total_bits = sum(sz.values()) * 8 / n
    assert abs(total_bits - (4 + res_bits + 32 / n)) < 1e-15
    assert round(total_bits, 3) == 4.127


def test_real_buffers_match_storage_formula():
    rng = np.random.default_rng(10)
    w = (rng.standard_normal((96, 640)) * 0.02).astype(np.float32)  # 960 blocks
    res = O.quantize(w)
    sz = O.nf4_storage_bytes(96, 640)
    assert res["codes"].nbytes == sz["codes"]
    assert res["absmax_q"].nbytes == sz["absmax_q"]
    assert res["absmax_scale"].nbytes == sz["absmax_scale"]   # 4 groups, last partial
    assert res["absmax_mean"].nbytes == sz["absmax_mean"]


@pytest.mark.parametrize("k", [63, 100])
def test_k_must_be_block_multiple(k):
    with pytest.raises(AssertionError):
        O.quantize(np.zeros((2, k), np.float32))


def test_dequantize_region_equals_full_dequantize():
    # the sampled-element form used on large weights must agree bit for bit
    # with the whole-matrix dequantisation, in any row/column order
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((48, 576)) * 0.02).astype(np.float32)   # 432 blocks, 2 groups
    res = O.quantize(w)
    full = O.dequantize(res)
    assert np.array_equal(O.dequantize_region(res, np.arange(48), np.arange(576)), full)
    rows = np.array([47, 0, 13, 13])
    cols = np.array([575, 0, 63, 64, 300])
    assert np.array_equal(O.dequantize_region(res, rows, cols), full[rows][:, cols])
