"""GPU parity of every call of the C ABI against the CPU oracle.

Bars: NF4 codes, FP8 constants, scales, mean and the dequantised bf16 weight
bit-exact; Y and dX within max|err|/max|ref| <= 1e-2; dA and dB within
2e-2; merge/unmerge within the fp32-accumulation bound of the exact result
plus half a bf16 ulp, and bit-exact when the adapter product is zero.
"""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from gpu_util import DEV, Layer, bf16_dev, bits_host, f32_dev, quant_host, rel

pytestmark = pytest.mark.gpu

TOL_Y = 1e-2
TOL_G = 2e-2


def _print_case(*args):
    print("case:", *args, flush=True)


# ------------------------------------------------------------ quantise --

def _check_quant(lib, W0_np):
    w = lib.quantize(f32_dev(W0_np))
    got = quant_host(w)
    ref = O.quantize(W0_np)
    assert np.array_equal(got["codes"], ref["codes"])
    assert np.array_equal(got["absmax_q"], ref["absmax_q"])
    assert np.array_equal(got["absmax_scale"].view(np.uint32), ref["absmax_scale"].view(np.uint32))
    assert np.array_equal(got["absmax_mean"].view(np.uint32), ref["absmax_mean"].view(np.uint32))
    Wt = bits_host(lib.merge(w))
    assert np.array_equal(Wt, O.dequantize(ref))
    return w, ref


@pytest.mark.parametrize("d,k", [(16, 64), (256, 256), (96, 640), (272, 320), (1024, 4096)])
def test_quantize_bitexact_random(lib, d, k):
    _print_case("quantize", d, k)
    _check_quant(lib, WL.normal_f32((d, k), 0.02, (0, 11, d, k, 0)))


def test_quantize_bitexact_special_blocks(lib):
    _print_case("quantize special")
    d, k = 32, 512
    W = WL.normal_f32((d, k), 0.02, (0, 12, 0, 0, 0))
    q = O.nf4_levels()
    mids = O.nf4_midpoints()
    W[0, :64] = 0.0                                    # all-zero block
    W[1, :64] = np.tile(q, 4) * np.float32(0.125)      # exact levels
    W[2, :16] = np.concatenate([[1.0], mids])[:16]     # values on thresholds
    W[2, 16:64] = 0.0
    W[3, 64:128] = np.nextafter(np.tile(mids, 5)[:64], np.float32(2))  # just above
    W[3, 64] = 1.0
    W[4, 5] = 3.0                                      # outlier block
    W[5, 128:192] = -0.5                               # constant negative block
    W[6, :] = -0.0
    W[7, 10] = 1e-30                                   # tiny absmax
    _check_quant(lib, W)


def test_quantize_many_groups_partial_tail(lib):
    # 1040 blocks = 4 full groups + a partial group of 16
    _print_case("quantize partial group")
    _check_quant(lib, WL.normal_f32((80, 832), 0.02, (0, 13, 0, 0, 0)))


# ------------------------------------------------------------- forward --

FWD_CASES = [
    # d, k, r, M        (M <= 64, and M <= 128 when k % 256 == 0, run the decode
    #                   kernels; larger M the tiled one)
    (256, 256, 8, 32),
    (256, 256, 8, 1),
    (272, 320, 8, 17),
    (256, 256, 0, 40),
    (512, 384, 64, 64),
    (208, 768, 64, 64),     # chunked decode: ragged rows, four token blocks, rank 64
    (144, 1280, 5, 49),
    (2048, 8704, 16, 16),   # three chunks per split, last split one chunk
    (256, 256, 8, 16),
    (8208, 256, 16, 5),
    (512, 2304, 3, 9),
    (1040, 1024, 0, 16),
    (256, 256, 8, 100),     # chunked decode, six token blocks (100 tokens)
    (512, 512, 16, 128),    # chunked decode, eight token blocks
    (208, 768, 64, 65),     # eight token blocks, one token in the last
    (272, 320, 8, 100),     # k % 256 != 0: the tiled kernel
    (1024, 2048, 16, 300),  # tiled kernel split in four K ranges (12 tiles of 128 x 256)
    (512, 1024, 8, 129),    # split in two, one token in the last row tile
    (272, 320, 3, 300),
    (512, 512, 16, 257),
    (1024, 1024, 64, 200),
    (256, 256, 0, 129),
]


@pytest.mark.parametrize("d,k,r,M", FWD_CASES)
def test_forward_parity(lib, d, k, r, M):
    _print_case("forward", d, k, r, M)
    L = Layer(lib, d, k, r, M)
    Y = lib.forward(L.X, L.w, L.A, L.B, L.alpha)
    Yref, _ = L.oracle_fwd()
    e = rel(bits_host(Y), Yref)
    assert e <= TOL_Y, e


# up to 16 tokens with k % 256 == 0 both token-poor forms apply: the single
# launch (the default without adapters or with k <= 4096) and the split-K
# pair; each is forced here.  The single launch issues every load at once
# for k <= 4096 (S = ceil(k / 1024) steps per wave) and runs its two-slot
# ring above that.  Cases: two steps (six waves idle), 68 steps (ring),
# three row blocks per work-group with the last one partly past d, 18 steps
# with an odd rank (S = 3), one token, no adapter, S = 2 with one row block,
# S = 2 with three waves past K, two row blocks with S = 3 and a rank that
# is not a multiple of 8, two row blocks with S = 4 and three tokens, and
# the ring without adapters (64 steps).
@pytest.mark.parametrize("form", ["single", "split"])
@pytest.mark.parametrize("d,k,r,M", [(256, 256, 8, 16), (2048, 8704, 16, 16), (8208, 256, 16, 5), (512, 2304, 3, 9),
                                     (272, 512, 8, 1), (1040, 1024, 0, 16), (2064, 2048, 16, 16),
                                     (1536, 1280, 16, 16), (4112, 3072, 12, 16), (4128, 4096, 16, 3),
                                     (1040, 8192, 0, 16)])
def test_forward_parity_small_m_both_forms(lib, monkeypatch, form, d, k, r, M):
    _print_case("forward small M", form, d, k, r, M)
    monkeypatch.setenv("QLORA_DECODE", form)
    L = Layer(lib, d, k, r, M)
    Y, T = lib.forward(L.X, L.w, L.A, L.B, L.alpha, save_t=True)
    Yref, Tref = L.oracle_fwd()
    assert rel(bits_host(Y), Yref) <= TOL_Y
    if r:
        ldt = (M + 63) // 64 * 64
        assert rel(bits_host(T)[: r * ldt].reshape(r, ldt)[:, :M], Tref.T) <= TOL_Y


# 16 one-hot tokens on the last 16 input features, B = 0: Y[m, :] =
# w~[:, k - 16 + m] bit for bit in both token-poor forms, including the last
# weight rows, whose last blocks' constants sit at the very end of the
# storage (the single launch reads a lane's constants with one 8-byte load,
# moved down where it would run past the end).
@pytest.mark.parametrize("form", ["single", "split"])
@pytest.mark.parametrize("d,k", [(272, 256), (1536, 1280), (4112, 3072), (4128, 4096)])
def test_forward_small_m_one_hot_last_columns_exact(lib, monkeypatch, form, d, k):
    _print_case("forward small M one-hot last columns", form, d, k)
    monkeypatch.setenv("QLORA_DECODE", form)
    L = Layer(lib, d, k, 8, 16, b_zero=True)
    Xh = np.zeros((16, k), np.float32)
    Xh[np.arange(16), k - 16 + np.arange(16)] = 1.0
    X = bf16_dev(WL.to_bf16_bits(Xh))
    Y = bits_host(lib.forward(X, L.w, L.A, L.B, L.alpha))
    assert np.array_equal(Y, L.Wt[:, k - 16 + np.arange(16)].T)


@pytest.mark.parametrize("M", [16, 300])
def test_forward_b_zero_is_base_output_bitexact(lib, M):
    _print_case("forward B=0", M)
    L = Layer(lib, 256, 512, 8, M, b_zero=True)
    Y1 = bits_host(lib.forward(L.X, L.w, L.A, L.B, L.alpha))
    Y0 = bits_host(lib.forward(L.X, L.w))
    assert np.array_equal(Y1, Y0)


@pytest.mark.parametrize("M", [7, 16, 64, 100, 128, 256, 384])
def test_forward_one_hot_tokens_return_dequantised_columns(lib, M):
    # X rows e_c (c < M) with B = 0: Y[c, :] = w~[:, c] exactly, which pins
    # the in-GEMM dequantisation bit for bit.
    _print_case("forward one-hot", M)
    L = Layer(lib, 256, 256, 8, M, b_zero=True)
    Xh = np.zeros((M, 256), np.float32)
    Xh[np.arange(M), np.arange(M) % 256] = 1.0
    X = bf16_dev(WL.to_bf16_bits(Xh))
    Y = bits_host(lib.forward(X, L.w, L.A, L.B, L.alpha))
    assert np.array_equal(Y, L.Wt[:, np.arange(M) % 256].T)


@pytest.mark.parametrize("d,k,M", [(512, 1024, 256), (1024, 2048, 384)])
def test_split_k_forward_one_hot_exact(lib, d, k, M):
    # token-rich forward split over K ranges: each output has one nonzero
    # product, so the summed partials still return w~ bit for bit
    _print_case("split-K one-hot", d, k, M)
    L = Layer(lib, d, k, 8, M, b_zero=True)
    Xh = np.zeros((M, k), np.float32)
    Xh[np.arange(M), (7 * np.arange(M)) % k] = 1.0
    Y = bits_host(lib.forward(bf16_dev(WL.to_bf16_bits(Xh)), L.w, L.A, L.B, L.alpha))
    assert np.array_equal(Y, L.Wt[:, (7 * np.arange(M)) % k].T)


def _layer_with_every_fp8_code(lib, d, k):
    # The stored block constants c2 are overwritten so that, along every
    # 64-column stripe, the blocks run through all 254 finite E4M3 bytes:
    # the in-kernel FP8 decode is compared with the oracle's decode table
    # code by code (a random weight reaches only a narrow band of codes).
    L = Layer(lib, d, k, 8, 1, b_zero=True)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    row, blk = np.meshgrid(np.arange(d), np.arange(k // 64), indexing="ij")
    c2 = finite[(row + 37 * blk) % finite.size].reshape(-1)
    L.q_ref["absmax_q"] = c2
    L.w.absmax_q.copy_(torch.from_numpy(c2).to(DEV))
    L.Wt = O.dequantize(L.q_ref)
    return L


@pytest.mark.parametrize("M", [16, 256])
def test_every_fp8_code_dequantises_exactly(lib, M):
    _print_case("every fp8 code", M)
    d = k = 256
    L = _layer_with_every_fp8_code(lib, d, k)
    assert np.array_equal(bits_host(lib.merge(L.w)), L.Wt)
    Xh = np.zeros((M, k), np.float32)
    Xh[np.arange(M), np.arange(M)] = 1.0
    Y = bits_host(lib.forward(bf16_dev(WL.to_bf16_bits(Xh)), L.w, L.A, L.B, L.alpha))
    assert np.array_equal(Y, L.Wt[:, :M].T)
    if M == d:
        dY = bf16_dev(WL.to_bf16_bits(np.eye(d, dtype=np.float32)))
        dX, _, _ = lib.backward(dY, bf16_dev(WL.to_bf16_bits(Xh)), L.w, L.A, L.B, L.alpha)
        assert np.array_equal(bits_host(dX), L.Wt)


# ------------------------------------------------------------ backward --

BWD_CASES = [
    (512, 1024, 16, 16),    # dX split in two K ranges (few tokens: 4 tiles)
    (2048, 1024, 16, 64),   # split in eight
    (1024, 512, 8, 300),    # split in four, ragged last row tile
    (256, 256, 8, 32),
    (272, 320, 8, 17),
    (256, 256, 1, 100),
    (512, 384, 16, 300),
    (1024, 1024, 64, 200),
    (256, 256, 0, 77),
    (512, 1024, 16, 2048),  # 2048 tokens, 32 tiles of 256 rows: those tiles, K in two
    (1024, 512, 64, 2100),  # 256-row tiles, K in four, ragged last row tile
    (768, 1024, 8, 1100),   # 1100 tokens: 256-row tiles, K in three, ragged last row tile
]


@pytest.mark.parametrize("d,k,r,M", BWD_CASES)
def test_backward_parity(lib, d, k, r, M):
    _print_case("backward", d, k, r, M)
    L = Layer(lib, d, k, r, M)
    dX, dA, dB = lib.backward(L.dY, L.X, L.w, L.A, L.B, L.alpha)
    rX, rA, rB = L.oracle_bwd()
    assert rel(bits_host(dX), rX) <= TOL_Y
    if r:
        assert rel(bits_host(dA), rA) <= TOL_G
        assert rel(bits_host(dB), rB) <= TOL_G


@pytest.mark.parametrize("M", [16, 40, 300])
def test_backward_with_saved_t_matches_recompute(lib, M):
    _print_case("backward saved T", M)
    L = Layer(lib, 256, 384, 16, M)
    _, T = lib.forward(L.X, L.w, L.A, L.B, L.alpha, save_t=True)
    g1 = lib.backward(L.dY, L.X, L.w, L.A, L.B, L.alpha, T_saved=T)
    g0 = lib.backward(L.dY, L.X, L.w, L.A, L.B, L.alpha)
    for a, b in zip(g1, g0):
        assert np.array_equal(bits_host(a), bits_host(b))


def test_backward_b_zero(lib):
    _print_case("backward B=0")
    L = Layer(lib, 256, 256, 8, 100, b_zero=True)
    dX, dA, dB = lib.backward(L.dY, L.X, L.w, L.A, L.B, L.alpha)
    assert not np.any(bits_host(dA) & 0x7FFF)           # exactly +-0
    dX0, _, _ = lib.backward(L.dY, L.X, L.w)
    assert np.array_equal(bits_host(dX), bits_host(dX0))
    _, _, rB = L.oracle_bwd()
    assert rel(bits_host(dB), rB) <= TOL_G


def test_backward_one_hot_output_gradient_returns_weight(lib):
    _print_case("backward one-hot dY")
    d = 256
    L = Layer(lib, d, 320, 8, d, b_zero=True)
    dY = bf16_dev(WL.to_bf16_bits(np.eye(d, dtype=np.float32)))
    dX, _, _ = lib.backward(dY, L.X, L.w, L.A, L.B, L.alpha)
    assert np.array_equal(bits_host(dX), L.Wt)


@pytest.mark.parametrize("d,k", [(1024, 512), (2048, 1024)])
def test_split_k_dx_one_hot_exact(lib, d, k):
    # dY = I: dX = w~; with the contraction split over row ranges each
    # output still has one nonzero product
    _print_case("split-K dX one-hot", d, k)
    L = Layer(lib, d, k, 8, d, b_zero=True)
    dY = bf16_dev(WL.to_bf16_bits(np.eye(d, dtype=np.float32)))
    dX, _, _ = lib.backward(dY, L.X, L.w, L.A, L.B, L.alpha)
    assert np.array_equal(bits_host(dX), L.Wt)


def test_backward_without_dx(lib):
    L = Layer(lib, 256, 256, 8, 50)
    dX, dA, dB = lib.backward(L.dY, L.X, L.w, L.A, L.B, L.alpha, need_dx=False)
    assert dX is None
    _, rA, rB = L.oracle_bwd()
    assert rel(bits_host(dA), rA) <= TOL_G and rel(bits_host(dB), rB) <= TOL_G


@pytest.mark.parametrize("tile", ["128", "256"])
@pytest.mark.parametrize("d,k,r,M", [(512, 512, 16, 300), (272, 320, 3, 513), (768, 256, 64, 257)])
def test_tiled_variants_parity(lib, monkeypatch, tile, d, k, r, M):
    # both tile heights of the token-rich forward and of dX, on ragged shapes
    _print_case("tile", tile, d, k, r, M)
    monkeypatch.setenv("QLORA_TILE", tile)
    L = Layer(lib, d, k, r, M)
    Y = lib.forward(L.X, L.w, L.A, L.B, L.alpha)
    dX, dA, dB = lib.backward(L.dY, L.X, L.w, L.A, L.B, L.alpha)
    Yref, _ = L.oracle_fwd()
    rX, rA, rB = L.oracle_bwd()
    assert rel(bits_host(Y), Yref) <= TOL_Y
    assert rel(bits_host(dX), rX) <= TOL_Y
    assert rel(bits_host(dA), rA) <= TOL_G and rel(bits_host(dB), rB) <= TOL_G


@pytest.mark.parametrize("tile", ["128", "256"])
def test_tiled_one_hot_exact(lib, monkeypatch, tile):
    monkeypatch.setenv("QLORA_TILE", tile)
    L = Layer(lib, 512, 256, 8, 256, b_zero=True)
    Xh = np.zeros((256, 256), np.float32)
    Xh[np.arange(256), np.arange(256)] = 1.0
    Y = bits_host(lib.forward(bf16_dev(WL.to_bf16_bits(Xh)), L.w, L.A, L.B, L.alpha))
    assert np.array_equal(Y, L.Wt.T)
    dY = bf16_dev(WL.to_bf16_bits(np.eye(512, dtype=np.float32)))
    L2 = Layer(lib, 512, 256, 8, 512, b_zero=True)
    dX, _, _ = lib.backward(dY, L2.X, L2.w, L2.A, L2.B, L2.alpha)
    assert np.array_equal(bits_host(dX), L2.Wt)


# ------------------------------------------------------- merge / unmerge --

def _merge_ok(got_bits, base_bits, Ab, Bb, alpha, sign, ref_bits):
    """Merge/unmerge bar derived from the arithmetic: the r-term product is
    accumulated in fp32 (error <= (r+2) 2^-24 (|base| + |s| |B| |A|)) and
    rounded once to bf16 (<= half an ulp of the result).  Almost every
    element must also equal the oracle's bf16 bit for bit."""
    r = Ab.shape[0]
    s = O.lora_scale(alpha, r)
    A = O.bf16_bits_to_f64(Ab)
    B = O.bf16_bits_to_f64(Bb)
    base = O.bf16_bits_to_f64(base_bits)
    exact = base + sign * s * (B @ A)
    mag = np.abs(base) + abs(s) * (np.abs(B) @ np.abs(A))
    got = O.bf16_bits_to_f64(got_bits)
    _, e = np.frexp(np.abs(got))
    half_ulp = np.where(got == 0, 2.0 ** -134, np.ldexp(1.0, np.maximum(e - 9, -134)))
    bound = half_ulp + (r + 2) * 2.0 ** -24 * 1.01 * mag
    assert np.all(np.abs(got - exact) <= bound)
    assert np.mean(got_bits == ref_bits) >= 0.99


# The last four take more than one tile per work-group slot (tile runs with
# the B operand kept per tile row; 3840 x 2368: ragged columns, runs that
# cross into the next row of tiles; r = 12: B rows not a whole number of
# 16-byte pieces; 1056 x 14720: 1035 tiles, runs of three, so pairs that end
# past a run, and a ragged last row of tiles).
@pytest.mark.parametrize("d,k,r", [(256, 256, 8), (272, 320, 1), (512, 1024, 64), (96, 2112, 16), (128, 448, 12),
                                   (384, 640, 40), (3840, 2368, 64), (2304, 4096, 16), (2304, 4096, 12),
                                   (1056, 14720, 64)])
def test_merge_unmerge_parity(lib, d, k, r):
    _print_case("merge", d, k, r)
    L = Layer(lib, d, k, r, 1)
    A, B = L.inp["A"], L.inp["B"]
    W = bits_host(lib.merge(L.w, L.A, L.B, L.alpha))
    Wref = O.merge(L.Wt, A, B, L.alpha)
    _merge_ok(W, L.Wt, A, B, L.alpha, +1, Wref)
    back = bits_host(lib.unmerge(bf16_dev(Wref), L.A, L.B, L.alpha))
    bref = O.unmerge(Wref, A, B, L.alpha)
    _merge_ok(back, Wref, A, B, L.alpha, -1, bref)


# Merge over runs of tiles (more tiles than work-group slots) with B = 0:
# W = w~ bit for bit, the product being exactly zero.  Ragged columns with
# 64 ranks, 12 ranks (B rows not a whole number of 16-byte pieces), and a
# ragged last row of tiles with runs of three.
@pytest.mark.parametrize("d,k,r", [(3840, 2368, 64), (2304, 4096, 12), (1056, 14720, 64)])
def test_merge_runs_b_zero_returns_dequantised_weight(lib, d, k, r):
    _print_case("merge runs B=0", d, k, r)
    L = Layer(lib, d, k, r, 1, b_zero=True)
    assert np.array_equal(bits_host(lib.merge(L.w, L.A, L.B, L.alpha)), L.Wt)


def test_merge_b_zero_and_unmerge_in_place(lib):
    L = Layer(lib, 256, 512, 8, 1, b_zero=True)
    W = lib.merge(L.w, L.A, L.B, L.alpha)
    assert np.array_equal(bits_host(W), L.Wt)
    L2 = Layer(lib, 256, 512, 8, 1, cfg=8)
    W2 = lib.merge(L2.w, L2.A, L2.B, L2.alpha)
    W2h = bits_host(W2)
    ref = O.unmerge(W2h, L2.inp["A"], L2.inp["B"], L2.alpha)
    lib.unmerge(W2, L2.A, L2.B, L2.alpha, out=W2)
    _merge_ok(bits_host(W2), W2h, L2.inp["A"], L2.inp["B"], L2.alpha, -1, ref)


def test_merged_layer_matches_unmerged_forward(lib):
    L = Layer(lib, 512, 512, 16, 300)
    Yu = bits_host(lib.forward(L.X, L.w, L.A, L.B, L.alpha))
    Wm = lib.merge(L.w, L.A, L.B, L.alpha)
    Ym = (L.X.float() @ Wm.float().T)
    Yref, _ = L.oracle_fwd()
    assert rel(Yu, Yref) <= TOL_Y
    assert O.rel_err(Ym.cpu().numpy(), Yref) <= TOL_Y


# --------------------------------------------------------- determinism --

def test_runs_are_bit_identical(lib):
    L = Layer(lib, 512, 512, 16, 300, oracle_quant=False)
    a = [bits_host(t) for t in lib.backward(L.dY, L.X, L.w, L.A, L.B, L.alpha)]
    b = [bits_host(t) for t in lib.backward(L.dY, L.X, L.w, L.A, L.B, L.alpha)]
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    y1 = bits_host(lib.forward(L.X, L.w, L.A, L.B, L.alpha))
    y2 = bits_host(lib.forward(L.X, L.w, L.A, L.B, L.alpha))
    assert np.array_equal(y1, y2)


# ----------------------------------------------------------- HIP graphs --

# The calls launch kernels only (no memsets, no host synchronisation), so a
# caller may capture them in a HIP graph.  Forward (decode-shaped and
# token-rich) and backward are captured together and the graph is replayed
# three times with eager calls in between; every replay must reproduce the
# eager results bit for bit.
@pytest.mark.parametrize("M", [16, 300])
def test_graph_capture_replays_match_eager(lib, M):
    _print_case("graph capture", 512, 512, 16, M)
    L = Layer(lib, 512, 512, 16, M, oracle_quant=False)
    Y0, T0 = lib.forward(L.X, L.w, L.A, L.B, L.alpha, save_t=True)
    ref = [bits_host(t) for t in (Y0,) + tuple(lib.backward(L.dY, L.X, L.w, L.A, L.B, L.alpha, T_saved=T0))]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture, as torch recommends
        Yw, Tw = lib.forward(L.X, L.w, L.A, L.B, L.alpha, save_t=True)
        lib.backward(L.dY, L.X, L.w, L.A, L.B, L.alpha, T_saved=Tw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        Y, T = lib.forward(L.X, L.w, L.A, L.B, L.alpha, save_t=True)
        outs = (Y,) + tuple(lib.backward(L.dY, L.X, L.w, L.A, L.B, L.alpha, T_saved=T))
    for rep in range(3):
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = [bits_host(t) for t in outs]
        for a, b in zip(got, ref):
            assert np.array_equal(a, b), rep
        # eager work between replays
        lib.forward(L.X, L.w, L.A, L.B, L.alpha)
        torch.cuda.synchronize()
