"""Plain numpy reference of the QLoRA adapted linear (TEST INFRASTRUCTURE ONLY).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
this module.  It shares no code with the HIP library.

Conventions (all from the pages' statement of the problem, "Mechanics",
section "The update LoRA is allowed to learn"; "PEFT Explained", first
mechanics paragraph):

* W0 is d x k (d = output features, k = input features), row-major fp32.
* A is r x k, B is d x r, scale s = alpha / r.
* Activations are row-major with one token per row: X is M x k, Y is M x d.
  The column form h = W0 x + s B A x becomes Y = X W0^T + s (X A^T) B^T.

Everything that is exact linear algebra (forward, backward, merge) is written
as its definition in float64.  The storage format (NF4 + double quantisation)
is an encoding, so it is spelled out step by step with every rounding fixed.

Parity unpinned: the tail probability DELTA of the outermost NF4 level.
"""

from __future__ import annotations

import math

import numpy as np
from scipy.special import ndtri

__all__ = [
    "NF4_BLOCK", "DQ_GROUP", "E4M3_MAX", "DELTA",
    "bf16_bits_to_f64", "bf16_rne_bits_from_f32", "bf16_rne_bits_from_f64",
    "e4m3_decode_table", "e4m3_encode", "nf4_levels", "nf4_midpoints",
    "nf4_storage_bytes", "quantize", "dequantize", "dequantize_region", "block_scales",
    "lora_scale", "forward", "backward", "forward_f64", "backward_f64", "merge", "unmerge", "delta_w",
    "forward_sections", "backward_sections", "forward_multi",
    "dropout_scale", "dropout_input", "forward_dropout", "backward_dropout", "backward_dropout_f64",
    "adam_step",
]

# Format constants ("Mechanics", section "What QLoRA freezes, and in how many
# bits": weight block 64, constant block 256; the bundle paragraph of "What to
# choose and why" repeats both sizes as part of the model's identity).
NF4_BLOCK = 64
DQ_GROUP = 256
# Largest finite OCP FP8 E4M3FN magnitude (1.75 * 2^8); the 8-bit float the
# pages name for the second-level constants ("FP8", double-quantisation
# paragraph).  E4M3FN is the reading taken for "FP8".
E4M3_MAX = 448.0

# Tail probability of the outermost level.  The pages say the levels sit at
# standard-normal quantiles with equal expected mass per bin; the outermost
# quantile of an equal-mass grid is infinite, so an offset is needed and the
# pages do not give it.  Reading: the mean of the upper-bin centre
# probabilities of a 16-bin and a 15-bin equal-mass grid,
# 1 - (1/32 + 1/30) / 2.  PARITY UNPINNED (no page fixes it).
DELTA = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0)


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (the top half of an fp32 word)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_rne_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest, ties to even.

    The pages compute in BF16 ("Mechanics", the forward equation of "What
    QLoRA freezes"); the rounding rule is IEEE's default.  Integer form: add
    0x7FFF plus the lowest kept bit and drop the low 16 bits.  NaN maps to a
    quiet NaN (never produced by the layer for finite inputs).
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    return np.where(nan, np.uint16(0x7FC0), r).astype(np.uint16)


def bf16_rne_bits_from_f64(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit pattern with a single round-to-nearest-even.

    Used where the oracle holds an exact (float64) result and the layer
    stores bf16 (merge / unmerge).  Rounding goes straight from float64 to the
    8-significant-bit grid, with no intermediate fp32 rounding.  Finite
    inputs only.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    m, e = np.frexp(ax)                      # ax = m * 2^e, m in [0.5, 1)
    # quantum of the bf16 grid at this magnitude: 8 significant bits for
    # normal numbers (exponent >= -126), fixed 2^-133 below that.
    q_exp = np.maximum(e - 8, -133)
    q = np.ldexp(1.0, q_exp)
    r = np.rint(ax / q) * q                   # ax / q is exact; rint is RNE
    # overflow past the largest finite bf16 goes to infinity
    big = r >= np.ldexp(1.0, 128)
    r32 = np.where(big, np.float32(np.inf), r.astype(np.float32))
    r32 = np.where(np.signbit(x), -r32, r32).astype(np.float32)
    return (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def e4m3_decode_table() -> np.ndarray:
    """Value of each of the 256 OCP FP8 E4M3FN byte patterns (float64).

    Layout: sign | 4 exponent bits (bias 7) | 3 mantissa bits.  Exponent
    field 0 holds subnormals m * 2^-9; S.1111.111 is NaN; there is no
    infinity.  This is the reading taken for the pages' "FP8" constants.
    """
    t = np.empty(256, dtype=np.float64)
    for b in range(256):
        s = -1.0 if (b >> 7) else 1.0
        e = (b >> 3) & 0xF
        m = b & 0x7
        if e == 0xF and m == 0x7:
            t[b] = np.nan
        elif e == 0:
            t[b] = s * m * 2.0 ** -9
        else:
            t[b] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """fp32 values -> E4M3FN bytes, round to nearest even, saturating at 448.

    Finite inputs only.  The sign of zero is kept (-0 -> 0x80).
    """
    x = np.asarray(x, dtype=np.float32)
    neg = np.signbit(x)
    ax = np.minimum(np.abs(x).astype(np.float64), E4M3_MAX)
    m, e = np.frexp(ax)                       # ax = m * 2^e, m in [0.5, 1)
    # grid spacing: 3 fraction bits in the normal range (ax >= 2^-6),
    # fixed 2^-9 in the subnormal range.
    q = np.where(ax >= 2.0 ** -6, np.ldexp(1.0, e - 4), 2.0 ** -9)
    r = np.rint(ax / q) * q                   # exact scaling, RNE
    r = np.minimum(r, E4M3_MAX)
    out = np.zeros(x.shape, dtype=np.uint8)
    sub = r < 2.0 ** -6
    msub = np.rint(r / 2.0 ** -9).astype(np.int64)
    rm, re_ = np.frexp(np.where(sub, 1.0, r))
    field = (re_ - 1 + 7).astype(np.int64)
    mant = np.rint((rm * 2.0 - 1.0) * 8.0).astype(np.int64)
    code = np.where(sub, msub, (field << 3) | mant)
    out[...] = (code | (neg.astype(np.int64) << 7)).astype(np.uint8)
    return out


# --------------------------------------------------------------------------
# NF4 code ("Mechanics", paragraph "4-bit NormalFloat"; "Budget", section
# "QLoRA: shrink the frozen part too")
# --------------------------------------------------------------------------

def nf4_levels() -> np.ndarray:
    """The 16 NF4 levels, ascending, as fp32 (code i <-> levels()[i]).

    Construction read from the pages: levels are standard-normal quantiles at
    equally spaced probabilities (equal expected count per bin); the code is
    asymmetric, built from 2^(k-1) = 8 negative-side quantiles and
    2^(k-1)+1 = 9 positive-side quantiles, each set containing zero, with one
    of the two zeros dropped, so zero is exact and all 16 codes are used.
    Levels are normalised by the outermost quantile so they span [-1, 1]
    (blocks are scaled by their absmax).  Quantiles are taken on the
    probability grid from 1/2 to DELTA.  Inverse normal: scipy's ndtri.
    """
    z = ndtri(DELTA)
    pos = [ndtri(0.5 + j * (DELTA - 0.5) / 8.0) for j in range(9)]
    neg = [-ndtri(0.5 + j * (DELTA - 0.5) / 7.0) for j in range(8)]
    vals = sorted([v / z for v in pos] + [v / z for v in neg[1:]])
    assert len(vals) == 16 and all(x < y for x, y in zip(vals, vals[1:]))
    return np.array(vals, dtype=np.float64).astype(np.float32)


def nf4_midpoints(levels: np.ndarray | None = None) -> np.ndarray:
    """Decision thresholds m_j = fl32((q_j + q_{j+1}) / 2), j = 0..14.

    Nearest-level rounding written as thresholds: code = #{j : n > m_j}, so a
    value exactly on a threshold takes the lower code.  The sum of two fp32
    levels and its halving are exact in float64; one fp32 rounding follows.
    """
    q = (nf4_levels() if levels is None else levels).astype(np.float64)
    return ((q[:-1] + q[1:]) / 2.0).astype(np.float32)


def nf4_storage_bytes(d: int, k: int) -> dict:
    """Byte count of each buffer of the quantised format."""
    n_b = d * k // NF4_BLOCK
    return {
        "codes": d * k // 2,
        "absmax_q": n_b,
        "absmax_scale": 4 * (-(-n_b // DQ_GROUP)),
        "absmax_mean": 4,
    }


# --------------------------------------------------------------------------
# Blockwise quantisation + double quantisation ("Mechanics", paragraphs
# "4-bit NormalFloat" and "Double quantisation"; forward equation of the
# same section for the decode)
# --------------------------------------------------------------------------

def _group_ranges(n_b: int):
    for g0 in range(0, n_b, DQ_GROUP):
        yield g0, min(g0 + DQ_GROUP, n_b)


def quantize(W0: np.ndarray) -> dict:
    """Quantise a d x k fp32 matrix to NF4 with double-quantised absmax.

    Steps, in the pages' order:
      1. cut the row-major flattening into blocks of 64 and take each
         block's absmax a_b (exact);
      2. code each weight against its own block constant: n = fl32(w / a_b),
         code = nearest NF4 level (thresholds, ties to the lower code); an
         all-zero block codes to the zero level;
      3. pack two codes per byte: within each aligned group of 8 consecutive
         elements, byte j (j = 0..3) holds element j in its low nibble and
         element j + 4 in its high nibble;
      4. double quantisation: subtract the mean mu of all a_b, then in groups
         of 256 consecutive constants scale so the largest |a - mu| maps to the
         8-bit float's maximum (c1, fp32) and round each to FP8 (c2).
    mu is an fp64 sum taken sequentially inside each group of 256 and then
    sequentially over the group sums, divided by n_b and rounded to fp32.
    """
    W0 = np.ascontiguousarray(W0, dtype=np.float32)
    d, k = W0.shape
    assert k % NF4_BLOCK == 0, "k must be a multiple of 64"
    n_b = d * k // NF4_BLOCK
    blocks = W0.reshape(n_b, NF4_BLOCK)

    # 1. absmax per block
    a = np.max(np.abs(blocks), axis=1).astype(np.float32)

    # 2. codes against the exact block absmax
    mids = nf4_midpoints()
    safe = np.where(a == 0, np.float32(1), a).astype(np.float32)
    n = (blocks / safe[:, None]).astype(np.float32)      # IEEE fp32 division
    codes = np.zeros(blocks.shape, dtype=np.uint8)
    for j in range(15):
        codes += (n > mids[j]).astype(np.uint8)
    codes[a == 0, :] = 7                                  # the exact-zero level

    # 3. pack: per group of 8 elements, byte j = element j | element j+4 << 4
    g8 = codes.reshape(-1, 8)
    packed = (g8[:, 0:4] | (g8[:, 4:8] << 4)).astype(np.uint8).reshape(-1)

    # 4. double quantisation
    a64 = a.astype(np.float64)
    S = 0.0
    for g0, g1 in _group_ranges(n_b):
        S += np.add.accumulate(a64[g0:g1])[-1]           # sequential in-group
    mu = np.float32(S / n_b)
    c2 = np.zeros(n_b, dtype=np.uint8)
    c1 = np.zeros(-(-n_b // DQ_GROUP), dtype=np.float32)
    for g, (g0, g1) in enumerate(_group_ranges(n_b)):
        e = (a[g0:g1] - mu).astype(np.float32)             # fp32 subtract
        c = np.float32(np.max(np.abs(e)) / np.float32(E4M3_MAX))
        c1[g] = c
        if c != 0:
            c2[g0:g1] = e4m3_encode((e / c).astype(np.float32))
    return {"d": d, "k": k, "codes": packed, "absmax_q": c2,
            "absmax_scale": c1, "absmax_mean": np.array([mu], np.float32),
            "absmax": a}


def block_scales(q: dict) -> np.ndarray:
    """Double-dequantised block constants a_hat (fp32), one per block.

    a_hat = fl32(fl32(dec(c2) * c1) + mu): the second-level constant and the
    mean are undone in the reverse order they were applied; two roundings,
    no fused multiply-add.
    """
    n_b = q["absmax_q"].shape[0]
    dec = e4m3_decode_table()[q["absmax_q"]].astype(np.float32)
    c1 = np.repeat(q["absmax_scale"], DQ_GROUP)[:n_b].astype(np.float32)
    prod = (dec * c1).astype(np.float32)
    return (prod + q["absmax_mean"][0]).astype(np.float32)


def unpack_codes(q: dict) -> np.ndarray:
    """Per-element NF4 codes (d x k, uint8) from the packed bytes."""
    p = q["codes"].reshape(-1, 4)
    out = np.empty((p.shape[0], 8), dtype=np.uint8)
    out[:, 0:4] = p & 0xF
    out[:, 4:8] = p >> 4
    return out.reshape(q["d"], q["k"])


def dequantize(q: dict) -> np.ndarray:
    """bf16 bits of the dequantised weight w~ (d x k).

    w~ = bf16_rne(fl32(level[code] * a_hat)): the pages' "doubleDequant" that
    turns the NF4 storage back into BF16 for the multiply ("Mechanics",
    forward equation; "Budget": forward passes de-quantise NF4 to bf16).
    """
    d, k = q["d"], q["k"]
    lv = nf4_levels()
    codes = unpack_codes(q).reshape(-1, NF4_BLOCK)
    ah = block_scales(q)
    prod = (lv[codes] * ah[:, None]).astype(np.float32)
    return bf16_rne_bits_from_f32(prod).reshape(d, k)


def dequantize_region(q: dict, rows, cols) -> np.ndarray:
    """bf16 bits of w~[rows][:, cols]: the same per-element rule as
    dequantize, evaluated only at the requested elements (for checks of
    large weights on sampled rows and columns).  Element (i, c) is element
    e = i*k + c of the row-major flattening; its code sits in byte
    4*(e // 8) + e % 4 (low nibble when e % 8 < 4, else high) and its block
    constant is that of block e // 64.
    """
    k = q["k"]
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    e = rows[:, None] * k + cols[None, :]
    byte = q["codes"][(e // 8) * 4 + (e % 4)]
    code = np.where(e % 8 < 4, byte & 0xF, byte >> 4)
    ah = block_scales(q)[e // NF4_BLOCK]
    prod = (nf4_levels()[code] * ah).astype(np.float32)
    return bf16_rne_bits_from_f32(prod)


# --------------------------------------------------------------------------
# The adapted linear ("Mechanics", "The update LoRA is allowed to learn";
# "Budget", "The LoRA hypothesis"; "Explained", "How LoRA reduces ...")
# --------------------------------------------------------------------------

def lora_scale(alpha: float, r: int) -> float:
    """s = fl32(alpha / r), the fixed LoRA scale (0 when r = 0)."""
    if r == 0:
        return 0.0
    return float(np.float32(np.float32(alpha) / np.float32(r)))


def forward_f64(X, W, A, B, s):
    """Y = X W^T + s (X A^T) B^T and T = X A^T, all float64 arrays.

    The same input goes through the frozen path and the low-rank path and the
    two outputs are added; with r = 0 only the frozen path remains.
    """
    Y = X @ W.T
    T = X @ A.T
    if A.shape[0]:
        Y = Y + s * (T @ B.T)
    return Y, T


def backward_f64(dY, X, W, A, B, s):
    """Gradients of L = sum(dY * Y) for the input and the adapters.

    Only the adapters A and B are trained (W0 stays frozen: no dW0 is
    formed); the input gradient flows through the dequantised base
    ("Mechanics", "What QLoRA freezes": the adapters are the only trained
    weights, yet the input gradient is formed with the bf16 expansion of
    the frozen base).
    With U = dY B:
        dX = dY W + s U A,   dA = s U^T X,   dB = s dY^T (X A^T).
    """
    dX = dY @ W
    U = dY @ B
    if A.shape[0]:
        dX = dX + s * (U @ A)
    dA = s * (U.T @ X)
    dB = s * (dY.T @ (X @ A.T))
    return dX, dA, dB


def forward(Xb, Wt_bits, Ab, Bb, alpha):
    """Forward on bf16 bit arrays: X (M x k), w~ (d x k), A (r x k),
    B (d x r); s = fl32(alpha / r).  Returns (Y, T) in float64."""
    r = Ab.shape[0]
    return forward_f64(bf16_bits_to_f64(Xb), bf16_bits_to_f64(Wt_bits),
                       bf16_bits_to_f64(Ab), bf16_bits_to_f64(Bb),
                       lora_scale(alpha, r))


def backward(dYb, Xb, Wt_bits, Ab, Bb, alpha):
    """Backward on bf16 bit arrays; returns dX (M x k), dA (r x k),
    dB (d x r) in float64."""
    r = Ab.shape[0]
    return backward_f64(bf16_bits_to_f64(dYb), bf16_bits_to_f64(Xb),
                        bf16_bits_to_f64(Wt_bits), bf16_bits_to_f64(Ab),
                        bf16_bits_to_f64(Bb), lora_scale(alpha, r))


def forward_sections(Xb, Wt_list, A_list, B_list, alpha):
    """Several adapted projections that read the same input (the pages'
    target modules: a layer's q, k, v projections, or gate and up; "LoRA vs
    QLoRA ... Explained", run configuration), each with its own frozen w~_p
    and adapter (A_p, B_p) of one rank r.  Returns Y = [Y_0 | Y_1 | ...]
    (M x sum d_p) and T = [T_0 | T_1 | ...] (M x nsec r) in float64: each
    projection is ``forward`` on its own, the outputs side by side."""
    outs = [forward(Xb, W, A, B, alpha) for W, A, B in zip(Wt_list, A_list, B_list)]
    return np.concatenate([o[0] for o in outs], axis=1), np.concatenate([o[1] for o in outs], axis=1)


def backward_sections(dYb, Xb, Wt_list, A_list, B_list, alpha):
    """Gradients for ``forward_sections`` given dY = [dY_0 | dY_1 | ...]:
    the shared input's gradient is the sum of the projections' input
    gradients; each adapter's gradient is its own projection's.  Returns
    dX (M x k), dA = [dA_0; dA_1; ...] and dB = [dB_0; dB_1; ...] in
    float64."""
    dX, dA, dB, c = None, [], [], 0
    for W, A, B in zip(Wt_list, A_list, B_list):
        d = W.shape[0]
        gx, ga, gb = backward(np.ascontiguousarray(dYb[:, c:c + d]), Xb, W, A, B, alpha)
        dX = gx if dX is None else dX + gx
        dA.append(ga)
        dB.append(gb)
        c += d
    return dX, np.concatenate(dA, axis=0), np.concatenate(dB, axis=0)


def forward_multi(Xb, Wt_bits, A_list, B_list, idx, alpha):
    """One frozen base serving several adapters in one batch ("Mechanics",
    "What to choose and why": a mixed-task batch keeps the adapters
    unmerged and picks one per example): token m goes through the base and
    through adapter idx[m]; an index outside the list means no adapter.
    Written token by token, in float64."""
    X = bf16_bits_to_f64(Xb)
    Y = X @ bf16_bits_to_f64(Wt_bits).T
    r = A_list[0].shape[0]
    s = lora_scale(alpha, r)
    for m in range(X.shape[0]):
        a = int(idx[m])
        if 0 <= a < len(A_list):
            t = bf16_bits_to_f64(A_list[a]) @ X[m]
            Y[m] = Y[m] + s * (bf16_bits_to_f64(B_list[a]) @ t)
    return Y


def dropout_scale(p: float) -> float:
    """fl32(1 / fl32(1 - p)): inverted dropout keeps the expected input."""
    return float(np.float32(np.float32(1.0) / np.float32(np.float32(1.0) - np.float32(p))))


def dropout_input(Xb, keep, p):
    """bf16 bits of the adapter path's input under LoRA dropout ("LoRA vs
    QLoRA ... Explained", run configuration: LoRA dropout 0.05 to 0.1).
    The mask is an input (the random draw is the caller's): kept elements
    are x * fl32(1/(1-p)) rounded once to bf16, dropped elements are 0.
    The frozen path keeps the undropped X."""
    x = bf16_bits_to_f64(Xb).astype(np.float32)
    prod = (x * np.float32(dropout_scale(p))).astype(np.float32)
    return np.where(np.asarray(keep) != 0, bf16_rne_bits_from_f32(prod), np.uint16(0)).astype(np.uint16)


def forward_dropout(Xb, Wt_bits, Ab, Bb, alpha, keep, p):
    """Y = X w~^T + s (Xd A^T) B^T with Xd the dropped input; returns
    (Y, T = Xd A^T) in float64."""
    r = Ab.shape[0]
    X = bf16_bits_to_f64(Xb)
    Xd = bf16_bits_to_f64(dropout_input(Xb, keep, p))
    T = Xd @ bf16_bits_to_f64(Ab).T
    Y = X @ bf16_bits_to_f64(Wt_bits).T
    if r:
        Y = Y + lora_scale(alpha, r) * (T @ bf16_bits_to_f64(Bb).T)
    return Y, T


def backward_dropout_f64(dY, X, W, A, B, s, D):
    """Gradients of L = sum(dY * Y) for Y = X W^T + s ((X * D) A^T) B^T,
    D the elementwise dropout multiplier (keep / (1 - p)), float64:
        dX = dY W + s (U A) * D,  dA = s U^T (X * D),  dB = s dY^T ((X * D) A^T)."""
    U = dY @ B
    dX = dY @ W + s * (U @ A) * D
    Xd = X * D
    return dX, s * (U.T @ Xd), s * (dY.T @ (Xd @ A.T))


def backward_dropout(dYb, Xb, Wt_bits, Ab, Bb, alpha, keep, p):
    """Backward of ``forward_dropout`` on bf16 bit arrays, float64 results.
    dA and dB use the dropped input as the forward rounded it."""
    r = Ab.shape[0]
    s = lora_scale(alpha, r)
    dY = bf16_bits_to_f64(dYb)
    A = bf16_bits_to_f64(Ab)
    B = bf16_bits_to_f64(Bb)
    D = (np.asarray(keep) != 0) * dropout_scale(p)
    U = dY @ B
    dX = dY @ bf16_bits_to_f64(Wt_bits) + s * (U @ A) * D
    Xd = bf16_bits_to_f64(dropout_input(Xb, keep, p))
    return dX, s * (U.T @ Xd), s * (dY.T @ (Xd @ A.T))


def adam_step(W, Gb, m, v, lr, step, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0):
    """One Adam step on adapter parameters with an fp32 master copy ("Budget",
    "Why full fine-tuning costs so much": a 32-bit master copy and Adam's two
    32-bit moments per trained parameter; "Mechanics": only the adapter has
    optimiser state).  Adam as published by Kingma and Ba (moments, bias
    corrections 1 - beta^step, eps added to the root), with decoupled weight
    decay when weight_decay > 0.  Float64 from the fp32 state and bf16
    gradients; returns (W, m, v) rounded to fp32 and the bf16 bits of W."""
    f32 = np.float32
    b1, b2, e, lr, wd = (float(f32(x)) for x in (beta1, beta2, eps, lr, weight_decay))
    g = bf16_bits_to_f64(Gb)
    m = b1 * np.asarray(m, np.float64) + (1.0 - b1) * g
    v = b2 * np.asarray(v, np.float64) + (1.0 - b2) * g * g
    mh = m / (1.0 - b1 ** step)
    vh = v / (1.0 - b2 ** step)
    W = np.asarray(W, np.float64)
    W = W - lr * (mh / (np.sqrt(vh) + e) + wd * W)
    W32 = W.astype(np.float32)
    return W32, m.astype(np.float32), v.astype(np.float32), bf16_rne_bits_from_f32(W32)


def delta_w(Ab, Bb, alpha):
    """The low-rank update s B A (d x k) in float64."""
    r = Ab.shape[0]
    A = bf16_bits_to_f64(Ab)
    B = bf16_bits_to_f64(Bb)
    return lora_scale(alpha, r) * (B @ A)


def merge(Wt_bits, Ab, Bb, alpha):
    """Deploy-time merge W = w~ + s B A, stored as bf16 bits.

    The merge target is the 16-bit dequantised base, never the 4-bit storage
    ("Budget", "What actually goes wrong": merging into the quantised weights
    locks in the quantisation error; "Explained": merging may need the
    weights dequantised).  One rounding from the exact float64 sum.
    """
    W = bf16_bits_to_f64(Wt_bits)
    if Ab.shape[0] == 0:
        return np.asarray(Wt_bits, dtype=np.uint16).copy()
    return bf16_rne_bits_from_f64(W + delta_w(Ab, Bb, alpha))


def unmerge(Wm_bits, Ab, Bb, alpha):
    """Task switch: subtract s B A from a merged bf16 W ("Mechanics": switch
    tasks by subtracting BA and adding B'A'), one rounding to bf16."""
    W = bf16_bits_to_f64(Wm_bits)
    if Ab.shape[0] == 0:
        return np.asarray(Wm_bits, dtype=np.uint16).copy()
    return bf16_rne_bits_from_f64(W - delta_w(Ab, Bb, alpha))


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max|got - ref| / max|ref| over the whole output."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(got - ref)) if ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return float(num / den)


__all__ += ["unpack_codes", "rel_err"]
