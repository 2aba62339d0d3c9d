"""GPU parity at the largest shapes the C ABI admits along one dimension.

The ABI takes d and k up to 2^31 - 1 as long as d*k, M*k and M*d stay below
2^31 elements.  The token-poor forward is the only path such shapes reach
(any M > 127 breaks the element bound), so it runs here with k just past
2^24 (d = 16) and with d just past 2^24 (k = 64): offsets of rows, tokens
and code words then need more than 24 bits.

The weights are built so that a small problem gives the exact answer: every
64-weight block has the same absmax a (one entry of each block is +-a, the
rest lie strictly inside), so the block constants are all a, their mean is
a, the second-level scales are 0 and every double-dequantised constant is a
again, in the large weight and in the small one alike.  The codes of a block
depend only on its values divided by a.  Hence

  k past 2^24:  W0 = the 16 x 64 matrix V repeated along k, with X and A
                zero except on the last block: Y = oracle(X_last, V, A_last).
  d past 2^24:  W0 = the rows of a 272 x 64 matrix V repeated along d
                (272 does not divide 2^24, so a row index cut to 24 bits
                lands on a different row of V), B likewise:
                Y[:, n] = oracle(X, V, A, B_V)[:, n % 272].

Bars as everywhere: max|err| / max|ref| <= 1e-2; the periodic columns of
the second case must also be bit-identical to each other.
"""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from gpu_util import DEV, bits_host, rel

pytestmark = pytest.mark.gpu

AMAX = np.float32(0.05)


def _equal_absmax_blocks(rows, seed):
    """rows x 64 fp32: N(0, 0.02^2) clipped inside (-a, a), one entry per
    row set to +-a (a = 0.05), so every block's absmax is exactly a."""
    rng = np.random.default_rng(seed)
    v = np.clip(rng.standard_normal((rows, 64)) * 0.02, -0.049, 0.049).astype(np.float32)
    pos = rng.integers(0, 64, rows)
    sign = np.where(rng.integers(0, 2, rows) == 1, 1.0, -1.0).astype(np.float32)
    v[np.arange(rows), pos] = sign * AMAX
    return v


def _bf16(a):
    return torch.from_numpy(WL.to_bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(DEV)


def test_k_past_2_to_24(lib):
    d, k, M, r, alpha = 16, (1 << 24) + 64, 2, 8, 16.0
    print(f"case: max-size k d={d} k={k} M={M} r={r}", flush=True)
    V = _equal_absmax_blocks(d, 401)
    rng = np.random.default_rng(402)
    Xs = WL.to_bf16_bits(rng.standard_normal((M, 64)).astype(np.float32))
    As = WL.to_bf16_bits((rng.standard_normal((r, 64)) / 8).astype(np.float32))
    Bb = WL.to_bf16_bits((rng.standard_normal((d, r)) * 0.3).astype(np.float32))
    Vt = O.dequantize(O.quantize(V))
    ref, _ = O.forward(Xs, Vt, As, Bb, alpha)

    W0 = torch.from_numpy(V).to(DEV).repeat(1, k // 64)
    w = lib.quantize(W0)
    del W0
    X = torch.zeros((M, k), dtype=torch.bfloat16, device=DEV)
    X[:, k - 64:] = _bf16(O.bf16_bits_to_f64(Xs).astype(np.float32))
    A = torch.zeros((r, k), dtype=torch.bfloat16, device=DEV)
    A[:, k - 64:] = _bf16(O.bf16_bits_to_f64(As).astype(np.float32))
    B = torch.from_numpy(Bb.view(np.int16)).view(torch.bfloat16).to(DEV)
    Y = lib.forward(X, w, A, B, alpha)
    torch.cuda.synchronize()
    e = rel(bits_host(Y), ref)
    print(f"  rel error Y {e:.2e}", flush=True)
    assert e <= 1e-2


def test_d_past_2_to_24(lib):
    P = 272                               # period of the rows; d = P * 61681
    d, k, M, r, alpha = (1 << 24) + 16, 64, 2, 8, 16.0
    assert d % P == 0 and (1 << 24) % P != 0
    print(f"case: max-size d d={d} k={k} M={M} r={r}", flush=True)
    V = _equal_absmax_blocks(P, 411)
    rng = np.random.default_rng(412)
    Xb = WL.to_bf16_bits(rng.standard_normal((M, k)).astype(np.float32))
    Ab = WL.to_bf16_bits((rng.standard_normal((r, k)) / 8).astype(np.float32))
    Bs = WL.to_bf16_bits((rng.standard_normal((P, r)) * 0.3).astype(np.float32))
    Vt = O.dequantize(O.quantize(V))
    ref, _ = O.forward(Xb, Vt, Ab, Bs, alpha)          # M x P

    W0 = torch.from_numpy(V).to(DEV).repeat(d // P, 1)
    w = lib.quantize(W0)
    del W0
    torch.cuda.empty_cache()
    B = torch.from_numpy(Bs.view(np.int16)).view(torch.bfloat16).to(DEV).repeat(d // P, 1)
    X = torch.from_numpy(Xb.view(np.int16)).view(torch.bfloat16).to(DEV)
    A = torch.from_numpy(Ab.view(np.int16)).view(torch.bfloat16).to(DEV)
    Y = lib.forward(X, w, A, B, alpha)
    torch.cuda.synchronize()
    Yh = bits_host(Y).reshape(M, d // P, P)
    # every period of output features is the same computation on the same
    # inputs: bit-identical results
    assert np.array_equal(Yh, np.broadcast_to(Yh[:, :1, :], Yh.shape))
    e = rel(Yh[:, 0, :], ref)
    print(f"  rel error Y {e:.2e}", flush=True)
    assert e <= 1e-2
