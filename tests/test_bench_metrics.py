"""The arithmetic behind the benchmark line, checked on the CPU.

The step's flop count is the sum of the products the layer computes,
counted term by term here (forward: X w~^T, T = X A^T, T B^T; backward:
U = dY B, dY w~, U A, dA = U^T X, dB = dY^T T; two flops per multiply-add),
and the NF4 storage size is the codes, the FP8 block constants, the fp32
second-level scales and the mean, counted from their definitions.  The
expected values at the benchmark's shapes are written out as integers.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (imports no GPU code at module level)


def _flops_by_term(M, d, k, r):
    fwd = 2 * M * d * k + 2 * M * k * r + 2 * M * r * d
    bwd = 2 * M * d * r + 2 * M * d * k + 2 * M * r * k + 2 * M * r * k + 2 * M * d * r
    return fwd + bwd


@pytest.mark.parametrize("M,d,k,r", [(32, 256, 256, 8), (4096, 4096, 4096, 8), (4096, 4096, 4096, 16),
                                     (2048, 11008, 4096, 16), (4096, 8192, 22016, 64)])
def test_step_flops_is_the_sum_of_the_products(M, d, k, r):
    assert bench.step_flops(M, d, k, r) == _flops_by_term(M, d, k, r)


def test_step_flops_at_the_headline_shapes():
    assert bench.step_flops(4096, 4096, 4096, 8) == 276_488_519_680
    assert bench.step_flops(4096, 4096, 4096, 16) == 278_099_132_416
    assert bench.step_flops(32, 256, 256, 8) == 9_175_040


def test_dominant_kernel_flops():
    # dX: dY w~ (2 M d k) plus the adapter term s U A (2 M k r)
    assert bench.kernel_flops("dx", 4096, 4096, 4096, 16) == 137_975_824_384
    assert bench.kernel_flops("fwd_rich", 4096, 4096, 4096, 16) == 137_975_824_384


@pytest.mark.parametrize("d,k,nbytes", [(256, 256, 33_812), (4096, 4096, 8_654_852), (11008, 4096, 23_259_908),
                                        (4096, 11008, 23_259_908)])
def test_nf4_bytes(d, k, nbytes):
    # d k / 2 code bytes, one FP8 constant per 64 weights, one fp32 scale per
    # 256 constants, one fp32 mean
    assert bench.nf4_bytes(d, k) == nbytes
    assert nbytes == d * k // 2 + d * k // 64 + 4 * -(-(d * k // 64) // 256) + 4


def test_more_than_one_gpu_is_refused_without_touching_a_gpu():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode != 0
    assert "one GPU" in (p.stdout + p.stderr)
