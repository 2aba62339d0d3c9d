"""GPU parity of the adapter's Adam step (qlora_adam_step) against the
oracle's adam_step: three steps in a row on a ragged parameter count, with
and without decoupled weight decay, and with the optimiser state in pinned
host memory (paged state read by the kernel in place).

Bars: the fp32 master copy and moments within max|err|/max|ref| <= 1e-5
(one fp32 operation order against float64); the bf16 copy within one bf16
ulp of the oracle's rounding of its master copy, elementwise.
"""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from gpu_util import DEV, bf16_dev, bits_host, rel

pytestmark = pytest.mark.gpu


def _print_case(*args):
    print("case:", *args, flush=True)


def _ulp_ok(got_bits, ref_bits):
    g = O.bf16_bits_to_f64(got_bits)
    r = O.bf16_bits_to_f64(ref_bits)
    ulp = np.maximum(np.abs(r) * 2.0 ** -7, 2.0 ** -133)
    return np.all(np.abs(g - r) <= ulp)


@pytest.mark.parametrize("wd", [0.0, 0.01])
def test_adam_steps_parity(lib, wd):
    n = 2 * 65536 + 13
    _print_case("adam", n, wd)
    W_h = WL.normal_f32((n,), 0.02, (0, 92, 0, 0, 0))
    m_h = np.zeros(n, np.float32)
    v_h = np.zeros(n, np.float32)
    W, m, v = (torch.from_numpy(a.copy()).to(DEV) for a in (W_h, m_h, v_h))
    P = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    for step in (1, 2, 3):
        G_h = WL.normal_bf16((n,), 1e-3, (step, 92, 0, 0, 4))
        lib.adam_step(P, W, bf16_dev(G_h), m, v, 2e-4, step, weight_decay=wd)
        W_h, m_h, v_h, P_ref = O.adam_step(W_h, G_h, m_h, v_h, 2e-4, step, weight_decay=wd)
        torch.cuda.synchronize()
        for got, ref in ((W, W_h), (m, m_h), (v, v_h)):
            assert O.rel_err(got.cpu().numpy(), ref) <= 1e-5
        assert _ulp_ok(bits_host(P), P_ref)
        # continue from the oracle's state so that each step is checked alone
        W.copy_(torch.from_numpy(W_h))
        m.copy_(torch.from_numpy(m_h))
        v.copy_(torch.from_numpy(v_h))


def test_adam_state_in_pinned_host_memory(lib):
    # the state may live outside device memory (paged optimiser state):
    # the kernel reads and writes it in place, with the same results
    n = 8 * 4096 + 5
    _print_case("adam pinned", n)
    W_h = WL.normal_f32((n,), 0.02, (0, 91, 0, 0, 0))
    G = bf16_dev(WL.normal_bf16((n,), 1e-3, (0, 91, 0, 0, 4)))
    dev_state = [torch.from_numpy(a).to(DEV) for a in (W_h.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32))]
    host_state = [torch.from_numpy(a).pin_memory() for a in (W_h.copy(), np.zeros(n, np.float32),
                                                             np.zeros(n, np.float32))]
    P1 = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    P2 = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    for step in (1, 2):
        lib.adam_step(P1, dev_state[0], G, dev_state[1], dev_state[2], 1e-3, step)
        lib.adam_step(P2, host_state[0], G, host_state[1], host_state[2], 1e-3, step)
    torch.cuda.synchronize()
    assert np.array_equal(bits_host(P1), bits_host(P2))
    for a, b in zip(dev_state, host_state):
        assert np.array_equal(a.cpu().numpy().view(np.uint32), b.numpy().view(np.uint32))
