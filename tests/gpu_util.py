"""Helpers shared by the GPU parity tests: upload seeded inputs, download
results as bf16 bit patterns, and run the oracle on the same bytes."""

import numpy as np
import torch

import oracle as O
import workloads as WL

DEV = "cuda:0"


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(DEV)


def bits_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def quant_host(w) -> dict:
    """NF4Weight buffers as numpy arrays in the oracle's dict layout."""
    torch.cuda.synchronize()
    return {"d": w.d, "k": w.k, "codes": w.codes.cpu().numpy(),
            "absmax_q": w.absmax_q.cpu().numpy(),
            "absmax_scale": w.absmax_scale.cpu().numpy(),
            "absmax_mean": w.absmax_mean.cpu().numpy()}


class Layer:
    """One adapted linear: seeded inputs on host and device, NF4 on both."""

    def __init__(self, lib, d, k, r, M, *, alpha=None, cfg=7, layer=0, proj=0, b_zero=False,
                 oracle_quant=True):
        self.d, self.k, self.r, self.M = d, k, r, M
        self.alpha = float(2 * r if alpha is None else alpha)
        self.inp = WL.layer_inputs(d, k, r, M, cfg=cfg, layer=layer, proj=proj, b_zero=b_zero)
        self.lib = lib
        self.W0 = f32_dev(self.inp["W0"])
        self.w = lib.quantize(self.W0)
        self.A = bf16_dev(self.inp["A"]) if r else None
        self.B = bf16_dev(self.inp["B"]) if r else None
        self.X = bf16_dev(self.inp["X"])
        self.dY = bf16_dev(self.inp["dY"])
        self.q_ref = O.quantize(self.inp["W0"]) if oracle_quant else None
        self.Wt = O.dequantize(self.q_ref) if oracle_quant else None

    def oracle_fwd(self):
        return O.forward(self.inp["X"], self.Wt, self.inp["A"], self.inp["B"], self.alpha)

    def oracle_bwd(self):
        return O.backward(self.inp["dY"], self.inp["X"], self.Wt, self.inp["A"], self.inp["B"],
                          self.alpha)


def rel(got_bits, ref):
    return O.rel_err(O.bf16_bits_to_f64(got_bits), ref)
