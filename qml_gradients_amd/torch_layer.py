"""PyTorch autograd bridge: the fused forward and adjoint passes as a differentiable op.

The pages wrap their fused kernels in a differentiable PyTorch module (hugo-pages
summary, section 3.3).  This module plays that role over the C ABI: the forward
runs ``hqml_forward`` (keeping the fused-pass outputs), the backward runs
``hqml_backward`` with the incoming dL/dE, so any loss built from the
expectation values gets its gradient from the fused adjoint kernels.  Gradients
flow to theta only; the encoding angles x are data.  Marshalling only: no
arithmetic of the method runs here.
"""
from __future__ import annotations

import math

import torch

from . import Context


class HEAExpectation(torch.autograd.Function):
    """E_b = <O> for a batch, differentiable in theta through the fused adjoint pass."""

    @staticmethod
    def forward(ctx, theta, x, hq_ctx):
        e = hq_ctx.forward(x, theta, save_for_backward=True)
        ctx.hq = hq_ctx
        ctx.fwd_id = hq_ctx.fwd_id
        return e

    @staticmethod
    def backward(ctx, grad_e):
        if ctx.hq.fwd_id != ctx.fwd_id:
            raise RuntimeError("this layer ran another forward after the one being differentiated; "
                               "a layer keeps the saved states of its latest forward only")
        return ctx.hq.backward(grad_e.contiguous()), None, None


class HEALayer(torch.nn.Module):
    """Hardware-efficient ansatz layer: angle encoding Ry(x_q), n_layers of Rx, Ry, Rz on
    every qubit plus the CZ chain (or the CNOT chain, entangler="cnot"), output <O> per
    sample (O = Z_0 unless obs_mask / obs_x_mask say otherwise).  theta
    [n_layers][n_qubits][3] is the trainable parameter.
    The remaining arguments are those of the C ABI's hqml_config; storage defaults to
    the compute type's (complex128 states with compute="fp64")."""

    def __init__(self, n_qubits, n_layers, max_batch, storage=None, ckpt_block=0, compute="fp32",
                 obs_mask=0, obs_x_mask=0, theta=None, device=None, entangler="cz"):
        super().__init__()
        if storage is None:
            storage = "fp64" if compute == "fp64" else "fp32"
        dtype = torch.float64 if compute == "fp64" else torch.float32
        dev = torch.device("cuda", torch.cuda.current_device() if device is None else int(device))
        if theta is None:
            theta = torch.rand(n_layers, n_qubits, 3, dtype=torch.float64) * (2.0 * math.pi)
        self.theta = torch.nn.Parameter(torch.as_tensor(theta).to(dev, dtype).contiguous())
        self.hq = Context(n_qubits, n_layers, max_batch, storage=storage, ckpt_block=ckpt_block,
                          device=dev.index, compute=compute, obs_mask=obs_mask, obs_x_mask=obs_x_mask,
                          entangler=entangler)

    def forward(self, x):
        return HEAExpectation.apply(self.theta, x, self.hq)
