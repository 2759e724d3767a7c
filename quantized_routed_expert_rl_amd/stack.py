"""Stacks of routed-expert MoE layers driven through the C ABI.

A stack applies L MoE layers in turn with a weightless RMSNorm before each
layer and a residual add after it: a_l = rmsnorm(x_l), y_l = MoE_l(a_l),
x_{l+1} = x_l + y_l, where a layer whose route raised the early-out flag
adds nothing ("Red Lite dev23 - per-layer early-out", "What changed": every
kernel downstream of a flagged layer returns at once).  The norm, the MoE
layer and the residual add all run in librlmoe's kernels; PyTorch only holds
the buffers.  Between two layers one launch (rl_residual_rmsnorm) writes
x_{l+1} and a_{l+1}, so a layer costs its three (decode) MoE launches plus
one, and every layer's input stays available for checking.

``DecodeStack`` runs single tokens through ``moe_decode_layer``;
``PrefillStack`` runs a prompt chunk by chunk through ``moe_prefill_chunk``
("Red Lite dev20 - batched prompt ingestion", "What changed": chunks of the
prompt go through every layer in turn).
"""
from __future__ import annotations

from typing import List, Sequence

import torch

from . import binding as B
from .device import DEV, DeviceModel, RouteBuffers

EPS = 1e-6


class DecodeStack:
    """One token at a time through all layers of ``model``.  After
    ``token(x0)``: ``x[l]`` is layer l's input (x[L] the output), ``a[l]``
    its normalised input, ``routes[l]`` its routing results and ``y[l]`` its
    MoE output (left untouched when the layer's flag is set)."""

    def __init__(self, model: DeviceModel):
        w = model.w
        self.model = model
        self.L, self.H = w.n_layers, w.hidden
        self.x = torch.empty(self.L + 1, self.H, device=DEV)
        self.a = torch.empty(self.L + 1, self.H, device=DEV)   # a[L]: norm of the output
        self.y = torch.empty(self.L, self.H, device=DEV)
        self.routes: List[RouteBuffers] = [
            RouteBuffers.alloc(1, w.top_k, w.n_experts, with_logits=False) for _ in range(self.L)]
        self.scratch = model.decode_scratch()

    def token(self, x0: torch.Tensor) -> torch.Tensor:
        """Runs x0 [H] (device) through the stack on the current stream."""
        self.x[0].copy_(x0.reshape(self.H))
        B.rl_rmsnorm(1, self.H, self.x[0], self.a[0], EPS)
        for l in range(self.L):
            self.model.decode(l, self.a[l], self.routes[l], self.scratch, self.y[l])
            B.rl_residual_rmsnorm(1, self.H, self.x[l], self.y[l], self.routes[l].early_out,
                                  self.x[l + 1], self.a[l + 1], EPS)
        return self.x[self.L]


class PrefillStack:
    """A prompt through all layers of ``model``, one chunk at a time.  After
    ``prompt(x0, chunks)``, for chunk c and layer l: ``xs[c][l]`` is the
    layer's input [n_c x H], ``as_[c][l]`` the normalised input,
    ``routes[c][l]`` the routing results and ``ys[c][l]`` the MoE output."""

    def __init__(self, model: DeviceModel, chunks: Sequence[int], plan_cap: int):
        w = model.w
        self.model = model
        self.L, self.H = w.n_layers, w.hidden
        self.chunks = list(chunks)
        self.plan_cap = plan_cap
        T = max(self.chunks)
        self.scratch = model.prefill_scratch(T)
        self.xs = [torch.empty(self.L + 1, n, self.H, device=DEV) for n in self.chunks]
        self.as_ = [torch.empty(self.L + 1, n, self.H, device=DEV) for n in self.chunks]
        self.ys = [torch.empty(self.L, n, self.H, device=DEV) for n in self.chunks]
        self.routes = [[RouteBuffers.alloc(n, w.top_k, w.n_experts, with_logits=False)
                        for _ in range(self.L)] for n in self.chunks]

    def prompt(self, x0: torch.Tensor) -> torch.Tensor:
        """Runs the prompt x0 [P x H] (device, P = sum of the chunks) through
        the stack on the current stream; returns the outputs [P x H]."""
        outs, t0 = [], 0
        for c, n in enumerate(self.chunks):
            x = self.xs[c]
            x[0].copy_(x0[t0:t0 + n])
            B.rl_rmsnorm(n, self.H, x[0], self.as_[c][0], EPS)
            for l in range(self.L):
                self.model.prefill(l, self.as_[c][l], self.plan_cap, self.routes[c][l],
                                   self.scratch, self.ys[c][l])
                B.rl_residual_rmsnorm(n, self.H, x[l], self.ys[c][l], self.routes[c][l].early_out,
                                      x[l + 1], self.as_[c][l + 1], EPS)
            outs.append(x[self.L])
            t0 += n
        return torch.cat(outs)
