"""Device buffers for one or more MoE layers, and calls through the C ABI.

PyTorch only provides device memory and streams here; every step of the
layer runs in librlmoe's kernels (see ``binding``).  Used by the tests, the
stack drivers and ``bench.py``.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from . import binding as B
from . import synth
from .workloads import Workload

DEV = "cuda"


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@dataclass
class RouteBuffers:
    ids: torch.Tensor
    weights: torch.Tensor
    slots: torch.Tensor
    miss_count: torch.Tensor
    early_out: torch.Tensor
    logits: Optional[torch.Tensor]

    @classmethod
    def alloc(cls, T: int, k: int, E: int, with_logits: bool = True) -> "RouteBuffers":
        return cls(torch.empty(T, k, dtype=torch.int32, device=DEV),
                   torch.empty(T, k, dtype=torch.float32, device=DEV),
                   torch.empty(T, k, dtype=torch.int32, device=DEV),
                   torch.empty(1, dtype=torch.int32, device=DEV),
                   torch.empty(1, dtype=torch.int32, device=DEV),
                   torch.empty(T, E, dtype=torch.float32, device=DEV) if with_logits else None)

    def c(self) -> B.RlRouteOut:
        return B.route_out(self.ids, self.weights, self.slots, self.miss_count,
                           self.early_out, self.logits)


class DeviceModel:
    """Router weights, biases, residency table and slot pool of L layers on
    the device, generated from the workload's seeded streams."""

    def __init__(self, w: Workload, seed: int = 0, layers: Optional[List[int]] = None,
                 table: Optional[np.ndarray] = None, pool: Optional[torch.Tensor] = None):
        self.w = w
        self.table = synth.residency(w, seed) if table is None else table
        # slots in the pool: table entries at or beyond it count as misses
        n_slots = synth.n_slots(self.table) if pool is None else int(pool.shape[0])
        self.desc = B.desc(w.hidden, w.n_experts, w.top_k, w.width, w.n_layers, w.qbits,
                           n_slots)
        self.slot_bytes = B.rl_slot_bytes(self.desc)
        assert self.slot_bytes == synth.slot_nbytes(w.hidden, w.width, w.qbits)
        layers = list(range(w.n_layers)) if layers is None else layers
        self.router = {l: to_dev(synth.router_weights(w, l, seed)) for l in layers}
        self.bias = {}
        for l in layers:
            b = synth.router_bias(w, l, seed)
            self.bias[l] = None if b is None else to_dev(b)
        self.residency = to_dev(self.table.astype(np.int32))
        if pool is None:
            pool = torch.empty(max(n_slots, 1), self.slot_bytes, dtype=torch.uint8, device=DEV)
            step = min(512, max(n_slots, 1))
            stage = torch.empty(step, self.slot_bytes, dtype=torch.uint8, pin_memory=True)
            for s0 in range(0, n_slots, step):
                cnt = min(step, n_slots - s0)
                synth.fill_slots(w, self.table, s0, cnt, seed, out=stage.numpy())
                pool[s0:s0 + cnt].copy_(stage[:cnt])
            del stage
        self.pool = pool
        self.seed = seed

    # ------------------------------------------------------------ calls
    def decode_scratch(self) -> torch.Tensor:
        return torch.zeros(B.rl_decode_scratch_bytes(self.desc), dtype=torch.uint8, device=DEV)

    def prefill_scratch(self, max_tokens: int) -> torch.Tensor:
        return torch.zeros(B.rl_prefill_scratch_bytes(self.desc, max_tokens), dtype=torch.uint8,
                           device=DEV)

    def route(self, layer, x, out: RouteBuffers, scratch, stream=None):
        return B.rl_route(self.desc, layer, x.shape[0], x, self.router[layer], self.bias[layer],
                          self.residency, out.c(), scratch, scratch.numel(), stream)

    def decode(self, layer, x, out: RouteBuffers, scratch, y, stream=None, desc=None):
        return B.moe_decode_layer(desc or self.desc, layer, x, self.router[layer], self.bias[layer],
                                  self.residency, self.pool, out.c(), scratch, scratch.numel(),
                                  y, stream)

    def decode_after(self, layer, x_prev, y_prev, flag_prev, eps, x_out, a_out,
                     out: RouteBuffers, scratch, y, stream=None, desc=None):
        """The step between two stack layers (residual add, RMSNorm) folded
        into this layer's decode call (moe_decode_layer_after)."""
        return B.moe_decode_layer_after(desc or self.desc, layer, x_prev, y_prev, flag_prev, eps,
                                        x_out, a_out, self.router[layer], self.bias[layer],
                                        self.residency, self.pool, out.c(), scratch,
                                        scratch.numel(), y, stream)

    def prefill(self, layer, x, plan_cap, out: RouteBuffers, scratch, y, stream=None):
        return B.moe_prefill_chunk(self.desc, layer, x.shape[0], plan_cap, x,
                                   self.router[layer], self.bias[layer], self.residency,
                                   self.pool, out.c(), scratch, scratch.numel(), y, stream)

    def read_slot(self, slot: int) -> np.ndarray:
        return self.pool[slot].cpu().numpy()

    def read_plan(self, scratch: torch.Tensor, max_tokens: int) -> dict:
        """The plan moe_prefill_chunk left in scratch (see rl_prefill_layout)."""
        lay = B.rl_prefill_plan_layout(self.desc, max_tokens)
        raw = scratch.cpu().numpy()

        def arr(off, n):
            return raw[off:off + 4 * n].view(np.int32).copy()

        ng = int(arr(lay.n_groups, 1)[0])
        nb = int(arr(lay.n_buckets, 1)[0])
        return {"n_groups": ng,
                "group_bounds": arr(lay.group_bounds, ng + 1),
                "n_buckets": nb,
                "group_bucket_start": arr(lay.group_bucket_start, ng + 1),
                "bucket_expert": arr(lay.bucket_expert, nb),
                "bucket_start": arr(lay.bucket_start, nb + 1),
                "pairs": lambda P: arr(lay.pairs, P)}
