"""Shared pieces of the GPU parity tests: oracle shapes, the tolerance, and
the oracle's inputs.

Tolerance: elementwise |gpu - ref| <= 1e-5 + 1e-4 * |ref| on float32 outputs
(logits, weights, y); ids, slots, miss counts, flags and plans exactly equal.

Every input the oracle sees is regenerated on the host from the seeded
streams (synth): router weights, biases and expert bytes are never read back
from the device buffers the kernels used, so a kernel that wrote into its
own inputs could not hide.  The oracle's expert evaluations are independent
of each other and run on a thread pool (NumPy releases the interpreter lock
inside its array operations).
"""
import os
from concurrent.futures import ThreadPoolExecutor
from functools import lru_cache

import numpy as np
import torch

from oracle import moe_oracle as O
from quantized_routed_expert_rl_amd import synth
from quantized_routed_expert_rl_amd.device import DeviceModel, RouteBuffers, to_dev  # noqa: F401

RTOL, ATOL = 1e-4, 1e-5

_POOL = None


def pool_map(fn, items):
    """map(fn, items) on a shared pool of host threads (results in order)."""
    global _POOL
    if _POOL is None:
        _POOL = ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1)))
    return list(_POOL.map(fn, items))


def close(gpu, ref, what=""):
    gpu = np.asarray(gpu, np.float32)
    ref = np.asarray(ref, np.float32)
    bad = ~np.isclose(gpu, ref, rtol=RTOL, atol=ATOL)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; "
                           f"worst |d|={np.abs(gpu - ref)[bad].max():.3e}")


def shape_of(w):
    return O.LayerShape(w.hidden, w.n_experts, w.top_k, w.width, w.qbits)


class HostInputs:
    """The oracle's view of a DeviceModel's workload, regenerated on the
    host: ``router(l)``, ``bias(l)`` and ``read_slot`` (slot -> that slot's
    bytes).  ``table`` is the residency table the device pool was filled
    from (slot s holds the expert whose entry is s)."""

    def __init__(self, w, table=None, seed=0):
        self.w, self.seed = w, seed
        self.table = synth.residency(w, seed) if table is None else np.asarray(table)
        flat = self.table.ravel()
        held = np.nonzero(flat >= 0)[0]
        self._owner = dict(zip(flat[held].tolist(), held.tolist()))
        self._router = lru_cache(maxsize=None)(lambda l: synth.router_weights(w, l, seed))
        self._bias = lru_cache(maxsize=None)(lambda l: synth.router_bias(w, l, seed))

    @classmethod
    def of(cls, model: DeviceModel):
        return cls(model.w, synth.residency(model.w, model.seed), model.seed)

    def router(self, layer):
        return self._router(layer)

    def bias(self, layer):
        return self._bias(layer)

    def read_slot(self, slot):
        key = self._owner[int(slot)]
        E = self.table.shape[1]
        return synth.expert_slot(self.w, key // E, key % E, self.seed)

    def expert(self, layer, expert):
        """Reader for a table whose 'slot' of every expert is its id (all
        resident): the oracle then evaluates the true expert bytes."""
        return synth.expert_slot(self.w, layer, expert, self.seed)


def oracle_route(model: DeviceModel, layer, x, host: HostInputs = None):
    host = host or HostInputs.of(model)
    return O.route(x, host.router(layer), host.bias(layer), model.table[layer], model.w.top_k)


def oracle_decode_many(host: HostInputs, layer, xs, table_row, read_slot=None):
    """oracle.decode_layer for every row of xs (one token each), in parallel:
    [(route, y, h)]."""
    shape = shape_of(host.w)
    rs = read_slot or host.read_slot
    return pool_map(lambda t: O.decode_layer(shape, xs[t], host.router(layer), host.bias(layer),
                                             table_row, rs), range(xs.shape[0]))


def oracle_prefill(host: HostInputs, layer, x, table_row, plan_cap, tokens=None,
                   read_slot=None):
    """oracle.prefill_chunk with its buckets evaluated in parallel."""
    return O.prefill_chunk(shape_of(host.w), x, host.router(layer), host.bias(layer), table_row,
                           read_slot or host.read_slot, plan_cap, tokens=tokens,
                           map_fn=lambda f, it: pool_map(f, list(it)))


def check_route(out: RouteBuffers, ref, with_logits=True):
    torch.cuda.synchronize()
    assert np.array_equal(out.ids.cpu().numpy(), ref.ids), "ids"
    assert np.array_equal(out.slots.cpu().numpy(), ref.slots), "slots"
    assert int(out.miss_count.cpu()[0]) == ref.miss_count, "miss_count"
    assert int(out.early_out.cpu()[0]) == ref.early_out, "early_out"
    close(out.weights.cpu().numpy(), ref.weights, "weights")
    if with_logits and out.logits is not None:
        close(out.logits.cpu().numpy(), ref.logits, "logits")
