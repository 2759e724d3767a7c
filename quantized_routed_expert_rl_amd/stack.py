"""Stacks of routed-expert MoE layers driven through the C ABI.

A stack applies L MoE layers in turn with a weightless RMSNorm before each
layer and a residual add after it: a_l = rmsnorm(x_l), y_l = MoE_l(a_l),
x_{l+1} = x_l + y_l, where a layer whose route raised the early-out flag
adds nothing ("Red Lite dev23 - per-layer early-out", "What changed": every
kernel downstream of a flagged layer returns at once).  The norm, the MoE
layer and the residual add all run in librlmoe's kernels; PyTorch only holds
the buffers.  Between two layers one launch (rl_residual_rmsnorm) writes
x_{l+1} and a_{l+1}, so a layer costs its three (decode) MoE launches plus
one, and every layer's input stays available for checking; single-token
decode folds that step into the next layer's first kernel instead
(moe_decode_layer_after), so a layer costs its three launches.

``DecodeStack`` runs single tokens through ``moe_decode_layer_after``;
``PrefillStack`` runs a prompt chunk by chunk through ``moe_prefill_chunk``
("Red Lite dev20 - batched prompt ingestion", "What changed": chunks of the
prompt go through every layer in turn).
"""
from __future__ import annotations

from typing import List, Sequence

import numpy as np
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
        """Runs x0 [H] (device) through the stack on the current stream.
        Each layer's call also does the step before it (the previous layer's
        residual add and this layer's RMSNorm) in its first kernel
        (moe_decode_layer_after), one launch less per layer, with the same
        bits as the separate launch."""
        self.x[0].copy_(x0.reshape(self.H))
        for l in range(self.L):
            first = l == 0
            self.model.decode_after(
                l, self.x[0] if first else self.x[l - 1], None if first else self.y[l - 1],
                None if first else self.routes[l - 1].early_out, EPS,
                None if first else self.x[l], self.a[l], self.routes[l], self.scratch,
                self.y[l])
        l = self.L - 1
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


class _nullcontext:
    def __enter__(self):
        return None

    def __exit__(self, *exc):
        return False


class HostExpertStore:
    """Every expert of a workload in pinned host memory: the backing store
    misses are loaded from, copied straight into pool slots.  ``build``
    fills it from the seeded streams (slot_bytes per expert, L*E experts)."""

    def __init__(self, w, seed: int = 0, build: bool = True):
        from . import synth
        self.w = w
        self.E = w.n_experts
        self.slot_bytes = synth.slot_nbytes(w.hidden, w.width, w.qbits)
        self.tensor = torch.empty(w.n_layers * w.n_experts, self.slot_bytes, dtype=torch.uint8,
                                  pin_memory=True)
        self.data = self.tensor.numpy()
        if build:
            for i in range(w.n_layers * w.n_experts):
                synth.expert_slot(w, i // self.E, i % self.E, seed, out=self.data[i])

    def __call__(self, layer: int, expert: int):
        return self.data[layer * self.E + expert]

    def row(self, layer: int, expert: int) -> torch.Tensor:
        return self.tensor[layer * self.E + expert]

    def device_pool(self, table, step: int = 256) -> torch.Tensor:
        """A device slot pool holding, for every resident entry of ``table``,
        that expert's bytes (the pool a cache seeded from the table needs)."""
        n_slots = int(table.max()) + 1
        pool = torch.empty(n_slots, self.slot_bytes, dtype=torch.uint8, device=DEV)
        key_of_slot = np.full(n_slots, -1, np.int64)
        held = np.nonzero(table.ravel() >= 0)[0]
        key_of_slot[table.ravel()[held]] = held
        stage = torch.empty(step, self.slot_bytes, dtype=torch.uint8, pin_memory=True)
        for s0 in range(0, n_slots, step):
            keys = key_of_slot[s0:s0 + step]
            n = keys.size
            stage.numpy()[:n] = self.data[np.maximum(keys, 0)]
            pool[s0:s0 + n].copy_(stage[:n])
        return pool


class ServicedDecodeStack:
    """Decode through L layers with a bounded expert pool: a layer whose
    selection names a non-resident expert raises its flag, and every kernel
    after it in that layer returns at once; the host then loads that layer's
    missing experts into least recently used slots (the library's expert
    cache), updates the device residency table, runs the layer again and
    resumes at the next layer ("Red Lite dev23 - per-layer early-out and
    pre-gated expert prefetch", "What changed": layers before f are
    complete, the CPU loads only layer f's missing experts, runs them and
    resumes at f+1).

    Two paths, as in the notes' policy: the early-out path replays the whole
    rest of the token as one HIP graph and looks at the layers' flags
    afterwards; the synchronous path replays one layer at a time and services
    a miss as soon as its layer shows it.  A token with more than
    ``early_out_limit`` early-outs sends the next tokens to the synchronous
    path; a token that needed no load sends them back ("Red Lite dev23",
    "What changed", policy).

    The layers after an early-out still run on the unfinished input; their
    results are overwritten when the token resumes, so every layer's
    output equals that of a fully resident stack.

    ``prefetch`` adds the notes' pre-gated prefetch to the synchronous path
    ("Red Lite dev23", "What changed", pre-gated prefetch): layer m's router
    applied to layer m-1's input predicts layer m's selection (rl_route into
    buffers of its own, so no layer flag is touched).  Layer l's graph ends
    with layer l+1's input, so it also predicts layer l+2; after layer l the
    host reserves the predicted experts in the cache with no victim among
    layer l+1's slots and queues their copies ahead of layer l+2 (layer 1 is
    predicted from layer 0's input before layer 0).  This is the order of the
    native driver, whose copies run on a stream of their own while layer l+1
    runs, so the cache decisions of the two agree step for step.
    ``stats`` counts the predictions and how many predicted experts layer
    l+1 then selected (the accuracy the notes did not measure).

    ``sticky`` gives every layer one shared early-out word in the library's
    RL_STICKY_EARLY_OUT mode (the notes' single flag of a token): after the
    first missing layer every kernel of the rest of the token returns at
    once, so the early-out path wastes almost nothing; the missing layer is
    the first whose miss count is nonzero, and the word is cleared before
    every replay."""

    def __init__(self, model: DeviceModel, source, early_out_limit: int = 4,
                 prefetch: bool = False, sticky: bool = False):
        w = model.w
        self.model, self.source, self.limit = model, source, early_out_limit
        self.L, self.E, self.k = w.n_layers, w.n_experts, w.top_k
        self.stack = DecodeStack(model)
        s = self.stack
        # one flag word per layer in one tensor, so one copy reads them all;
        # sticky: one word for every layer, and the miss counts in one tensor
        self.sticky = sticky
        self.flags = torch.zeros(1 if sticky else self.L, dtype=torch.int32, device=DEV)
        self.misses = torch.zeros(self.L, dtype=torch.int32, device=DEV)
        self.ddesc = model.desc
        if sticky:
            d = model.desc
            self.ddesc = B.desc(d.hidden, d.n_experts, d.top_k, d.width, d.n_layers, d.qbits,
                                d.n_slots, flags=B.RL_STICKY_EARLY_OUT)
        for l in range(self.L):
            s.routes[l].early_out = self.flags[0:1] if sticky else self.flags[l:l + 1]
            s.routes[l].miss_count = self.misses[l:l + 1]
        self.table = np.array(model.table, dtype=np.int32)
        n_slots = int(model.pool.shape[0])
        self.cache = B.ExpertCache(n_slots, self.L, self.E)
        for l, e in zip(*np.nonzero(self.table >= 0)):
            self.cache.insert(int(l), int(e), int(self.table[l, e]))
        self.stage = torch.empty(self.k, model.slot_bytes, dtype=torch.uint8, pin_memory=True)
        self.pstage = torch.empty(self.k, model.slot_bytes, dtype=torch.uint8, pin_memory=True)
        self.table_h = torch.from_numpy(self.table).pin_memory()
        self.sync_path = False
        self.prefetch = prefetch
        self.stats = dict(tokens=0, early_outs=0, loads=0, sync_tokens=0, evictions=0,
                          predictions=0, predicted_selected=0, prefetch_loads=0)
        self.pred = RouteBuffers.alloc(1, self.k, self.E, with_logits=False)
        self.pred_scratch = torch.zeros(B.rl_route_scratch_bytes(model.desc, 1),
                                        dtype=torch.uint8, device=DEV)
        self.h_flags = torch.empty(self.flags.numel(), dtype=torch.int32, pin_memory=True)
        self.h_miss = torch.empty(self.L, dtype=torch.int32, pin_memory=True)
        self.h_pred = torch.empty(self.k, dtype=torch.int32, pin_memory=True)
        self.stream = torch.cuda.Stream()
        self.suffix = [self._capture(l, self.L) for l in range(self.L)]
        self.single = [self._capture(l, l + 1) for l in range(self.L)]
        # layer l, then the prediction of layer l+2's selection from layer l+1's
        # input; and layer 1's prediction from layer 0's input
        self.single_pf = ([self._capture(l, l + 1, predict=True) for l in range(self.L - 2)]
                          if prefetch else [])
        self.first_pf = self._capture(0, 0, predict=True) if prefetch and self.L > 1 else None

    def _predict(self, l):
        """Layer l+1's router on layer l's input, into the prediction buffers."""
        self.model.route(l + 1, self.stack.a[l:l + 1], self.pred, self.pred_scratch)

    def _layer(self, l):
        s = self.stack
        self.model.decode(l, s.a[l], s.routes[l], s.scratch, s.y[l], desc=self.ddesc)
        B.rl_residual_rmsnorm(1, s.H, s.x[l], s.y[l], s.routes[l].early_out, s.x[l + 1],
                              s.a[l + 1], EPS)

    def _capture(self, l0, l1, predict=False):
        """Layers l0 .. l1-1, then (predict) layer l1+1's router on layer l1's input."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(self.stream):
            for rep in range(2):              # once to warm up, once captured
                with (torch.cuda.graph(g, stream=self.stream) if rep else _nullcontext()):
                    for l in range(l0, l1):
                        self._layer(l)
                    if predict:
                        self._predict(l1)
        return g

    def _load(self, layer, ids, stage, exclude_layer=-1):
        """Reserve layer's ids in the cache (no victim among exclude_layer's
        experts when >= 0; a reservation refused for want of such slots loads
        nothing) and queue the copies of the missing ones (from the pinned
        rows ``stage``) and the table update on the stream; returns (loads,
        slots, gens)."""
        n, slots, load, evicted, gens = self.cache.reserve(layer, ids, exclude_layer, raw=True)
        if n == B.RL_E_RANGE and exclude_layer >= 0:
            return 0, slots, gens
        B.check(min(n, 0), "rl_cache_reserve")
        pool = self.model.pool
        for i in np.nonzero(load)[0] if n else ():
            if hasattr(self.source, "row"):      # pinned store: one copy, host to slot
                pool[int(slots[i])].copy_(self.source.row(layer, int(ids[i])), non_blocking=True)
            else:
                stage[i].numpy()[:] = self.source(layer, int(ids[i]))
                pool[int(slots[i])].copy_(stage[i], non_blocking=True)
            self.table[layer, ids[i]] = slots[i]
            if evicted[i] >= 0:
                self.table[evicted[i] // self.E, evicted[i] % self.E] = -1
                self.stats["evictions"] += 1
        if n:
            self.table_h.numpy()[:] = self.table
            self.model.residency.copy_(self.table_h, non_blocking=True)
        self.cache.commit()
        return n, slots, gens

    def _service(self, f, graph=None):
        """Load layer f's missing experts, then run layer f again (``graph``:
        layer f's graph with the next prediction, recomputed on the finished
        input)."""
        s = self.stack
        ids = s.routes[f].ids[0].cpu().numpy()
        n, slots, gens = self._load(f, ids, self.stage)
        self.stats["loads"] += n
        if self.sticky:
            self.flags.zero_()
        (graph or self.single[f]).replay()
        flag = int(self.flags[0 if self.sticky else f].item())
        assert flag == 0, f"layer {f} still misses after its experts were loaded"
        for sl, g in zip(slots, gens):        # no slot of the run was reloaded meanwhile
            assert self.cache.generation(int(sl)) == int(g)

    def token(self, x0: torch.Tensor) -> torch.Tensor:
        s = self.stack
        with torch.cuda.stream(self.stream):
            s.x[0].copy_(x0.reshape(s.H))
            B.rl_rmsnorm(1, s.H, s.x[0], s.a[0], EPS)
            n_eo, l = 0, 0
            sync = self.sync_path
            predicted = {}
            while l < self.L:
                if not sync:
                    if self.sticky:
                        self.flags.zero_()
                        self.misses[l:].zero_()
                    self.suffix[l].replay()
                    if self.sticky:
                        self.h_flags.copy_(self.flags, non_blocking=True)
                        self.h_miss.copy_(self.misses, non_blocking=True)
                        self.stream.synchronize()
                        if int(self.h_flags[0]) == 0:
                            break
                        f = l + int(np.nonzero(self.h_miss.numpy()[l:])[0][0])
                    else:
                        flags = self.flags.cpu().numpy()
                        hit = np.nonzero(flags[l:])[0]
                        if hit.size == 0:
                            break
                        f = l + int(hit[0])
                else:
                    def prefetch(m):          # queued ahead of layer m; layer m-1 runs first
                        pids = self.pred.ids[0].cpu().numpy()
                        predicted[m] = pids
                        self.stats["prefetch_loads"] += self._load(m, pids, self.pstage,
                                                                   exclude_layer=m - 1)[0]
                    if l == 0 and self.first_pf is not None:
                        self.first_pf.replay()
                        prefetch(1)
                    predict = self.prefetch and l + 2 < self.L
                    g = self.single_pf[l] if predict else self.single[l]
                    if self.sticky:
                        self.flags.zero_()
                    g.replay()
                    self.h_flags.copy_(self.flags, non_blocking=True)
                    self.stream.synchronize()
                    if int(self.h_flags[0 if self.sticky else l]) != 0:
                        n_eo += 1
                        self._service(l, g)
                    if predict:
                        prefetch(l + 2)
                    l += 1
                    continue
                n_eo += 1
                self._service(f)
                l = f + 1
            # the experts every layer used become the most recently used
            # ("Red Lite dev21", "What changed": LRU stamps refreshed after
            # the token); a later layer's loads may have evicted some
            ids = torch.stack([r.ids[0] for r in s.routes]).cpu().numpy()
            for layer in range(self.L):
                self.cache.touch(layer, ids[layer])
            for layer, pids in predicted.items():
                self.stats["predictions"] += 1
                self.stats["predicted_selected"] += len(set(pids.tolist()) & set(ids[layer].tolist()))
            self.stream.synchronize()
        self.stats["tokens"] += 1
        self.stats["early_outs"] += n_eo
        self.stats["sync_tokens"] += int(sync)
        if n_eo > self.limit:
            self.sync_path = True
        elif n_eo == 0:
            self.sync_path = False
        return s.x[self.L]


class NativeServicedDecode:
    """The miss-servicing decode of ``ServicedDecodeStack`` run by the
    library's native driver (rl_driver_*): the same policy, graphs and
    statistics, with the per-layer host work (waits, cache calls, copies,
    table updates) in C++ instead of Python.  ``x`` [L+1, H] holds every
    layer's input after a token."""

    def __init__(self, model: DeviceModel, store: "HostExpertStore", early_out_limit: int = 4,
                 prefetch: bool = False, sticky: bool = False):
        w = model.w
        self.model, self.store = model, store
        self.L, self.H = w.n_layers, w.hidden
        d = model.desc
        self.desc = B.desc(d.hidden, d.n_experts, d.top_k, d.width, d.n_layers, d.qbits, d.n_slots,
                           flags=B.RL_STICKY_EARLY_OUT if sticky else 0)
        self.cache = B.ExpertCache(int(model.pool.shape[0]), self.L, w.n_experts)
        for l, e in zip(*np.nonzero(model.table >= 0)):
            self.cache.insert(int(l), int(e), int(model.table[l, e]))
        self.x = torch.empty(self.L + 1, self.H, device=DEV)
        self.stream = torch.cuda.Stream()
        self.drv = B.DecodeDriver(self.desc, [model.router[l] for l in range(self.L)],
                                  [model.bias[l] for l in range(self.L)], model.residency,
                                  model.pool, store.tensor, self.cache, self.x,
                                  early_out_limit=early_out_limit, prefetch=prefetch, eps=EPS,
                                  stream=self.stream)

    def token(self, x0: torch.Tensor) -> torch.Tensor:
        x0 = x0.reshape(self.H)
        self.stream.wait_stream(torch.cuda.current_stream())
        self.drv.token(x0)
        return self.x[self.L]

    @property
    def stats(self) -> dict:
        return self.drv.stats()
