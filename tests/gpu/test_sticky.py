"""The shared, only-raised early-out flag of the decode calls
(RL_STICKY_EARLY_OUT; "Red Lite dev23 - per-layer early-out", "What
changed": every decode kernel takes the flag and returns at once when it
is set).

A call that finds the flag set must leave every output untouched (routing
results, miss count, y); a call that misses must raise it and report its
misses; a call without misses must leave it at zero and match the oracle.
A three-layer chain that shares one flag stops at the first missing layer:
the layer after it does nothing.  Both expert paths (matrix cores for
widths that are multiples of 256, the VALU path otherwise) run each case.
"""
import numpy as np
import pytest
import torch

from gpu.common import HostInputs, close, oracle_decode_many
from oracle import moe_oracle as O
from quantized_routed_expert_rl_amd import binding as B
from quantized_routed_expert_rl_amd import synth
from quantized_routed_expert_rl_amd.device import DeviceModel, RouteBuffers, to_dev
from quantized_routed_expert_rl_amd.workloads import Workload

pytestmark = pytest.mark.gpu

SENT = -7


def _model(F, table=None):
    w = Workload("sticky", 11, 256, 16, 2, F, 3, 4)
    return DeviceModel(w, table=table)


def _call(m, layer, x, out, flag, y):
    w = m.w
    d = B.desc(w.hidden, w.n_experts, w.top_k, w.width, w.n_layers, w.qbits,
               int(m.pool.shape[0]), flags=B.RL_STICKY_EARLY_OUT)
    scratch = torch.zeros(B.rl_decode_scratch_bytes(d), dtype=torch.uint8, device="cuda")
    ro = B.route_out(out.ids, out.weights, out.slots, out.miss_count, flag)
    B.moe_decode_layer(d, layer, to_dev(x[None]), m.router[layer], m.bias[layer], m.residency,
                       m.pool, ro, scratch, scratch.numel(), y)
    torch.cuda.synchronize()


def _fresh(m):
    w = m.w
    out = RouteBuffers.alloc(1, w.top_k, w.n_experts, with_logits=False)
    out.ids.fill_(SENT)
    out.slots.fill_(SENT)
    out.miss_count.fill_(123)
    y = torch.full((w.hidden,), float("nan"), device="cuda")
    return out, y


@pytest.mark.parametrize("F", [256, 64])
def test_set_flag_stops_the_call(F):
    m = _model(F)
    x = synth.activations(m.w, 1)[0]
    out, y = _fresh(m)
    flag = torch.ones(1, dtype=torch.int32, device="cuda")
    _call(m, 0, x, out, flag, y)
    assert int(flag.cpu()[0]) == 1
    assert (out.ids.cpu().numpy() == SENT).all() and (out.slots.cpu().numpy() == SENT).all()
    assert int(out.miss_count.cpu()[0]) == 123
    assert torch.isnan(y).all()


@pytest.mark.parametrize("F", [256, 64])
def test_clear_flag_stays_clear_without_misses(F):
    m = _model(F)
    x = synth.activations(m.w, 1)[0]
    out, y = _fresh(m)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    _call(m, 1, x, out, flag, y)
    assert int(flag.cpu()[0]) == 0 and int(out.miss_count.cpu()[0]) == 0
    r, y_ref, _ = oracle_decode_many(HostInputs.of(m), 1, x[None], m.table[1])[0]
    assert np.array_equal(out.ids.cpu().numpy()[0], r.ids[0])
    close(y.cpu().numpy(), y_ref, "y")


@pytest.mark.parametrize("F", [256, 64])
def test_chain_stops_at_the_first_miss(F):
    m0 = _model(F)
    x = synth.activations(m0.w, 1)[0]
    # layer 1 loses the expert it selects first; layers 0 and 2 keep theirs
    host = HostInputs.of(m0)
    r1 = O.route(x[None], host.router(1), host.bias(1), m0.table[1], m0.w.top_k)
    table = m0.table.copy()
    table[1, r1.ids[0][0]] = -1
    m = _model(F, table=table)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    outs, ys = zip(*[_fresh(m) for _ in range(3)])
    for l in range(3):                   # the same input to each layer is enough here
        _call(m, l, x, outs[l], flag, ys[l])
    assert int(flag.cpu()[0]) == 1
    assert not torch.isnan(ys[0]).any()                       # ran
    assert int(outs[1].miss_count.cpu()[0]) >= 1 and torch.isnan(ys[1]).all()   # missed
    assert (outs[2].ids.cpu().numpy() == SENT).all() and torch.isnan(ys[2]).all()  # stopped
    assert int(outs[2].miss_count.cpu()[0]) == 123
