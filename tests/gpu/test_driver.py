"""The native decode driver (rl_driver_*) against the Python miss-servicing
stack ("Red Lite dev23 - per-layer early-out and pre-gated expert prefetch",
"What changed": stop at the first missing layer, load its experts, run it
again, resume; the early-out / layer-by-layer policy; the pre-gated
prefetch).  Both drive the same kernels with the same policy from the same
seeded model, so every layer's input after every token, the statistics, the
cache's counters and the device residency table must agree exactly; the
layer inputs must also equal those of an all-resident stack."""
import numpy as np
import pytest
import torch

from gpu.common import RTOL, ATOL, HostInputs, pool_map
from oracle import moe_oracle as O
from quantized_routed_expert_rl_amd import synth
from quantized_routed_expert_rl_amd.device import DeviceModel, to_dev
from quantized_routed_expert_rl_amd.stack import (DecodeStack, HostExpertStore,
                                                  NativeServicedDecode, ServicedDecodeStack)
from quantized_routed_expert_rl_amd.workloads import Workload

pytestmark = pytest.mark.gpu


def oracle_replay_layer_inputs(x, host: HostInputs):
    """The native driver exposes each layer's input x_l; every layer is
    checked against the oracle from it: the oracle runs layer l on
    rmsnorm(x_l) with every expert's true bytes, and x_{l+1} must be the
    float32 sum of x_l and a y within the tolerance of the oracle's:
    |x_{l+1} - (x_l + y_ref)| <= 1e-5 + 1e-4 |y_ref| + half an ulp of x_{l+1}
    (the one rounding of the residual sum).  A wrong selection, a wrong
    expert in a slot or a skipped layer moves x_{l+1} far outside that."""
    w = host.w
    shape = O.LayerShape(w.hidden, w.n_experts, w.top_k, w.width, w.qbits)
    every = np.arange(w.n_experts, dtype=np.int32)
    refs = pool_map(lambda l: O.decode_layer(shape, O.rmsnorm(x[l])[0], host.router(l),
                                             host.bias(l), every, lambda e: host.expert(l, e)),
                    range(w.n_layers))
    for l, (r, y_ref, _) in enumerate(refs):
        assert not r.early_out
        want = x[l].astype(np.float64) + y_ref.astype(np.float64)
        bound = ATOL + RTOL * np.abs(y_ref.astype(np.float64)) + 0.5 * np.spacing(
            np.abs(x[l + 1])).astype(np.float64)
        err = np.abs(x[l + 1].astype(np.float64) - want)
        assert (err <= bound).all(), f"layer {l}: worst excess {float((err - bound).max()):.3e}"


def _workloads(per_layer):
    hot = Workload("serviced", 9, 256, 32, 4, 256, 6, 10, zipf=True, resident=6 * per_layer,
                   popular=True)
    full = Workload(**{**hot.__dict__, "resident": -1, "popular": False})
    return hot, full


@pytest.mark.parametrize("per_layer,limit,prefetch,sticky", [
    (8, 4, False, False), (8, 0, False, False), (16, 4, False, False), (8, 0, True, False),
    (8, 4, False, True), (8, 0, True, True), (8, 100, False, True)])
def test_native_driver_equals_python_stack(per_layer, limit, prefetch, sticky):
    hot, full = _workloads(per_layer)
    xs = synth.activations(hot, hot.tokens)
    ref = DecodeStack(DeviceModel(full))
    store = HostExpertStore(hot)
    py = ServicedDecodeStack(DeviceModel(hot), store, early_out_limit=limit, prefetch=prefetch,
                             sticky=sticky)
    nat = NativeServicedDecode(DeviceModel(hot), store, early_out_limit=limit, prefetch=prefetch,
                               sticky=sticky)
    host = HostInputs(hot)
    for t in range(hot.tokens):
        print("token", t, flush=True)
        x0 = to_dev(xs[t])
        ref.token(x0)
        py.token(x0)
        nat.token(x0)
        torch.cuda.synchronize()
        want = ref.x.cpu().numpy()
        assert np.array_equal(py.stack.x.cpu().numpy(), want), f"python stack, token {t}"
        assert np.array_equal(nat.x.cpu().numpy(), want), f"native driver, token {t}"
        oracle_replay_layer_inputs(nat.x.cpu().numpy(), host)
    assert nat.stats == py.stats, (nat.stats, py.stats)
    assert nat.cache.stats() == py.cache.stats()
    assert np.array_equal(nat.model.residency.cpu().numpy(), nat.cache.table())
    assert np.array_equal(nat.cache.table(), py.cache.table())
    st = nat.stats
    assert st["loads"] > 0 and st["early_outs"] > 0
    if prefetch:
        assert st["predictions"] > 0 and st["prefetch_loads"] > 0


def test_driver_refuses_after_an_error():
    """A pool smaller than one layer's selection: the cache refuses the
    reservation (RL_E_RANGE from the token), and the driver then refuses
    every further token (RL_E_STATE), since cache and pool may be out of step.
    The error comes from the host-side cache; no kernel misbehaves."""
    from quantized_routed_expert_rl_amd import binding as B
    hot = Workload("serviced", 9, 256, 32, 4, 256, 6, 10, zipf=True, resident=2, popular=True)
    m = DeviceModel(hot)
    assert int(m.pool.shape[0]) < hot.top_k
    nat = NativeServicedDecode(m, HostExpertStore(hot), early_out_limit=0)
    xs = synth.activations(hot, 2)
    with pytest.raises(B.RlError, match=r"\(-3\)"):
        nat.token(to_dev(xs[0]))
    with pytest.raises(B.RlError, match=r"\(-6\)"):
        nat.token(to_dev(xs[1]))
