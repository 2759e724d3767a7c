"""Parity of rl_route and moe_decode_layer with the CPU oracle on the GPU."""
import numpy as np
import pytest
import torch

from gpu.common import HostInputs, check_route, close, oracle_decode_many, oracle_route, shape_of
from oracle import moe_oracle as O
from quantized_routed_expert_rl_amd import binding as B, synth, workloads
from quantized_routed_expert_rl_amd.device import DeviceModel, RouteBuffers, to_dev

pytestmark = pytest.mark.gpu


def _model(name, qbits=2):
    return DeviceModel(workloads.get(name, qbits))


@pytest.fixture(scope="module")
def tiny():
    return _model("tiny")


@pytest.fixture(scope="module")
def real():
    return _model("decode_1l")


@pytest.fixture(scope="module")
def real3():
    return _model("decode_1l", 3)


def _decode_tokens(model, xs, layer=0):
    w = model.w
    scratch = model.decode_scratch()
    outs, ys = [], []
    for t in range(xs.shape[0]):
        out = RouteBuffers.alloc(1, w.top_k, w.n_experts)
        y = torch.full((w.hidden,), float("nan"), device="cuda")
        model.decode(layer, to_dev(xs[t:t + 1]), out, scratch, y)
        outs.append(out)
        ys.append(y)
    torch.cuda.synchronize()
    return outs, ys


def test_route_tiny_gemv_and_gemm(tiny):
    w = tiny.w
    x = synth.activations(w, 4)
    ref = oracle_route(tiny, 0, x)
    for T in (1, 4):     # T=1 takes the router GEMV, T=4 the GEMM; both then the top-k kernel
        out = RouteBuffers.alloc(T, w.top_k, w.n_experts)
        scratch = torch.zeros(64 << 10, dtype=torch.uint8, device="cuda")
        tiny.route(0, to_dev(x[:T]), out, scratch)
        check_route(out, oracle_route(tiny, 0, x[:T]))
    assert ref.ids.shape == (4, 2)


@pytest.mark.parametrize("table", ["resident", "half"])
def test_route_one_token_real_shape(real, table):
    """rl_route with one token at the real shape (router GEMV, then the top-k)
    against the oracle, with every expert resident and with every second
    expert missing.  The call zeroes its own miss count and flag, so the
    values an earlier call left there (7 and 1 here) do not leak in."""
    w = real.w
    host = HostInputs.of(real)
    row = real.table[0].copy()
    if table == "half":
        row[1::2] = -1
    tab = to_dev(row[None, :].astype(np.int32))
    x = synth.activations(w, 6, stream=3)
    scratch = torch.zeros(B.rl_route_scratch_bytes(real.desc, 1), dtype=torch.uint8, device="cuda")
    misses = 0
    for t in range(x.shape[0]):
        out = RouteBuffers.alloc(1, w.top_k, w.n_experts)
        out.miss_count.fill_(7)
        out.early_out.fill_(1)
        B.rl_route(real.desc, 0, 1, to_dev(x[t:t + 1]), real.router[0], real.bias[0], tab, out.c(),
                   scratch, scratch.numel())
        ref = O.route(x[t:t + 1], host.router(0), host.bias(0), row, w.top_k)
        check_route(out, ref)
        misses += ref.miss_count
    assert (misses > 0) == (table == "half")


def test_decode_tiny(tiny):
    w = tiny.w
    x = synth.activations(w, 4)
    outs, ys = _decode_tokens(tiny, x)
    host = HostInputs.of(tiny)
    for t, (r, y_ref, _) in enumerate(oracle_decode_many(host, 0, x, tiny.table[0])):
        check_route(outs[t], r)
        close(ys[t].cpu().numpy(), y_ref, f"y token {t}")


def _check_real(model, x, what):
    """Every token: ids, slots, miss count and flag exact; logits, weights and
    all H values of y within tolerance of the oracle."""
    outs, ys = _decode_tokens(model, x)
    host = HostInputs.of(model)
    refs = oracle_decode_many(host, 0, x, model.table[0])
    for t, (r, y_ref, _) in enumerate(refs):
        check_route(outs[t], r)
        close(ys[t].cpu().numpy(), y_ref, f"y token {t} ({what})")


def test_decode_real_shape(real):
    """Single-token decode at hidden 2048, 512 experts, top-10, width 512:
    64 tokens, every output against the oracle."""
    _check_real(real, synth.activations(real.w, 64, stream=7), "2-bit")


def test_decode_real_shape_3bit(real3):
    """The same layer with 3-bit block weights (third code bit in its own
    plane): 32 tokens, every output against the oracle."""
    _check_real(real3, synth.activations(real3.w, 32, stream=8), "3-bit")


def test_decode_early_out_leaves_y(real):
    w = real.w
    x = synth.activations(w, 3, stream=9)
    ref = oracle_route(real, 0, x)
    table = real.table.copy()
    table[0, ref.ids[1][3]] = -1          # one selected expert of token 1 missing
    hole = DeviceModel(w, table=table, pool=real.pool)
    outs, ys = _decode_tokens(hole, x)
    torch.cuda.synchronize()
    assert int(outs[1].early_out.cpu()[0]) == 1
    assert int(outs[1].miss_count.cpu()[0]) == 1
    assert int(outs[1].slots.cpu()[0, 3]) == -1
    assert torch.isnan(ys[1]).all()                      # not written
    for t in (0, 2):
        if ref.ids[1][3] not in ref.ids[t]:
            assert int(outs[t].early_out.cpu()[0]) == 0
            assert not torch.isnan(ys[t]).any()


def test_out_of_range_entries_count_as_misses(tiny):
    w = tiny.w
    x = synth.activations(w, 1)
    r = oracle_route(tiny, 0, x)
    table = tiny.table.copy()
    table[0, r.ids[0][0]] = 10_000                     # beyond n_slots
    m = DeviceModel(w, table=table, pool=tiny.pool)     # n_slots = 16 pool rows
    assert m.desc.n_slots == 16
    outs, ys = _decode_tokens(m, x)
    assert int(outs[0].early_out.cpu()[0]) == 1 and int(outs[0].slots.cpu()[0, 0]) == -1
    assert torch.isnan(ys[0]).all()


def test_decode_reruns_bit_identical(real):
    x = synth.activations(real.w, 4, stream=11)
    _, y1 = _decode_tokens(real, x)
    _, y2 = _decode_tokens(real, x)
    for a, b in zip(y1, y2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("H,E,k,F,qbits", [
    (256, 16, 2, 64, 3), (512, 100, 5, 128, 2), (1024, 1024, 32, 256, 2),
    (256, 8, 1, 32, 3), (2048, 64, 8, 2048, 2), (512, 200, 7, 1024, 3),
    (256, 1, 1, 64, 2), (512, 6, 6, 256, 3)])       # one expert; every expert selected
def test_decode_shapes(H, E, k, F, qbits):
    rng = np.random.default_rng(H + E + k + F + qbits)
    n = H * F
    W = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    table = rng.permutation(E).astype(np.int32)[None, :]
    pool_np = np.stack([np.concatenate([synth.random_tensor(rng, n, qbits) for _ in range(3)])
                        for _ in range(E)])
    from quantized_routed_expert_rl_amd import binding as B
    d = B.desc(H, E, k, F, 1, qbits, E)
    pool = to_dev(pool_np)
    Wd, res = to_dev(W), to_dev(table)
    scratch = torch.zeros(B.rl_decode_scratch_bytes(d), dtype=torch.uint8, device="cuda")
    shape = O.LayerShape(H, E, k, F, qbits)
    for t in range(3):
        x = rng.standard_normal((1, H)).astype(np.float32)
        out = RouteBuffers.alloc(1, k, E)
        y = torch.full((H,), float("nan"), device="cuda")
        B.moe_decode_layer(d, 0, to_dev(x), Wd, None, res, pool, out.c(), scratch,
                           scratch.numel(), y)
        r, y_ref, _ = O.decode_layer(shape, x[0], W, None, table[0], lambda s: pool_np[s])
        check_route(out, r)
        close(y.cpu().numpy(), y_ref, f"y {H},{E},{k},{F},{qbits} token {t}")
