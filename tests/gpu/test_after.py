"""moe_decode_layer_after: the step between two layers of a stack (residual
add skipped when the previous layer's flag is set, then a weightless RMSNorm;
"Red Lite dev23 - per-layer early-out", "What changed": a flagged layer
contributes nothing) folded into the layer's first kernel.  Every output
(the residual stream r, the normalised input a, the routing results, the
logits and y) must equal, bit for bit, rl_residual_rmsnorm (rl_rmsnorm for a
first layer) followed by moe_decode_layer on a; with the shared sticky flag
set, r and a are still written and nothing else is.  Matrix-core and
vector-unit widths, 2-bit and 3-bit."""
import numpy as np
import pytest
import torch

from quantized_routed_expert_rl_amd import binding as B
from quantized_routed_expert_rl_amd import synth
from quantized_routed_expert_rl_amd.device import DeviceModel, RouteBuffers, to_dev
from quantized_routed_expert_rl_amd.workloads import Workload

pytestmark = pytest.mark.gpu

EPS = 1e-6
SENT = -7


def _model(H, F, qbits):
    return DeviceModel(Workload("after", 21, H, 64, 8, F, 2, 4, zipf=True, qbits=qbits))


def _bits(t):
    return t.detach().cpu().numpy().view(np.uint8)


def _run(m, fused, layer, x_prev, y_prev, flag, desc=None):
    w = m.w
    out = RouteBuffers.alloc(1, w.top_k, w.n_experts)
    out.ids.fill_(SENT)
    y = torch.full((w.hidden,), float("nan"), device="cuda")
    r = torch.full((w.hidden,), float("nan"), device="cuda")
    a = torch.full((w.hidden,), float("nan"), device="cuda")
    scratch = m.decode_scratch()
    if fused:
        m.decode_after(layer, x_prev, y_prev, flag, EPS, r if y_prev is not None else None, a,
                       out, scratch, y, desc=desc)
    else:
        if y_prev is None:
            B.rl_rmsnorm(1, w.hidden, x_prev, a, EPS)
        else:
            B.rl_residual_rmsnorm(1, w.hidden, x_prev, y_prev, flag, r, a, EPS)
        m.decode(layer, a, out, scratch, y, desc=desc)
    torch.cuda.synchronize()
    return out, y, r, a


def _same(o1, o2, what):
    for t1, t2, name in [(o1[0].ids, o2[0].ids, "ids"), (o1[0].weights, o2[0].weights, "weights"),
                         (o1[0].slots, o2[0].slots, "slots"),
                         (o1[0].miss_count, o2[0].miss_count, "miss"),
                         (o1[0].early_out, o2[0].early_out, "flag"),
                         (o1[0].logits, o2[0].logits, "logits"),
                         (o1[1], o2[1], "y"), (o1[2], o2[2], "r"), (o1[3], o2[3], "a")]:
        assert np.array_equal(_bits(t1), _bits(t2)), f"{what}: {name}"


@pytest.mark.parametrize("H,F,qbits", [(2048, 512, 2), (2048, 512, 3), (512, 256, 2),
                                       (256, 64, 2), (1024, 128, 3)])
def test_after_equals_separate_step(H, F, qbits):
    m = _model(H, F, qbits)
    rng = np.random.default_rng(H + F + qbits)
    xs = synth.activations(m.w, 3)
    for t in range(3):
        x_prev = to_dev(xs[t])
        y_prev = to_dev((rng.standard_normal(H) * 0.5).astype(np.float32))
        # first layer: no previous output
        _same(_run(m, True, 0, x_prev, None, None), _run(m, False, 0, x_prev, None, None),
              f"token {t} first layer")
        for flag_val in (0, 1):               # previous layer ran / stopped
            flag = torch.full((1,), flag_val, dtype=torch.int32, device="cuda")
            f1 = _run(m, True, 1, x_prev, y_prev, flag)
            f2 = _run(m, False, 1, x_prev, y_prev, flag)
            _same(f1, f2, f"token {t} flag {flag_val}")
            want_r = xs[t] if flag_val else (xs[t] + y_prev.cpu().numpy())
            assert np.array_equal(f1[2].cpu().numpy(), want_r.astype(np.float32))


@pytest.mark.parametrize("F", [512, 64])
def test_after_with_the_sticky_flag_set(F):
    m = _model(2048, F, 2)
    w = m.w
    d = B.desc(w.hidden, w.n_experts, w.top_k, w.width, w.n_layers, w.qbits,
               int(m.pool.shape[0]), flags=B.RL_STICKY_EARLY_OUT)
    x_prev = to_dev(synth.activations(w, 1)[0])
    y_prev = to_dev(np.ones(w.hidden, np.float32))
    flag = torch.ones(1, dtype=torch.int32, device="cuda")
    out = RouteBuffers.alloc(1, w.top_k, w.n_experts)
    out.ids.fill_(SENT)
    out.early_out.fill_(1)                      # the shared word: set by an earlier layer
    y = torch.full((w.hidden,), float("nan"), device="cuda")
    r = torch.full((w.hidden,), float("nan"), device="cuda")
    a = torch.full((w.hidden,), float("nan"), device="cuda")
    scratch = m.decode_scratch()
    B.moe_decode_layer_after(d, 1, x_prev, y_prev, out.early_out, EPS, r, a, m.router[1],
                             m.bias[1], m.residency, m.pool, out.c(), scratch, scratch.numel(), y)
    r2 = torch.empty_like(r)
    a2 = torch.empty_like(a)
    B.rl_residual_rmsnorm(1, w.hidden, x_prev, y_prev, flag, r2, a2, EPS)
    torch.cuda.synchronize()
    assert torch.equal(r, r2) and torch.equal(a, a2) and torch.equal(r, x_prev)
    assert (out.ids.cpu().numpy() == SENT).all()
    assert torch.isnan(y).all()


def test_stack_graph_replays_equal_eager_runs():
    """A token of DecodeStack (the step between layers inside each layer's
    first kernel) captured once as a HIP graph and replayed for several
    tokens, with eager work between the replays, gives the same bits in
    every layer's input, normalised input, routing results and output as
    the same stack run eagerly; some layers miss and stop."""
    from quantized_routed_expert_rl_amd.stack import DecodeStack
    w = Workload("after_stack", 23, 2048, 32, 4, 512, 6, 5, zipf=True, resident=6 * 20,
                 popular=True)
    m = DeviceModel(w)
    eager, graphed = DecodeStack(m), DecodeStack(m)
    xs = synth.activations(w, w.tokens)
    x_in = torch.empty(w.hidden, device="cuda")
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        x_in.copy_(to_dev(xs[0]))
        graphed.token(x_in)                      # warm-up outside the capture
        st.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            graphed.token(x_in)
    flags = 0
    for t in range(w.tokens):
        with torch.cuda.stream(st):
            x_in.copy_(to_dev(xs[t]))
            for buf in (graphed.y, eager.y):
                buf.fill_(float("nan"))
            g.replay()
            eager.token(to_dev(xs[t]))
            st.synchronize()
        for name in ("x", "a", "y"):
            assert np.array_equal(_bits(getattr(graphed, name)), _bits(getattr(eager, name))), \
                f"token {t}: {name}"
        for l in range(w.n_layers):
            for field in ("ids", "weights", "slots", "miss_count", "early_out"):
                assert np.array_equal(_bits(getattr(graphed.routes[l], field)),
                                      _bits(getattr(eager.routes[l], field))), f"token {t} layer {l} {field}"
            flags += int(eager.routes[l].early_out.cpu()[0])
    assert 0 < flags < w.tokens * w.n_layers
