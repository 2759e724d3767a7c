"""moe_decode_layer_noalloc (the decode call for callers that cannot
allocate: its scratch is a fixed device array inside the library) against
moe_decode_layer with a caller-allocated scratch buffer: the same kernels,
so every output must be identical to the last bit.  Two calls in a row,
the second on a smaller layer, so the second runs over what the first left
in the shared array; then the first shape again."""
import numpy as np
import pytest
import torch

from quantized_routed_expert_rl_amd import binding as B
from quantized_routed_expert_rl_amd import synth
from quantized_routed_expert_rl_amd.device import RouteBuffers, to_dev

pytestmark = pytest.mark.gpu


def _layer(H, E, k, F, qbits, seed):
    rng = np.random.default_rng(seed)
    W = to_dev((rng.standard_normal((E, H)) * 0.05).astype(np.float32))
    table = to_dev(rng.permutation(E).astype(np.int32)[None, :])
    pool = to_dev(np.stack([np.concatenate([synth.random_tensor(rng, H * F, qbits)
                                            for _ in range(3)]) for _ in range(E)]))
    x = to_dev(rng.standard_normal((1, H)).astype(np.float32))
    return B.desc(H, E, k, F, 1, qbits, E), W, table, pool, x


def _outputs(d, W, table, pool, x, noalloc):
    out = RouteBuffers.alloc(1, d.top_k, d.n_experts, with_logits=False)
    y = torch.full((d.hidden,), float("nan"), device="cuda")
    if noalloc:
        B.moe_decode_layer_noalloc(d, 0, x, W, None, table, pool, out.c(), y)
    else:
        scratch = torch.empty(B.rl_decode_scratch_bytes(d), dtype=torch.uint8, device="cuda")
        B.moe_decode_layer(d, 0, x, W, None, table, pool, out.c(), scratch, scratch.numel(), y)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (out.ids, out.weights, out.slots, out.miss_count,
                                      out.early_out, y)]


def _same(a, b, what):
    for u, v, name in zip(a, b, ["ids", "weights", "slots", "miss_count", "early_out", "y"]):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), f"{what}: {name} differs"


def test_noalloc_decode_equals_decode():
    big = _layer(2048, 512, 10, 512, 2, 1)        # the real layer shape, matrix-core kernels
    small = _layer(256, 16, 2, 64, 3, 2)          # a smaller layer, vector-unit kernels
    for what, layer in [("real shape", big), ("smaller layer", small), ("real shape again", big)]:
        got = _outputs(*layer, noalloc=True)
        want = _outputs(*layer, noalloc=False)
        assert int(got[4][0]) == 0 and np.isfinite(got[5]).all()
        _same(got, want, what)
