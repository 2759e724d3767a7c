"""Bit-exact parity on dyadic layers: inputs and weights chosen so that every
step of the expert path is exact in float32, so the kernels' y must equal the
exact value to the last bit (decode and prefill, 2-bit and 3-bit, at
hidden = width = 256 and at the real shape hidden 2048, width 512), a
stronger check than the tolerance the other parity tests apply.  Width 128
takes the vector-unit kernels.

The layer follows the definitions of the routed expert (SwiGLU gate/up,
down, rank-ordered sum; "Red Lite dev20 - batched prompt ingestion" and
"Red Lite dev21 - GPU-routed decode", "What changed") with k = 1:
- every x row takes values in {0, 16, 32}, in pairs around 16, so that it
  sums to 16 H;
- gate weights are positive multiples of 1/32 (codes with 2c - 3 > 0, or
  2c - 7 > 0 for 3-bit), so g_j >= 16 H / 32 >= 128: exp(-g) underflows and
  silu(g) = g in float32 and in float64; g sits on a grid of 1/2;
- up weights are all 1/32, so u_j = H / 2 and h_j = (H / 2) g_j exactly;
- down weights are multiples of 2^-10;
- the code and group-scale sets of each case keep every partial sum of g
  and e below 2^24 steps of its grid (checked below);
- with k = 1 the routing weight is exactly 1.
So y = e = W_d ((H/2) W_g x) exactly.  The expected value is computed here in
integers from the fields the tensors were written from, independently of the
oracle and of the kernels; the oracle's own y is checked against it too.
"""
import numpy as np
import pytest
import torch

from blockfmt import pack_tensor_fast
from gpu.common import check_route
from oracle import moe_oracle as O
from quantized_routed_expert_rl_amd import binding as B
from quantized_routed_expert_rl_amd import synth
from quantized_routed_expert_rl_amd.device import RouteBuffers, to_dev

pytestmark = pytest.mark.gpu

E, K, T = 4, 1, 6

# (codes, group scales, d) per tensor kind; codes given as the allowed set
FIELDS = {
    # hidden = width = 256: every down code and group scales 0/1
    (256, 2): {"gate": ([2, 3], [0, 1], 1.0), "up": ([2], [0], 1.0),
               "down": ([0, 1, 2, 3], [0, 1], 2.0 ** -5)},
    (256, 3): {"gate": ([4, 5, 6, 7], [0], 2.0), "up": ([4], [0], 2.0),
               "down": (list(range(8)), [0, 1], 2.0 ** -4)},
    # hidden 2048, width 512: group scale 0 and gate levels <= 3 keep e's sums in range
    (2048, 2): {"gate": ([2, 3], [0], 1.0), "up": ([2], [0], 1.0),
                "down": ([0, 1, 2, 3], [0], 2.0 ** -5)},
    (2048, 3): {"gate": ([4, 5], [0], 2.0), "up": ([4], [0], 2.0),
                "down": ([2, 3, 4, 5], [0], 2.0 ** -4)},
}
SHAPES = [(256, 256, 2), (256, 256, 3), (2048, 512, 2), (2048, 512, 3),
          (256, 128, 2), (256, 128, 3)]                  # width 128: vector-unit kernels


def _x_rows(rng, n, H):
    """Rows of {0, 16, 32}: each of H/2 disjoint index pairs holds (0, 32),
    (32, 0) or (16, 16)."""
    rows = np.empty((n, H), np.float32)
    for t in range(n):
        perm = rng.permutation(H)
        a, b = perm[:H // 2], perm[H // 2:]
        dv = rng.choice([-16, 0, 16], H // 2)
        rows[t, a] = 16 + dv
        rows[t, b] = 16 - dv
    return rows


def _tensor(rng, H, F, qbits, kind):
    """One F x H (gate, up) or H x F (down) tensor in the block format, and
    its weights as integers in units of 1/32 (gate, up) or 2^-10 (down)."""
    n = H * F
    nb = n // 256
    cset, sset, d = FIELDS[(H, qbits)][kind]
    c = rng.choice(cset, n)
    s = rng.choice(sset, (nb, 8))
    buf = pack_tensor_fast(c, s, np.full(nb, d), qbits)
    m = 2 * np.repeat(s.reshape(-1), 32) + 1               # group scale factor of each value
    lvl = (2 * c - 3) if qbits == 2 else (2 * c - 7)
    unit = 32 if kind != "down" else 1024
    num = d * m * lvl * unit / (32 if qbits == 2 else 64)  # weight / (1 / unit)
    assert np.all(num == np.round(num))
    return buf, np.round(num).astype(np.int64).reshape(H if kind == "down" else F, -1)


def _layer(H, F, qbits, seed):
    rng = np.random.default_rng(1000 * qbits + H + seed)
    slots, nums = [], []
    for _ in range(E):
        parts = [_tensor(rng, H, F, qbits, kind) for kind in ("gate", "up", "down")]
        slots.append(np.concatenate([p[0] for p in parts]))
        nums.append([p[1] for p in parts])
    W = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    return np.stack(slots), nums, W, _x_rows(rng, T, H)


def _exact_y(nums, expert, x_row):
    """y = e = W_d (silu(g) u) with silu(g) = g, in integers; also checks
    that every partial sum of g and e has fewer than 2^24 steps of its grid."""
    gn, un, dn = nums[expert]
    H = x_row.size
    xi = x_row.astype(np.int64)
    g32 = gn @ xi                                          # 32 g, multiples of 16
    assert g32.min() >= 128 * 32 and np.all(un @ xi == 16 * H)
    assert (np.abs(gn) @ xi).max() // 16 < 2 ** 24
    h = g32 * (H // 2) // 32                               # h = g u, u = H / 2
    assert np.all(g32 * (H // 2) % 32 == 0)
    grid = np.gcd.reduce(h)                                # e's grid, in units of 2^-10
    assert (np.abs(dn) @ h).max() // grid < 2 ** 24
    y = (dn @ h).astype(np.float64) / 1024
    assert np.all(y.astype(np.float32).astype(np.float64) == y)
    return y.astype(np.float32)


def _same_bits(got, want, what):
    got = np.asarray(got, np.float32)
    bad = got.view(np.uint32) != want.view(np.uint32)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} differ; "
                           f"worst |d|={np.abs(got - want)[bad].max():.3e}")


@pytest.mark.parametrize("H,F,qbits", SHAPES)
def test_decode_exact(H, F, qbits):
    pool_np, nums, W, x = _layer(H, F, qbits, 1)
    table = np.arange(E, dtype=np.int32)[None, :]
    d = B.desc(H, E, K, F, 1, qbits, E)
    pool, Wd, res = to_dev(pool_np), to_dev(W), to_dev(table)
    scratch = torch.zeros(B.rl_decode_scratch_bytes(d), dtype=torch.uint8, device="cuda")
    shape = O.LayerShape(H, E, K, F, qbits)
    for t in range(T):
        out = RouteBuffers.alloc(1, K, E)
        y = torch.full((H,), float("nan"), device="cuda")
        B.moe_decode_layer(d, 0, to_dev(x[t:t + 1]), Wd, None, res, pool, out.c(), scratch,
                           scratch.numel(), y)
        r, y_ref, _ = O.decode_layer(shape, x[t], W, None, table[0], lambda s: pool_np[s])
        torch.cuda.synchronize()
        check_route(out, r)
        assert float(out.weights.cpu()[0, 0]) == 1.0
        want = _exact_y(nums, int(r.ids[0][0]), x[t])
        _same_bits(y_ref, want, f"oracle token {t}")
        _same_bits(y.cpu().numpy(), want, f"decode {H}x{F} {qbits}-bit token {t}")


@pytest.mark.parametrize("H,F,qbits", SHAPES)
def test_prefill_exact(H, F, qbits):
    pool_np, nums, W, x = _layer(H, F, qbits, 2)
    table = np.arange(E, dtype=np.int32)[None, :]
    d = B.desc(H, E, K, F, 1, qbits, E)
    pool = to_dev(pool_np)
    scratch = torch.zeros(B.rl_prefill_scratch_bytes(d, T), dtype=torch.uint8, device="cuda")
    out = RouteBuffers.alloc(T, K, E)
    y = torch.full((T, H), float("nan"), device="cuda")
    B.moe_prefill_chunk(d, 0, T, E, to_dev(x), to_dev(W), None, to_dev(table), pool, out.c(),
                        scratch, scratch.numel(), y)
    r, _, y_ref = O.prefill_chunk(O.LayerShape(H, E, K, F, qbits), x, W, None, table[0],
                                  lambda s: pool_np[s], E)
    torch.cuda.synchronize()
    check_route(out, r)
    got = y.cpu().numpy()
    for t in range(T):
        want = _exact_y(nums, int(r.ids[t][0]), x[t])
        _same_bits(y_ref[t], want, f"oracle token {t}")
        _same_bits(got[t], want, f"prefill {H}x{F} {qbits}-bit token {t}")


@pytest.mark.parametrize("path,T", [("route", 1), ("route", 37), ("decode", 1)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_route_logits_exact(path, T, with_bias):
    """Router logits on a dyadic grid (W in 2^-10 Z with |numerator| <= 2^6,
    x in 2^-6 Z with |numerator| <= 2^7, bias in 2^-16 Z): every product and
    partial sum is exact in float64, so each logit is the single float32
    rounding of the integer sum, to the last bit ("Red Lite dev23", "What
    changed": the router GEMV in float32 with the sum kept exact), and the
    ids, slots and flags equal the oracle's.  rl_route takes the float64
    matrix-core GEMM for several tokens and the GEMV for one; a decode call
    takes the GEMV."""
    H, E, k, F = 2048, 64, 8, 256
    rng = np.random.default_rng(T + 100 * with_bias + 7 * (path == "decode"))
    nw = rng.integers(-64, 65, (E, H))
    nx = rng.integers(-128, 129, (T, H))
    W = (nw / 1024).astype(np.float32)
    x = (nx / 64).astype(np.float32)
    nb = rng.integers(-2 ** 20, 2 ** 20, E) if with_bias else np.zeros(E, np.int64)
    bias = (nb / 65536).astype(np.float32) if with_bias else None
    table = np.arange(E, dtype=np.int32)[None, :]
    want = ((nx @ nw.T + nb[None, :]).astype(np.float64) / 65536).astype(np.float32)
    d = B.desc(H, E, k, F, 1, 2, E)
    out = RouteBuffers.alloc(T, k, E)
    bd = None if bias is None else to_dev(bias)
    if path == "route":
        scratch = torch.zeros(B.rl_route_scratch_bytes(d, T), dtype=torch.uint8, device="cuda")
        B.rl_route(d, 0, T, to_dev(x), to_dev(W), bd, to_dev(table), out.c(), scratch,
                   scratch.numel())
    else:
        pool = to_dev(np.stack([np.concatenate([synth.random_tensor(rng, H * F, 2)
                                                for _ in range(3)]) for _ in range(E)]))
        scratch = torch.zeros(B.rl_decode_scratch_bytes(d), dtype=torch.uint8, device="cuda")
        y = torch.empty(H, device="cuda")
        B.moe_decode_layer(d, 0, to_dev(x), to_dev(W), bd, to_dev(table), pool, out.c(),
                           scratch, scratch.numel(), y)
    r = O.route(x, W, bias, table[0], k)
    check_route(out, r)
    _same_bits(r.logits, want, "oracle logits")
    _same_bits(out.logits.cpu().numpy(), want, f"{path} logits T={T}")
