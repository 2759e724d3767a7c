"""CPU oracle of the routed mixture-of-experts FFN -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64.  The HIP library is checked against this module; the
library never calls it.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with
the HIP path and imports nothing from the library package: callers hand it
NumPy arrays (activations, router weights, residency rows) and a function that
returns one expert slot's bytes.

Sources, the four Red Lite development notes:
  [dev21] "Red Lite dev21 - GPU-routed decode (full residency)",
          section "What changed" (router selection rule, renormalised
          weights, residency table, slot table, per-layer miss count).
  [dev23] "Red Lite dev23 - per-layer early-out and pre-gated expert
          prefetch", section "What changed" (early-out flag: a set flag makes
          every later kernel of the layer return at once).
  [dev20] "Red Lite dev20 - batched prompt ingestion", section "What
          changed" (chunks, bounded plans of at most 512 distinct experts,
          consecutive token groups past the cap, (expert, token) pairs sorted
          by expert, per-token sum in router selection order).
  [dev38] "Red Lite dev38 - decode: expert down-projection lanes", section
          "Finding" (down projection = 2048 rows of 512 columns per expert).

Block format (the workload's 2- and 3-bit expert weight format).  A tensor's
elements, row-major and flattened, form blocks of 256 values; a block holds one
binary16 scale d, eight 4-bit group scales s (one per 32 values) and one code
per value.  The 2-bit code c maps to the level c - 1.5, i.e. {-1.5, -0.5, 0.5,
1.5}; the 3-bit code maps to (c - 3.5)/2, eight evenly spaced levels in
[-1.75, 1.75].  Weight = d * (2s+1)/16 * level.  Byte planes (each 256-byte
aligned, in this order): Q (2 low code bits, element j of block b at byte
64b + j//4, bits 2(j%4)..2(j%4)+1), Hb (3-bit only: bit 2 of the code at byte
32b + j//8, bit j%8), S (group g of block b at byte 4b + g//2, low nibble when
g is even), D (binary16, little endian, at byte 2b).  A slot is the gate
[F x H], up [F x H] and down [H x F] tensors back to back.

Readings the notes leave open (each one also listed in the design notes):
  * router dot products accumulate in float64 and round once to float32;
  * selection compares float32 logits (so -0 == +0), ties to the lower index;
  * renormalised weights = softmax over the k selected logits;
  * residency entries are slot indices, -1 = not resident;
  * one miss count and one flag per call; a flagged call produces no output;
  * SwiGLU: h = silu(g) * u with silu(g) = g / (1 + exp(-g));
  * an expert's contribution is w_r * (W_down h_r), summed in rank order;
  * float32 rounding at the storage points h, e_r and y, float64 elsewhere.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Callable, List, Optional

import numpy as np

F32, F64 = np.float32, np.float64


# --------------------------------------------------------------------------
# Block format
# --------------------------------------------------------------------------
def block_layout(n_elems: int, qbits: int) -> dict:
    """Offsets of the Q, Hb, S, D planes of a tensor of ``n_elems`` values."""
    assert n_elems % 256 == 0 and qbits in (2, 3)
    nb = n_elems // 256

    def up256(n):
        return -(-n // 256) * 256

    q_off = 0
    end = nb * 64
    hb_off = None
    if qbits == 3:
        hb_off = up256(end)
        end = hb_off + nb * 32
    s_off = up256(end)
    d_off = up256(s_off + nb * 4)
    total = up256(d_off + nb * 2)
    return {"nb": nb, "q": q_off, "hb": hb_off, "s": s_off, "d": d_off,
            "total": total}


def dequantize(buf: np.ndarray, n_elems: int, qbits: int) -> np.ndarray:
    """All ``n_elems`` weights of one block-format tensor, as float64."""
    lay = block_layout(n_elems, qbits)
    nb = lay["nb"]
    j = np.arange(256)                      # element index inside a block
    q = buf[lay["q"]:lay["q"] + nb * 64].reshape(nb, 64).astype(np.int64)
    code = (q[:, j // 4] >> (2 * (j % 4))) & 3
    if qbits == 3:
        hb = buf[lay["hb"]:lay["hb"] + nb * 32].reshape(nb, 32).astype(np.int64)
        code = code | (((hb[:, j // 8] >> (j % 8)) & 1) << 2)
        level = (code - 3.5) / 2.0
    else:
        level = code - 1.5
    g = j // 32                             # group of each element
    sb = buf[lay["s"]:lay["s"] + nb * 4].reshape(nb, 4).astype(np.int64)
    s = (sb[:, g // 2] >> (4 * (g % 2))) & 15
    d = buf[lay["d"]:lay["d"] + nb * 2].copy().view("<f2").astype(F64)
    w = d[:, None] * ((2 * s + 1) / 16.0) * level
    return w.reshape(-1)


def slot_bytes(hidden: int, width: int, qbits: int) -> int:
    return 3 * block_layout(hidden * width, qbits)["total"]


def expert_matrices(slot: np.ndarray, hidden: int, width: int, qbits: int):
    """(W_gate [F x H], W_up [F x H], W_down [H x F]) of one slot, float64."""
    n = hidden * width
    tb = block_layout(n, qbits)["total"]
    wg = dequantize(slot[0:tb], n, qbits).reshape(width, hidden)
    wu = dequantize(slot[tb:2 * tb], n, qbits).reshape(width, hidden)
    wd = dequantize(slot[2 * tb:3 * tb], n, qbits).reshape(hidden, width)
    return wg, wu, wd


# --------------------------------------------------------------------------
# Routing: router GEMV, softmax top-k, renormalisation, residency lookup
# --------------------------------------------------------------------------
def router_logits(x: np.ndarray, w_router: np.ndarray,
                  bias: Optional[np.ndarray]) -> np.ndarray:
    """logit[t, e] = fl32(sum_i W[e, i] x[t, i] + b[e]), summed in float64.

    The router is a float32 GEMV in the notes ([dev23] "What changed", the
    pre-gate router); every float32 product is exact in float64, so the only
    rounding that matters is the final one to float32.
    """
    acc = np.atleast_2d(x).astype(F64) @ w_router.astype(F64).T
    if bias is not None:
        acc = acc + bias.astype(F64)[None, :]
    return acc.astype(F32)


def select_experts(logits_row: np.ndarray, k: int) -> List[int]:
    """The k experts taken in router order: largest logit first, ties to the
    lower expert index ([dev21] "What changed").  Softmax is monotone, so the
    order by probability is the same as the order by logit.

    Taken one at a time: at each step the best remaining candidate, compared
    as float32 values (so -0 and +0 are equal); argmax returns the first
    maximum, i.e. the lower index.  Logits must be finite.
    """
    vals = logits_row.astype(F64)
    taken = np.zeros(vals.shape[0], bool)
    ids = []
    for _ in range(k):
        cand = np.where(taken, -np.inf, vals)
        e = int(np.argmax(cand))
        ids.append(e)
        taken[e] = True
    return ids


def renormalized_weights(logits_row: np.ndarray, ids: List[int]) -> np.ndarray:
    """Softmax weights renormalised over the selected experts ([dev21]).

    a_r = exp(l_r - l_0) with l_0 the top logit; w_r = fl32(a_r / sum_j a_j),
    the sum taken in rank order.  The full softmax denominator cancels.
    """
    l0 = float(logits_row[ids[0]])
    a = [math.exp(float(logits_row[e]) - l0) for e in ids]
    total = 0.0
    for v in a:
        total += v
    return np.array([v / total for v in a], dtype=F64).astype(F32)


def residency_lookup(ids: List[int], residency_row: np.ndarray):
    """Slots of the selected experts and the number that are not resident."""
    slots = [int(residency_row[e]) for e in ids]
    misses = sum(1 for s in slots if s == -1)
    return slots, misses


@dataclass
class Route:
    logits: np.ndarray      # [T, E] float32
    ids: np.ndarray         # [T, k] int32, rank order
    weights: np.ndarray     # [T, k] float32
    slots: np.ndarray       # [T, k] int32
    miss_count: int
    early_out: int


def route(x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray],
          residency_row: np.ndarray, k: int) -> Route:
    """Router, selection, renormalisation, lookup, miss count and flag for T
    tokens.  The flag is raised when any selected expert is not resident
    ([dev21] per-layer miss count; [dev23] early-out flag)."""
    logits = router_logits(x, w_router, bias)
    T = logits.shape[0]
    ids = np.zeros((T, k), np.int32)
    wts = np.zeros((T, k), F32)
    slots = np.zeros((T, k), np.int32)
    misses = 0
    for t in range(T):
        sel = select_experts(logits[t], k)
        ids[t] = sel
        wts[t] = renormalized_weights(logits[t], sel)
        sl, m = residency_lookup(sel, residency_row)
        slots[t] = sl
        misses += m
    return Route(logits, ids, wts, slots, misses, int(misses > 0))


# --------------------------------------------------------------------------
# Expert FFN and the ordered sum
# --------------------------------------------------------------------------
def silu(g: np.ndarray) -> np.ndarray:
    """SiLU g * sigmoid(g) = g / (1 + exp(-g)), float64."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def expert_forward(x_rows: np.ndarray, wg: np.ndarray, wu: np.ndarray,
                   wd: np.ndarray):
    """SwiGLU expert on token rows x [n x H]:
    h = fl32(silu(x Wg^T) * (x Wu^T)), e = fl32(h Wd^T).  Returns (h, e)."""
    xs = np.atleast_2d(x_rows).astype(F64)
    g = xs @ wg.T
    u = xs @ wu.T
    h = (silu(g) * u).astype(F32)
    e = (h.astype(F64) @ wd.T).astype(F32)
    return h, e


def ordered_sum(weights: np.ndarray, outs: List[np.ndarray]) -> np.ndarray:
    """y = fl32(sum_r w_r e_r) with r ascending: each token's experts are added
    in router selection order ([dev20] "What changed")."""
    acc = np.zeros(outs[0].shape, F64)
    for w, e in zip(weights, outs):
        acc = acc + F64(w) * e.astype(F64)
    return acc.astype(F32)


SlotReader = Callable[[int], np.ndarray]


@dataclass
class LayerShape:
    hidden: int
    n_experts: int
    top_k: int
    width: int
    qbits: int


def decode_layer(shape: LayerShape, x_row: np.ndarray, w_router, bias,
                 residency_row, read_slot: SlotReader):
    """One single-token decode step of the routed FFN.

    Returns (route, y, h): y [H] float32 and h [k, F] float32, or y = h =
    None when the early-out flag is raised (nothing downstream of the router
    runs, [dev23] "What changed").
    """
    r = route(np.atleast_2d(x_row), w_router, bias, residency_row, shape.top_k)
    if r.early_out:
        return r, None, None
    outs, hs = [], []
    for slot in r.slots[0]:
        wg, wu, wd = expert_matrices(read_slot(int(slot)), shape.hidden,
                                     shape.width, shape.qbits)
        h, e = expert_forward(x_row, wg, wu, wd)
        hs.append(h[0])
        outs.append(e[0])
    return r, ordered_sum(r.weights[0], outs), np.stack(hs)


# --------------------------------------------------------------------------
# Prefill: token groups, expert-sorted pairs, batched experts, per-token sum
# --------------------------------------------------------------------------
def token_groups(ids: np.ndarray, plan_cap: int) -> List[int]:
    """Boundaries of consecutive token groups whose selected experts' union
    stays within ``plan_cap`` ([dev20]: a chunk whose union exceeds the plan
    limit is split into consecutive token groups).  Greedy: a token joins the
    current group unless that would push the union past the cap."""
    bounds = [0]
    union = set()
    for t in range(ids.shape[0]):
        row = set(int(e) for e in ids[t])
        if t > bounds[-1] and len(union | row) > plan_cap:
            bounds.append(t)
            union = row
        else:
            union |= row
    bounds.append(ids.shape[0])
    return bounds


@dataclass
class Plan:
    group_bounds: np.ndarray        # [n_groups+1] token boundaries
    pairs: np.ndarray               # [T*k] pair ids p = t*k + r, sorted
    bucket_expert: np.ndarray       # [n_buckets] expert of each bucket
    bucket_start: np.ndarray        # [n_buckets+1] offsets into pairs
    group_bucket_start: np.ndarray  # [n_groups+1] first bucket of each group


def pair_plan(ids: np.ndarray, n_experts: int, plan_cap: int) -> Plan:
    """(expert, token) pairs sorted by expert, per token group ([dev20]).

    Within a group the pairs p = t*k + r are ordered by expert, then by p
    (a stable counting sort: histogram, exclusive scan, placement in input
    order).  Buckets are the group's distinct experts in ascending order.
    """
    T, k = ids.shape
    bounds = token_groups(ids, plan_cap)
    flat = ids.reshape(-1)
    pairs = np.zeros(T * k, np.int32)
    b_exp, b_start, g_start = [], [], []
    for g in range(len(bounds) - 1):
        p0, p1 = bounds[g] * k, bounds[g + 1] * k
        counts = [0] * n_experts
        for p in range(p0, p1):
            counts[int(flat[p])] += 1
        offset = [0] * n_experts
        run = p0
        g_start.append(len(b_exp))
        for e in range(n_experts):
            offset[e] = run
            if counts[e]:
                b_exp.append(e)
                b_start.append(run)
            run += counts[e]
        for p in range(p0, p1):
            e = int(flat[p])
            pairs[offset[e]] = p
            offset[e] += 1
    b_start.append(T * k)
    g_start.append(len(b_exp))
    return Plan(np.array(bounds, np.int32), pairs, np.array(b_exp, np.int32),
                np.array(b_start, np.int32), np.array(g_start, np.int32))


def prefill_chunk(shape: LayerShape, x: np.ndarray, w_router, bias,
                  residency_row, read_slot: SlotReader, plan_cap: int,
                  tokens: Optional[List[int]] = None, map_fn=map):
    """One prefill chunk of T tokens through the routed FFN ([dev20]).

    Returns (route, plan, y).  The chunk's flag is raised by any miss among
    its T*k selections; then plan and y are None.  ``tokens`` restricts y to
    a subset of rows (the others stay NaN) so that a large chunk can be
    checked on a sample; routing and the plan always cover the whole chunk.
    ``map_fn`` maps the evaluation over the buckets, which are independent of
    one another (the builtin map by default; a thread pool's map gives the
    same results sooner).
    """
    r = route(x, w_router, bias, residency_row, shape.top_k)
    if r.early_out:
        return r, None, None
    plan = pair_plan(r.ids, shape.n_experts, plan_cap)
    T, k = r.ids.shape
    want = set(range(T)) if tokens is None else set(tokens)

    def bucket_outputs(b):
        """(pair ids, expert outputs) of bucket b's wanted pairs."""
        ps = [int(p) for p in plan.pairs[plan.bucket_start[b]:plan.bucket_start[b + 1]]
              if int(p) // k in want]
        if not ps:
            return ps, None
        slot = int(r.slots[ps[0] // k, ps[0] % k])
        wg, wu, wd = expert_matrices(read_slot(slot), shape.hidden,
                                     shape.width, shape.qbits)
        _, e = expert_forward(x[[p // k for p in ps]], wg, wu, wd)
        return ps, e

    pair_out = {}
    for ps, e in map_fn(bucket_outputs, range(len(plan.bucket_expert))):
        for i, p in enumerate(ps):
            pair_out[p] = e[i]
    y = np.full((T, shape.hidden), np.nan, F32)
    for t in sorted(want):
        y[t] = ordered_sum(r.weights[t], [pair_out[t * k + q] for q in range(k)])
    return r, plan, y


# --------------------------------------------------------------------------
# Stacks of layers (bench and test harness only, not part of the MoE layer)
# --------------------------------------------------------------------------
def rmsnorm(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """Weightless RMSNorm x / sqrt(mean(x^2) + eps) per row, float64 -> f32."""
    xs = np.atleast_2d(x).astype(F64)
    return (xs / np.sqrt(np.mean(xs * xs, axis=1, keepdims=True) + eps)).astype(F32)


def residual_add(x: np.ndarray, y: Optional[np.ndarray]) -> np.ndarray:
    """x + y in float32 (one rounding); a flagged layer adds nothing."""
    if y is None:
        return x.copy()
    return (x.astype(F64) + y.astype(F64)).astype(F32)
