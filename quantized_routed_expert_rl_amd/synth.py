"""Seeded synthetic inputs: router weights, activations, block-format expert
bytes, residency tables.

This module draws random numbers and places them in buffers.  It holds none
of the MoE layer's arithmetic (no dequantisation, no dot products, no
selection).  Both sides of every parity check take their inputs from here:
the HIP library through the Python binding, and the CPU oracle through the
tests.

Streams.  Every tensor has its own NumPy PCG64 stream seeded with
``SeedSequence([seed, workload_id, tensor_kind, layer, index])`` so that any
expert of any layer can be regenerated on its own, without building the
whole pool on the host.

Block format planes.  An expert tensor of ``n`` elements (row-major,
flattened) is cut into ``n/256`` blocks.  Its bytes hold four planes, each
starting at a 256-byte aligned offset, in this order:

    Q   n/256 * 64 bytes   low two bits of every code, four codes per byte
    Hb  n/256 * 32 bytes   third code bit, eight codes per byte (3-bit only)
    S   n/256 *  4 bytes   eight 4-bit group scales per block
    D   n/256 *  2 bytes   one IEEE binary16 block scale per block

and the tensor's size is rounded up to a multiple of 256 bytes.  An expert
slot is the gate [F x H], up [F x H] and down [H x F] tensors back to back.
Uniform random bytes in Q, Hb and S make every code and every group scale
uniform; D holds d ~ U(0.01, 0.05) drawn in float64 and rounded to binary16.
"""
from __future__ import annotations

import numpy as np

from .workloads import Workload

# tensor kinds (third word of every seed)
K_ROUTER, K_BIAS, K_EXPERT, K_X, K_RESIDENCY = 1, 2, 3, 4, 5


def _rng(seed, wid, kind, layer=0, index=0) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([seed, wid, kind, layer, index])))


def _align(n: int, a: int = 256) -> int:
    return (n + a - 1) // a * a


def plane_offsets(n_elems: int, qbits: int) -> dict:
    """Byte offsets of the Q, Hb, S and D planes and the tensor's total size."""
    if n_elems % 256:
        raise ValueError("tensor size must be a multiple of 256 elements")
    nb = n_elems // 256
    q = 0
    off = _align(nb * 64)
    hb = None
    if qbits == 3:
        hb = off
        off = _align(off + nb * 32)
    s = off
    off = _align(off + nb * 4)
    d = off
    off = _align(off + nb * 2)
    return {"nb": nb, "q": q, "hb": hb, "s": s, "d": d, "total": off}


def tensor_nbytes(n_elems: int, qbits: int) -> int:
    return plane_offsets(n_elems, qbits)["total"]


def slot_nbytes(hidden: int, width: int, qbits: int) -> int:
    return 3 * tensor_nbytes(hidden * width, qbits)


def _random_bytes(rng: np.random.Generator, n: int) -> np.ndarray:
    """n uniform random bytes (whole 64-bit draws, the fastest numpy path)."""
    words = rng.integers(0, 2**64 - 1, (n + 7) // 8, dtype=np.uint64, endpoint=True)
    return words.view(np.uint8)[:n]


def random_tensor(rng: np.random.Generator, n_elems: int, qbits: int,
                  d_low: float = 0.01, d_high: float = 0.05, out: np.ndarray = None) -> np.ndarray:
    """One block-format tensor of random codes and group scales, with block
    scales d ~ U(d_low, d_high) rounded to float16; written into ``out``
    (tensor_nbytes long) when given.  Padding between planes is zero."""
    lay = plane_offsets(n_elems, qbits)
    nb = lay["nb"]
    buf = np.zeros(lay["total"], np.uint8) if out is None else out
    if out is not None:
        buf[:] = 0
    buf[lay["q"]:lay["q"] + nb * 64] = _random_bytes(rng, nb * 64)
    if qbits == 3:
        buf[lay["hb"]:lay["hb"] + nb * 32] = _random_bytes(rng, nb * 32)
    buf[lay["s"]:lay["s"] + nb * 4] = _random_bytes(rng, nb * 4)
    d = rng.uniform(d_low, d_high, nb).astype(np.float16)
    buf[lay["d"]:lay["d"] + nb * 2] = d.view(np.uint8)
    return buf


def expert_slot(w: Workload, layer: int, expert: int, seed: int = 0,
                out: np.ndarray = None) -> np.ndarray:
    """Bytes of one expert slot (gate, up, down) of ``layer``/``expert``,
    written into ``out`` (slot_nbytes long) when given."""
    rng = _rng(seed, w.wid, K_EXPERT, layer, expert)
    n = w.hidden * w.width
    tb = tensor_nbytes(n, w.qbits)
    buf = np.empty(3 * tb, np.uint8) if out is None else out
    for i in range(3):
        random_tensor(rng, n, w.qbits, out=buf[i * tb:(i + 1) * tb])
    return buf


def router_weights(w: Workload, layer: int, seed: int = 0) -> np.ndarray:
    """Router matrix [E x H], float32 entries N(0, 0.05)."""
    rng = _rng(seed, w.wid, K_ROUTER, layer)
    return (rng.standard_normal((w.n_experts, w.hidden)) * 0.05).astype(np.float32)


def router_bias(w: Workload, layer: int, seed: int = 0):
    """Per-expert Zipf(1.1) bias, or None when the workload has no skew.

    A seeded permutation assigns each expert a popularity rank rho in 1..E and
    the bias is -1.1 * ln(rho), so the softmax prior of an expert is
    proportional to rho**-1.1.
    """
    if not w.zipf:
        return None
    rng = _rng(seed, w.wid, K_BIAS, layer)
    rank = rng.permutation(w.n_experts) + 1
    return (-1.1 * np.log(rank.astype(np.float64))).astype(np.float32)


def activations(w: Workload, n_tokens: int, stream: int = 0, seed: int = 0) -> np.ndarray:
    """[n_tokens x H] float32 activations N(0, 1)."""
    rng = _rng(seed, w.wid, K_X, 0, stream)
    return rng.standard_normal((n_tokens, w.hidden)).astype(np.float32)


def residency(w: Workload, seed: int = 0) -> np.ndarray:
    """[L x E] int32 table of slot indices, -1 where an expert is not resident.

    All-resident workloads place the L*E experts at a random permutation of
    the slots.  A workload with ``resident`` = R picks R (layer, expert)
    entries uniformly without replacement and gives them a random permutation
    of slots 0..R-1; with ``popular`` it picks each layer's R/L most popular
    experts instead (lowest Zipf rank, the ranks ``router_bias`` uses).
    """
    rng = _rng(seed, w.wid, K_RESIDENCY)
    n = w.n_layers * w.n_experts
    if w.resident < 0:
        table = rng.permutation(n).astype(np.int32)
    elif w.popular:
        per = w.resident // w.n_layers
        chosen = []
        for layer in range(w.n_layers):
            rank = _rng(seed, w.wid, K_BIAS, layer).permutation(w.n_experts) + 1
            chosen.append(layer * w.n_experts + np.nonzero(rank <= per)[0])
        chosen = np.concatenate(chosen)
        table = np.full(n, -1, np.int32)
        table[chosen] = rng.permutation(chosen.size).astype(np.int32)
    else:
        table = np.full(n, -1, np.int32)
        chosen = rng.choice(n, size=w.resident, replace=False)
        table[chosen] = rng.permutation(w.resident).astype(np.int32)
    return table.reshape(w.n_layers, w.n_experts)


def n_slots(table: np.ndarray) -> int:
    return int(table.max()) + 1 if table.size else 0


def build_pool(w: Workload, table: np.ndarray, seed: int = 0) -> np.ndarray:
    """Host slot pool [n_slots x slot_bytes] for every resident expert.

    Only for pools that fit comfortably in host memory; the stacked
    workloads fill the device pool in pieces with ``fill_slots``.
    """
    sb = slot_nbytes(w.hidden, w.width, w.qbits)
    pool = np.zeros((n_slots(table), sb), np.uint8)
    for layer, expert in zip(*np.nonzero(table >= 0)):
        pool[table[layer, expert]] = expert_slot(w, int(layer), int(expert), seed)
    return pool


def fill_slots(w: Workload, table: np.ndarray, start: int, count: int,
               seed: int = 0, out: np.ndarray = None) -> np.ndarray:
    """Bytes of slots [start, start+count) as a [count x slot_bytes] array,
    written into ``out`` (at least count rows) when given: reusing one
    buffer keeps page faults out of large pools."""
    sb = slot_nbytes(w.hidden, w.width, w.qbits)
    if out is None:
        out = np.zeros((count, sb), np.uint8)
    else:
        out = out[:count]
        out[:] = 0
    flat = table.ravel()
    E = table.shape[1]
    held = np.nonzero((flat >= start) & (flat < start + count))[0]
    for i in held:
        expert_slot(w, int(i) // E, int(i) % E, seed, out=out[int(flat[i]) - start])
    return out
