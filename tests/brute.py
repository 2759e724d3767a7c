"""Pure-Python brute force of the routed-expert layer for tiny shapes.

A second, independent computation used to pin the oracle: it walks the bytes
of each expert element by element with Python integers, sums dot products
with ``math.fsum`` (correctly rounded float64), ranks experts with a full
sort, and evaluates every expert densely before masking by the selection.
It shares no code with ``oracle/`` or with the library.
"""
from __future__ import annotations

import math
import struct

import numpy as np


def _f32(v: float) -> float:
    return struct.unpack("<f", struct.pack("<f", v))[0]


def _half(lo: int, hi: int) -> float:
    return struct.unpack("<e", bytes([lo, hi]))[0]


class Tensor:
    """Element access into one block-format tensor, decoding on demand."""

    def __init__(self, raw: bytes, n_elems: int, qbits: int):
        self.raw, self.n, self.qbits = raw, n_elems, qbits
        nb = n_elems // 256
        pos = nb * 64
        pos = (pos + 255) // 256 * 256
        if qbits == 3:
            self.hb = pos
            pos = (pos + nb * 32 + 255) // 256 * 256
        self.s = pos
        pos = (pos + nb * 4 + 255) // 256 * 256
        self.d = pos
        self.total = (pos + nb * 2 + 255) // 256 * 256

    def weight(self, flat: int) -> float:
        b, j = divmod(flat, 256)
        code = (self.raw[64 * b + j // 4] >> ((j % 4) * 2)) & 0b11
        if self.qbits == 3:
            code += 4 * ((self.raw[self.hb + 32 * b + j // 8] >> (j % 8)) & 1)
            num = 2 * code - 7          # level (c - 3.5)/2 = (2c - 7)/4
            den = 4
        else:
            num = 2 * code - 3          # level c - 1.5 = (2c - 3)/2
            den = 2
        grp = j // 32
        sbyte = self.raw[self.s + 4 * b + grp // 2]
        s = (sbyte >> 4) if grp % 2 else (sbyte & 0xF)
        d = _half(self.raw[self.d + 2 * b], self.raw[self.d + 2 * b + 1])
        return d * (2 * s + 1) * num / (16 * den)


def expert(raw: bytes, hidden: int, width: int, qbits: int):
    n = hidden * width
    t0 = Tensor(raw, n, qbits)
    tb = t0.total
    return (t0, Tensor(raw[tb:], n, qbits), Tensor(raw[2 * tb:], n, qbits))


def layer(x, w_router, bias, residency_row, slots_raw, hidden, n_experts, k,
          width, qbits):
    """Brute force of one MoE layer on token rows ``x``.

    Returns a dict with logits, ids, weights, slots, miss and, when no
    selected expert is missing, y.
    """
    T = len(x)
    logits = []
    for t in range(T):
        row = []
        for e in range(n_experts):
            terms = [float(w_router[e][i]) * float(x[t][i]) for i in range(hidden)]
            if bias is not None:
                terms.append(float(bias[e]))
            row.append(_f32(math.fsum(terms)))
        logits.append(row)
    ids = []
    for t in range(T):
        order = sorted(range(n_experts), key=lambda e: (-logits[t][e], e))
        ids.append(order[:k])
    weights = []
    for t in range(T):
        top = logits[t][ids[t][0]]
        a = [math.exp(logits[t][e] - top) for e in ids[t]]
        z = 0.0
        for v in a:
            z += v
        weights.append([_f32(v / z) for v in a])
    slots = [[int(residency_row[e]) for e in ids[t]] for t in range(T)]
    miss = sum(1 for t in range(T) for s in slots[t] if s < 0)
    out = {"logits": logits, "ids": ids, "weights": weights, "slots": slots,
           "miss": miss}
    if miss:
        return out
    # Dense evaluation: every expert on every token, masked afterwards.
    dense = {}
    for e in range(n_experts):
        if residency_row[e] < 0:
            continue
        tens = expert(slots_raw(int(residency_row[e])), hidden, width, qbits)
        gate, up, down = ([tn.weight(f) for f in range(hidden * width)] for tn in tens)
        for t in range(T):
            xt = [float(v) for v in x[t]]
            h = []
            for j in range(width):
                g = math.fsum(gate[j * hidden + i] * xt[i] for i in range(hidden))
                u = math.fsum(up[j * hidden + i] * xt[i] for i in range(hidden))
                h.append(_f32(g / (1.0 + math.exp(-g)) * u))
            dense[(e, t)] = [_f32(math.fsum(down[i * width + j] * h[j]
                                            for j in range(width)))
                             for i in range(hidden)]
    y = []
    for t in range(T):
        row = []
        for i in range(hidden):
            acc = 0.0
            for r, e in enumerate(ids[t]):
                acc += weights[t][r] * dense[(e, t)][i]
            row.append(_f32(acc))
        y.append(row)
    out["y"] = np.array(y, np.float32)
    return out
