"""Block-format tensors written from explicit fields (codes, group scales,
block scales), byte by byte at the positions the format defines, and the
exact rational weight of a field combination.  Used by the oracle pins and
by the GPU tests that need weights of a chosen structure; independent of
the package's generator and of the oracle's decoder."""
from fractions import Fraction

import numpy as np


def pack_tensor(codes, scales, d, qbits):
    """Write a block-format tensor from explicit fields, byte by byte, at the
    positions the format defines (independent of every other packer)."""
    codes = np.asarray(codes, np.int64).reshape(-1)
    nb = codes.size // 256
    up = lambda n: -(-n // 256) * 256
    q_end = nb * 64
    hb_off = up(q_end) if qbits == 3 else None
    s_off = up(hb_off + nb * 32) if qbits == 3 else up(q_end)
    d_off = up(s_off + nb * 4)
    buf = np.zeros(up(d_off + nb * 2), np.uint8)
    for f, c in enumerate(codes):
        b, j = divmod(f, 256)
        buf[64 * b + j // 4] |= (int(c) & 3) << (2 * (j % 4))
        if qbits == 3:
            buf[hb_off + 32 * b + j // 8] |= ((int(c) >> 2) & 1) << (j % 8)
    scales = np.asarray(scales, np.int64).reshape(nb, 8)
    for b in range(nb):
        for g in range(8):
            buf[s_off + 4 * b + g // 2] |= int(scales[b, g]) << (4 * (g % 2))
    dh = np.asarray(d, np.float16).reshape(nb)
    buf[d_off:d_off + 2 * nb] = dh.view(np.uint8)
    return buf


def exact_weight(c, s, d, qbits):
    if qbits == 2:
        return Fraction(d) * (2 * s + 1) * (2 * c - 3) / 32
    return Fraction(d) * (2 * s + 1) * (2 * c - 7) / 64


def pack_tensor_fast(codes, scales, d, qbits):
    """pack_tensor with whole-array operations, for large tensors: same bytes."""
    codes = np.asarray(codes, np.int64).reshape(-1)
    nb = codes.size // 256
    up = lambda n: -(-n // 256) * 256
    q_end = nb * 64
    hb_off = up(q_end) if qbits == 3 else None
    s_off = up(hb_off + nb * 32) if qbits == 3 else up(q_end)
    d_off = up(s_off + nb * 4)
    buf = np.zeros(up(d_off + nb * 2), np.uint8)
    c4 = (codes & 3).reshape(nb * 64, 4)                  # four 2-bit fields per byte
    buf[:q_end] = (c4 << (2 * np.arange(4))).sum(axis=1).astype(np.uint8)
    if qbits == 3:
        b8 = ((codes >> 2) & 1).reshape(nb * 32, 8)       # eight third bits per byte
        buf[hb_off:hb_off + nb * 32] = (b8 << np.arange(8)).sum(axis=1).astype(np.uint8)
    s2 = np.asarray(scales, np.int64).reshape(nb * 4, 2)  # two 4-bit group scales per byte
    buf[s_off:s_off + nb * 4] = (s2[:, 0] | (s2[:, 1] << 4)).astype(np.uint8)
    buf[d_off:d_off + 2 * nb] = np.asarray(d, np.float16).reshape(nb).view(np.uint8)
    return buf
