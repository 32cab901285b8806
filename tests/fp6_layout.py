"""Host-side FP6 tiled layout of int4 codes, written from its definition in
include/svdq.h (the precision enum): per row and group of 64, two 192-bit
strings, one per half h of the group; field j (bits 6j .. 6j+5) is the E2M3
encoding of q/2 for channel 64g + 32h + j; the group is three 16-byte chunks
[h0 words 0-3 | h1 words 0-3 | h0 words 4-5, h1 words 4-5], the two halves of
the last chunk swapped when s(r) = 1; with p = r % 128,
rot(r) = ((p >> 2) xor (p >> 3)) & 1 and s(r) = ((p >> 3) xor (p >> 4)) & 1,
chunk c of group g of row r sits at
  ((r / 128) * ceil(K/128) + g / 2) * 12288 + p * 96
    + 16 * ((3 * (g % 2) + c + rot(r)) mod 6).

E2M3 (the OCP microscaling FP6 format): sign bit 5, exponent bits 3-4 with
bias 1, mantissa bits 0-2; exponent 0 encodes the subnormals m/8, exponent
e > 0 the value 2^(e-1) * (1 + m/8).  This module is test infrastructure:
the tests compare the library's FP6 encoders (the activation step's and the
weight packer's) with it, and feed the FP6 GEMM from it.  Bytes the layout
leaves as padding are given a fill value (the GPU tests' 0xFF poison)."""
from __future__ import annotations

import numpy as np


def e2m3_value(f):
    """Value of 6-bit E2M3 codes (array of ints)."""
    f = np.asarray(f, np.int64)
    s = np.where(f & 32, -1.0, 1.0)
    e, m = (f >> 3) & 3, f & 7
    mag = np.where(e == 0, m / 8.0, np.ldexp(1.0 + m / 8.0, e - 1))
    return s * mag


def e2m3_encode(v):
    """E2M3 code of values that the format holds exactly (raises otherwise)."""
    v = np.asarray(v, np.float64)
    table = {float(e2m3_value(f)): f for f in range(64) if not (f == 32)}   # -0 -> +0
    out = np.empty(v.shape, np.int64)
    for idx, x in np.ndenumerate(v):
        if float(x) not in table:
            raise ValueError(f"{x} is not an E2M3 value")
        out[idx] = table[float(x)]
    return out


def _strings_to_block(fields):
    """fields [..., 2, 32] (half, field) -> 48 bytes per block [..., 48]."""
    lead = fields.shape[:-2]
    words = np.zeros(lead + (2, 6), np.uint64)
    for j in range(32):
        b = 6 * j
        f = fields[..., j].astype(np.uint64)
        w, o = b // 32, b % 32
        words[..., w] |= (f << np.uint64(o)) & np.uint64(0xFFFFFFFF)
        if o > 26:
            words[..., w + 1] |= f >> np.uint64(32 - o)
    words = words.astype(np.uint32)
    order = np.concatenate([words[..., 0, 0:4], words[..., 1, 0:4], words[..., 0, 4:6], words[..., 1, 4:6]],
                           axis=-1)
    return order.view(np.uint8).reshape(lead + (48,))


def fp6_codes_bytes(R, K):
    return -(-R // 128) * -(-K // 128) * 12288


def rot(r):
    p = r % 128
    return ((p >> 2) ^ (p >> 3)) & 1


def half_swap(r):
    p = r % 128
    return ((p >> 3) ^ (p >> 4)) & 1


def chunk_offset(r, g, c, K):
    """Byte offset of chunk c (0..2) of group g of row r (the documented formula)."""
    NP = -(-K // 128)
    slot = (3 * (g % 2) + c + rot(r)) % 6
    return ((r // 128) * NP + g // 2) * 12288 + (r % 128) * 96 + 16 * slot


def _swap_last_chunk(blocks, R):
    """Swap the two 8-byte halves of chunk 2 in the rows with s(r) = 1
    (blocks [R, NG, 48]; an involution)."""
    out = blocks.copy()
    rows = np.array([half_swap(r) for r in range(R)], bool)
    out[rows, :, 32:40] = blocks[rows, :, 40:48]
    out[rows, :, 40:48] = blocks[rows, :, 32:40]
    return out


def fp6_layout_from_q(q, fill=0xFF):
    """Integer codes q [R, K] in [-8, 7] -> the FP6 tiled layout (uint8, 1-D)."""
    q = np.asarray(q, np.int64)
    R, K = q.shape
    NG = K // 64
    blocks = _swap_last_chunk(_strings_to_block(e2m3_encode(q / 2.0).reshape(R, NG, 2, 32)), R)   # [R, NG, 48]
    out = np.full(fp6_codes_bytes(R, K), fill, np.uint8)
    r = np.arange(R)[:, None]
    g = np.arange(NG)[None, :]
    for c in range(3):
        off = np.vectorize(chunk_offset)(r, g, c, K)                              # [R, NG]
        idx = off[..., None] + np.arange(16)
        out[idx] = blocks[..., 16 * c:16 * c + 16]
    return out


def q_from_fp6_layout(b, R, K):
    """The FP6 tiled layout -> integer codes [R, K] (2 * the E2M3 values)."""
    b = np.asarray(b, np.uint8)
    NG = K // 64
    r = np.arange(R)[:, None]
    g = np.arange(NG)[None, :]
    blocks = np.empty((R, NG, 48), np.uint8)
    for c in range(3):
        off = np.vectorize(chunk_offset)(r, g, c, K)
        blocks[..., 16 * c:16 * c + 16] = b[off[..., None] + np.arange(16)]
    blocks = _swap_last_chunk(blocks, R)
    words = blocks.view(np.uint32).astype(np.uint64)                             # [R, NG, 12]
    halves = [np.concatenate([words[..., 0:4], words[..., 8:10]], axis=-1),
              np.concatenate([words[..., 4:8], words[..., 10:12]], axis=-1)]
    out = np.empty((R, NG, 2, 32), np.int64)
    for h, wd in enumerate(halves):
        for j in range(32):
            bit = 6 * j
            w, o = bit // 32, bit % 32
            v = wd[..., w] >> np.uint64(o)
            if o > 26:
                v |= wd[..., w + 1] << np.uint64(32 - o)
            out[..., h, j] = (v & np.uint64(63)).astype(np.int64)
    return (e2m3_value(out) * 2.0).reshape(R, K).astype(np.int64)


def nibbles_to_q(codes, K):
    c = np.asarray(codes, np.uint8)
    lo = (c & 15).astype(np.int64)
    hi = (c >> 4).astype(np.int64)
    q = np.empty((c.shape[0], K), np.int64)
    q[:, 0::2] = np.where(lo >= 8, lo - 16, lo)
    q[:, 1::2] = np.where(hi >= 8, hi - 16, hi)
    return q


def fp6_layout_from_nibbles(codes, K, fill=0xFF):
    """Packed two's-complement nibbles [R, K/2] -> the FP6 tiled layout."""
    return fp6_layout_from_q(nibbles_to_q(codes, K), fill)
