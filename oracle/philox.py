"""Philox4x32-10 counter-based generator and the dropout keep-mask built on it.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The generator is the published one: J. K. Salmon, M. A. Moraes, R. O. Dror,
D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11), section
"Philox": a 4 x 32-bit counter and a 2 x 32-bit key; ten rounds, each
multiplying counter words 0 and 2 by the constants below into 64-bit
products and recombining the halves with the other words and the key; the
key is bumped by two Weyl constants between rounds.  Written here in numpy
from that description, vectorised over counters.

The pages only show dropout switched off (TE-2448 "Steps/Code to reproduce
bug": ``dropout=0.0``, an ``rng`` state tensor); the mask layout below is
this implementation's own specification, shared with the HIP kernels by
definition only (no code):

* one generator call per sequence b, query head h and 4 x 4 block of
  (query i, key j) positions of the sequence: counter
  (j >> 2, i >> 2, b, offset * hq + h), key (seed_lo, seed_hi);
* its four output words x0..x3 give 16 bytes; element (i, j) takes byte
  (j & 3) of word x[i & 3] (byte k of a word = bits 8k..8k+7);
* the element is kept iff that byte >= t, t = round(256 p) in [0, 255]: the
  dropout probability is t / 256 and kept elements are scaled by
  256 / (256 - t).
"""
from __future__ import annotations

import numpy as np

__all__ = ["philox4x32_10", "dropout_threshold", "keep_mask"]

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = np.uint32(0x9E3779B9)
W1 = np.uint32(0xBB67AE85)
MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key):
    """ctr: uint32 [..., 4]; key: uint32 [..., 2] (broadcast).  Returns uint32 [..., 4]."""
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    c0, c1, c2, c3 = (c[..., n].astype(np.uint64) for n in range(4))
    k0, k1 = k[..., 0].astype(np.uint32), k[..., 1].astype(np.uint32)
    with np.errstate(over="ignore"):
        for rnd in range(10):
            if rnd:
                k0 = (k0 + W0).astype(np.uint32)
                k1 = (k1 + W1).astype(np.uint32)
            p0 = M0 * c0                      # exact 64-bit products of 32-bit words
            p1 = M1 * c2
            hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
            hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
            c0, c1, c2, c3 = (hi1 ^ c1 ^ k0.astype(np.uint64), lo1,
                              hi0 ^ c3 ^ k1.astype(np.uint64), lo0)
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def dropout_threshold(p: float) -> int:
    """Byte threshold t = round(256 p) for a dropout probability p in [0, 255.5/256)."""
    if not (0.0 <= p < 255.5 / 256.0):
        raise ValueError("dropout probability must be in [0, 255.5/256)")
    return int(np.floor(256.0 * p + 0.5))


def keep_mask(lq: int, lk: int, b: int, h: int, hq: int, seed: int, offset: int, t: int):
    """Boolean [lq, lk]: element (i, j) of sequence b, query head h is kept."""
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    ctr = np.stack(np.broadcast_arrays((j >> 2).astype(np.uint32), (i >> 2).astype(np.uint32),
                                       np.uint32(b & 0xFFFFFFFF),
                                       np.uint32((offset * hq + h) & 0xFFFFFFFF)), axis=-1)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint32)
    words = philox4x32_10(ctr, key)                       # [lq, lk, 4]
    word = np.take_along_axis(words, (i & 3)[..., None].repeat(lk, axis=1), axis=-1)[..., 0]
    byte = (word >> (8 * (j & 3)).astype(np.uint32)) & np.uint32(0xFF)
    return byte >= t
