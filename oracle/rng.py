"""CPU oracle of the router's counter-based noise generator.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module.  Plain Python / NumPy;
it imports neither torch nor the GPU library and shares no code with it.

[P3] 三 (MoERouter.forward) adds, at training time, noise_std times a
standard normal draw to every router logit; the page draws it with
torch.randn_like and names no generator.  To draw the same numbers on the
GPU without a [T, N] tensor, the draws come from a counter-based generator:
Philox-4x32 with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3", SC 2011, section 4), and each pair of its
32-bit outputs becomes two normals by the Box-Muller transform (Box and
Muller, "A Note on the Generation of Random Normal Deviates", Ann. Math.
Statist. 29, 1958).

The stream (a reading of this library; the pages fix none of it):
  * normal number i of the stream (seed, offset) comes from Philox block
    b = i // 4 with counter words (b mod 2^32, b div 2^32, offset mod 2^32,
    offset div 2^32) and key words (seed mod 2^32, seed div 2^32);
  * the block's outputs (x0, x1, x2, x3) give normals 4b .. 4b+3 as the
    Box-Muller pairs (x0, x1) -> (r cos a, r sin a) and likewise (x2, x3),
    with u1 = (x_even + 1) / 2^32 in (0, 1], u2 = x_odd / 2^32 in [0, 1),
    r = sqrt(-2 ln u1), a = 2 pi u2;
  * these are evaluated in float64 and rounded once (to nearest even) to
    float32;
  * the router's noise for token t and expert e is normal number t*N + e.
"""
from __future__ import annotations

import numpy as np

# Philox-4x32 constants (Salmon et al. 2011): the two round multipliers and
# the two Weyl increments of the key schedule (golden ratio and sqrt(3) - 1
# in 0.32 fixed point).
M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
ROUNDS = 10
MASK = 0xFFFFFFFF


def philox4x32_block(ctr, key, rounds=ROUNDS):
    """One Philox-4x32 block in plain Python integers.

    Each round multiplies words 0 and 2 by the two multipliers (64-bit
    products split into high and low halves), and the new words are
    (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key
    advances by the Weyl increments between rounds."""
    c0, c1, c2, c3 = (int(v) & MASK for v in ctr)
    k0, k1 = (int(v) & MASK for v in key)
    for r in range(rounds):
        if r:
            k0 = (k0 + W0) & MASK
            k1 = (k1 + W1) & MASK
        p0 = M0 * c0
        p1 = M1 * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0), p1 & MASK, ((p0 >> 32) ^ c3 ^ k1), p0 & MASK
    return c0, c1, c2, c3


def philox4x32_blocks(blocks, offset, seed, rounds=ROUNDS):
    """The same generator vectorised over many block numbers: uint64 numpy
    arithmetic on arrays of the four counter words (a second, independent
    implementation of the round).  Returns uint32 [n, 4]."""
    b = np.asarray(blocks, dtype=np.uint64)
    m32 = np.uint64(MASK)
    c0 = b & m32
    c1 = b >> np.uint64(32)
    off = int(offset)
    c2 = np.full_like(c0, np.uint64(off & MASK))
    c3 = np.full_like(c0, np.uint64((off >> 32) & MASK))
    k0 = int(seed) & MASK
    k1 = (int(seed) >> 32) & MASK
    for r in range(rounds):
        if r:
            k0 = (k0 + W0) & MASK
            k1 = (k1 + W1) & MASK
        # products of two 32-bit values fit in uint64 exactly
        p0 = c0 * np.uint64(M0)
        p1 = c2 * np.uint64(M1)
        n0 = (p1 >> np.uint64(32)) ^ c1 ^ np.uint64(k0)
        n1 = p1 & m32
        n2 = (p0 >> np.uint64(32)) ^ c3 ^ np.uint64(k1)
        n3 = p0 & m32
        c0, c1, c2, c3 = n0, n1, n2, n3
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def box_muller(x_even, x_odd):
    """Two float64 normals from two uint32 words: u1 = (x_even + 1) / 2^32 in
    (0, 1] (never 0, so the logarithm is finite), u2 = x_odd / 2^32 in [0, 1);
    r = sqrt(-2 ln u1), a = 2 pi u2; returns (r cos a, r sin a)."""
    u1 = (np.asarray(x_even, np.float64) + 1.0) * 2.0 ** -32
    u2 = np.asarray(x_odd, np.float64) * 2.0 ** -32
    r = np.sqrt(-2.0 * np.log(u1))
    a = (2.0 * np.pi) * u2
    return r * np.cos(a), r * np.sin(a)


def normals(seed, offset, first, count):
    """Normals number first .. first+count-1 of the stream (seed, offset):
    (float32 values, the float64 values they were rounded from)."""
    if count <= 0:
        return np.zeros(0, np.float32), np.zeros(0)
    i = np.arange(first, first + count, dtype=np.int64)
    b0, b1 = int(i[0] // 4), int(i[-1] // 4)
    x = philox4x32_blocks(np.arange(b0, b1 + 1, dtype=np.uint64), offset, seed)
    z0, z1 = box_muller(x[:, 0], x[:, 1])
    z2, z3 = box_muller(x[:, 2], x[:, 3])
    z = np.stack([z0, z1, z2, z3], axis=-1).reshape(-1)
    z64 = z[i - 4 * b0]
    return z64.astype(np.float32), z64


def router_noise(seed, offset, T, N):
    """The router's standard-normal draws [T, N] (float32): token t, expert e
    takes normal number t*N + e of the stream (seed, offset)."""
    z32, _ = normals(seed, offset, 0, int(T) * int(N))
    return z32.reshape(int(T), int(N))
