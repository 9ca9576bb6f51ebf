"""Pins of the noise generator's oracle (oracle/rng.py), CPU only.

  * Philox-4x32-10 against the published known-answer vectors
    (tests/golden/philox4x32_10_kat.json), for both implementations of the
    round (plain Python integers; vectorised uint64 NumPy);
  * the two implementations against each other on random 64-bit seeds,
    offsets and block numbers;
  * the Box-Muller normals against the standard normal distribution
    (Kolmogorov-Smirnov with scipy, moments, pairwise correlation), and
    its special points (u1 = 1 gives 0; a = 0 gives (r, 0));
  * the stream layout: normal i in block i // 4, word i % 4; offsets select
    disjoint streams.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.stats

from oracle import rng

GOLD = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")


def kat_cases():
    return json.load(open(GOLD))["cases"]


@pytest.mark.parametrize("case", kat_cases(), ids=["zeros", "ones", "pi"])
def test_philox_known_answers(case):
    ctr = [int(v, 16) for v in case["ctr"]]
    key = [int(v, 16) for v in case["key"]]
    want = [int(v, 16) for v in case["out"]]
    assert list(rng.philox4x32_block(ctr, key)) == want
    # the vectorised route takes the block number (c0, c1) and the offset
    # (c2, c3) and seed (k0, k1) as 64-bit integers
    b = ctr[0] | (ctr[1] << 32)
    off = ctr[2] | (ctr[3] << 32)
    seed = key[0] | (key[1] << 32)
    got = rng.philox4x32_blocks(np.array([b], dtype=np.uint64), off, seed)[0]
    assert [int(v) for v in got] == want


def test_two_implementations_agree():
    r = np.random.default_rng(5)
    for _ in range(200):
        seed = int(r.integers(0, 2 ** 63)) * 2 + int(r.integers(0, 2))
        off = int(r.integers(0, 2 ** 63)) * 2 + int(r.integers(0, 2))
        blocks = r.integers(0, 2 ** 63, size=7, dtype=np.uint64)
        vec = rng.philox4x32_blocks(blocks, off, seed)
        for b, row in zip(blocks, vec):
            b = int(b)
            ref = rng.philox4x32_block([b & 0xFFFFFFFF, b >> 32, off & 0xFFFFFFFF, off >> 32],
                                       [seed & 0xFFFFFFFF, seed >> 32])
            assert tuple(int(v) for v in row) == ref


def test_normals_are_standard_normal():
    z32, z64 = rng.normals(seed=1234, offset=7, first=0, count=1 << 20)
    assert z32.dtype == np.float32 and np.array_equal(z32, z64.astype(np.float32))
    n = z64.size
    assert abs(z64.mean()) < 5.0 / math.sqrt(n)
    assert abs(z64.var() - 1.0) < 5.0 * math.sqrt(2.0 / n)
    assert abs(np.mean(z64 ** 4) - 3.0) < 5.0 * math.sqrt(96.0 / n)
    ks = scipy.stats.kstest(z64, "norm")
    assert ks.pvalue > 1e-3, ks
    # the two normals of a Box-Muller pair, and neighbouring pairs, are
    # uncorrelated
    for lag in (1, 2, 4):
        c = np.corrcoef(z64[:-lag], z64[lag:])[0, 1]
        assert abs(c) < 5.0 / math.sqrt(n), (lag, c)


def test_box_muller_special_points():
    # u1 = 1 (x_even = 2^32 - 1): r = 0, both normals 0
    z0, z1 = rng.box_muller(np.array([0xFFFFFFFF]), np.array([12345]))
    assert z0[0] == 0.0 and z1[0] == 0.0
    # u2 = 0: angle 0, so (r, 0) with r = sqrt(-2 ln u1); u1 = 1/2 -> sqrt(2 ln 2)
    z0, z1 = rng.box_muller(np.array([0x7FFFFFFF]), np.array([0]))
    assert abs(z0[0] - math.sqrt(2.0 * math.log(2.0))) < 1e-15 and z1[0] == 0.0
    # the smallest u1 = 2^-32 bounds every draw: |z| <= sqrt(64 ln 2) ~ 6.66
    z0, _ = rng.box_muller(np.array([0]), np.array([0]))
    assert abs(z0[0] - math.sqrt(64.0 * math.log(2.0))) < 1e-14


def test_stream_layout():
    seed, off = 99, 3
    z, _ = rng.normals(seed, off, 0, 40)
    x = rng.philox4x32_blocks(np.arange(10, dtype=np.uint64), off, seed)
    a0, a1 = rng.box_muller(x[:, 0], x[:, 1])
    a2, a3 = rng.box_muller(x[:, 2], x[:, 3])
    want = np.stack([a0, a1, a2, a3], axis=-1).reshape(-1).astype(np.float32)
    assert np.array_equal(z, want)
    # any window of the stream is the same numbers
    w, _ = rng.normals(seed, off, 13, 17)
    assert np.array_equal(w, z[13:30])
    # router noise: token t, expert e is number t*N + e
    T, N = 5, 7
    rn = rng.router_noise(seed, off, T, N)
    assert rn.shape == (T, N) and np.array_equal(rn.reshape(-1), z[:T * N])
    # another offset or seed is another stream
    assert not np.any(rng.normals(seed, off + 1, 0, 40)[0] == z)
    assert not np.any(rng.normals(seed + 1, off, 0, 40)[0] == z)
