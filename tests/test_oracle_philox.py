"""Pins of the oracle's Philox4x64-10 against numpy's independent implementation."""
import numpy as np
import pytest

from oracle import philox

MASK = (1 << 64) - 1


def numpy_block(ctr, key):
    """Block at counter ``ctr`` from numpy.random.Philox.

    numpy increments its 256-bit counter before producing a block, so the
    block at counter c is the first block after setting the counter to c - 1.
    """
    c = 0
    for i, w in enumerate(ctr):
        c |= (int(w) & MASK) << (64 * i)
    c = (c - 1) % (1 << 256)
    words = np.array([(c >> (64 * i)) & MASK for i in range(4)], dtype=np.uint64)
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=words)
    return [int(v) for v in bg.random_raw(4)]


CASES = [
    ((0, 0, 0, 0), (0, 0)),
    ((1, 0, 0, 0), (0, 0)),
    ((7, 2, 3, 4), (123, 456)),
    ((MASK, 0, 0, 0), (1, 2)),             # carry into word 1 on numpy's side
    ((0, 2052, 0, 0), (0x5EED0003, 0)),
    ((65535, 2048, 7, 1), (0x5EED0005, 0)),
    ((MASK, MASK, MASK, MASK), (MASK, MASK)),
]


@pytest.mark.parametrize("ctr,key", CASES)
def test_scalar_matches_numpy(ctr, key):
    assert philox.philox4x64_10(ctr, key) == numpy_block(ctr, key)


def test_vectorised_matches_scalar():
    rng = np.random.default_rng(5)
    c = rng.integers(0, 2 ** 63, size=(4, 300), dtype=np.int64).astype(np.uint64) * np.uint64(2) + np.uint64(1)
    k = rng.integers(0, 2 ** 63, size=2, dtype=np.int64).astype(np.uint64)
    out = philox.philox4x64_10_np(c[0], c[1], c[2], c[3], k[0], k[1])
    for j in range(300):
        ref = philox.philox4x64_10([int(c[i, j]) for i in range(4)], [int(k[0]), int(k[1])])
        assert [int(out[i][j]) for i in range(4)] == ref


def test_vectorised_random_against_numpy():
    rng = np.random.default_rng(6)
    for _ in range(50):
        ctr = [int(x) for x in rng.integers(0, 2 ** 62, size=4)]
        key = [int(x) for x in rng.integers(0, 2 ** 62, size=2)]
        out = philox.philox4x64_10_np(*ctr, *key)
        assert [int(o) for o in out] == numpy_block(ctr, key)


def test_uniform_grids():
    u = philox.accept_uniform(99, np.arange(1000), 17)
    assert np.all((u >= 0) & (u < 1))
    assert np.all(u * 2 ** 24 == np.floor(u * 2 ** 24))
    assert np.all(u.astype(np.float32).astype(np.float64) == u)
    g = philox.gumbel_uniform(99, 3, 17, np.arange(4096))
    assert np.all((g > 0) & (g < 1))
    assert np.all(g.astype(np.float32).astype(np.float64) == g)
    # the word layout: vocab entry v is word v & 3 of block v >> 2
    w = philox.philox4x64_10((5, 17, 3, philox.TAG_GUMBEL), (99, 0))
    for j in range(4):
        assert g[20 + j] == ((w[j] >> 41) + 0.5) * 2.0 ** -23
    w0 = philox.philox4x64_10((0, 17, 4, philox.TAG_ACCEPT), (99, 0))[0]
    assert u[4] == (w0 >> 40) * 2.0 ** -24


def test_uniformity():
    u = philox.accept_uniform(1, np.arange(200000), 3)
    hist, _ = np.histogram(u, bins=20, range=(0, 1))
    exp = len(u) / 20
    chi2 = ((hist - exp) ** 2 / exp).sum()
    assert chi2 < 50  # 19 dof; p ~ 1e-4


def test_gumbel_rows_match_elementwise():
    seq = np.array([0, 5, 1 << 40])
    pos = np.array([3, 2048, 77])
    rows = philox.gumbel_uniform_rows(11, seq, pos, 13)
    ref = philox.gumbel_uniform(11, seq[:, None], pos[:, None], np.arange(13)[None, :])
    assert np.array_equal(rows, ref)
