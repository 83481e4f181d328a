"""Philox4x64-10 and the verify step's random stream (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Philox is the counter-based generator of Salmon, Moraes, Dror and Shaw,
"Parallel random numbers: as easy as 1, 2, 3" (SC'11).  The 4x64 variant with
10 rounds: the state is four 64-bit words (the counter) and the key is two
64-bit words.  One round multiplies words 0 and 2 by two fixed odd constants,
keeping the 128-bit products' high and low halves, and permutes/xors them with
words 1 and 3 and the round key; the key is advanced by two Weyl constants
between rounds.  The constants below are those published with the generator.

Why a counter-based stream: [Self-spec] section 3.3 says every position must
draw its own independent random numbers, shaped like the candidate batch; a
shared draw across a batch biases the output.  Keying every draw by
(seed, sequence, absolute position, purpose) gives that, and makes the GPU and
this oracle draw identical numbers without sharing any state.

Stream layout used by the verify step (a reading; the pages fix no layout):

* key     = (seed, 0)
* counter = (block, position, sequence, tag)
* tag 0   -- the acceptance uniform for the draft decided at ``position``;
             block 0, word 0:  u = (w >> 40) * 2**-24, in [0, 1).
* tag 1   -- the Gumbel noise of the correction/bonus sample at ``position``;
             vocab entry v uses block v >> 2, word v & 3:
             U = ((w >> 41) + 0.5) * 2**-23, in (0, 1).
* tag 2   -- the drafter's Gumbel noise for the draft token at ``position``,
             laid out as tag 1 (a stream of its own, so drafting and verifying
             never share random numbers).

Pinned by: bit-exact comparison with ``numpy.random.Philox`` (a library
implementation of the same generator), see tests/test_oracle_philox.py.
"""
import numpy as np

M0 = 0xD2E7470EE14C6C93
M1 = 0xCA5A826395121157
W0 = 0x9E3779B97F4A7C15
W1 = 0xBB67AE8584CAA73B
_MASK64 = (1 << 64) - 1

TAG_ACCEPT = 0
TAG_GUMBEL = 1
TAG_DRAFT = 2


def philox4x64_10(ctr, key):
    """Philox4x64-10 on Python integers: the plain definition, one block.

    ``ctr`` is four 64-bit words, ``key`` two; returns four 64-bit words.
    """
    x0, x1, x2, x3 = (int(c) & _MASK64 for c in ctr)
    k0, k1 = (int(k) & _MASK64 for k in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + W0) & _MASK64
            k1 = (k1 + W1) & _MASK64
        p0 = M0 * x0
        p1 = M1 * x2
        hi0, lo0 = p0 >> 64, p0 & _MASK64
        hi1, lo1 = p1 >> 64, p1 & _MASK64
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return [x0, x1, x2, x3]


_M32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo(a, m):
    """128-bit product of uint64 array ``a`` and constant ``m``: (hi, lo)."""
    a = a.astype(np.uint64, copy=False)
    m = np.uint64(m)
    a_lo, a_hi = a & _M32, a >> _S32
    m_lo, m_hi = m & _M32, m >> _S32
    ll = a_lo * m_lo
    lh = a_lo * m_hi
    hl = a_hi * m_lo
    hh = a_hi * m_hi
    mid = (ll >> _S32) + (lh & _M32) + (hl & _M32)
    hi = hh + (lh >> _S32) + (hl >> _S32) + (mid >> _S32)
    lo = a * m  # wraps modulo 2**64
    return hi, lo


def philox4x64_10_np(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x64-10 over broadcastable uint64 arrays.

    Same arithmetic as :func:`philox4x64_10`, element-wise; returns four
    uint64 arrays.
    """
    with np.errstate(over="ignore"):
        x0, x1, x2, x3 = np.broadcast_arrays(*(np.asarray(c, dtype=np.uint64) for c in (c0, c1, c2, c3)))
        x0, x1, x2, x3 = (a.copy() for a in (x0, x1, x2, x3))
        k0 = np.asarray(k0, dtype=np.uint64)
        k1 = np.asarray(k1, dtype=np.uint64)
        for rnd in range(10):
            if rnd:
                k0 = k0 + np.uint64(W0)
                k1 = k1 + np.uint64(W1)
            hi0, lo0 = _mulhilo(x0, M0)
            hi1, lo1 = _mulhilo(x2, M1)
            x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return x0, x1, x2, x3


def accept_uniform(seed, seq, pos):
    """Acceptance uniform u in [0, 1) with 24 random bits.

    One per (sequence, absolute position); ``pos`` is the position of the token
    being decided.  The 24-bit grid makes u exact in float32 and float64.
    Broadcasts over array arguments; returns float64.
    """
    w0, _, _, _ = philox4x64_10_np(0, np.asarray(pos, dtype=np.int64).astype(np.uint64),
                                   np.asarray(seq, dtype=np.int64).astype(np.uint64),
                                   TAG_ACCEPT, np.uint64(seed), 0)
    return (w0 >> np.uint64(40)).astype(np.float64) * 2.0 ** -24


def gumbel_uniform(seed, seq, pos, v):
    """Uniform U in (0, 1) with 23 random bits for vocab entry ``v``.

    U = ((w >> 41) + 0.5) * 2**-23 never equals 0 or 1, so -log(-log U) is
    finite.  Exact in float32.  Broadcasts; returns float64.
    """
    v = np.asarray(v, dtype=np.int64).astype(np.uint64)
    words = philox4x64_10_np(v >> np.uint64(2),
                             np.asarray(pos, dtype=np.int64).astype(np.uint64),
                             np.asarray(seq, dtype=np.int64).astype(np.uint64),
                             TAG_GUMBEL, np.uint64(seed), 0)
    sel = (v & np.uint64(3)).astype(np.int64)
    w = np.choose(np.broadcast_to(sel, words[0].shape), words)
    return ((w >> np.uint64(41)).astype(np.float64) + 0.5) * 2.0 ** -23


def gumbel_uniform_rows(seed, seq, pos, V, tag=TAG_GUMBEL):
    """The uniforms of :func:`gumbel_uniform` for entries 0..V-1 of one row per
    sequence: [B, V] float64 from ``seq``, ``pos`` of shape [B].  Each Philox
    block is computed once and its four words laid out in vocab order.  ``tag``
    selects the stream (TAG_GUMBEL for the verify's draw, TAG_DRAFT for the
    drafter's)."""
    seq = np.asarray(seq, dtype=np.int64).astype(np.uint64)[:, None]
    pos = np.asarray(pos, dtype=np.int64).astype(np.uint64)[:, None]
    nb = (int(V) + 3) // 4
    blocks = np.arange(nb, dtype=np.uint64)[None, :]
    words = philox4x64_10_np(blocks, pos, seq, np.uint64(tag), np.uint64(seed), 0)
    w = np.stack(words, axis=-1).reshape(seq.shape[0], nb * 4)[:, :int(V)]
    return ((w >> np.uint64(41)).astype(np.float64) + 0.5) * 2.0 ** -23
