"""Philox4x32-10, written from its published definition — oracle side.

Source: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC'11, section 3 (the Philox S-box built from
two 32x32->64 bit multiplies per round, a Weyl sequence on the key, and 10
rounds for Philox4x32-10).

One round maps counter (c0, c1, c2, c3) under key (k0, k1) to
    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))
and then bumps the key by the Weyl constants (W0, W1).

The pages draw uniforms for the acceptance test (innvotechnologies.co, section
"Verification Acceptance Probabilities and Speedup Math", eq. alpha_i) without
saying how; this project's reading is a counter-based generator so that every
(sequence, position, vocabulary entry) draw is reproducible on any device.
"""
import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF

# Purposes, stored in the top 16 bits of counter word 3.
PURPOSE_ACCEPT = 1
PURPOSE_SAMPLE = 2


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10.  Counter words may be arrays (broadcast);
    key words are Python ints.  Returns four uint32 arrays."""
    c0 = np.asarray(c0, dtype=np.uint64) & MASK32
    c1 = np.asarray(c1, dtype=np.uint64) & MASK32
    c2 = np.asarray(c2, dtype=np.uint64) & MASK32
    c3 = np.asarray(c3, dtype=np.uint64) & MASK32
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    k0 = int(k0) & MASK32
    k1 = int(k1) & MASK32
    for _ in range(10):
        p0 = np.uint64(M0) * c0          # < 2**64, exact in uint64
        p1 = np.uint64(M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK32)
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1,
                          hi0 ^ c3 ^ np.uint64(k1), lo0)
        k0 = (k0 + W0) & MASK32
        k1 = (k1 + W1) & MASK32
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def uniform_open01(word):
    """Map a 32-bit word to u in (0, 1): u = (floor(w / 2**9) + 1/2) * 2**-23.

    Every value is a dyadic rational with at most 24 significant bits, so it
    is exact in fp32 and fp64 alike; 0 and 1 are excluded (needed by the
    Gumbel transform -log(-log u))."""
    w = np.asarray(word, dtype=np.uint64)
    return ((w >> np.uint64(9)).astype(np.float64) + 0.5) * 2.0 ** -23


def _key(seed):
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & MASK32, seed >> 32


def accept_uniform(seed, step, b, i):
    """Uniform for the acceptance test of draft position i of sequence b."""
    k0, k1 = _key(seed)
    w = philox4x32_10(0, b, step, i | (PURPOSE_ACCEPT << 16), k0, k1)[0]
    return float(uniform_open01(w))


def sample_uniforms(seed, step, b, i, vocab):
    """Uniforms u[x], x in [0, vocab), for sampling a token at position i of
    sequence b.  Entry x uses counter (x // 4, b, step, i | SAMPLE << 16) and
    output word x % 4."""
    k0, k1 = _key(seed)
    nblk = (vocab + 3) // 4
    words = philox4x32_10(np.arange(nblk), b, step, i | (PURPOSE_SAMPLE << 16), k0, k1)
    w = np.stack(words, axis=1).reshape(-1)[:vocab]
    return uniform_open01(w)
