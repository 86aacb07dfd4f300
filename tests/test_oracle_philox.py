"""Pins for oracle.philox: published known-answer vectors and the uniform map."""
import os

import numpy as np

from oracle import philox

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        w = [int(x, 16) for x in line.split()]
        rows.append((w[0:4], w[4:6], w[6:10]))
    return rows


def test_known_answer_vectors():
    rows = _kat()
    assert len(rows) == 3
    for ctr, key, out in rows:
        got = philox.philox4x32_10(*ctr, *key)
        assert [int(x) for x in got] == out


def test_vectorised_matches_scalar():
    c0 = np.arange(17)
    vec = philox.philox4x32_10(c0, 5, 7, 9, 123, 456)
    for i in range(17):
        sc = philox.philox4x32_10(i, 5, 7, 9, 123, 456)
        assert all(int(vec[w][i]) == int(sc[w]) for w in range(4))


def test_uniform_open_interval_and_exact():
    w = np.array([0, 1, 511, 512, 0xFFFFFFFF, 0x80000000], dtype=np.uint64)
    u = philox.uniform_open01(w)
    assert u[0] == 2.0 ** -24 and u[1] == 2.0 ** -24 and u[2] == 2.0 ** -24
    assert u[3] == 3 * 2.0 ** -24
    assert u[4] == 1 - 2.0 ** -24
    assert u[5] == 0.5 + 2.0 ** -24
    # exact in fp32
    assert np.all(u.astype(np.float32).astype(np.float64) == u)


def test_uniform_distribution_chi2():
    words = philox.philox4x32_10(np.arange(50000), 1, 2, 3, 99, 7)
    u = philox.uniform_open01(np.concatenate(words))
    counts, _ = np.histogram(u, bins=20, range=(0, 1))
    exp = len(u) / 20
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert chi2 < 50          # 19 dof: p ~ 1e-4 at 50


def test_sample_uniforms_layout():
    u = philox.sample_uniforms(42, 3, 5, 2, 10)
    words = philox.philox4x32_10(np.arange(3), 5, 3, 2 | (philox.PURPOSE_SAMPLE << 16), 42, 0)
    flat = np.stack(words, 1).reshape(-1)[:10]
    assert np.array_equal(u, philox.uniform_open01(flat))
    a = philox.accept_uniform(42, 3, 5, 2)
    w = philox.philox4x32_10(0, 5, 3, 2 | (philox.PURPOSE_ACCEPT << 16), 42, 0)[0]
    assert a == float(philox.uniform_open01(w))
