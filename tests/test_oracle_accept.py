"""Pins for oracle.accept (O-C): the pages' closed forms and worked numbers,
Monte-Carlo against E[K], exactness of the emitted distribution, special cases."""
import os

import numpy as np

from oracle import accept as oc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "speedup_worked_example.txt")


def test_speedup_worked_example():
    for line in open(GOLDEN):
        if not line.strip() or line.startswith("#"):
            continue
        gamma, alpha, r, ek, eta_min = line.split()
        gamma, alpha, r, ek, eta_min = int(gamma), float(alpha), float(r), float(ek), float(eta_min)
        got = oc.expected_accepted([alpha] * gamma)
        assert abs(got - ek) < 1e-12
        assert oc.speedup(got, gamma, r) >= eta_min


def _softmax(x):
    e = np.exp(x - x.max())
    return e / e.sum()


def _draw(rng, p):
    return int(np.searchsorted(np.cumsum(p), rng.random() * p.sum(), side="right"))


def _independent_positions(rng, gamma, V, noise):
    T = rng.standard_normal((gamma + 1, V)) * 1.5
    D = T[:gamma] + rng.standard_normal((gamma, V)) * noise
    return T, D


def test_monte_carlo_expected_accepted_length():
    """With per-position distributions fixed and x_i ~ Q_i drawn
    independently, each position is accepted with probability
    beta_i = sum_x min(P_i, Q_i), so E[K] = sum_i prod_{j<=i} beta_j exactly and
    Pr(K >= i) = prod_{j<=i} beta_j (futurestack.online, section 2.2)."""
    rng = np.random.default_rng(7)
    gamma, V, trials = 4, 8, 6000
    T, D = _independent_positions(rng, gamma, V, 0.6)
    P = np.array([_softmax(t) for t in T])
    Q = np.array([_softmax(d) for d in D])
    beta = np.minimum(P[:gamma], Q).sum(1)
    closed = oc.expected_accepted(beta)
    ks = np.empty(trials, dtype=int)
    for b in range(trials):
        x = np.array([_draw(rng, Q[i]) for i in range(gamma)])
        ks[b] = oc.accept_one(T, D, x, seed=11, step=0, b=b)["k"]
    se = ks.std() / np.sqrt(trials)
    assert abs(ks.mean() - closed) < 5 * se
    for i in range(1, gamma + 1):
        p_i = np.prod(beta[:i])
        frac = (ks >= i).mean()
        assert abs(frac - p_i) < 5 * np.sqrt(p_i * (1 - p_i) / trials) + 1e-9


def test_first_token_follows_target_distribution():
    """The first emitted token (the accepted x_1, or the resample at a reject
    of position 0) must be distributed as P_0 (futurestack.online, sections
    2.1-2.2: verification preserves the target distribution)."""
    rng = np.random.default_rng(8)
    gamma, V, trials = 2, 6, 12000
    T, D = _independent_positions(rng, gamma, V, 1.2)
    P0 = _softmax(T[0])
    Q = [_softmax(d) for d in D]
    counts = np.zeros(V)
    for b in range(trials):
        x = np.array([_draw(rng, Q[i]) for i in range(gamma)])
        r = oc.accept_one(T, D, x, seed=3, step=1, b=b)
        counts[x[0] if r["k"] >= 1 else r["token"]] += 1
    exp = P0 * trials
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert chi2 < 25          # 5 dof, p ~ 1.4e-4


def test_bonus_token_follows_target_distribution():
    rng = np.random.default_rng(9)
    V, trials = 5, 10000
    T = rng.standard_normal((2, V))
    D = T[:1].copy()                  # identical -> always accepted
    counts = np.zeros(V)
    for b in range(trials):
        r = oc.accept_one(T, D, np.array([0]), seed=5, step=2, b=b)
        assert r["k"] == 1 and r["source"] == "bonus"
        counts[r["token"]] += 1
    exp = _softmax(T[1]) * trials
    assert ((counts - exp) ** 2 / exp).sum() < 23


def test_special_cases():
    rng = np.random.default_rng(10)
    V, gamma = 16, 4
    T = rng.standard_normal((gamma + 1, V))
    # P == Q: every draft accepted
    for b in range(50):
        x = rng.integers(0, V, gamma)
        assert oc.accept_one(T, T[:gamma], x, 1, 0, b)["k"] == gamma
    # disjoint supports: rejected at 0, token from the target's support
    Tm = np.full((gamma + 1, V), -1e4)
    Tm[:, :8] = rng.standard_normal((gamma + 1, 8))
    Dm = np.full((gamma, V), -1e4)
    Dm[:, 8:] = rng.standard_normal((gamma, 8))
    for b in range(50):
        r = oc.accept_one(Tm, Dm, np.full(gamma, 9), 1, 0, b)
        assert r["k"] == 0 and r["token"] < 8 and r["source"] == "residual"
    # one-hot target agreeing with one-hot draft: greedy match
    Th = np.full((gamma + 1, V), -1e4)
    Dh = np.full((gamma, V), -1e4)
    toks = rng.integers(0, V, gamma)
    for i, t in enumerate(toks):
        Th[i, t] = 0
        Dh[i, t] = 0
    Th[gamma, 3] = 0
    r = oc.accept_one(Th, Dh, toks, 1, 0, 0)
    assert r["k"] == gamma and r["token"] == 3
    # first mismatch of a one-hot pair: rejected there, target token emitted
    toks2 = toks.copy()
    Dh2 = Dh.copy()
    Dh2[2] = -1e4
    Dh2[2, (toks[2] + 1) % V] = 0
    toks2[2] = (toks[2] + 1) % V
    r = oc.accept_one(Th, Dh2, toks2, 1, 0, 0)
    assert r["k"] == 2 and r["token"] == toks[2]


def test_out_of_vocabulary_draft_is_a_zero_probability_token():
    """A draft token outside [0, V) is no token of the target's vocabulary:
    the rule must treat it as a token the target gives probability 0, which
    min(1, P/Q) rejects with certainty; the next token is then the resample at
    that position.  Pinned against a real in-vocabulary token whose target
    probability is exactly 0 (the same decisions, the same draw)."""
    rng = np.random.default_rng(12)
    V, gamma = 40, 4
    for trial in range(30):
        T = rng.standard_normal((gamma + 1, V)) * 2
        D = rng.standard_normal((gamma, V)) * 2
        D[:2] = T[:2]                         # positions 0 and 1 always accepted
        z = int(rng.integers(0, V))
        Tz = T.copy()
        Tz[2, z] = -np.inf                    # P_2(z) = 0 exactly
        x = rng.integers(0, V, gamma)
        x[2] = z
        ref = oc.accept_one(Tz, D, x, 4, trial, trial)
        assert ref["k"] == 2 and ref["source"] == "residual"
        for bad in (-1, V, V + 7, -(2 ** 31)):
            xb = x.copy()
            xb[2] = bad
            # the rejected position's residual uses P_2 = softmax(Tz[2]) only
            # through tokens other than z; the OOV case reads T unchanged, so
            # compare against the same zero-probability target row
            got = oc.accept_one(Tz, D, xb, 4, trial, trial)
            assert (got["k"], got["token"], got["source"]) == (ref["k"], ref["token"], ref["source"])
            got_plain = oc.accept_one(T, D, xb, 4, trial, trial)
            assert got_plain["k"] == 2
