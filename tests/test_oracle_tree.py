"""Pins for the oracle's draft-tree acceptance and path commit.

Tree acceptance (oracle.accept.accept_tree_one) is pinned by facts outside its
own code: on a chain it is the per-token rule (itself pinned by Monte-Carlo
against the pages' E[K]); the first and second emitted tokens follow the
target distributions exactly when the candidates are drawn from the draft
(chi-square); the probability that every candidate at a node is rejected is
the product of the per-round rejection masses; a point-mass target is greedy
decoding; identical target and draft accept the first child at every level.

Path commit (oracle.pool.PoolModel.commit_path) is pinned against brute force:
a float pool ends holding exactly the context, the root and the accepted nodes'
K/V, with the same pages as a pool that never appended the rejected nodes; an
FP8 pool keeps codes within a page and re-encodes across pages exactly as
torch's float8_e4m3fn conversion does.
"""
import numpy as np
import pytest
import torch

from oracle import accept as oc
from oracle import fp8 as of
from oracle import pool as op


def _softmax(x):
    e = np.exp(x - x.max())
    return e / e.sum()


def _draw(rng, p):
    return min(int(np.searchsorted(np.cumsum(p), rng.random() * p.sum(), side="right")), len(p) - 1)


def test_chain_tree_is_the_chain_rule():
    rng = np.random.default_rng(3)
    V, gamma = 40, 4
    parents = [-1, 0, 1, 2, 3]
    for b in range(150):
        T = rng.standard_normal((gamma + 1, V)) * 2
        D = T + rng.standard_normal((gamma + 1, V)) * (0.3 + (b % 3))
        x = np.array([_draw(rng, _softmax(D[i])) for i in range(gamma)])
        tokens = np.concatenate([[-1], x])
        r1 = oc.accept_one(T, D[:gamma], x, seed=5, step=2, b=b)
        r2 = oc.accept_tree_one(T, D, parents, tokens, seed=5, step=2, b=b)
        assert r2["k"] == r1["k"] and r2["token"] == r1["token"]
        assert r2["path"] == list(range(1, r1["k"] + 1))
        assert np.allclose(r2["accept_margins"], r1["accept_margins"], rtol=0, atol=1e-12)
        assert (r2["source"] == "bonus") == (r1["source"] == "bonus")


def _two_level_tree(m1, m2):
    parents = [-1] + [0] * m1
    for c in range(1, m1 + 1):
        parents += [c] * m2
    return parents


def test_emitted_tokens_follow_the_target():
    """Root with 3 candidates, each with 2 candidates below; the target and
    draft at a node depend only on the node's token, as for a real model.
    Candidates are drawn i.i.d. from the draft at their parent.  The first
    emitted token must follow P_root and, given first token a, the second
    must follow P_a (chi-square at p = 1e-4)."""
    rng = np.random.default_rng(11)
    V, trials = 5, 9000
    parents = _two_level_tree(3, 2)
    n = len(parents)
    T_root, D_root = rng.standard_normal(V) * 1.2, rng.standard_normal(V) * 1.2
    T_tok, D_tok = rng.standard_normal((V, V)) * 1.2, rng.standard_normal((V, V)) * 1.2
    first = np.zeros(V)
    second = np.zeros((V, V))
    for b in range(trials):
        tokens = np.full(n, -1)
        T = np.zeros((n, V))
        D = np.zeros((n, V))
        T[0], D[0] = T_root, D_root
        for c in range(1, n):
            tokens[c] = _draw(rng, _softmax(D[parents[c]]))
            T[c], D[c] = T_tok[tokens[c]], D_tok[tokens[c]]
        r = oc.accept_tree_one(T, D, parents, tokens, seed=9, step=1, b=b)
        emitted = [tokens[c] for c in r["path"]] + [r["token"]]
        first[emitted[0]] += 1
        if len(emitted) > 1:
            second[emitted[0], emitted[1]] += 1
    P = _softmax(T_root)
    chi = ((first - trials * P) ** 2 / (trials * P)).sum()
    assert chi < 26.0, chi                     # 4 dof, p ~ 3e-5
    for a in range(V):
        cnt = second[a].sum()
        if cnt < 400:
            continue
        Pa = _softmax(T_tok[a])
        chi = ((second[a] - cnt * Pa) ** 2 / (cnt * Pa)).sum()
        assert chi < 26.0, (a, chi)


def test_probability_that_every_candidate_is_rejected():
    """At a node with m candidates drawn i.i.d. from Q, round j accepts with
    probability sum_x min(P_{j-1}(x), Q(x)), P_j the residual after j
    rejections, so Pr(k = 0) = prod_j (1 - sum_x min(P_{j-1}, Q))."""
    rng = np.random.default_rng(21)
    V, m, trials = 6, 3, 8000
    parents = [-1] + [0] * m
    T0, D0 = rng.standard_normal(V) * 1.5, rng.standard_normal(V) * 1.5
    P, Q = _softmax(T0), _softmax(D0)
    rej, p = 1.0, P.copy()
    for _ in range(m):
        rej *= 1.0 - np.minimum(p, Q).sum()
        r = np.maximum(p - Q, 0)
        p = r / r.sum()
    T = np.tile(T0, (m + 1, 1))
    D = np.tile(D0, (m + 1, 1))
    zero = 0
    for b in range(trials):
        tokens = np.array([-1] + [_draw(rng, Q) for _ in range(m)])
        zero += oc.accept_tree_one(T, D, parents, tokens, seed=4, step=0, b=b)["k"] == 0
    frac = zero / trials
    assert abs(frac - rej) < 5 * np.sqrt(rej * (1 - rej) / trials), (frac, rej)


def test_point_mass_target_is_greedy():
    rng = np.random.default_rng(2)
    V = 30
    parents = _two_level_tree(4, 2)
    n = len(parents)
    for b in range(60):
        T = rng.standard_normal((n, V))
        best = rng.integers(0, V, size=n)
        T[np.arange(n), best] += 60.0
        D = rng.standard_normal((n, V))
        tokens = np.array([-1] + [int(rng.integers(0, V)) for _ in range(n - 1)])
        r = oc.accept_tree_one(T, D, parents, tokens, seed=1, step=0, b=b)
        emitted = [tokens[c] for c in r["path"]] + [r["token"]]
        nodes = [0] + r["path"]
        for d, tok in enumerate(emitted):
            assert tok == best[nodes[d]]


def test_identical_distributions_accept_first_children():
    rng = np.random.default_rng(8)
    V = 50
    parents = _two_level_tree(3, 2)
    n = len(parents)
    T = rng.standard_normal((n, V))
    tokens = np.array([-1] + [int(rng.integers(0, V)) for _ in range(n - 1)])
    for b in range(30):
        r = oc.accept_tree_one(T, T.copy(), parents, tokens, seed=3, step=0, b=b)
        assert r["path"] == [1, 4] and r["source"] == "bonus"


# ---------------------------------------------------------------------------
# path commit
# ---------------------------------------------------------------------------

def _tree_path(rng, parents):
    """A root path of the tree, as the acceptance would return it."""
    kids = oc.children_of(parents)
    path, u = [], 0
    while kids[u] and rng.random() < 0.8:
        u = int(rng.choice(kids[u]))
        path.append(u)
    return path


@pytest.mark.parametrize("ctx", [0, 13, 29, 32])
def test_commit_path_float_pool(ctx):
    rng = np.random.default_rng(ctx)
    H, d, S = 2, 4, 16
    parents = [-1, 0, 0, 0, 1, 1, 2, 3, 4, 4, 6, 8]
    n_tree = len(parents)
    order = rng.permutation(40)
    for trial in range(12):
        a = op.PoolModel(40, S, H, d, free_order=order)
        b = op.PoolModel(40, S, H, d, free_order=order)
        kc, vc = rng.standard_normal((ctx, H, d)), rng.standard_normal((ctx, H, d))
        kt, vt = rng.standard_normal((n_tree, H, d)), rng.standard_normal((n_tree, H, d))
        path = _tree_path(rng, parents)
        a.alloc(0)
        a.append(0, kc, vc)
        a.append(0, kt, vt)
        a.commit_path(0, n_tree, path)
        keep = [0] + path
        b.alloc(0)
        b.append(0, kc, vc)
        b.append(0, kt[keep], vt[keep])
        K, V = a.gather(0)
        assert np.array_equal(K, np.concatenate([kc, kt[keep]]))
        assert np.array_equal(V, np.concatenate([vc, vt[keep]]))
        assert a.tables == b.tables and a.free == b.free and a.lens == b.lens
        a.check_invariants()


def test_commit_path_fp8_pool():
    rng = np.random.default_rng(5)
    H, d, S = 2, 8, 16
    parents = [-1, 0, 0, 0, 1, 1, 2, 3, 4, 4, 6, 8, 9, 9, 12, 14]
    n_tree = len(parents)
    moved_across = 0
    for trial in range(20):
        ctx = int(rng.integers(0, 40))
        a = op.PoolModel(16, S, H, d, kv_dtype="fp8")
        a.alloc(0)
        a.append(0, rng.standard_normal((ctx, H, d)).astype(np.float32),
                 rng.standard_normal((ctx, H, d)).astype(np.float32))
        scale = np.float32(rng.choice([0.5, 1.0, 3.0]))
        kt = (rng.standard_normal((n_tree, H, d)) * scale).astype(np.float32)
        vt = (rng.standard_normal((n_tree, H, d)) * scale).astype(np.float32)
        a.append(0, kt, vt)
        base = ctx
        before = {t: (a.tables[0][t // S], t % S) for t in range(base, base + n_tree)}
        kc_before, vc_before = a.kc.copy(), a.vc.copy()
        ks, vs = a.ks.copy(), a.vs.copy()
        path = _tree_path(rng, parents)
        a.commit_path(0, n_tree, path)
        assert a.lens[0] == base + 1 + len(path)
        for dpt, c in enumerate(path):
            ps, os_ = before[base + c]
            pd, od = before[base + 1 + dpt]
            for codes_b, codes_a, sc in ((kc_before, a.kc, ks), (vc_before, a.vc, vs)):
                for h in range(H):
                    if ps == pd or sc[ps, h] == sc[pd, h]:
                        assert np.array_equal(codes_a[pd, h, od], codes_b[ps, h, os_])
                    else:
                        moved_across += 1
                        x = torch.from_numpy(of.decode(codes_b[ps, h, os_]).astype(np.float32)) * float(sc[ps, h])
                        inv = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(float(sc[pd, h]))
                        y = torch.clamp(x * inv, -448.0, 448.0)
                        want = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
                        assert np.array_equal(codes_a[pd, h, od], want)
        a.check_invariants()
    assert moved_across > 0


def test_commit_path_rejects_bad_paths():
    a = op.PoolModel(8, 16, 1, 2)
    a.alloc(0)
    a.append(0, np.zeros((20, 1, 2)), np.zeros((20, 1, 2)))
    with pytest.raises(ValueError):
        a.commit_path(0, 6, [2, 1])          # not increasing
    with pytest.raises(ValueError):
        a.commit_path(0, 6, [6])             # outside the tree
    with pytest.raises(ValueError):
        a.commit_path(0, 21, [])             # tree longer than the sequence
    a.alloc(1, 0, 20)                        # another sequence shares every page
    with pytest.raises(ValueError):
        a.commit_path(0, 6, [3])
    a.commit_path(0, 6, [])                  # nothing moves: plain truncation
    assert a.lens[0] == 15
