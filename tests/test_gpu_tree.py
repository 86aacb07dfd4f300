"""GPU parity of draft-tree acceptance (spec_accept_tree) and of the path
commit (paged_kv_commit_path) against the oracle, and the exactness of the
tree rule checked on the GPU's own draws.

Decisions must equal the oracle's except where the oracle reports a tie the
fp32 kernels may resolve either way (an acceptance test within 1e-5 of its
threshold, or a draw whose two best Gumbel keys are within 1e-4)."""
import numpy as np
import pytest
import torch

from oracle import accept as oc
from oracle import pool as opool
from paged_kv_speculative_amd import Pool, PkvError, spec_accept, spec_accept_tree
from paged_kv_speculative_amd import workloads as wl
from layout_ref import detile_k, detile_v

pytestmark = pytest.mark.gpu

ACCEPT_TIE = 1e-5
SAMPLE_TIE = 1e-4


def _dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=dtype)).cuda()


def _gpu_tree(T, D, parents, tokens, seed, step, max_children=None):
    k, nodes, tok = spec_accept_tree(_dev(T, np.float32), _dev(D, np.float32),
                                     _dev(parents, np.int32), _dev(tokens, np.int32), seed, step,
                                     max_children=max_children)
    torch.cuda.synchronize()
    return k.cpu().numpy(), nodes.cpu().numpy(), tok.cpu().numpy()


def _check_tree(T, D, parents, tokens, seed, step):
    k, nodes, tok = _gpu_tree(T, D, parents, tokens, seed, step)
    ties = 0
    for b in range(len(k)):
        r = oc.accept_tree_one(T[b], D[b], list(parents[b]), tokens[b], seed, step, b)
        if min(r["accept_margins"], default=1.0) < ACCEPT_TIE:
            ties += 1
            continue
        assert k[b] == r["k"], (b, k[b], r["k"])
        assert list(nodes[b, :k[b]]) == r["path"] and np.all(nodes[b, k[b]:] == -1)
        if r["sample_gap"] < SAMPLE_TIE:
            ties += 1
            continue
        assert tok[b] == r["token"], (b, tok[b], r["token"], r["source"])
    return k, nodes, tok, ties


@pytest.mark.parametrize("small", [True, False])
def test_tree_workload_acceptance_parity(small):
    """The FP8 tree workload's trees (16 nodes, branching 4, 2, 2) with logits
    N(0, 2^2) over the Llama-3 vocabulary at full size."""
    w = wl.make(4, small=small)
    parents = np.array(w.tree_parents, dtype=np.int32)
    print(f"tree accept B={w.batch} n={w.n_q} V={w.accept_vocab}", flush=True)
    steps = range(4) if small else range(1)
    for step in steps:
        T, D, x = w.tree_accept_inputs(step=step)
        k, nodes, tok, ties = _check_tree(T, D, parents, x, seed=77, step=step)
        assert ties <= max(1, w.batch // 50)
        assert np.all((tok >= 0) & (tok < w.accept_vocab))


def test_tree_with_close_target_and_draft():
    """Target close to the draft so that deep paths and bonus draws occur."""
    w = wl.make(4, small=True, batch=12)
    parents = np.array(w.tree_parents, dtype=np.int32)
    T, D, x = w.tree_accept_inputs(step=5)
    rng = np.random.default_rng(0)
    T = (D + 0.15 * rng.standard_normal(D.shape)).astype(np.float32)
    x = np.full_like(x, -1)
    for b in range(w.batch):
        for c in range(1, w.n_q):
            p = np.exp(D[b, parents[b][c]] - D[b, parents[b][c]].max())
            x[b, c] = min(int(np.searchsorted(np.cumsum(p), rng.random() * p.sum(), side="right")),
                          w.accept_vocab - 1)
    k, nodes, tok, ties = _check_tree(T, D, parents, x, seed=5, step=1)
    assert k.max() >= 2


def test_random_trees_unaligned_vocab_many_children():
    """Random trees of up to 64 nodes (a root with up to 12 children, so up
    to 11 residual levels), an unaligned vocabulary and out-of-range tokens."""
    rng = np.random.default_rng(3)
    for n, V, B in [(2, 5, 9), (13, 37, 16), (40, 1001, 6), (64, 258, 5)]:
        parents = np.zeros((B, n), dtype=np.int32)
        for b in range(B):
            parents[b, 0] = -1
            root_kids = min(n - 1, int(rng.integers(1, 13)))
            for c in range(1, n):
                parents[b, c] = 0 if c <= root_kids else int(rng.integers(0, c))
        T = (rng.standard_normal((B, n, V)) * 1.5).astype(np.float32)
        D = (T + rng.standard_normal((B, n, V)) * 0.7).astype(np.float32)
        tokens = rng.integers(0, V, size=(B, n)).astype(np.int32)
        tokens[:, 0] = -1
        tokens[0, -1] = V + 3                       # never accepted
        _check_tree(T, D, parents, tokens, seed=11, step=3)


def test_chain_tree_equals_spec_accept():
    w = wl.make(5, small=True)
    T, D, x = w.accept_inputs(step=2)
    B, g = x.shape
    parents = np.tile(np.arange(-1, g, dtype=np.int32), (B, 1))
    Dn = np.concatenate([D, np.zeros((B, 1, D.shape[2]), np.float32)], 1)
    tokens = np.concatenate([np.full((B, 1), -1, np.int32), x], 1)
    k, nodes, tok = _gpu_tree(T, Dn, parents, tokens, 99, 2)
    kc, tc = spec_accept(_dev(T, np.float32), _dev(D, np.float32), _dev(x, np.int32), 99, 2)
    kc, tc = kc.cpu().numpy(), tc.cpu().numpy()
    _, _, info = oc.spec_accept(T, D, x, 99, 2)
    for b in range(B):
        if min(info[b]["accept_margins"], default=1.0) < ACCEPT_TIE:
            continue
        assert k[b] == kc[b] and list(nodes[b, :k[b]]) == list(range(1, k[b] + 1))
        if info[b]["sample_gap"] >= SAMPLE_TIE:
            assert tok[b] == tc[b]


def test_invalid_trees_are_flagged():
    rng = np.random.default_rng(1)
    B, n, V = 4, 6, 64
    T = rng.standard_normal((B, n, V)).astype(np.float32)
    D = rng.standard_normal((B, n, V)).astype(np.float32)
    tokens = rng.integers(0, V, size=(B, n)).astype(np.int32)
    parents = np.array([[-1, 0, 0, 1, 1, 2],        # valid, max 2 children
                        [-1, 0, 2, 1, 1, 2],        # parent after child
                        [0, 0, 0, 1, 1, 2],         # root with a parent
                        [-1, 0, 0, 0, 1, 2]],       # three children > max_children
                       dtype=np.int32)
    k, nodes, tok = _gpu_tree(T, D, parents, tokens, 1, 0, max_children=2)
    assert k[0] >= 0 and tok[0] >= 0
    assert list(k[1:]) == [-1, -1, -1] and list(tok[1:]) == [-1, -1, -1]
    assert np.all(nodes[1:] == -1)
    with pytest.raises(PkvError):
        _gpu_tree(T, D, parents, tokens, 1, 0, max_children=6)


def test_first_token_exact_on_gpu_draws():
    """20000 sequences with the same distributions: root with 3 candidates,
    each with 2 below, candidates drawn i.i.d. from the draft at their
    parent.  The first emitted token follows P_root (chi-square), and the
    fraction with nothing accepted is prod_j (1 - sum min(P_{j-1}, Q))."""
    rng = np.random.default_rng(17)
    B, V = 20000, 8
    parents1 = [-1, 0, 0, 0, 1, 1, 2, 2, 3, 3]
    n = len(parents1)
    Tn = rng.standard_normal((n, V)) * 1.3
    Dn = rng.standard_normal((n, V)) * 1.3
    sm = lambda z: np.exp(z - z.max()) / np.exp(z - z.max()).sum()
    tokens = np.full((B, n), -1, dtype=np.int32)
    for c in range(1, n):
        q = sm(Dn[parents1[c]])
        tokens[:, c] = np.minimum(np.searchsorted(np.cumsum(q), rng.random(B) * q.sum(), side="right"), V - 1)
    T = np.broadcast_to(Tn, (B, n, V)).astype(np.float32)
    D = np.broadcast_to(Dn, (B, n, V)).astype(np.float32)
    parents = np.tile(np.array(parents1, dtype=np.int32), (B, 1))
    k, nodes, tok = _gpu_tree(T, D, parents, tokens, 2024, 0)
    first = np.where(k >= 1, tokens[np.arange(B), np.maximum(nodes[:, 0], 0)], tok)
    P = sm(Tn[0].astype(np.float32).astype(np.float64))
    cnt = np.bincount(first, minlength=V)
    chi = ((cnt - B * P) ** 2 / (B * P)).sum()
    assert chi < 30.0, chi                           # 7 dof, p ~ 1e-4
    Q = sm(Dn[0].astype(np.float32).astype(np.float64))
    rej, p = 1.0, P.copy()
    for _ in range(3):
        rej *= 1.0 - np.minimum(p, Q).sum()
        r = np.maximum(p - Q, 0)
        p = r / r.sum()
    frac = float(np.mean(k == 0))
    assert abs(frac - rej) < 5 * np.sqrt(rej * (1 - rej) / B), (frac, rej)


# ---------------------------------------------------------------------------
# path commit
# ---------------------------------------------------------------------------

def _gpu_tokens(pool, seq, dtype, H, d):
    """Per-position K/V of a sequence read back from the device pool: bf16
    bits, FP8 codes or fp32 values, [len, H, d]."""
    pages, n, _ = pool.table(seq)
    view = {"bf16": np.uint16, "fp8": np.uint8, "f32": np.float32}[dtype]
    kp = pool.k_pages.cpu().numpy().view(view)
    vp = pool.v_pages.cpu().numpy().view(view)
    if dtype == "f32":
        K = np.concatenate([kp[p].reshape(H, 16, d).transpose(1, 0, 2) for p in pages])[:n]
        V = np.concatenate([vp[p].reshape(H, 16, d).transpose(1, 0, 2) for p in pages])[:n]
        return K, V
    K = np.concatenate([np.stack([detile_k(kp[p, h], dtype, d) for h in range(H)], 1) for p in pages])[:n]
    V = np.concatenate([np.stack([detile_v(vp[p, h], dtype, d) for h in range(H)], 1) for p in pages])[:n]
    return K, V


def _oracle_tokens(pm, seq, dtype):
    n, table = pm.lens[seq], pm.tables[seq]
    if dtype == "fp8":
        K = np.stack([pm.kc[table[t // 16], :, t % 16] for t in range(n)]) if n else None
        V = np.stack([pm.vc[table[t // 16], :, t % 16] for t in range(n)]) if n else None
        return K, V
    K = np.stack([pm.k[table[t // 16], :, t % 16] for t in range(n)])
    V = np.stack([pm.v[table[t // 16], :, t % 16] for t in range(n)])
    if dtype == "bf16":
        return wl.bf16_bits(K.astype(np.float32)), wl.bf16_bits(V.astype(np.float32))
    return K.astype(np.float32), V.astype(np.float32)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp8", 128), ("f32", 64), ("bf16", 64)])
def test_commit_path_matches_oracle(dtype, d):
    rng = np.random.default_rng({"bf16": 1, "fp8": 2, "f32": 3}[dtype] * 1000 + d)
    H, S, B = 3, 16, 9
    parents = [-1, 0, 0, 0, 0, 1, 1, 2, 2, 3, 3, 4, 4, 5, 7, 10]
    n_tree = len(parents)
    kids = oc.children_of(parents)
    pages = 80
    order = rng.permutation(pages).astype(np.int32)
    pool = Pool(pages, H, d, dtype, max_seqs=B, max_pages_per_seq=16, free_order=order, device="cuda")
    pool.fill_nan()
    pm = opool.PoolModel(pages, S, H, d, kv_dtype="fp8" if dtype == "fp8" else "f64", free_order=order)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def vals(n, scale=1.0):
        x = (rng.standard_normal((n, H, d)) * scale).astype(np.float32)
        return wl.bf16_to_f32(wl.bf16_bits(x)) if dtype == "bf16" else x

    for rnd in range(3):
        ctxs = [int(rng.integers(0, 40)) for _ in range(B)] if rnd == 0 else [0] * B
        if rnd == 0:
            for b in range(B):
                pool.alloc(b)
                pm.alloc(b)
        for phase in ("ctx", "tree"):
            ks, vs, ns = [], [], []
            for b in range(B):
                n = ctxs[b] if phase == "ctx" else n_tree
                k, v = vals(n, 1.0 if phase == "ctx" else float(rng.choice([0.3, 2.0, 40.0]))), vals(n)
                ks.append(k)
                vs.append(v)
                ns.append(n)
                pm.append(b, k.astype(np.float64) if dtype != "fp8" else k,
                          v.astype(np.float64) if dtype != "fp8" else v)
            pool.append(range(B), ns, torch.from_numpy(np.concatenate(ks)).to(tdt).cuda(),
                        torch.from_numpy(np.concatenate(vs)).to(tdt).cuda())
        paths = []
        for b in range(B):
            path, u = [], 0
            while kids[u] and rng.random() < 0.85:
                u = int(rng.choice(kids[u]))
                path.append(u)
            paths.append(path)
        paths[0] = []
        pool.commit_path(range(B), [n_tree] * B, paths)
        for b in range(B):
            pm.commit_path(b, n_tree, paths[b])
        torch.cuda.synchronize()
        for b in range(B):
            assert pool.table(b)[0] == pm.tables[b] and pool.table(b)[1] == pm.lens[b]
            Kg, Vg = _gpu_tokens(pool, b, dtype, H, d)
            Ko, Vo = _oracle_tokens(pm, b, dtype)
            assert np.array_equal(Kg, Ko), (rnd, b, dtype)
            assert np.array_equal(Vg, Vo), (rnd, b, dtype)
        assert np.array_equal(pool.seq_lens.cpu().numpy()[:B], [pm.lens[b] for b in range(B)])


def test_commit_then_verify_equals_never_drafted():
    """After committing a tree branch, the next verification step sees the
    same K/V as a pool that appended only the accepted tokens."""
    w = wl.make(2, small=True, batch=4)
    H, d = w.num_kv_heads, w.head_dim
    parents = [-1, 0, 0, 1, 1, 2, 3, 4]
    n_tree = len(parents)
    rng = np.random.default_rng(6)
    from harness import GpuSide
    g1, g2 = GpuSide(w), GpuSide(w)
    tree = wl.bf16_to_f32(wl.bf16_bits(rng.standard_normal((w.batch, n_tree, H, d)).astype(np.float32)))
    paths = [[2, 5], [], [1, 3, 6], [1, 4, 7]]
    t1 = torch.from_numpy(tree.reshape(-1, H, d)).to(torch.bfloat16).cuda()
    g1.pool.append(range(w.batch), [n_tree] * w.batch, t1, t1.clone())
    g1.pool.commit_path(range(w.batch), [n_tree] * w.batch, paths)
    keep = np.concatenate([tree[b, [0] + paths[b]] for b in range(w.batch)])
    t2 = torch.from_numpy(keep).to(torch.bfloat16).cuda()
    g2.pool.append(range(w.batch), [1 + len(p) for p in paths], t2, t2.clone())
    q = torch.randn((w.batch, 3, w.num_q_heads, d)).to(torch.bfloat16).cuda()
    kn = torch.randn((w.batch * 3, H, d)).to(torch.bfloat16).cuda()
    for g in (g1, g2):
        g.pool.append(range(w.batch), [3] * w.batch, kn, kn.clone())
    O1, L1 = (x.clone() for x in g1.pool.verify(q, 3))
    O2, L2 = g2.pool.verify(q, 3)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
