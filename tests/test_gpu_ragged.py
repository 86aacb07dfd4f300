"""Per-sequence draft counts: verification with n_q_seq and acceptance with
gammas, against the oracle run sequence by sequence with each sequence's own
count (oracle.attention.verify_attention with n_q = n_b; oracle.accept.accept_one
on the first g_b drafts)."""
import numpy as np
import pytest
import torch

from oracle import accept as oc
from oracle import attention as oa
from oracle import pool as opool
from paged_kv_speculative_amd import Pool, spec_accept, tree_ancestor_masks
from paged_kv_speculative_amd import VerifyBuffers
from paged_kv_speculative_amd import workloads as wl
import harness as H

pytestmark = pytest.mark.gpu


def _ragged_side(w, nqs):
    """Pool holding every sequence's context followed by its own n_b
    verification tokens, and the oracle's K/V of the same tokens."""
    B = w.batch
    dt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    pool = Pool(w.num_pages, w.num_kv_heads, w.head_dim, w.kv_dtype, max_seqs=B,
                max_pages_per_seq=H.max_pages(w), free_order=w.free_order, device="cuda")
    pool.fill_nan()
    Ks, Vs = [], []
    for b in range(B):
        pool.alloc(b)
        k, v = w.private_kv(b)
        n = int(w.cached_lens[b]) + int(nqs[b])
        ctx = int(w.cached_lens[b])
        for sl in (slice(0, ctx), slice(ctx, n)):
            pool.append([b], [sl.stop - sl.start], torch.from_numpy(np.ascontiguousarray(k[sl])).to(dt).cuda(),
                        torch.from_numpy(np.ascontiguousarray(v[sl])).to(dt).cuda())
        pm = opool.PoolModel(-(-n // 16) + 2, 16, w.num_kv_heads, w.head_dim,
                             kv_dtype="fp8" if w.kv_dtype == "fp8" else "f64")
        pm.alloc(0)
        pm.append(0, k[:ctx], v[:ctx])
        pm.append(0, k[ctx:n], v[ctx:n])
        K, V = pm.gather(0)
        Ks.append(K)
        Vs.append(V)
    return pool, Ks, Vs


def _q(w):
    q = w.q()
    if w.q_dtype == "bf16":
        return torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(q).cuda()


@pytest.mark.parametrize("cfg,splits", [(2, 0), (2, 1), (3, 0), (3, 64), (1, 0), (4, 0)])
def test_ragged_verify_matches_oracle(cfg, splits):
    w = wl.make(cfg, small=True)
    rng = np.random.default_rng(cfg * 10 + splits)
    nqs = rng.integers(1, w.n_q + 1, size=w.batch).astype(np.int32)
    nqs[0] = w.n_q
    nqs[-1] = 1
    print(f"ragged cfg {cfg} splits {splits} n_b {nqs.tolist()}", flush=True)
    pool, Ks, Vs = _ragged_side(w, nqs)
    q = _q(w)
    anc = None
    if w.tree_parents is not None:
        m = [tree_ancestor_masks(p) for p in w.tree_parents]
        anc = torch.tensor(np.array(m, dtype=np.uint64).view(np.int64), device="cuda")
    nq_t = torch.from_numpy(nqs).cuda()
    B, nq, Hq, d = q.shape
    # outputs pre-filled with a sentinel: padding slots must stay untouched
    buf = VerifyBuffers(B, nq, Hq, d, 1 << 27, "cuda")
    buf.out.fill_(12345.0)
    buf.lse.fill_(12345.0)
    O, L = pool.verify(q, nq, anc_mask=anc, sm_scale=w.sm_scale, buffers=buf, num_splits=splits,
                       n_q_seq=nq_t)
    O, L = O.cpu().numpy(), L.cpu().numpy()
    qf = w.q_f32().astype(np.float64)
    tol = 1e-4 if w.kv_dtype == "f32" else H.TOL[w.kv_dtype]
    for b in range(B):
        n_b = int(nqs[b])
        a = None if anc is None else [oa.tree_masks(w.tree_parents[b])[:n_b]]
        Or, Lr = oa.verify_attention(qf[b:b + 1, :n_b], [Ks[b]], [Vs[b]], n_b, a, float(w.sm_scale))
        H.compare(O[b:b + 1, :n_b], L[b:b + 1, :n_b], Or, Lr, tol)
        assert np.all(O[b, n_b:] == 12345.0) and np.all(L[b, n_b:] == 12345.0), b


@pytest.mark.parametrize("splits", [0, 1, 7])
def test_ragged_zero_and_negative_counts(splits):
    """Counts of 0 and below are clamped to one slot (the documented [1, n_q]
    range): the result equals a call with those sequences' counts set to 1,
    bitwise, and the oracle with one query slot."""
    w = wl.make(2, small=True, batch=6)
    nqs = np.array([0, 5, -3, 2, 1, -2147483648], dtype=np.int32)
    print(f"ragged clamp splits {splits} n_b {nqs.tolist()}", flush=True)
    clamped = np.clip(nqs, 1, w.n_q)
    pool, Ks, Vs = _ragged_side(w, clamped)
    q = _q(w)
    B, nq, Hq, d = q.shape
    outs = []
    for counts in (nqs, clamped):
        buf = VerifyBuffers(B, nq, Hq, d, 1 << 27, "cuda")
        buf.out.fill_(12345.0)
        buf.lse.fill_(12345.0)
        O, L = pool.verify(q, nq, sm_scale=w.sm_scale, buffers=buf, num_splits=splits,
                           n_q_seq=torch.from_numpy(counts).cuda())
        outs.append((O.cpu().numpy(), L.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    O, L = outs[0]
    qf = w.q_f32().astype(np.float64)
    for b in range(B):
        n_b = int(clamped[b])
        Or, Lr = oa.verify_attention(qf[b:b + 1, :n_b], [Ks[b]], [Vs[b]], n_b, None, float(w.sm_scale))
        H.compare(O[b:b + 1, :n_b], L[b:b + 1, :n_b], Or, Lr, H.TOL["bf16"])
        assert np.all(O[b, n_b:] == 12345.0) and np.all(L[b, n_b:] == 12345.0), b


def test_full_counts_equal_no_counts_bitwise():
    w = wl.make(2, small=True, batch=6)
    g = H.GpuSide(w)
    O1, L1 = (x.clone() for x in g.verify())
    nq_t = torch.full((w.batch,), w.n_q, dtype=torch.int32, device="cuda")
    O2, L2 = g.verify(n_q_seq=nq_t)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


@pytest.mark.parametrize("small", [True, False])
def test_ragged_acceptance_matches_oracle(small):
    w = wl.make(5, small=small)
    B = w.batch if small else 64
    T, D, x = w.accept_inputs(step=3, batch=B)
    rng = np.random.default_rng(9)
    gam = rng.integers(1, w.gamma + 1, size=B).astype(np.int32)
    gam[0] = w.gamma
    gam[1] = 1
    dev = lambda a, t: torch.from_numpy(np.ascontiguousarray(a, dtype=t)).cuda()
    k, tok = spec_accept(dev(T, np.float32), dev(D, np.float32), dev(x, np.int32), 31, 3,
                         gammas=dev(gam, np.int32))
    k, tok = k.cpu().numpy(), tok.cpu().numpy()
    ties = 0
    for b in range(B):
        g_b = int(gam[b])
        r = oc.accept_one(T[b, :g_b + 1], D[b, :g_b], x[b, :g_b], 31, 3, b)
        if min(r["accept_margins"], default=1.0) < 1e-5:
            ties += 1
            continue
        assert k[b] == r["k"] and k[b] <= g_b, (b, k[b], r["k"])
        if r["sample_gap"] < 1e-4:
            ties += 1
            continue
        assert tok[b] == r["token"], (b, tok[b], r["token"], r["source"])
    assert ties <= max(1, B // 50)


def test_ragged_acceptance_with_close_distributions():
    """Drafts close to the target, so that sequences run to their own count
    and take the bonus from row g_b."""
    rng = np.random.default_rng(4)
    B, g, V = 24, 5, 777
    T = rng.standard_normal((B, g + 1, V)).astype(np.float32) * 2
    D = (T[:, :g] + 0.05 * rng.standard_normal((B, g, V))).astype(np.float32)
    x = np.empty((B, g), dtype=np.int32)
    for b in range(B):
        for i in range(g):
            p = np.exp(D[b, i] - D[b, i].max())
            x[b, i] = min(int(np.searchsorted(np.cumsum(p), rng.random() * p.sum(), side="right")), V - 1)
    gam = rng.integers(1, g + 1, size=B).astype(np.int32)
    dev = lambda a, t: torch.from_numpy(np.ascontiguousarray(a, dtype=t)).cuda()
    k, tok = spec_accept(dev(T, np.float32), dev(D, np.float32), dev(x, np.int32), 5, 0,
                         gammas=dev(gam, np.int32))
    k, tok = k.cpu().numpy(), tok.cpu().numpy()
    bonus = 0
    for b in range(B):
        r = oc.accept_one(T[b, :gam[b] + 1], D[b, :gam[b]], x[b, :gam[b]], 5, 0, b)
        if min(r["accept_margins"], default=1.0) < 1e-5 or r["sample_gap"] < 1e-4:
            continue
        assert k[b] == r["k"] and tok[b] == r["token"]
        bonus += r["source"] == "bonus"
    assert bonus >= 5
