"""GPU parity of the pool's copy-on-write append and of rollback followed by a
later verification step, against the oracle's pool model replaying the same
operations.

Copy-on-write (paurushmuley.com, PagedKVCacheManager.EnsureCapacityAndAppendToken:
a block with reference count > 1 is copied before a write; diagram
"PagedAttention virtual memory manager": shared block, copy on generation):
a sequence that shares a partly valid page with another gets its own copy of
that page on its first append, the source's page stays as it was, and the
copy carries the page's FP8 scales (per page-head fp32, or the per-token E8M0
bytes of the 64-channel tiles).

Rollback (innvotechnologies.co, pipeline diagram: commit to the block table,
discard invalid KV blocks): after the rejected tail of every sequence is
dropped, the next step's tokens land where the rejected ones were and a fresh
verification sees exactly context + accepted tokens + the new tokens.
"""
import numpy as np
import pytest
import torch

import harness as H
from oracle import attention as oa
from oracle import pool as opool
from paged_kv_speculative_amd import Pool
from paged_kv_speculative_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _vals(rng, n, Hkv, d, kv):
    x = rng.standard_normal((n, Hkv, d)).astype(np.float32) * 1.5
    if kv == "bf16":
        x = wl.bf16_to_f32(wl.bf16_bits(x))
    return x


def _dev(x, kv):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return (t.to(torch.bfloat16) if kv == "bf16" else t).cuda()


def _page_state(pool, p):
    """Raw bytes of page p (K, V and, for FP8 kinds, both scale arrays)."""
    parts = [pool.k_pages[p].clone(), pool.v_pages[p].clone()]
    if pool.k_scale is not None:
        parts += [pool.k_scale[p].clone(), pool.v_scale[p].clone()]
    return parts


@pytest.mark.parametrize("kv,d", [("bf16", 128), ("bf16", 64), ("fp8", 128), ("fp8mx", 128)])
def test_copy_on_write_append(kv, d):
    rng = np.random.default_rng({"bf16": 1, "fp8": 2, "fp8mx": 3}[kv] + d)
    Hkv, Hq, P = 2, 8, 48
    free = rng.permutation(P).astype(np.int32)
    pool = Pool(P, Hkv, d, kv, max_seqs=4, max_pages_per_seq=8, free_order=free, device="cuda")
    pool.fill_nan()
    pm = opool.PoolModel(P, 16, Hkv, d, kv_dtype="f64" if kv == "bf16" else kv, free_order=free)
    # (op, seq, argument); every append's values are fresh draws
    ops = [("alloc", 0, None), ("append", 0, 24),
           ("share", 1, 20),           # shares both pages; 4 of page 1's slots visible to seq 1
           ("share", 2, 24),           # shares both pages
           ("append", 1, 7),           # page 1 has 3 holders: seq 1 copies it
           ("append", 0, 5),           # still 2 holders (seq 0, seq 2): seq 0 copies it
           ("append", 2, 30),          # now held by seq 2 alone: written in place
           ("append", 1, 12)]          # seq 1's copy is its own: in place, then a new page
    print(f"cow kv={kv} d={d}", flush=True)
    for op, seq, arg in ops:
        if op == "alloc":
            pool.alloc(seq)
            pm.alloc(seq)
        elif op == "share":
            pool.alloc(seq, 0, arg)
            pm.alloc(seq, 0, arg)
        else:
            k, v = _vals(rng, arg, Hkv, d, kv), _vals(rng, arg, Hkv, d, kv)
            src_pages = list(pm.tables[seq])
            shared_tail = (pm.lens[seq] % 16 != 0 and pm.refcount[src_pages[pm.lens[seq] // 16]] > 1)
            before = None
            blk = pm.lens[seq] // 16                      # block the append starts in
            if shared_tail:
                tail = src_pages[blk]
                before = (tail, _page_state(pool, tail))
            pool.append([seq], [arg], _dev(k, kv), _dev(v, kv))
            pm.append(seq, k.astype(np.float64) if kv == "bf16" else k,
                      v.astype(np.float64) if kv == "bf16" else v)
            torch.cuda.synchronize()
            if before is not None:
                # the shared page itself is untouched by the copy and the write
                tail, state = before
                assert all(torch.equal(a, b) for a, b in zip(state, _page_state(pool, tail)))
                assert pool.table(seq)[0][blk] != tail    # the writer holds its own copy
        for s in pm.tables:
            assert pool.table(s)[0] == pm.tables[s] and pool.table(s)[1] == pm.lens[s]
        assert pool.stats()["cow_copies"] == pm.cow_copies
    assert pm.cow_copies == 2
    for s in pm.tables:
        H.check_sequence_pages(pool, pm, s, kv, d)
    # the three sequences' verification against the oracle's gathered K/V
    n_q = 3
    seqs = sorted(pm.tables)
    q = wl.bf16_to_f32(wl.bf16_bits(rng.standard_normal((len(seqs), n_q, Hq, d)).astype(np.float32)))
    qt = torch.from_numpy(q).to(torch.bfloat16).cuda()
    slots = torch.tensor([pool.slot(s) for s in seqs], dtype=torch.int32, device="cuda")
    O, L = pool.verify(qt, n_q, slots=slots)
    Ks, Vs = zip(*[pm.gather(s) for s in seqs])
    O_ref, L_ref = oa.verify_attention(q.astype(np.float64), list(Ks), list(Vs), n_q, None,
                                       float(np.float32(1 / np.sqrt(d))))
    H.compare(O.cpu().numpy(), L.cpu().numpy(), O_ref, L_ref, H.TOL[kv])


@pytest.mark.parametrize("small", [True, False])
def test_config3_rollback_then_next_step(small):
    """Workload 3 ("plus rollback of rejected tails"): after verification each
    sequence keeps 1 + k_b of its gamma + 1 tokens (k_b with Pr(K >= i) =
    0.85^i), the next step appends gamma + 1 new tokens and verifies fresh
    queries.  Block tables equal the oracle allocator's for every sequence;
    outputs equal the oracle's (all sequences at small size, a sample at full
    size, in the benchmark's launch configuration)."""
    w = wl.make(3, small=small)
    B, n_q = w.batch, w.n_q
    print(f"cfg 3 rollback small={small} B={B} k={w.rollback_k.tolist()}", flush=True)
    g = H.GpuSide(w)
    g.verify()
    drop = (n_q - 1 - w.rollback_k).astype(np.int32)
    g.pool.rollback(range(B), drop)
    kn, vn = w.step_kv(1)
    g.pool.append(range(B), [n_q] * B, _dev(kn.reshape(-1, w.num_kv_heads, w.head_dim), "bf16"),
                  _dev(vn.reshape(-1, w.num_kv_heads, w.head_dim), "bf16"))
    q2 = w.step_q(1)
    qt = torch.from_numpy(q2.view(np.int16)).view(torch.bfloat16).cuda()
    O, L = g.pool.verify(qt, n_q, sm_scale=w.sm_scale)
    O, L = O.cpu().numpy(), L.cpu().numpy()
    # integer state: the oracle allocator replaying the same calls for the batch
    pm = opool.PoolModel(w.num_pages, 16, 1, 1, free_order=w.free_order)
    z = lambda n: np.zeros((int(n), 1, 1))
    for b in range(B):
        pm.alloc(b)
    for b in range(B):
        pm.append(b, z(w.cached_lens[b]), z(w.cached_lens[b]))
    for b in range(B):
        pm.append(b, z(n_q), z(n_q))
    for b in range(B):
        pm.rollback(b, int(drop[b]))
    for b in range(B):
        pm.append(b, z(n_q), z(n_q))
    for b in range(B):
        pages, n, _ = g.pool.table(b)
        assert pages == pm.tables[b] and n == pm.lens[b] == int(w.cached_lens[b]) + 1 + int(w.rollback_k[b]) + n_q
    # values: each sampled sequence's K/V replayed into the oracle's pool
    if small:
        sample = list(range(B))
    else:
        rng = np.random.default_rng(33)
        sample = sorted(set([0, B - 1, int(np.argmax(w.seq_lens))] + list(rng.choice(B, 2, replace=False))))
    Ks, Vs = [], []
    for b in sample:
        k, v = w.private_kv(b)
        n = int(w.seq_lens[b]) + n_q
        m = opool.PoolModel(-(-n // 16) + 2, 16, w.num_kv_heads, w.head_dim)
        m.alloc(0)
        ctx = int(w.cached_lens[b])
        m.append(0, k[:ctx].astype(np.float64), v[:ctx].astype(np.float64))
        m.append(0, k[ctx:].astype(np.float64), v[ctx:].astype(np.float64))
        m.rollback(0, int(drop[b]))
        m.append(0, kn[b].astype(np.float64), vn[b].astype(np.float64))
        K, V = m.gather(0)
        Ks.append(K)
        Vs.append(V)
    qf = wl.bf16_to_f32(q2)[sample].astype(np.float64)
    O_ref, L_ref = oa.verify_attention(qf, Ks, Vs, n_q, None, float(w.sm_scale))
    H.compare(O[sample], L[sample], O_ref, L_ref, H.TOL["bf16"])
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
