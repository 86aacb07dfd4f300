"""GPU parity of spec_verify_attention_append: the new tokens appended and
verified in one launch (atozofsoftwareengineering.blog, diagram "Speculative
Decoding Memory Pipeline": FP8 pages flow straight into the fused
verification attention).

Two checks per case:
  * the pool state the fused call leaves (K/V pages, FP8 scales, block table,
    lengths and the host bookkeeping) equals, byte for byte, the state of the
    same pool after paged_kv_append of the same tokens, and (page-boundary
    cases) every visible slot's bf16 values or FP8 codes and scales equal the
    oracle pool model's quantisation of the same tokens;
  * the outputs equal the oracle's attention over the oracle pool model's
    replay of the same appends, within the accuracy targets (2e-3 of rms(O)
    and 2e-3 nats for bf16 KV, 2e-2 for the FP8 kinds).
"""
import zlib

import numpy as np
import pytest
import torch

import harness as H
from oracle import attention as oa
from oracle import pool as opool
from paged_kv_speculative_amd import Pool, PkvError, tree_ancestor_masks
from paged_kv_speculative_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _same_state(pa, pb, seqs):
    torch.cuda.synchronize()
    assert torch.equal(pa.k_pages, pb.k_pages) and torch.equal(pa.v_pages, pb.v_pages)
    if pa.k_scale is not None:
        assert torch.equal(pa.k_scale, pb.k_scale) and torch.equal(pa.v_scale, pb.v_scale)
    assert torch.equal(pa.block_table, pb.block_table) and torch.equal(pa.seq_lens, pb.seq_lens)
    for s in seqs:
        assert pa.table(s) == pb.table(s)
    assert pa.stats() == pb.stats()


def _workload(cfg, kv=None, small=True):
    w = wl.make(cfg, small=small)
    if kv is not None:
        w.kv_dtype = kv
    return w


@pytest.mark.parametrize("cfg,kv,splits", [(2, "bf16", 0), (2, "fp8", 0), (2, "fp8mx", 0), (2, "bf16", 11),
                                           (4, "fp8", 0), (4, "fp8mx", 0), (4, "bf16", 5), (5, "bf16", 0),
                                           (5, "fp8", 0), (5, "fp8", 7), (3, "bf16", 0)])
def test_fused_equals_append_then_verify(cfg, kv, splits):
    w = _workload(cfg, kv)
    print(f"fused cfg {cfg} kv={kv} splits={splits} B={w.batch} n_q={w.n_q}", flush=True)
    kw = {"num_splits": splits}
    if w.prefix_len:
        kw["shared_prefix_pages"] = w.prefix_len // 16
    a = H.GpuSide(w)
    Oa, La = a.verify(**kw)
    b = H.GpuSide(w, verify_tokens=False)
    Ob, Lb = b.verify_append(**kw)
    _same_state(a.pool, b.pool, range(w.batch))
    O_ref, L_ref = H.oracle_verify(w, range(w.batch))
    H.compare(Ob.cpu().numpy(), Lb.cpu().numpy(), O_ref, L_ref, H.TOL[kv])
    H.compare(Oa.cpu().numpy(), La.cpu().numpy(), O_ref, L_ref, H.TOL[kv])


def _vals(rng, n, Hkv, d, kv):
    x = rng.standard_normal((n, Hkv, d)).astype(np.float32) * 1.5
    if kv == "bf16":
        x = wl.bf16_to_f32(wl.bf16_bits(x))
    return x


def _dev(x, kv):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return (t.to(torch.bfloat16) if kv == "bf16" else t).cuda()


@pytest.mark.parametrize("kv,d,n_q,G,tree", [("bf16", 128, 16, 4, False), ("bf16", 64, 16, 4, True),
                                             ("fp8", 128, 16, 4, False), ("fp8", 64, 3, 8, True),
                                             ("fp8mx", 128, 16, 2, True), ("fp8mx", 64, 1, 4, False),
                                             ("bf16", 128, 1, 1, False)])
def test_fused_page_boundaries(kv, d, n_q, G, tree):
    """Cached lengths at and around page boundaries (0, 1, 15, 16, 17, 31,
    47): the new tokens start a page, fill a page's tail, or straddle two
    pages; an empty sequence attends only its new tokens."""
    rng = np.random.default_rng(zlib.crc32(repr((kv, d, n_q, G, tree)).encode()))
    Hkv = 2
    Hq = Hkv * G
    lens = [0, 16, 15, 31, 1, 47, 17]
    B = len(lens)
    P = 64
    free = rng.permutation(P).astype(np.int32)
    pools = [Pool(P, Hkv, d, kv, max_seqs=B, max_pages_per_seq=6, free_order=free, device="cuda")
             for _ in range(2)]
    pm = opool.PoolModel(P, 16, Hkv, d, kv_dtype="f64" if kv == "bf16" else kv, free_order=free)
    for p in pools:
        p.fill_nan()
    ctx = [(_vals(rng, n, Hkv, d, kv), _vals(rng, n, Hkv, d, kv)) for n in lens]
    for s in range(B):
        for p in pools:
            p.alloc(s)
        pm.alloc(s)
    for p in pools:
        p.append(list(range(B)), lens, _dev(np.concatenate([k for k, _ in ctx]), kv),
                 _dev(np.concatenate([v for _, v in ctx]), kv))
    for s in range(B):
        pm.append(s, *(x.astype(np.float64) if kv == "bf16" else x for x in ctx[s]))
    new = [(_vals(rng, n_q, Hkv, d, kv), _vals(rng, n_q, Hkv, d, kv)) for _ in range(B)]
    kn = np.stack([k for k, _ in new])
    vn = np.stack([v for _, v in new])
    q = wl.bf16_to_f32(wl.bf16_bits(rng.standard_normal((B, n_q, Hq, d)).astype(np.float32)))
    qt = torch.from_numpy(q).to(torch.bfloat16).cuda()
    anc, anc_t = None, None
    if tree:
        parents = [[-1] + [int(rng.integers(0, i)) for i in range(1, n_q)] for _ in range(B)]
        anc = [oa.tree_masks(pp) for pp in parents]
        anc_t = torch.tensor(np.array([tree_ancestor_masks(pp) for pp in parents], dtype=np.uint64)
                             .view(np.int64), device="cuda")
    print(f"fused boundaries kv={kv} d={d} n_q={n_q} G={G} tree={tree}", flush=True)
    pools[0].append(list(range(B)), [n_q] * B, _dev(kn.reshape(-1, Hkv, d), kv), _dev(vn.reshape(-1, Hkv, d), kv))
    Oa, La = pools[0].verify(qt, n_q, anc_mask=anc_t)
    Ob, Lb = pools[1].verify_append(range(B), qt, _dev(kn, kv), _dev(vn, kv), anc_mask=anc_t)
    _same_state(pools[0], pools[1], range(B))
    for s in range(B):
        pm.append(s, *(x.astype(np.float64) if kv == "bf16" else x for x in new[s]))
        assert pools[1].table(s)[0] == pm.tables[s] and pools[1].table(s)[1] == pm.lens[s]
        # codes and scales the fused call wrote equal the oracle's quantisation
        H.check_sequence_pages(pools[1], pm, s, kv, d)
    Ks, Vs = zip(*[pm.gather(s) for s in range(B)])
    O_ref, L_ref = oa.verify_attention(q.astype(np.float64), list(Ks), list(Vs), n_q, anc,
                                       float(np.float32(1 / np.sqrt(d))))
    H.compare(Ob.cpu().numpy(), Lb.cpu().numpy(), O_ref, L_ref, H.TOL[kv])
    H.compare(Oa.cpu().numpy(), La.cpu().numpy(), O_ref, L_ref, H.TOL[kv])


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_fused_steps_with_rollback(kv):
    """Workload 3's step sequence through the fused call: verify, roll back
    the rejected tails (Pr(K >= i) = 0.85^i), then a second fused step whose
    streaming pass reads the lengths and block-table entries the first one
    wrote.  The state equals the separate-call path's after every call."""
    w = _workload(3, kv)
    B, n_q = w.batch, w.n_q
    print(f"fused steps kv={kv} B={B} k={w.rollback_k.tolist()}", flush=True)
    a = H.GpuSide(w)
    a.verify()
    b = H.GpuSide(w, verify_tokens=False)
    b.verify_append()
    _same_state(a.pool, b.pool, range(B))
    drop = (n_q - 1 - w.rollback_k).astype(np.int32)
    for g in (a, b):
        g.pool.rollback(range(B), drop)
    _same_state(a.pool, b.pool, range(B))
    kn, vn = w.step_kv(1)
    q2 = w.step_q(1)
    qt = (torch.from_numpy(q2.view(np.int16)).view(torch.bfloat16) if w.q_dtype == "bf16"
          else torch.from_numpy(q2)).cuda()
    a.pool.append(range(B), [n_q] * B, _dev(kn.reshape(-1, w.num_kv_heads, w.head_dim), kv),
                  _dev(vn.reshape(-1, w.num_kv_heads, w.head_dim), kv))
    Oa, La = a.pool.verify(qt, n_q, sm_scale=w.sm_scale)
    Ob, Lb = b.pool.verify_append(range(B), qt, _dev(kn, kv), _dev(vn, kv), sm_scale=w.sm_scale)
    _same_state(a.pool, b.pool, range(B))
    Ks, Vs = [], []
    for s in range(B):
        k, v = w.private_kv(s)
        ctx = int(w.cached_lens[s])
        n = int(w.seq_lens[s]) + n_q
        m = opool.PoolModel(-(-n // 16) + 2, 16, w.num_kv_heads, w.head_dim,
                            kv_dtype="f64" if kv == "bf16" else kv)
        m.alloc(0)
        f = (lambda x: x.astype(np.float64)) if kv == "bf16" else (lambda x: x)
        m.append(0, f(k[:ctx]), f(v[:ctx]))
        m.append(0, f(k[ctx:]), f(v[ctx:]))
        m.rollback(0, int(drop[s]))
        m.append(0, f(kn[s]), f(vn[s]))
        K, V = m.gather(0)
        Ks.append(K)
        Vs.append(V)
    qf = (wl.bf16_to_f32(q2) if w.q_dtype == "bf16" else q2).astype(np.float64)
    O_ref, L_ref = oa.verify_attention(qf, Ks, Vs, n_q, None, float(w.sm_scale))
    H.compare(Ob.cpu().numpy(), Lb.cpu().numpy(), O_ref, L_ref, H.TOL[kv])


def test_fused_full_size_bench_workload():
    """The 32-sequence workload (contexts 512..4096, 5 verification tokens,
    32 query / 8 KV heads) at full size in the benchmark's launch
    configuration: pool state equals the separate-call path's, and a sample
    of sequences (all heads and rows) equals the oracle."""
    w = wl.make(2)
    a = H.GpuSide(w)
    Oa, La = a.verify()
    b = H.GpuSide(w, verify_tokens=False)
    Ob, Lb = b.verify_append()
    _same_state(a.pool, b.pool, range(w.batch))
    rng = np.random.default_rng(2)
    sample = sorted(set([0, w.batch - 1, int(np.argmax(w.seq_lens))] + list(rng.choice(w.batch, 2, replace=False))))
    O_ref, L_ref = H.oracle_verify(w, sample)
    H.compare(Ob.cpu().numpy()[sample], Lb.cpu().numpy()[sample], O_ref, L_ref, H.TOL["bf16"])
    assert torch.isfinite(Ob).all() and torch.isfinite(Lb).all()


def test_fused_refusals_change_nothing():
    """Calls the fused path does not take are refused before anything
    changes: a shared (copy-on-write) tail page, more than 16 new tokens,
    an fp32 pool, and a sequence that is not in its own block-table row."""
    d, Hkv, Hq = 64, 2, 4
    rng = np.random.default_rng(7)
    pool = Pool(32, Hkv, d, "bf16", max_seqs=4, max_pages_per_seq=6, device="cuda")
    pool.alloc(0)
    pool.append([0], [20], _dev(_vals(rng, 20, Hkv, d, "bf16"), "bf16"), _dev(_vals(rng, 20, Hkv, d, "bf16"), "bf16"))
    pool.alloc(1, 0, 20)                 # shares the partly filled second page
    before = (pool.table(0), pool.table(1), pool.stats(), pool.seq_lens.clone(), pool.block_table.clone())

    def call(n_q, seqs=(0, 1)):
        B = len(seqs)
        q = torch.zeros((B, n_q, Hq, d), dtype=torch.bfloat16, device="cuda")
        kn = torch.zeros((B, n_q, Hkv, d), dtype=torch.bfloat16, device="cuda")
        return pool.verify_append(list(seqs), q, kn, kn.clone())

    with pytest.raises(PkvError) as e:
        call(2)
    assert e.value.status == 5                      # PKV_ERR_UNSUPPORTED: shared tail page
    with pytest.raises(PkvError) as e:
        call(17)
    assert e.value.status == 5                      # more than 16 new tokens
    with pytest.raises(PkvError) as e:
        call(2, seqs=(1, 0))
    assert e.value.status == 1                      # PKV_ERR_INVALID_ARG: not in its own row
    after = (pool.table(0), pool.table(1), pool.stats(), pool.seq_lens.clone(), pool.block_table.clone())
    assert before[:3] == after[:3]
    assert torch.equal(before[3], after[3]) and torch.equal(before[4], after[4])
    p32 = Pool(8, 1, 64, "f32", max_seqs=1, max_pages_per_seq=2, device="cuda")
    p32.alloc(0)
    with pytest.raises(PkvError):
        p32.verify_append([0], torch.zeros((1, 1, 1, 64), dtype=torch.float32, device="cuda"),
                          torch.zeros((1, 1, 1, 64), dtype=torch.float32, device="cuda"),
                          torch.zeros((1, 1, 1, 64), dtype=torch.float32, device="cuda"))
