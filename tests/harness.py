"""Test harness: builds the same seeded workload on the GPU path (through the
C ABI) and on the oracle, and compares them.

The oracle never reads anything the GPU produced: it replays the same
append calls into its own pool model from the generator's arrays.
"""
import math

import numpy as np
import torch

from oracle import attention as oa
from oracle import pool as opool
from paged_kv_speculative_amd import Pool, tree_ancestor_masks
from paged_kv_speculative_amd.workloads import bf16_bits, bf16_to_f32
from layout_ref import detile_k, detile_v

TOL = {"f32": 2e-3, "bf16": 2e-3, "fp8": 2e-2, "fp8mx": 2e-2}


def max_pages(w):
    return int(max(-(-int(n) // 16) for n in w.seq_lens)) + 2


def _to_torch(x, kv_dtype, device):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if kv_dtype == "bf16":
        t = t.to(torch.bfloat16)             # exact: values are bf16-valued
    return t.to(device)


class GpuSide:
    """The workload's pool filled through paged_kv_alloc/append, plus queries."""

    def __init__(self, w, device="cuda", free_order=None, chunk_tokens=32768, verify_tokens=True):
        self.w = w
        order = w.free_order if free_order is None else free_order
        self.pool = Pool(w.num_pages, w.num_kv_heads, w.head_dim, w.kv_dtype, max_seqs=w.batch,
                         max_pages_per_seq=max_pages(w), free_order=order, device=device)
        self.pool.fill_nan()
        B = w.batch
        # context: shared prefix first, then every sequence's own context
        if w.prefix_len:
            self.pool.alloc(0)
            pk, pv = w.prefix_kv()
            self.pool.append([0], [w.prefix_len], _to_torch(pk, w.kv_dtype, device),
                             _to_torch(pv, w.kv_dtype, device))
            for b in range(1, B):
                self.pool.alloc(b, 0, w.prefix_len)
        else:
            for b in range(B):
                self.pool.alloc(b)
        self._append_private(range(B), context=True, chunk_tokens=chunk_tokens)
        if verify_tokens:
            self._append_private(range(B), context=False, chunk_tokens=chunk_tokens)
        q = w.q()
        if w.q_dtype == "bf16":
            self.q = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).to(device)
        else:
            self.q = torch.from_numpy(q).to(device)
        self.anc = None
        if w.tree_parents is not None:
            m = [tree_ancestor_masks(p) for p in w.tree_parents]
            self.anc = torch.tensor(np.array(m, dtype=np.uint64).view(np.int64), device=device)
        torch.cuda.synchronize()

    def _append_private(self, seqs, context, chunk_tokens):
        w = self.w
        seqs = list(seqs)
        i = 0
        while i < len(seqs):
            ks, vs, ns, ids = [], [], [], []
            tot = 0
            while i < len(seqs) and (tot == 0 or tot < chunk_tokens):
                b = seqs[i]
                k, v = w.private_kv(b)
                ctx = int(w.cached_lens[b]) - w.prefix_len
                sl = slice(0, ctx) if context else slice(ctx, None)
                ks.append(k[sl])
                vs.append(v[sl])
                ns.append(len(k[sl]))
                ids.append(b)
                tot += len(k[sl])
                i += 1
            kt = _to_torch(np.concatenate(ks), w.kv_dtype, "cuda")
            vt = _to_torch(np.concatenate(vs), w.kv_dtype, "cuda")
            self.pool.append(ids, ns, kt, vt)
            del kt, vt

    def verify(self, **kw):
        return self.pool.verify(self.q, self.w.n_q, anc_mask=self.anc, sm_scale=self.w.sm_scale, **kw)

    def new_kv(self):
        """K, V [B, n_q, Hkv, d] of the verification tokens, as the fused call
        takes them (bf16 for bf16 pools, fp32 for the FP8 kinds)."""
        w = self.w
        ks, vs = [], []
        for b in range(w.batch):
            k, v = w.private_kv(b)
            ctx = int(w.cached_lens[b]) - w.prefix_len
            ks.append(k[ctx:])
            vs.append(v[ctx:])
        return _to_torch(np.stack(ks), w.kv_dtype, "cuda"), _to_torch(np.stack(vs), w.kv_dtype, "cuda")

    def verify_append(self, **kw):
        """Append the verification tokens and verify them in one call
        (a pool built with verify_tokens=False)."""
        kn, vn = self.new_kv()
        return self.pool.verify_append(range(self.w.batch), self.q, kn, vn, anc_mask=self.anc,
                                       sm_scale=self.w.sm_scale, **kw)


def oracle_sequence_kv(w, b):
    """Oracle K, V (fp64) of sequence b: the same appends replayed into the
    oracle's own single-sequence pool model and gathered back."""
    S = 16
    n = int(w.seq_lens[b])
    pm = opool.PoolModel(-(-n // S) + 2, S, w.num_kv_heads, w.head_dim,
                         kv_dtype=w.kv_dtype if w.kv_dtype in ("fp8", "fp8mx") else "f64")
    pm.alloc(0)
    k, v = w.private_kv(b)
    if w.prefix_len:
        pk, pv = w.prefix_kv()
        pm.append(0, pk, pv)
    ctx = int(w.cached_lens[b]) - w.prefix_len
    pm.append(0, k[:ctx], v[:ctx])
    pm.append(0, k[ctx:], v[ctx:])
    return pm.gather(0)


def oracle_verify(w, seqs):
    """Oracle O [len(seqs), n_q, Hq, d] and LSE for the listed sequences."""
    q = w.q_f32()[list(seqs)].astype(np.float64)
    Ks, Vs = zip(*[oracle_sequence_kv(w, b) for b in seqs])
    anc = None
    if w.tree_parents is not None:
        anc = [oa.tree_masks(w.tree_parents[b]) for b in seqs]
    return oa.verify_attention(q, list(Ks), list(Vs), w.n_q, anc, float(w.sm_scale))


def oracle_block_tables(w):
    """Block tables the oracle's allocator gives for the harness's call order."""
    pm = opool.PoolModel(w.num_pages, 16, 1, 1, free_order=w.free_order)
    z = lambda n: np.zeros((n, 1, 1))
    if w.prefix_len:
        pm.alloc(0)
        pm.append(0, z(w.prefix_len), z(w.prefix_len))
        for b in range(1, w.batch):
            pm.alloc(b, 0, w.prefix_len)
    else:
        for b in range(w.batch):
            pm.alloc(b)
    for b in range(w.batch):
        n = int(w.cached_lens[b]) - w.prefix_len
        pm.append(b, z(n), z(n))
    for b in range(w.batch):
        pm.append(b, z(w.n_q), z(w.n_q))
    return pm.tables


def compare(O, L, O_ref, L_ref, tol):
    """Max |dO| / rms(O_ref) and max |dLSE| (nats)."""
    O = np.asarray(O, dtype=np.float64)
    L = np.asarray(L, dtype=np.float64)
    rms = math.sqrt(float(np.mean(O_ref ** 2)))
    err_o = float(np.max(np.abs(O - O_ref))) / rms
    err_l = float(np.max(np.abs(L - L_ref)))
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L)), "non-finite output"
    assert err_o <= tol, f"max|dO|/rms = {err_o:.3e} > {tol}"
    assert err_l <= tol, f"max|dLSE| = {err_l:.3e} > {tol}"
    return err_o, err_l


def check_sequence_pages(pool, pm, seq, kv, d):
    """GPU pages of `seq` hold exactly the oracle model's values in every
    slot the sequence can see (codes and scales for FP8 kinds)."""
    pages, n, _ = pool.table(seq)
    assert pages == pm.tables[seq] and n == pm.lens[seq]
    kp = pool.k_pages.cpu().numpy()
    vp = pool.v_pages.cpu().numpy()
    if kv != "bf16":
        ks = pool.k_scale.cpu().numpy()
        vs = pool.v_scale.cpu().numpy()
    layout = "bf16" if kv == "bf16" else "fp8"
    for j, p in enumerate(pages):
        valid = min(16, n - 16 * j)
        for h in range(pm.H):
            if kv == "bf16":
                K = detile_k(kp[p, h].view(np.uint16), layout, d)[:valid]
                V = detile_v(vp[p, h].view(np.uint16), layout, d)[:valid]
                assert np.array_equal(K, bf16_bits(pm.k[p, h, :valid])), (seq, j, h)
                assert np.array_equal(V, bf16_bits(pm.v[p, h, :valid])), (seq, j, h)
            else:
                K = detile_k(kp[p, h], layout, d)[:valid]
                V = detile_v(vp[p, h], layout, d)[:valid]
                assert np.array_equal(K, pm.kc[p, h, :valid]), (seq, j, h)
                assert np.array_equal(V, pm.vc[p, h, :valid]), (seq, j, h)
        if kv == "fp8":
            assert np.array_equal(ks[p], pm.ks[p]) and np.array_equal(vs[p], pm.vs[p]), (seq, j)
        elif kv == "fp8mx":
            assert np.array_equal(ks[p, :, :valid], pm.kx[p, :, :valid]), (seq, j)
            assert np.array_equal(vs[p, :, :valid], pm.vx[p, :, :valid]), (seq, j)
