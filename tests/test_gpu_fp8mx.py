"""FP8 KV with a power-of-two scale per 64 channels of each token
(PKV_FP8_E4M3_MX64): the append quantiser bit-exact against the oracle's
(codes and E8M0 bytes), verification attention against the oracle on chain
and tree workloads (one- and two-wave kernels, head_dim 64 and 128, full size
sampled), tokens of very different magnitudes (the scaled conversion of K on
gfx950), and path commits."""
import numpy as np
import pytest
import torch

from oracle import accept as oc
from oracle import attention as oa
from oracle import pool as opool
from paged_kv_speculative_amd import Pool
from paged_kv_speculative_amd import workloads as wl
from layout_ref import detile_k, detile_v
import harness as H

pytestmark = pytest.mark.gpu


def _mx(cfg, small=True, head_dim=None, **kw):
    w = wl.make(cfg, small=small, **kw)
    w.kv_dtype = "fp8mx"
    if head_dim:
        w.head_dim = head_dim
    return w


def _gpu_codes(pool, seq, H_, d):
    pages, n, _ = pool.table(seq)
    kp = pool.k_pages.cpu().numpy()
    vp = pool.v_pages.cpu().numpy()
    ke = pool.k_scale.cpu().numpy()
    ve = pool.v_scale.cpu().numpy()
    K = np.concatenate([np.stack([detile_k(kp[p, h], "fp8", d) for h in range(H_)], 1) for p in pages])[:n]
    V = np.concatenate([np.stack([detile_v(vp[p, h], "fp8", d) for h in range(H_)], 1) for p in pages])[:n]
    KE = np.concatenate([ke[p].transpose(1, 0, 2) for p in pages])[:n]     # [token][head][tile]
    VE = np.concatenate([ve[p].transpose(1, 0, 2) for p in pages])[:n]
    return K, V, KE, VE


def test_append_codes_and_exponents_bit_exact():
    w = _mx(4, batch=2)
    g = H.GpuSide(w)
    for b in range(w.batch):
        K, V, KE, VE = _gpu_codes(g.pool, b, w.num_kv_heads, w.head_dim)
        pm = opool.PoolModel(64, 16, w.num_kv_heads, w.head_dim, kv_dtype="fp8mx")
        pm.alloc(0)
        k, v = w.private_kv(b)
        ctx = int(w.cached_lens[b])
        pm.append(0, k[:ctx], v[:ctx])
        pm.append(0, k[ctx:], v[ctx:])
        n = pm.lens[0]
        t = pm.tables[0]
        Ko = np.stack([pm.kc[t[i // 16], :, i % 16] for i in range(n)])
        KEo = np.stack([pm.kx[t[i // 16], :, i % 16] for i in range(n)])
        Vo = np.stack([pm.vc[t[i // 16], :, i % 16] for i in range(n)])
        VEo = np.stack([pm.vx[t[i // 16], :, i % 16] for i in range(n)])
        assert np.array_equal(K, Ko) and np.array_equal(KE, KEo)
        assert np.array_equal(V, Vo) and np.array_equal(VE, VEo)


@pytest.mark.parametrize("cfg,d", [(4, 128), (2, 128), (3, 128), (2, 64), (4, 64)])
def test_verify_matches_oracle(cfg, d):
    w = _mx(cfg, head_dim=d)
    print(f"fp8mx cfg {cfg} d {d} rows {w.n_q * w.num_q_heads // w.num_kv_heads}", flush=True)
    g = H.GpuSide(w)
    O, L = g.verify()
    O_ref, L_ref = H.oracle_verify(w, range(w.batch))
    H.compare(O.cpu().numpy(), L.cpu().numpy(), O_ref, L_ref, H.TOL["fp8mx"])


def test_verify_full_size_sampled():
    w = _mx(4, small=False)
    g = H.GpuSide(w)
    O, L = g.verify()
    O, L = O.cpu().numpy(), L.cpu().numpy()
    sample = [0, 7, w.batch - 1]
    O_ref, L_ref = H.oracle_verify(w, sample)
    H.compare(O[sample], L[sample], O_ref, L_ref, H.TOL["fp8mx"])


def test_tokens_of_very_different_magnitudes():
    """Per-token scales from 2^-28 (K) / 2^-24 (V) up to 2^-2 (K) / 2^20 (V):
    the K scale enters through the scaled FP8 -> bf16 conversion, the V scale
    through P; results match the oracle as closely as with unit scales."""
    rng = np.random.default_rng(3)
    Hkv, Hq, d, n_q = 2, 8, 128, 3
    for trial in range(3):
        N = int(rng.integers(20, 90))
        mag = 2.0 ** rng.integers(-24, 3, size=(N, Hkv, 1))
        k = (rng.standard_normal((N, Hkv, d)) * mag * 2.0 ** -4).astype(np.float32)
        v = (rng.standard_normal((N, Hkv, d)) * 2.0 ** rng.integers(-24, 21, size=(N, Hkv, 1))).astype(np.float32)
        pool = Pool(16, Hkv, d, "fp8mx", max_seqs=1, max_pages_per_seq=8, device="cuda")
        pool.fill_nan()
        pool.alloc(0)
        pool.append([0], [N], torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
        pm = opool.PoolModel(16, 16, Hkv, d, kv_dtype="fp8mx")
        pm.alloc(0)
        pm.append(0, k, v)
        K, V = pm.gather(0)
        q = wl.bf16_to_f32(wl.bf16_bits(rng.standard_normal((1, n_q, Hq, d)).astype(np.float32)))
        qt = torch.from_numpy(wl.bf16_bits(q).view(np.int16)).view(torch.bfloat16).cuda()
        O, L = pool.verify(qt, n_q, sm_scale=np.float32(1 / np.sqrt(d)))
        Or, Lr = oa.verify_attention(q.astype(np.float64), [K], [V], n_q, None, float(np.float32(1 / np.sqrt(d))))
        H.compare(O.cpu().numpy(), L.cpu().numpy(), Or, Lr, 2e-2)


def test_commit_path_moves_codes_and_scales():
    rng = np.random.default_rng(8)
    Hkv, d, B = 3, 128, 6
    parents = [-1, 0, 0, 0, 1, 1, 2, 3, 4, 4, 6, 8]
    n_tree = len(parents)
    kids = oc.children_of(parents)
    order = rng.permutation(60).astype(np.int32)
    pool = Pool(60, Hkv, d, "fp8mx", max_seqs=B, max_pages_per_seq=10, free_order=order, device="cuda")
    pool.fill_nan()
    pm = opool.PoolModel(60, 16, Hkv, d, kv_dtype="fp8mx", free_order=order)
    ks, vs, ns = [], [], []
    for b in range(B):
        pool.alloc(b)
        pm.alloc(b)
        n = int(rng.integers(0, 40)) + n_tree
        k = (rng.standard_normal((n, Hkv, d)) * 2.0 ** rng.integers(-6, 7, size=(n, Hkv, 1))).astype(np.float32)
        v = rng.standard_normal((n, Hkv, d)).astype(np.float32)
        pm.append(b, k, v)
        ks.append(k)
        vs.append(v)
        ns.append(n)
    pool.append(range(B), ns, torch.from_numpy(np.concatenate(ks)).cuda(),
                torch.from_numpy(np.concatenate(vs)).cuda())
    paths = []
    for b in range(B):
        path, u = [], 0
        while kids[u] and rng.random() < 0.85:
            u = int(rng.choice(kids[u]))
            path.append(u)
        paths.append(path)
    pool.commit_path(range(B), [n_tree] * B, paths)
    for b in range(B):
        pm.commit_path(b, n_tree, paths[b])
    torch.cuda.synchronize()
    for b in range(B):
        K, V, KE, VE = _gpu_codes(pool, b, Hkv, d)
        n, t = pm.lens[b], pm.tables[b]
        assert pool.table(b)[0] == t
        assert np.array_equal(K, np.stack([pm.kc[t[i // 16], :, i % 16] for i in range(n)]))
        assert np.array_equal(KE, np.stack([pm.kx[t[i // 16], :, i % 16] for i in range(n)]))
        assert np.array_equal(V, np.stack([pm.vc[t[i // 16], :, i % 16] for i in range(n)]))
        assert np.array_equal(VE, np.stack([pm.vx[t[i // 16], :, i % 16] for i in range(n)]))
