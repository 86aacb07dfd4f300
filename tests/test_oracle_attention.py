"""Pins for oracle.attention (O-A): brute force, a library routine, closed
forms and textbook reductions."""
import math

import numpy as np
import torch

from oracle import attention as oa


def _rand(rng, B, n_q, Hq, Hkv, d, lens):
    q = rng.standard_normal((B, n_q, Hq, d))
    K = [rng.standard_normal((n, Hkv, d)) for n in lens]
    V = [rng.standard_normal((n, Hkv, d)) for n in lens]
    return q, K, V


def _brute(q, K, V, n_q, masks, scale):
    """Element-by-element loops with math.exp: no numpy reductions."""
    B, _, Hq, d = q.shape
    O = np.zeros_like(q)
    LSE = np.zeros(q.shape[:3])
    for b in range(B):
        N, Hkv, _ = K[b].shape
        L = N - n_q
        for i in range(n_q):
            for h in range(Hq):
                g = h // (Hq // Hkv)
                s = []
                for t in range(N):
                    vis = t < L or (masks[b][i] >> (t - L)) & 1
                    if vis:
                        acc = 0.0
                        for c in range(d):
                            acc += q[b, i, h, c] * K[b][t, g, c]
                        s.append((t, acc * scale))
                m = max(v for _, v in s)
                tot = sum(math.exp(v - m) for _, v in s)
                for c in range(d):
                    O[b, i, h, c] = sum(math.exp(v - m) * V[b][t, g, c] for t, v in s) / tot
                LSE[b, i, h] = m + math.log(tot)
    return O, LSE


def test_brute_force_chain_and_tree():
    rng = np.random.default_rng(1)
    lens = [7, 12]
    q, K, V = _rand(rng, 2, 4, 4, 2, 8, lens)
    scale = float(np.float32(1 / math.sqrt(8)))
    O, LSE = oa.verify_attention(q, K, V, 4, None, scale)
    Ob, Lb = _brute(q, K, V, 4, [oa.chain_masks(4)] * 2, scale)
    assert np.allclose(O, Ob, atol=1e-12) and np.allclose(LSE, Lb, atol=1e-12)
    parents = [[-1, 0, 0, 1], [-1, 0, 1, 1]]
    anc = [oa.tree_masks(p) for p in parents]
    O, LSE = oa.verify_attention(q, K, V, 4, anc, scale)
    Ob, Lb = _brute(q, K, V, 4, anc, scale)
    assert np.allclose(O, Ob, atol=1e-12) and np.allclose(LSE, Lb, atol=1e-12)


def test_matches_torch_sdpa_float64():
    rng = np.random.default_rng(2)
    lens = [40, 23, 66]
    n_q, Hq, Hkv, d = 5, 8, 2, 16
    q, K, V = _rand(rng, 3, n_q, Hq, Hkv, d, lens)
    scale = 0.3
    O, _ = oa.verify_attention(q, K, V, n_q, None, scale)
    for b, N in enumerate(lens):
        L = N - n_q
        mask = torch.zeros(n_q, N, dtype=torch.bool)
        mask[:, :L] = True
        for i in range(n_q):
            mask[i, L:L + i + 1] = True
        qt = torch.from_numpy(q[b]).permute(1, 0, 2)                  # [Hq, n_q, d]
        kt = torch.from_numpy(K[b]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        vt = torch.from_numpy(V[b]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
        assert np.allclose(O[b], ref.permute(1, 0, 2).numpy(), atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(3)
    n_q, d = 3, 8
    q = np.zeros((1, n_q, 2, d))
    K = [rng.standard_normal((10, 1, d))]
    V = [rng.standard_normal((10, 1, d))]
    O, LSE = oa.verify_attention(q, K, V, n_q, None, 1.0)
    L = 10 - n_q
    for i in range(n_q):
        nvis = L + i + 1
        assert np.allclose(O[0, i, 0], V[0][:nvis, 0].mean(0), atol=1e-13)
        assert abs(LSE[0, i, 0] - math.log(nvis)) < 1e-13
    # single visible token: L = 0, chain row 0 sees only itself
    q = rng.standard_normal((1, n_q, 1, d))
    K = [rng.standard_normal((n_q, 1, d))]
    V = [rng.standard_normal((n_q, 1, d))]
    O, LSE = oa.verify_attention(q, K, V, n_q, None, 0.5)
    assert np.allclose(O[0, 0, 0], V[0][0, 0])
    assert abs(LSE[0, 0, 0] - 0.5 * q[0, 0, 0] @ K[0][0, 0]) < 1e-12
    # identical keys -> uniform weights
    K = [np.repeat(rng.standard_normal((1, 1, d)), 9, 0)]
    V = [rng.standard_normal((9, 1, d))]
    O, _ = oa.verify_attention(q, K, V, n_q, None, 0.5)
    assert np.allclose(O[0, 2, 0], V[0].mean(0)[0])


def test_gqa_equals_repeated_mha():
    rng = np.random.default_rng(4)
    q, K, V = _rand(rng, 2, 5, 8, 2, 16, [30, 41])
    O, L = oa.verify_attention(q, K, V, 5)
    Kr = [np.repeat(k, 4, axis=1) for k in K]
    Vr = [np.repeat(v, 4, axis=1) for v in V]
    O2, L2 = oa.verify_attention(q, Kr, Vr, 5)
    assert np.allclose(O, O2) and np.allclose(L, L2)


def test_chain_row_is_single_query_decode():
    rng = np.random.default_rng(5)
    n_q = 5
    q, K, V = _rand(rng, 1, n_q, 4, 2, 16, [50])
    O, L = oa.verify_attention(q, K, V, n_q)
    for i in range(n_q):
        N = 50 - n_q + i + 1
        O1, L1 = oa.verify_attention(q[:, i:i + 1], [K[0][:N]], [V[0][:N]], 1)
        assert np.allclose(O[:, i], O1[:, 0]) and np.allclose(L[:, i], L1[:, 0])


def test_tree_node_is_contiguous_path():
    rng = np.random.default_rng(6)
    parents = [-1, 0, 0, 0, 1, 1, 2, 4]
    n_q = len(parents)
    q, K, V = _rand(rng, 1, n_q, 2, 1, 8, [30])
    anc = [oa.tree_masks(parents)]
    O, L = oa.verify_attention(q, K, V, n_q, anc)
    Lc = 30 - n_q
    for i in range(n_q):
        path, j = [], i
        while j >= 0:
            path.append(j)
            j = parents[j]
        path = sorted(path)
        idx = list(range(Lc)) + [Lc + j for j in path]
        O1, L1 = oa.verify_attention(q[:, i:i + 1], [K[0][idx]], [V[0][idx]], 1)
        assert np.allclose(O[:, i], O1[:, 0]) and np.allclose(L[:, i], L1[:, 0])
    # a chain-shaped tree equals the chain mask
    assert oa.tree_masks([-1, 0, 1, 2, 3]) == oa.chain_masks(5)
