"""GPU parity of the FP8 page-scale growth: a page filled by several short
appends (a decode loop appends gamma + 1 tokens a step) doubles its scale when
new values exceed its range and encodes its cached codes again
(atozofsoftwareengineering.blog, section "Custom FP8 Quantized Memory Block
Layout", per-block scales; the growth rule is the reading documented in
oracle/fp8.py).  The pool-update kernel and the fused append of
spec_verify_attention_append must give the oracle pool model's codes and
scales bit for bit, and verification over the pages equals the oracle's."""
import numpy as np
import pytest
import torch

import harness as H
from oracle import attention as oa
from oracle import pool as opool
from paged_kv_speculative_amd import Pool

pytestmark = pytest.mark.gpu


def _steps(rng, n_total, step, Hkv, d):
    """Token values in chunks of `step`, each chunk scaled by a factor that
    grows now and then, so that later chunks exceed earlier pages' ranges."""
    out = []
    t = 0
    while t < n_total:
        n = min(step, n_total - t)
        f = float(rng.choice([0.5, 1.0, 1.0, 3.0, 9.0]))
        out.append((f * rng.standard_normal((n, Hkv, d)).astype(np.float32),
                    f * rng.standard_normal((n, Hkv, d)).astype(np.float32)))
        t += n
    return out


@pytest.mark.parametrize("step,d", [(1, 128), (5, 128), (5, 64), (3, 64)])
def test_short_appends_grow_page_scales_like_the_oracle(step, d):
    rng = np.random.default_rng(100 * step + d)
    Hkv, G, B, n_total, n_q = 2, 4, 3, 70, 4
    P = 48
    free = rng.permutation(P).astype(np.int32)
    pool = Pool(P, Hkv, d, "fp8", max_seqs=B, max_pages_per_seq=8, free_order=free, device="cuda")
    pool.fill_nan()
    pm = opool.PoolModel(P, 16, Hkv, d, kv_dtype="fp8", free_order=free)
    for s in range(B):
        pool.alloc(s)
        pm.alloc(s)
    chunks = [_steps(rng, n_total, step, Hkv, d) for _ in range(B)]
    print(f"fp8 growth step={step} d={d}", flush=True)
    for i in range(max(len(c) for c in chunks)):
        seqs = [s for s in range(B) if i < len(chunks[s])]
        ks = np.concatenate([chunks[s][i][0] for s in seqs])
        vs = np.concatenate([chunks[s][i][1] for s in seqs])
        pool.append(seqs, [len(chunks[s][i][0]) for s in seqs], torch.from_numpy(ks).cuda(),
                    torch.from_numpy(vs).cuda())
        for s in seqs:
            pm.append(s, *chunks[s][i])
    torch.cuda.synchronize()
    assert pm.scale_growths > 0          # the appends did exceed earlier pages' ranges
    for s in range(B):
        H.check_sequence_pages(pool, pm, s, "fp8", d)
    # verification over the grown pages
    q = rng.standard_normal((B, n_q, Hkv * G, d)).astype(np.float32)
    qb = torch.from_numpy(q).to(torch.bfloat16)
    kn = [rng.standard_normal((n_q, Hkv, d)).astype(np.float32) * 5 for _ in range(B)]
    vn = [rng.standard_normal((n_q, Hkv, d)).astype(np.float32) * 5 for _ in range(B)]
    pool.append(list(range(B)), [n_q] * B, torch.from_numpy(np.concatenate(kn)).cuda(),
                torch.from_numpy(np.concatenate(vn)).cuda())
    for s in range(B):
        pm.append(s, kn[s], vn[s])
    O, L = pool.verify(qb.cuda(), n_q)
    for s in range(B):
        H.check_sequence_pages(pool, pm, s, "fp8", d)
    Ks, Vs = zip(*[pm.gather(s) for s in range(B)])
    O_ref, L_ref = oa.verify_attention(qb.float().numpy().astype(np.float64), list(Ks), list(Vs), n_q, None,
                                       float(np.float32(1 / np.sqrt(d))))
    H.compare(O.cpu().numpy(), L.cpu().numpy(), O_ref, L_ref, H.TOL["fp8"])


@pytest.mark.parametrize("n_q", [1, 5])
def test_fused_steps_grow_page_scales_like_the_separate_path(n_q):
    """A decode loop of fused steps (append inside the verification launch)
    with growing magnitudes: after every step the pool equals, byte for byte,
    a pool driven by paged_kv_append + spec_verify_attention, and the pages
    equal the oracle's; outputs equal the oracle's."""
    rng = np.random.default_rng(7 + n_q)
    Hkv, G, B, d = 2, 4, 4, 128
    P = 64
    free = rng.permutation(P).astype(np.int32)
    pools = [Pool(P, Hkv, d, "fp8", max_seqs=B, max_pages_per_seq=8, free_order=free, device="cuda")
             for _ in range(2)]
    pm = opool.PoolModel(P, 16, Hkv, d, kv_dtype="fp8", free_order=free)
    for p in pools:
        p.fill_nan()
    ctx = [3, 16, 9, 21]
    for s in range(B):
        for p in pools:
            p.alloc(s)
        pm.alloc(s)
    k0 = [rng.standard_normal((n, Hkv, d)).astype(np.float32) for n in ctx]
    v0 = [rng.standard_normal((n, Hkv, d)).astype(np.float32) for n in ctx]
    for p in pools:
        p.append(list(range(B)), ctx, torch.from_numpy(np.concatenate(k0)).cuda(),
                 torch.from_numpy(np.concatenate(v0)).cuda())
    for s in range(B):
        pm.append(s, k0[s], v0[s])
    print(f"fused fp8 growth n_q={n_q}", flush=True)
    for it in range(6):
        f = [0.5, 2.0, 1.0, 6.0, 1.0, 20.0][it]
        kn = (f * rng.standard_normal((B, n_q, Hkv, d))).astype(np.float32)
        vn = (f * rng.standard_normal((B, n_q, Hkv, d))).astype(np.float32)
        q = torch.from_numpy(rng.standard_normal((B, n_q, Hkv * G, d)).astype(np.float32)).to(torch.bfloat16)
        pools[0].append(list(range(B)), [n_q] * B, torch.from_numpy(kn.reshape(-1, Hkv, d)).cuda(),
                        torch.from_numpy(vn.reshape(-1, Hkv, d)).cuda())
        Oa, La = pools[0].verify(q.cuda(), n_q)
        Ob, Lb = pools[1].verify_append(range(B), q.cuda(), torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda())
        torch.cuda.synchronize()
        assert torch.equal(pools[0].k_pages, pools[1].k_pages) and torch.equal(pools[0].v_pages, pools[1].v_pages)
        assert torch.equal(pools[0].k_scale, pools[1].k_scale) and torch.equal(pools[0].v_scale, pools[1].v_scale)
        for s in range(B):
            pm.append(s, kn[s], vn[s])
            H.check_sequence_pages(pools[1], pm, s, "fp8", d)
        Ks, Vs = zip(*[pm.gather(s) for s in range(B)])
        O_ref, L_ref = oa.verify_attention(q.float().numpy().astype(np.float64), list(Ks), list(Vs), n_q, None,
                                           float(np.float32(1 / np.sqrt(d))))
        H.compare(Ob.cpu().numpy(), Lb.cpu().numpy(), O_ref, L_ref, H.TOL["fp8"])
        H.compare(Oa.cpu().numpy(), La.cpu().numpy(), O_ref, L_ref, H.TOL["fp8"])
    assert pm.scale_growths > 0
