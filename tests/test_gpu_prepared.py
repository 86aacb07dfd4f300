"""Prepared pool updates (Pool.prepare_append / prepare_rollback: arguments
marshalled once, as a serving loop calls them every step) leave the pool in
exactly the state Pool.append / Pool.rollback leave it in: pages, FP8
scales, block tables and lengths, byte for byte, over a few steps of
append + partial rollback, for bf16, FP8 and FP8-MX pools."""
import numpy as np
import pytest
import torch

from paged_kv_speculative_amd import Pool

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv", ["bf16", "fp8", "fp8mx"])
def test_prepared_append_and_rollback_equal_plain_calls(kv):
    Hkv, d, B, nq = 2, 128, 5, 5
    order = np.random.default_rng(3).permutation(96)
    pools = [Pool(96, Hkv, d, kv, max_seqs=B, max_pages_per_seq=24, free_order=order, device="cuda")
             for _ in range(2)]
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    dt = torch.bfloat16 if kv == "bf16" else torch.float32
    ctx = [3, 16, 31, 40, 0]
    seqs = np.arange(B, dtype=np.int64)
    for p in pools:
        p.fill_nan()                   # unwritten slots hold the same bytes in both pools
        for s in range(B):
            p.alloc(s)
    k0 = (torch.randn((sum(ctx), Hkv, d), generator=g, device="cuda") * 2).to(dt)
    v0 = (torch.randn((sum(ctx), Hkv, d), generator=g, device="cuda") * 2).to(dt)
    for p in pools:
        p.append(seqs, ctx, k0, v0)
    knew = torch.empty((B * nq, Hkv, d), dtype=dt, device="cuda")
    vnew = torch.empty_like(knew)
    n_new = np.full(B, nq, dtype=np.int32)
    app = pools[1].prepare_append(seqs, n_new, knew, vnew)
    rb = pools[1].prepare_rollback(seqs)
    rng = np.random.default_rng(5)
    for step in range(4):
        knew.copy_((torch.randn(knew.shape, generator=g, device="cuda") * (1 + step)).to(dt))
        vnew.copy_((torch.randn(vnew.shape, generator=g, device="cuda") * (1 + step)).to(dt))
        pools[0].append(seqs, n_new, knew, vnew)
        app()
        drop = rng.integers(0, nq, size=B).astype(np.int32)
        pools[0].rollback(seqs, drop)
        rb(drop)
        torch.cuda.synchronize()
        a, b = pools
        assert [a.table(s) for s in range(B)] == [b.table(s) for s in range(B)]
        assert torch.equal(a.seq_lens, b.seq_lens) and torch.equal(a.block_table, b.block_table)
        assert torch.equal(a.k_pages.view(torch.uint8), b.k_pages.view(torch.uint8))
        assert torch.equal(a.v_pages.view(torch.uint8), b.v_pages.view(torch.uint8))
        if a.k_scale is not None:
            assert torch.equal(a.k_scale.view(torch.uint8), b.k_scale.view(torch.uint8))
            assert torch.equal(a.v_scale.view(torch.uint8), b.v_scale.view(torch.uint8))
