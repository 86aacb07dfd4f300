"""spec_verify_attention_static, the entry point that allocates nothing (its
scratch is a static array the library holds per GPU), against
spec_verify_attention with a caller workspace: the same kernels, so the same
outputs bit for bit, on consecutive calls whose sizes shrink (the array keeps
the previous call's contents), and within the accuracy target of the oracle.
Calls through the C ABI (the binding marshals arguments only)."""
import numpy as np
import pytest
import torch

import harness as H
from paged_kv_speculative_amd import PkvError, spec_verify_attention_static
from paged_kv_speculative_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _outputs(g):
    B, nq, Hq, d = g.q.shape
    return (torch.full((B, nq, Hq, d), 12345.0, dtype=torch.float32, device="cuda"),
            torch.full((B, nq, Hq), 12345.0, dtype=torch.float32, device="cuda"))


def _static(g, outputs=None, **kw):
    w = g.w
    nq = g.q.shape[1]
    out, lse = outputs if outputs is not None else _outputs(g)
    pool = g.pool
    return spec_verify_attention_static(g.q, pool.k_pages, pool.v_pages, pool.block_table, pool.seq_lens,
                                        n_q=nq, num_kv_heads=w.num_kv_heads, kv_dtype=w.kv_dtype,
                                        out=out, lse=lse, k_scale=pool.k_scale, v_scale=pool.v_scale,
                                        anc_mask=g.anc, sm_scale=w.sm_scale, **kw)


def _case(cfg, small=True, batch=None, kv=None, **kw):
    w = wl.make(cfg, small=small, batch=batch)
    if kv is not None:
        w.kv_dtype = kv
    print(f"no-alloc cfg {cfg} small={small} B={w.batch} kv={w.kv_dtype} {kw}", flush=True)
    g = H.GpuSide(w)
    O_ws, L_ws = (x.clone() for x in g.verify(**kw))
    O_st, L_st = _static(g, **kw)
    torch.cuda.synchronize()
    assert torch.equal(O_st, O_ws) and torch.equal(L_st, L_ws)
    return w, O_st.cpu().numpy(), L_st.cpu().numpy()


def test_static_scratch_matches_workspace_on_shrinking_calls():
    # larger first (48 rows per KV head, long contexts split over many waves),
    # then smaller calls that find the first call's partials in the array
    calls = [dict(cfg=3), dict(cfg=2, batch=3), dict(cfg=2, batch=3, num_splits=5),
             dict(cfg=4), dict(cfg=5), dict(cfg=2, batch=1)]
    for c in calls:
        kw = {k: v for k, v in c.items() if k not in ("cfg", "batch")}
        if c["cfg"] == 5:
            kw["shared_prefix_pages"] = wl.make(5, small=True).prefix_len // 16
        w, O, L = _case(c["cfg"], batch=c.get("batch"), **kw)
        O_ref, L_ref = H.oracle_verify(w, range(w.batch))
        H.compare(O, L, O_ref, L_ref, H.TOL[w.kv_dtype])


def test_static_scratch_fp8_cascade():
    """The cascade over FP8 pages (per-page scales) through the static
    scratch, then a smaller plain call that finds its partials there."""
    pages = wl.make(5, small=True).prefix_len // 16
    for c in (dict(cfg=5, kv="fp8", shared_prefix_pages=pages),
              dict(cfg=5, kv="fp8", shared_prefix_pages=pages, num_splits=7),
              dict(cfg=2, batch=2)):
        w, O, L = _case(**c)
        O_ref, L_ref = H.oracle_verify(w, range(w.batch))
        H.compare(O, L, O_ref, L_ref, H.TOL[w.kv_dtype])


def test_static_scratch_full_size_llama_layer():
    """The benchmark's workload at full size in its launch configuration
    (auto split count) fits the static scratch; sampled against the oracle."""
    w, O, L = _case(2, small=False)
    sample = [0, w.batch - 1, int(np.argmax(w.seq_lens))]
    O_ref, L_ref = H.oracle_verify(w, sample)
    H.compare(O[sample], L[sample], O_ref, L_ref, H.TOL["bf16"])


def test_static_scratch_refuses_oversized_calls():
    """A call whose scratch exceeds the static array is refused before
    anything is enqueued (outputs keep their sentinel)."""
    w = wl.make(3, small=True)
    g = H.GpuSide(w)
    outputs = _outputs(g)
    with pytest.raises(PkvError) as e:
        _static(g, outputs, num_splits=1024)
    torch.cuda.synchronize()
    assert e.value.status == 7 and "static scratch" in str(e.value)
    assert bool(torch.all(outputs[0] == 12345.0)) and bool(torch.all(outputs[1] == 12345.0))
    O, L = _static(g, num_splits=64)            # a smaller split count fits
    O_ws, L_ws = g.verify(num_splits=64)
    torch.cuda.synchronize()
    assert torch.equal(O, O_ws) and torch.equal(L, L_ws)
