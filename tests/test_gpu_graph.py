"""Verification + acceptance captured in a HIP graph (torch.cuda.CUDAGraph)
and replayed: every replay must equal the eager calls bit for bit.  The
acceptance reads its step counter from device memory (step_ptr), which the
graph increments, so each replay draws new random numbers.  Replays are
interleaved with eager library calls, other device work and
synchronisations."""
import numpy as np
import pytest
import torch

from paged_kv_speculative_amd import PreparedAccept
from paged_kv_speculative_amd import workloads as wl
import harness as H

pytestmark = pytest.mark.gpu


def test_graph_replays_equal_eager():
    w = wl.make(5, small=True)
    g = H.GpuSide(w)
    T, D, x = w.accept_inputs(step=0)
    Tt, Dt = torch.from_numpy(T).cuda(), torch.from_numpy(D).cuda()
    xt = torch.from_numpy(x).cuda()
    step_t = torch.zeros(1, dtype=torch.int32, device="cuda")
    verify = g.pool.prepare_verify(g.q, w.n_q, anc_mask=g.anc, sm_scale=w.sm_scale)
    accept = PreparedAccept(Tt, Dt, xt, seed=77, step_tensor=step_t)
    eager_acc = PreparedAccept(Tt, Dt, xt, seed=77)
    ref = {}
    for s in (1, 2, 3, 4):
        O, L = verify()
        k, tok = eager_acc(step=s)
        torch.cuda.synchronize()
        ref[s] = (O.clone(), L.clone(), k.clone(), tok.clone())
    # the step counter through device memory gives the same draws
    step_t.fill_(2)
    k, tok = accept(step=0)
    torch.cuda.synchronize()
    assert torch.equal(k, ref[2][2]) and torch.equal(tok, ref[2][3])

    step_t.zero_()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step_t.add_(1)
        verify()
        accept(step=0)
    torch.cuda.synchronize()
    step_t.zero_()
    torch.cuda.synchronize()
    for s in (1, 2, 3, 4):
        graph.replay()
        torch.cuda.synchronize()
        O, L = verify.buffers.out, verify.buffers.lse
        k, tok = accept.buffers.accepted_len, accept.buffers.next_token
        assert int(step_t.item()) == s
        assert torch.equal(O, ref[s][0]) and torch.equal(L, ref[s][1]), s
        assert torch.equal(k, ref[s][2]) and torch.equal(tok, ref[s][3]), s
        # eager work between replays: another library call and a torch op
        eager_acc(step=99)
        _ = (Tt[:1] * 2).sum()
        torch.cuda.synchronize()
