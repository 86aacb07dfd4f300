"""Cascade attention over a shared prefix (shared_prefix_pages): the prefix
pages common to every sequence are attended once for all sequences and merged
with each sequence's own pages.  Checked against the oracle (which gathers
every sequence's full K/V and knows nothing of the sharing), for the split
counts that put units in place and across workers, at full size, with
per-sequence draft counts, through batch_slots, and against the plain call;
for bf16 KV and for FP8 KV with per-page scales."""
import numpy as np
import pytest
import torch

from paged_kv_speculative_amd import PkvError
from paged_kv_speculative_amd import workloads as wl
import harness as H

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("splits", [0, 1, 7, 64])
def test_cascade_matches_oracle(splits):
    w = wl.make(5, small=True)
    g = H.GpuSide(w)
    pref = w.prefix_len // 16
    O, L = g.verify(shared_prefix_pages=pref, num_splits=splits)
    O_ref, L_ref = H.oracle_verify(w, range(w.batch))
    H.compare(O.cpu().numpy(), L.cpu().numpy(), O_ref, L_ref, H.TOL["bf16"])


def test_cascade_equals_plain_call():
    w = wl.make(5, small=True, batch=9)
    g = H.GpuSide(w)
    O1, L1 = (x.clone() for x in g.verify())
    O2, L2 = g.verify(shared_prefix_pages=w.prefix_len // 16)
    O1, L1, O2, L2 = (x.cpu().numpy() for x in (O1, L1, O2, L2))
    rms = float(np.sqrt(np.mean(O1.astype(np.float64) ** 2)))
    assert np.max(np.abs(O1 - O2)) <= 1e-4 * rms and np.max(np.abs(L1 - L2)) <= 1e-4
    # a shorter shared part (the first page only) is a valid cascade as well
    O3, L3 = g.verify(shared_prefix_pages=1)
    assert np.max(np.abs(O1 - O3.cpu().numpy())) <= 1e-4 * rms


def test_cascade_full_size_sampled():
    w = wl.make(5)
    print(f"cascade full: B={w.batch} prefix={w.prefix_len}", flush=True)
    g = H.GpuSide(w)
    O, L = g.verify(shared_prefix_pages=w.prefix_len // 16)
    O, L = O.cpu().numpy(), L.cpu().numpy()
    rng = np.random.default_rng(5)
    sample = sorted(set([0, w.batch - 1, int(np.argmax(w.seq_lens))] + list(rng.choice(w.batch, 2, replace=False))))
    O_ref, L_ref = H.oracle_verify(w, sample)
    H.compare(O[sample], L[sample], O_ref, L_ref, H.TOL["bf16"])


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_cascade_with_per_sequence_counts(kv):
    """Per-sequence slot counts with the cascade: only slots i < n_b are
    computed and written."""
    w = wl.make(5, small=True)
    w.kv_dtype = kv
    g = H.GpuSide(w)
    nq = torch.tensor([5, 1, 3, 5, 2, 4][:w.batch], dtype=torch.int32, device="cuda")
    from paged_kv_speculative_amd import VerifyBuffers
    B, n_q, Hq, d = g.q.shape
    buf = VerifyBuffers(B, n_q, Hq, d, 1 << 27, "cuda")
    buf.out.fill_(7.0)
    O, L = g.verify(shared_prefix_pages=w.prefix_len // 16, n_q_seq=nq, buffers=buf)
    # with n_b slots the last n_b tokens are the verification slots and the
    # tokens before them are context: the oracle run per sequence with n_b
    from oracle import attention as oa
    qf = w.q_f32().astype(np.float64)
    O, L = O.cpu().numpy(), L.cpu().numpy()
    for b in range(B):
        n_b = int(nq[b])
        K, V = H.oracle_sequence_kv(w, b)
        Or, Lr = oa.verify_attention(qf[b:b + 1, :n_b], [K], [V], n_b, None, float(w.sm_scale))
        H.compare(O[b:b + 1, :n_b], L[b:b + 1, :n_b], Or, Lr, H.TOL[kv])
        assert np.all(O[b, n_b:] == 7.0)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("splits", [0, 5])
def test_cascade_with_batch_slots(splits, kv):
    """A permuted subset of the pool's rows (batch_slots) with the cascade:
    the prefix pass reads the shared pages through the first listed row (not
    row 0), and every listed sequence matches the oracle."""
    w = wl.make(5, small=True)
    w.kv_dtype = kv
    g = H.GpuSide(w)
    rows = [w.batch - 1, 0, w.batch // 2]
    slots = torch.tensor(rows, dtype=torch.int32, device="cuda")
    q = g.q[rows].contiguous()
    from paged_kv_speculative_amd import spec_verify_attention
    O, L = spec_verify_attention(q, g.pool.k_pages, g.pool.v_pages, g.pool.block_table, g.pool.seq_lens,
                                 n_q=w.n_q, num_kv_heads=w.num_kv_heads, kv_dtype=kv, batch_slots=slots,
                                 k_scale=g.pool.k_scale, v_scale=g.pool.v_scale,
                                 sm_scale=w.sm_scale, num_splits=splits,
                                 shared_prefix_pages=w.prefix_len // 16)
    O_ref, L_ref = H.oracle_verify(w, rows)
    H.compare(O.cpu().numpy(), L.cpu().numpy(), O_ref, L_ref, H.TOL[kv])


def _fp8(w, kv="fp8"):
    w.kv_dtype = kv
    return w


@pytest.mark.parametrize("splits", [0, 1, 7])
def test_cascade_fp8_matches_oracle(splits):
    """FP8 KV with per-page scales: the prefix pass decodes each page while
    staging it and applies the page's K and V scales; against the oracle's
    replay of the same quantised appends."""
    w = _fp8(wl.make(5, small=True))
    g = H.GpuSide(w)
    O, L = g.verify(shared_prefix_pages=w.prefix_len // 16, num_splits=splits)
    O_ref, L_ref = H.oracle_verify(w, range(w.batch))
    H.compare(O.cpu().numpy(), L.cpu().numpy(), O_ref, L_ref, H.TOL["fp8"])


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("splits", [0, 7])
def test_cascade_head_dim_64(kv, splits):
    """The d = 64 prefix pass (half the tiles per page; for FP8 half the
    threads stage a page) against the oracle."""
    w = _fp8(wl.make(5, small=True), kv)
    w.head_dim = 64
    g = H.GpuSide(w)
    O, L = g.verify(shared_prefix_pages=w.prefix_len // 16, num_splits=splits)
    O_ref, L_ref = H.oracle_verify(w, range(w.batch))
    H.compare(O.cpu().numpy(), L.cpu().numpy(), O_ref, L_ref, H.TOL[kv])


def test_cascade_fp8_equals_plain_call():
    """Same FP8 pool with and without the cascade: the same decoded values and
    scales, combined in another order.  Both passes feed each weight p to the
    bf16 products as a truncated high half plus a rounded remainder, which
    keeps p to 2^-16 of itself, so each side's O is within 2^-16 max|V| of
    the exact combination of the same decoded pages, and the two sides within
    twice that (plus fp32 reordering, far below it)."""
    w = _fp8(wl.make(5, small=True, batch=9))
    g = H.GpuSide(w)
    O1, L1 = (x.clone() for x in g.verify())
    O2, L2 = g.verify(shared_prefix_pages=w.prefix_len // 16)
    O1, L1, O2, L2 = (x.cpu().numpy() for x in (O1, L1, O2, L2))
    vmax = max([float(np.abs(w.prefix_kv()[1]).max())] +
               [float(np.abs(w.private_kv(b)[1]).max()) for b in range(w.batch)])
    tol = 2.0 ** -15 * vmax * 1.1                 # 1.1: FP8 rounding may round a value up
    assert np.max(np.abs(O1 - O2)) <= tol and np.max(np.abs(L1 - L2)) <= 1e-4


def test_cascade_fp8_full_size_sampled():
    w = _fp8(wl.make(5))
    print(f"cascade fp8 full: B={w.batch} prefix={w.prefix_len}", flush=True)
    g = H.GpuSide(w)
    O, L = g.verify(shared_prefix_pages=w.prefix_len // 16)
    O, L = O.cpu().numpy(), L.cpu().numpy()
    rng = np.random.default_rng(6)
    sample = sorted(set([0, w.batch - 1, int(np.argmax(w.seq_lens))] + list(rng.choice(w.batch, 2, replace=False))))
    O_ref, L_ref = H.oracle_verify(w, sample)
    H.compare(O[sample], L[sample], O_ref, L_ref, H.TOL["fp8"])


def test_cascade_rejects_fp8mx():
    """Per-64-channel FP8 scales are not supported by the prefix pass."""
    w = _fp8(wl.make(5, small=True, batch=2), "fp8mx")
    g = H.GpuSide(w)
    with pytest.raises(PkvError):
        g.verify(shared_prefix_pages=w.prefix_len // 16)
