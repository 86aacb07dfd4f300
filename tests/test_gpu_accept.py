"""GPU parity of spec_accept against the oracle, and the pages' closed forms
checked on the GPU's own draws.

Decisions (accepted length, token) must equal the oracle's exactly, except
where the oracle reports a tie the fp32 kernel may resolve either way:
an acceptance test with |u - min(1, P/Q)| < 1e-5, or a Gumbel-max draw whose
two best keys are closer than 1e-4."""
import numpy as np
import pytest
import torch

from oracle import accept as oc
from paged_kv_speculative_amd import spec_accept
from paged_kv_speculative_amd import workloads as wl

pytestmark = pytest.mark.gpu

ACCEPT_TIE = 1e-5
SAMPLE_TIE = 1e-4


def _gpu(T, D, x, seed, step):
    Tt = torch.from_numpy(np.ascontiguousarray(T, dtype=np.float32)).cuda()
    Dt = torch.from_numpy(np.ascontiguousarray(D, dtype=np.float32)).cuda()
    xt = torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()
    k, tok = spec_accept(Tt, Dt, xt, seed, step)
    torch.cuda.synchronize()
    return k.cpu().numpy(), tok.cpu().numpy()


def _check_against_oracle(T, D, x, seed, step):
    k, tok = _gpu(T, D, x, seed, step)
    ko, to, info = oc.spec_accept(T, D, x, seed, step)
    ties = 0
    for b in range(len(k)):
        if min(info[b]["accept_margins"], default=1.0) < ACCEPT_TIE:
            ties += 1
            continue
        assert k[b] == ko[b], (b, k[b], ko[b])
        if info[b]["sample_gap"] < SAMPLE_TIE:
            ties += 1
            continue
        assert tok[b] == to[b], (b, tok[b], to[b], info[b]["source"])
    return k, tok, ties


@pytest.mark.parametrize("small", [True, False])
def test_config5_acceptance_parity(small):
    w = wl.make(5, small=small)
    T, D, x = w.accept_inputs(step=0)
    print(f"accept B={w.batch} V={w.accept_vocab}", flush=True)
    k, tok, ties = _check_against_oracle(T, D, x, seed=1234, step=0)
    assert ties <= max(1, w.batch // 50)
    assert np.all((k >= 0) & (k <= w.gamma)) and np.all((tok >= 0) & (tok < w.accept_vocab))


def test_unaligned_vocab_and_steps():
    rng = np.random.default_rng(1)
    B, g, V = 7, 3, 1001
    T = rng.standard_normal((B, g + 1, V)).astype(np.float32)
    D = (T[:, :g] + 0.3 * rng.standard_normal((B, g, V))).astype(np.float32)
    x = rng.integers(0, V, (B, g)).astype(np.int32)
    for step in (0, 1, 77):
        _check_against_oracle(T, D, x, seed=99, step=step)


def _independent(rng, gamma, V, noise):
    T = rng.standard_normal((gamma + 1, V)) * 1.5
    Dl = T[:gamma] + rng.standard_normal((gamma, V)) * noise
    return T, Dl


def _softmax(z):
    e = np.exp(z - z.max(-1, keepdims=True))
    return e / e.sum(-1, keepdims=True)


def test_monte_carlo_expected_length_on_gpu():
    """E[K] = sum_i prod_{j<=i} beta_j (innvotechnologies.co, eq. E[K]) with
    beta_j = sum_x min(P_j, Q_j), on the GPU's own acceptance draws."""
    rng = np.random.default_rng(2)
    gamma, V, B = 4, 32, 100000
    T, Dl = _independent(rng, gamma, V, 0.5)
    P, Q = _softmax(T), _softmax(Dl)
    beta = np.minimum(P[:gamma], Q).sum(1)
    closed = oc.expected_accepted(beta)
    x = np.stack([rng.choice(V, size=B, p=Q[i]) for i in range(gamma)], 1).astype(np.int32)
    Tb = np.broadcast_to(T.astype(np.float32), (B, gamma + 1, V))
    Db = np.broadcast_to(Dl.astype(np.float32), (B, gamma, V))
    k, tok = _gpu(Tb, Db, x, seed=7, step=3)
    se = k.std() / np.sqrt(B)
    assert abs(k.mean() - closed) < 5 * se, (k.mean(), closed, se)
    for i in range(1, gamma + 1):
        p = np.prod(beta[:i])
        assert abs((k >= i).mean() - p) < 5 * np.sqrt(p * (1 - p) / B) + 1e-9
    # first emitted token ~ P_0 (exactness of the resample)
    first = np.where(k >= 1, x[:, 0], tok)
    counts = np.bincount(first, minlength=V)
    exp = P[0] * B
    keep = exp > 5
    chi2 = (((counts - exp) ** 2 / exp)[keep]).sum()
    dof = keep.sum() - 1
    assert chi2 < dof + 6 * np.sqrt(2 * dof), (chi2, dof)


def test_pages_regime_alpha_085():
    """Correlated draft (alpha ~ 0.85, the pages' regime): GPU mean accepted
    length against the closed form, and eta from the pages' formula."""
    rng = np.random.default_rng(3)
    gamma, V, B = 4, 64, 60000
    T = rng.standard_normal((gamma + 1, V)) * 2.0
    Dl = T[:gamma] + rng.standard_normal((gamma, V)) * 0.37
    P, Q = _softmax(T), _softmax(Dl)
    beta = np.minimum(P[:gamma], Q).sum(1)
    assert np.all(beta > 0.75)
    x = np.stack([rng.choice(V, size=B, p=Q[i]) for i in range(gamma)], 1).astype(np.int32)
    k, _ = _gpu(np.broadcast_to(T.astype(np.float32), (B, gamma + 1, V)),
                np.broadcast_to(Dl.astype(np.float32), (B, gamma, V)), x, seed=11, step=0)
    closed = oc.expected_accepted(beta)
    assert abs(k.mean() - closed) < 5 * k.std() / np.sqrt(B)
    assert oc.speedup(k.mean(), gamma, 0.08) > 2.0


def test_special_cases():
    rng = np.random.default_rng(4)
    B, g, V = 64, 4, 50
    T = rng.standard_normal((B, g + 1, V)).astype(np.float32)
    x = rng.integers(0, V, (B, g)).astype(np.int32)
    k, _ = _gpu(T, T[:, :g].copy(), x, 5, 0)          # P == Q: all accepted
    assert np.all(k == g)
    Tm = np.full((B, g + 1, V), -30.0, np.float32)
    Tm[..., :25] = rng.standard_normal((B, g + 1, 25))
    Dm = np.full((B, g, V), -30.0, np.float32)
    Dm[..., 25:] = rng.standard_normal((B, g, 25))
    k, tok = _gpu(Tm, Dm, np.full((B, g), 30, np.int32), 5, 0)
    assert np.all(k == 0) and np.all(tok < 25)
    bad = x.copy()
    bad[:, 1] = V + 3                                    # invalid draft token: rejected there
    k, _ = _gpu(T, T[:, :g].copy(), bad, 5, 0)
    assert np.all(k == 1)


@pytest.mark.parametrize("bad_token", [-1, "V", "V+5"])
def test_out_of_vocabulary_drafts_match_oracle(bad_token):
    """Draft tokens -1, V and V+5 at a random position of each sequence: the
    kernel's decisions and resampled tokens equal the oracle's, which rejects
    such a token at its position."""
    rng = np.random.default_rng(21)
    B, g, V = 48, 4, 3000
    T = (rng.standard_normal((B, g + 1, V)) * 2).astype(np.float32)
    D = T[:, :g] + (rng.standard_normal((B, g, V)) * 0.4).astype(np.float32)
    x = rng.integers(0, V, (B, g)).astype(np.int32)
    pos = rng.integers(0, g, B)
    bad = {"V": V, "V+5": V + 5}.get(bad_token, bad_token)
    x[np.arange(B), pos] = bad
    k, tok, ties = _check_against_oracle(T, D, x, seed=17, step=3)
    assert ties <= 1
    assert np.all(k <= pos)


def test_prepared_accept_matches():
    from paged_kv_speculative_amd import PreparedAccept
    rng = np.random.default_rng(11)
    B, gamma, V = 6, 4, 5000
    T = (rng.standard_normal((B, gamma + 1, V)) * 2).astype(np.float32)
    D = (rng.standard_normal((B, gamma, V)) * 2).astype(np.float32)
    x = rng.integers(0, V, (B, gamma)).astype(np.int32)
    Tt, Dt, xt = (torch.from_numpy(a).cuda() for a in (T, D, x))
    call = PreparedAccept(Tt, Dt, xt, seed=99)
    for step in (0, 5):
        k1, t1 = (a.clone() for a in call(step))
        k2, t2 = spec_accept(Tt, Dt, xt, 99, step)
        assert torch.equal(k1, k2) and torch.equal(t1, t2)


def test_accepted_lengths_written_to_pinned_host_memory():
    """accepted_len in pinned host memory: the kernels store the lengths there
    directly; after the stream passes the call they equal the device-buffer
    call's on several steps (workload-5 shapes, small)."""
    from paged_kv_speculative_amd import PreparedAccept
    w = wl.make(5, small=True)
    T, D, x = w.accept_inputs(step=0)
    Tt, Dt, xt = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (T, D, x))
    host = torch.full((w.batch,), -7, dtype=torch.int32, pin_memory=True)
    direct = PreparedAccept(Tt, Dt, xt, seed=4321, accepted_len_out=host)
    plain = PreparedAccept(Tt, Dt, xt, seed=4321)
    for step in (0, 3, 17):
        direct(step)
        k_dev, t_dev = (a.clone() for a in plain(step))
        torch.cuda.synchronize()
        assert torch.equal(host, k_dev.cpu())
        assert torch.equal(direct.buffers.next_token, t_dev)
    with pytest.raises(ValueError):
        PreparedAccept(Tt, Dt, xt, seed=1, accepted_len_out=torch.zeros(w.batch, dtype=torch.int32))
