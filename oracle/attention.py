"""O-A: attention of the verification queries over a sequence's KV — oracle side.

What is computed (atozofsoftwareengineering.blog, section "Speculative Decoding
Mechanics & The K-Token Penalty", eq. A_speculative):

    A = Softmax((Q K^T + M) / sqrt(d_k)) V

with M an additive 0 / -inf mask.  Readings where the pages are silent:
  * the n_q = gamma + 1 verification queries (last emitted token plus the
    gamma drafts) have their own K/V appended to the sequence before
    attention, so a sequence of total length N has L = N - n_q cached tokens
    followed by the n_q verification slots (futurestack.online, section 2.3:
    the KV extension for the whole bundle happens before any decision);
  * cached tokens are visible to every query; verification slot j is visible
    to query i iff j is an ancestor-or-self of i in the draft tree (bit j of
    anc[i]); the chain (a plain draft sequence) is anc[i] = 2^(i+1) - 1;
  * GQA: query head h reads KV head h // (Hq / Hkv);
  * the softmax scale is passed explicitly as an fp32 number (1/sqrt(d));
  * outputs are fp32-or-better O and the natural-log log-sum-exp of the
    scaled, masked scores.

Everything here is fp64 with no blocking, splitting or online softmax: the
scores of a row are formed, the maximum subtracted, exponentiated, summed.
"""
import numpy as np


def chain_masks(n_q):
    """Ancestor-or-self bitmasks of a chain: anc[i] = 2^(i+1) - 1."""
    return [(1 << (i + 1)) - 1 for i in range(n_q)]


def tree_masks(parents):
    """Ancestor-or-self bitmasks from a parent list (parents[0] = -1 for the
    root, parents[i] < i).  Walks each node up to the root."""
    masks = []
    for i in range(len(parents)):
        m, j = 0, i
        while j >= 0:
            m |= 1 << j
            j = parents[j]
        masks.append(m)
    return masks


def visible(n_tokens, n_q, i, anc_i):
    """Boolean visibility of tokens 0..n_tokens-1 for verification query i."""
    L = n_tokens - n_q
    t = np.arange(n_tokens)
    vis = t < L
    for j in range(n_q):
        if (anc_i >> j) & 1:
            vis[L + j] = True
    return vis


def attend_one(q, K, V, vis, sm_scale):
    """One query row: q [d], K/V [N, d], vis [N] -> (o [d], lse)."""
    s = (K[vis] @ q) * float(sm_scale)
    m = s.max()
    e = np.exp(s - m)
    l = e.sum()
    o = (e[:, None] * V[vis]).sum(axis=0) / l
    return o, m + np.log(l)


def verify_attention(q, K_seqs, V_seqs, n_q, anc=None, sm_scale=None):
    """Verification attention for a batch.

    q       [B, n_q, Hq, d] (any float dtype; used exactly in fp64)
    K_seqs  list of [N_b, Hkv, d] fp64 arrays, the full sequences (cached
            tokens then the n_q verification slots)
    V_seqs  same shapes as K_seqs
    anc     None (chain) or [B][n_q] ancestor-or-self bitmasks
    Returns O [B, n_q, Hq, d] fp64 and LSE [B, n_q, Hq] fp64 (natural log).
    """
    q = np.asarray(q, dtype=np.float64)
    B, nq, Hq, d = q.shape
    assert nq == n_q
    if sm_scale is None:
        sm_scale = np.float32(1.0 / np.sqrt(d))
    O = np.zeros((B, n_q, Hq, d))
    LSE = np.zeros((B, n_q, Hq))
    for b in range(B):
        K = np.asarray(K_seqs[b], dtype=np.float64)
        V = np.asarray(V_seqs[b], dtype=np.float64)
        N, Hkv, _ = K.shape
        G = Hq // Hkv
        masks = chain_masks(n_q) if anc is None else [int(a) for a in anc[b]]
        for i in range(n_q):
            vis = visible(N, n_q, i, masks[i])
            for h in range(Hq):
                g = h // G
                O[b, i, h], LSE[b, i, h] = attend_one(q[b, i, h], K[:, g], V[:, g], vis, sm_scale)
    return O, LSE
