"""O-C: speculative acceptance, accepted length and the next token — oracle side.

Rule (innvotechnologies.co, section "Verification Acceptance Probabilities and
Speedup Math", eq. alpha_i): draft token x_i is accepted with probability
alpha_i = min(1, P(x_i) / Q(x_i)), P the target and Q the draft distribution at
that position; verification stops at the first rejection, so the accepted
length k is the number of leading accepts (its mean is eq. E[K]).  On a
rejection the pipeline diagram resamples ("Rejection Recovery (Resample)");
when all gamma drafts are accepted the target's distribution at the next
position yields one more token (the "+1" of eq. eta).

Readings where the pages are silent or disagree:
  * P and Q are plain softmaxes of the logits (temperature 1);
  * the acceptance test is u_i < min(1, P/Q) with u_i a counter-based uniform
    (oracle.philox.accept_uniform); a draft token outside [0, V) is not a
    token of the target's vocabulary, so P(x_i) = 0 and it is rejected at its
    position (the same reading as for draft trees below);
  * on rejection at position k the token is drawn from the residual
    R(x) = max(0, P_k(x) - Q_k(x)) normalised, which is what makes the output
    follow the target distribution exactly (futurestack.online, section 2.1,
    asks for that exactness; its bundle-product rule of section 2.2 is not
    used).  If R is zero everywhere the token is drawn from P_k;
  * drawing from weights w uses the Gumbel-max construction:
    token = argmax_x log w(x) + g(x), g(x) = -log(-log u_x), u_x counter-based
    uniforms (oracle.philox.sample_uniforms); ties go to the smaller index.
    argmax over independent Gumbel-perturbed log weights is distributed as
    w / sum(w) (Gumbel 1954; the "Gumbel-max trick").

All arithmetic is fp64.  Besides the decisions, the functions report the
margins a lower-precision implementation may legitimately disagree on.
"""
import numpy as np

from . import philox


def log_softmax(x):
    x = np.asarray(x, dtype=np.float64)
    m = x.max()
    return x - (m + np.log(np.exp(x - m).sum()))


def gumbel(u):
    return -np.log(-np.log(u))


def _argmax_with_gap(keys):
    j = int(np.argmax(keys))
    best = keys[j]
    rest = np.delete(keys, j)
    second = rest.max() if rest.size else -np.inf
    return j, float(best - second)


def accept_one(T, D, x, seed, step, b):
    """One sequence.  T [gamma+1, V] target logits, D [gamma, V] draft logits,
    x [gamma] draft tokens.  Returns dict with k, token, bonus flag and the
    decision margins (|u - min(1, ratio)| per tested position, and the gap
    between the two best Gumbel keys of the sampling step)."""
    gamma = D.shape[0]
    V = T.shape[1]
    margins = []
    k = gamma
    for i in range(gamma):
        xi = int(x[i])
        if 0 <= xi < V:
            lp = log_softmax(T[i])
            lq = log_softmax(D[i])
            a = min(1.0, float(np.exp(lp[xi] - lq[xi])))
        else:
            a = 0.0             # a token outside the vocabulary has P = 0: always rejected
        u = philox.accept_uniform(seed, step, b, i)
        margins.append(abs(u - a))
        if not u < a:
            k = i
            break
    g = gumbel(philox.sample_uniforms(seed, step, b, k, V))
    if k < gamma:
        p = np.exp(log_softmax(T[k]))
        q = np.exp(log_softmax(D[k]))
        r = np.maximum(p - q, 0.0)
        if np.any(r > 0):
            with np.errstate(divide="ignore"):
                keys = np.where(r > 0, np.log(r), -np.inf) + g
            source = "residual"
        else:
            keys = log_softmax(T[k]) + g
            source = "target"
    else:
        keys = np.asarray(T[gamma], dtype=np.float64) + g
        source = "bonus"
    token, gap = _argmax_with_gap(keys)
    return {"k": k, "token": token, "source": source, "accept_margins": margins,
            "sample_gap": gap}


def spec_accept(target_logits, draft_logits, draft_tokens, seed, step):
    """Batch version.  target_logits [B, gamma+1, V], draft_logits [B, gamma, V],
    draft_tokens [B, gamma].  Returns (k [B], token [B], per-sequence info)."""
    B = target_logits.shape[0]
    ks, toks, info = [], [], []
    for b in range(B):
        r = accept_one(target_logits[b], draft_logits[b], draft_tokens[b], seed, step, b)
        ks.append(r["k"])
        toks.append(r["token"])
        info.append(r)
    return np.array(ks, dtype=np.int32), np.array(toks, dtype=np.int32), info


def expected_accepted(alphas):
    """Closed form E[K] = sum_i prod_{j<=i} alpha_j (innvotechnologies.co,
    eq. E[K])."""
    total, prod = 0.0, 1.0
    for a in alphas:
        prod *= a
        total += prod
    return total


def speedup(expected_k, gamma, r):
    """eta = (E[K] + 1) / (gamma * r + 1) (innvotechnologies.co, eq. eta)."""
    return (expected_k + 1.0) / (gamma * r + 1.0)


# ----------------------------------------------------------------------------
# Draft trees
# ----------------------------------------------------------------------------
# The pages verify a whole draft tree in one pass and then commit the accepted
# branch (atozofsoftwareengineering.blog, pipeline diagram: "Tree-Attention
# Verification" followed by "Dynamic KV Rollback/Commit") but state no
# acceptance rule for several candidates at one position.  Reading taken: the
# per-token rule of eq. alpha_i applied child by child with the residual
# update between candidates (multi-candidate speculative sampling, as in
# SpecInfer, Miao et al., ASPLOS 2024):
#   at node u with target P and draft Q, the children c_1 < c_2 < ... of u
#   (drafted i.i.d. from Q) are tried in index order; child c_j is accepted iff
#   u_{c_j} < min(1, P_{j-1}(x_{c_j}) / Q(x_{c_j})), where P_0 = P and
#   P_j = max(0, P_{j-1} - Q) normalised (P_j = P_{j-1} if that is zero
#   everywhere).  An accepted child becomes the new node; if every child is
#   rejected the next token is drawn from P_m (m = number of children); at a
#   leaf the next token is drawn from the leaf's P (the bonus).
# On a chain (one child per node) this is exactly accept_one with draft i =
# node i + 1, which is why the counters are indexed the same way: the test of
# node c uses accept_uniform(.., c - 1) and the draw at node u uses
# sample_uniforms(.., u, V).


def children_of(parents):
    n = len(parents)
    kids = [[] for _ in range(n)]
    for c in range(1, n):
        kids[parents[c]].append(c)
    return kids


def accept_tree_one(T, D, parents, tokens, seed, step, b):
    """One sequence.  T, D [n, V]: target and draft logits at each node (the
    distributions of that node's children); parents [n] (parents[0] = -1,
    parents[c] < c); tokens [n] (tokens[0], the root's, is not used).
    Returns dict with the accepted path (node ids, depth order, root
    excluded), k = its length, the next token, its source and the decision
    margins."""
    n, V = T.shape
    kids = children_of(parents)
    margins = []
    path = []
    u = 0
    while True:
        if not kids[u]:
            keys = np.asarray(T[u], dtype=np.float64) + gumbel(philox.sample_uniforms(seed, step, b, u, V))
            source = "bonus"
            break
        p = np.exp(log_softmax(T[u]))
        q = np.exp(log_softmax(D[u]))
        taken = None
        for c in kids[u]:
            x = int(tokens[c])
            a = min(1.0, p[x] / q[x]) if 0 <= x < V else 0.0   # a token outside the vocabulary is rejected
            uc = philox.accept_uniform(seed, step, b, c - 1)
            margins.append(abs(uc - a))
            if uc < a:
                taken = c
                break
            r = np.maximum(p - q, 0.0)
            if np.any(r > 0):
                p = r / r.sum()
        if taken is not None:
            path.append(taken)
            u = taken
            continue
        with np.errstate(divide="ignore"):
            keys = np.log(p) + gumbel(philox.sample_uniforms(seed, step, b, u, V))
        source = "residual"
        break
    token, gap = _argmax_with_gap(keys)
    return {"k": len(path), "path": path, "node": u, "token": token, "source": source,
            "accept_margins": margins, "sample_gap": gap}


def spec_accept_tree(target_logits, draft_logits, parents, tokens, seed, step):
    """Batch version.  target_logits, draft_logits [B, n, V]; parents, tokens
    [B, n].  Returns (k [B], token [B], paths, per-sequence info)."""
    B = target_logits.shape[0]
    out = [accept_tree_one(target_logits[b], draft_logits[b], list(parents[b]), tokens[b],
                           seed, step, b) for b in range(B)]
    k = np.array([r["k"] for r in out], dtype=np.int32)
    tok = np.array([r["token"] for r in out], dtype=np.int32)
    return k, tok, [r["path"] for r in out], out
