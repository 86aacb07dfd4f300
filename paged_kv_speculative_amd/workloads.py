"""Seeded synthetic inputs for paged-KV speculative verification.

This module only draws random inputs (lengths, token K/V values, queries,
draft trees, logits, page orders).  It holds none of the method's arithmetic:
no attention, no paging, no quantisation, no acceptance.  Both the GPU path
and the CPU oracle consume its arrays.

Shapes follow the workloads the pages discuss: Llama-class GQA heads
(head_dim 128, 8 KV heads), page size 16 (paurushmuley.com, diagram
"PagedAttention virtual memory manager": block size 16), gamma = 4..5 drafts
(innvotechnologies.co: 4-token candidates; atozofsoftwareengineering.blog:
K = 5), contexts up to 32k (futurestack.online, section 3), FP8 KV with
per-block scales and draft trees (atozofsoftwareengineering.blog).

Every array is reproducible from (config, seed, index): per-sequence draws use
numpy's PCG64 seeded with (seed, tag, b) so one sequence can be regenerated
without the others.
"""
from dataclasses import dataclass, field

import numpy as np

PAGE = 16
VOCAB = 128256          # Llama-3 tokenizer size, the acceptance workload's vocab


def bf16_bits(x):
    """Round float32 values to bfloat16 (nearest, ties to even); returns the
    uint16 bit patterns.  Used to make bf16-valued inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(seed, tag, b=0):
    return np.random.default_rng([int(seed), int(tag), int(b)])


@dataclass
class Workload:
    name: str
    seed: int
    batch: int
    gamma: int
    n_q: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    kv_dtype: str                 # "f32" | "bf16" | "fp8" | "fp8mx"
    q_dtype: str                  # "f32" | "bf16"
    cached_lens: np.ndarray       # L_b
    prefix_len: int = 0           # tokens shared by every sequence (in common pages)
    tree_parents: list = None     # per sequence parent lists, or None (chain)
    num_pages: int = 0
    free_order: np.ndarray = None
    rollback_k: np.ndarray = None  # accepted lengths to commit (rollback of the rest)
    accept_vocab: int = 0
    accept_std: float = 2.0
    extras: dict = field(default_factory=dict)

    @property
    def seq_lens(self):
        return self.cached_lens + self.n_q

    @property
    def page_size(self):
        return PAGE

    @property
    def sm_scale(self):
        return np.float32(1.0 / np.sqrt(self.head_dim))

    # -- per-sequence token K/V -----------------------------------------------
    def _tokens(self, tag, b, n):
        """n tokens of [Hkv, d] N(0,1) values as float32 (bf16-valued for
        bf16 KV)."""
        x = _rng(self.seed, tag, b).standard_normal((n, self.num_kv_heads, self.head_dim),
                                                    dtype=np.float32)
        if self.kv_dtype == "bf16":
            x = bf16_to_f32(bf16_bits(x))
        return x

    def prefix_kv(self):
        return self._tokens(11, 0, self.prefix_len), self._tokens(12, 0, self.prefix_len)

    def private_kv(self, b):
        """K, V [N_b - prefix_len, Hkv, d] of sequence b's own tokens (its
        tail of the context followed by the n_q verification tokens)."""
        n = int(self.seq_lens[b]) - self.prefix_len
        return self._tokens(21, b, n), self._tokens(22, b, n)

    def seq_kv(self, b):
        """Full K, V [N_b, Hkv, d] of sequence b (float32 values)."""
        k, v = self.private_kv(b)
        if self.prefix_len:
            pk, pv = self.prefix_kv()
            k, v = np.concatenate([pk, k]), np.concatenate([pv, v])
        return k, v

    def step_kv(self, step):
        """K, V [B, n_q, Hkv, d] of the n_q tokens a later verification step
        appends (float32; bf16-valued for bf16 KV)."""
        x = [self._tokens(61 + 2 * step, b, self.n_q) for b in range(self.batch)]
        y = [self._tokens(62 + 2 * step, b, self.n_q) for b in range(self.batch)]
        return np.stack(x), np.stack(y)

    def step_q(self, step):
        """Queries [B, n_q, Hq, d] of a later verification step (bf16 bit
        patterns for bf16 queries)."""
        x = _rng(self.seed, 71, step).standard_normal(
            (self.batch, self.n_q, self.num_q_heads, self.head_dim), dtype=np.float32)
        return bf16_bits(x) if self.q_dtype == "bf16" else x

    # -- queries and masks ----------------------------------------------------
    def q(self):
        x = _rng(self.seed, 31).standard_normal(
            (self.batch, self.n_q, self.num_q_heads, self.head_dim), dtype=np.float32)
        if self.q_dtype == "bf16":
            return bf16_bits(x)
        return x

    def q_f32(self):
        q = self.q()
        return bf16_to_f32(q) if self.q_dtype == "bf16" else q

    # -- acceptance inputs ----------------------------------------------------
    def accept_inputs(self, step=0, batch=None):
        """Target logits [B, gamma+1, V], draft logits [B, gamma, V] ~ N(0, std)
        float32, and draft tokens x_i drawn from the draft distribution with
        the generator's own stream."""
        B = self.batch if batch is None else batch
        V, g = self.accept_vocab, self.gamma
        rng = _rng(self.seed, 41, step)
        T = (rng.standard_normal((B, g + 1, V), dtype=np.float32) * np.float32(self.accept_std))
        D = (rng.standard_normal((B, g, V), dtype=np.float32) * np.float32(self.accept_std))
        # draft tokens sampled from softmax(D) by inverse CDF with the harness's RNG
        u = rng.random((B, g))
        x = np.empty((B, g), dtype=np.int32)
        for b in range(B):
            for i in range(g):
                z = D[b, i].astype(np.float64)
                w = np.exp(z - z.max())
                c = np.cumsum(w)
                x[b, i] = min(int(np.searchsorted(c, u[b, i] * c[-1], side="right")), V - 1)
        return T, D, x

    def tree_accept_inputs(self, step=0, batch=None):
        """Draft-tree acceptance inputs: target and draft logits [B, n, V] ~
        N(0, std) float32 at every node, and node tokens [B, n] where node c's
        token is drawn from the draft distribution at its parent (siblings
        independently) with the generator's own stream; token 0 (the root,
        already emitted) is -1."""
        B = self.batch if batch is None else batch
        V, n = self.accept_vocab, self.n_q
        rng = _rng(self.seed, 43, step)
        T = rng.standard_normal((B, n, V), dtype=np.float32) * np.float32(self.accept_std)
        D = rng.standard_normal((B, n, V), dtype=np.float32) * np.float32(self.accept_std)
        u = rng.random((B, n))
        x = np.full((B, n), -1, dtype=np.int32)
        for b in range(B):
            par = self.tree_parents[b % len(self.tree_parents)]
            for c in range(1, n):
                z = D[b, par[c]].astype(np.float64)
                w = np.exp(z - z.max())
                cs = np.cumsum(w)
                x[b, c] = min(int(np.searchsorted(cs, u[b, c] * cs[-1], side="right")), V - 1)
        return T, D, x


def _pool_pages(seq_lens, prefix_len, factor=1.25):
    pages = sum(-(-int(n) // PAGE) for n in seq_lens)
    if prefix_len:
        # the shared prefix pages are stored once
        pages -= (len(seq_lens) - 1) * (prefix_len // PAGE)
    return int(np.ceil(factor * pages)) + 4


def _tree(rng, n_nodes=16, branching=(4, 2, 2)):
    """Draft tree of n_nodes including the root (slot 0): full levels by the
    branching factors, the last level cut at random to reach n_nodes.  Nodes
    in breadth-first order; returns the parent list."""
    parents = [-1]
    level = [0]
    for br in branching:
        cand = [(p, c) for p in level for c in range(br)]
        room = n_nodes - len(parents)
        if room <= 0:
            break
        if len(cand) > room:
            keep = sorted(rng.choice(len(cand), size=room, replace=False))
            cand = [cand[i] for i in keep]
        nxt = []
        for p, _ in cand:
            parents.append(p)
            nxt.append(len(parents) - 1)
        level = nxt
    return parents


CONFIG_NAMES = {
    1: "tiny-verify",
    2: "llama3-8b-layer",
    3: "70b-layer-splitk-rollback",
    4: "tree-fp8",
    5: "shared-prefix-accept",
}


def make(cfg, small=False, batch=None, seed=None):
    """Build config cfg (1..5).  small=True keeps the structure but shrinks the
    batch and contexts so the oracle finishes in seconds."""
    seed = 1000 + cfg if seed is None else seed
    rng = _rng(seed, 1)
    if cfg == 1:
        w = Workload("tiny-verify", seed, 2, 4, 5, 2, 2, 64, "f32", "f32",
                     np.array([37, 100]))
        w.num_pages = 16
    elif cfg == 2:
        B = batch or (4 if small else 32)
        lo, hi = (40, 300) if small else (512, 4096)
        w = Workload("llama3-8b-layer", seed, B, 4, 5, 32, 8, 128, "bf16", "bf16",
                     rng.integers(lo, hi + 1, size=B))
    elif cfg == 3:
        B = batch or (3 if small else 64)
        lo, hi = (200, 700) if small else (1024, 32768)
        w = Workload("70b-layer-splitk-rollback", seed, B, 5, 6, 64, 8, 128, "bf16", "bf16",
                     rng.integers(lo, hi + 1, size=B))
        # accepted lengths with Pr(K >= i) = 0.85^i, capped at gamma
        u = rng.random(B)
        w.rollback_k = np.minimum(np.floor(np.log(u) / np.log(0.85)), 5).astype(np.int32)
    elif cfg == 4:
        B = batch or (3 if small else 16)
        L = 100 if small else 8192
        w = Workload("tree-fp8", seed, B, 15, 16, 32, 8, 128, "fp8", "bf16",
                     np.full(B, L))
        w.tree_parents = [_tree(_rng(seed, 51, b)) for b in range(B)]
        w.accept_vocab = 1000 if small else VOCAB
    elif cfg == 5:
        B = batch or (6 if small else 256)
        prefix = 48 if small else 800
        med, cap = (60, 300) if small else (1200, 8000)
        tails = np.floor(np.minimum(cap, np.exp(np.log(med) + 1.0 * rng.standard_normal(B))))
        w = Workload("shared-prefix-accept", seed, B, 4, 5, 32, 8, 128, "bf16", "bf16",
                     prefix + tails.astype(np.int64))
        w.prefix_len = prefix
        w.accept_vocab = 1000 if small else VOCAB
    else:
        raise ValueError(cfg)
    w.cached_lens = np.asarray(w.cached_lens, dtype=np.int64)
    if not w.num_pages:
        w.num_pages = _pool_pages(w.seq_lens, w.prefix_len)
    w.free_order = _rng(seed, 2).permutation(w.num_pages).astype(np.int32)
    if cfg in (2, 3) and not w.accept_vocab:
        # the acceptance step of a full verify step uses the same logit model
        w.accept_vocab = 1000 if small else VOCAB
    return w
