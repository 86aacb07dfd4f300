"""Benchmark: one speculative verification step over a paged KV cache on one GPU.

A step is one pass of the whole path over the batch, as a serving loop runs it:
  1. paged_kv_append       the gamma+1 verification tokens' K/V of every sequence
  2. spec_verify_attention verification queries over each sequence's pages
  3. spec_accept           acceptance rule, accepted length, next token
  4. paged_kv_rollback     commit 1+k tokens, drop the rejected gamma-k
For a draft-tree workload steps 3 and 4 are spec_accept_tree (accepted branch)
and paged_kv_commit_path (the branch's K/V moved into place, the rest dropped).
With --fused, steps 1 and 2 are one spec_verify_attention_append call (the
verification kernels write the new tokens themselves).
(the accepted lengths are read back to the host each step, as a serving loop
must to emit tokens).  Inputs are resident in HBM before the timed region.
Several independent pool instances (independent batches) are used round-robin
so that no step finds its KV in the 256 MB last-level cache.  The host issues
step s + 1 (the next instance) before it waits for step s's accepted lengths,
as a serving loop overlaps its host work with the GPU; each instance's commit
still precedes its next append.  --serial issues one step at a time.

Output: one JSON line.  `value` is whole-step throughput in query tokens per
second (batch * (gamma+1) / step time); `roofline` is measured on the
verification attention launch (partial + merge kernels) with HIP events on
the launch stream.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]
"""
import argparse
import ctypes as C
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
METRIC = "verify-attn KV GB/s & % of HBM peak; query-tokens/s at γ=4, 1 GPU"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--config", type=int, default=2, choices=[2, 3, 4, 5])
    ap.add_argument("--instances", type=int, default=0, help="pool copies used round-robin (0: auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--kv-dtype", choices=["bf16", "fp8", "fp8mx"], default=None,
                    help="override the workload's KV type (fp8mx: FP8 with a power-of-two scale per "
                         "64 channels of each token)")
    ap.add_argument("--no-cascade", action="store_true",
                    help="attend a shared prefix once per sequence instead of once for all sequences")
    ap.add_argument("--graph", action="store_true",
                    help="replay verification and acceptance from HIP graphs (measured slower than "
                         "eager launches on MI355X: 177 vs 168 us per step)")
    ap.add_argument("--fused", action="store_true",
                    help="append the new tokens inside the verification launch "
                         "(spec_verify_attention_append) instead of a separate paged_kv_append")
    ap.add_argument("--serial", action="store_true",
                    help="issue one step at a time (the host reads a step's accepted lengths before it "
                         "issues the next step) instead of keeping the next instance's step queued")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="kept for the counter commands; the 1 GiB reference copy always runs after the steps")
    return ap.parse_args()


TRAFFIC_PROFILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                               "verify_traffic_llama3-8b-layer.md")


SAMPLE_EVERY = 4          # timed steps per sampled verification (and acceptance) timing


def kernel_build_digest(sources):
    """sha256 over the given source files (repository-relative) followed by
    the hipcc flags the build script compiles the first of them with."""
    import hashlib
    import importlib.util
    root = os.path.dirname(os.path.abspath(__file__))
    spec = importlib.util.spec_from_file_location(
        "_pkv_build_flags", os.path.join(root, "paged_kv_speculative_amd", "csrc", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    h = hashlib.sha256()
    for name in sources:
        h.update(open(os.path.join(root, name), "rb").read())
    rel = os.path.relpath(os.path.join(root, sources[0]),
                          os.path.join(root, "paged_kv_speculative_amd", "csrc"))
    h.update(" ".join(b.FLAGS + b.EXTRA.get(rel, [])).encode())
    return h.hexdigest()


def measured_traffic(config):
    """HBM-side bytes per verification call from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy), or None when the
    summary is for another workload or the kernel has changed since: the
    summary names the source files that make the kernel and the sha256 of
    their contents followed by the kernel file's compile flags."""
    if config != 2 or not os.path.exists(TRAFFIC_PROFILE):
        return None
    fields = {}
    for line in open(TRAFFIC_PROFILE):
        k, sep, v = line.strip().partition(": ")
        if sep:
            fields[k] = v.strip()
    try:
        if kernel_build_digest(fields["kernel_source"].split()) != fields["kernel_source_sha256"]:
            return None
        return float(fields["traffic_bytes_per_call"])
    except (KeyError, OSError, ValueError):
        return None


def kv_bytes(lens, w):
    """Algorithmic KV bytes of one verification call: every K and V element of
    every token of every sequence once (the shared prefix counted once), plus
    the FP8 scales of the pages read."""
    elem = {"bf16": 2, "f32": 4, "fp8": 1, "fp8mx": 1}[w.kv_dtype]
    per_tok = w.num_kv_heads * 2 * w.head_dim * elem
    toks = int(np.sum(lens)) - (len(lens) - 1) * w.prefix_len if w.prefix_len else int(np.sum(lens))
    total = toks * per_tok
    if w.kv_dtype == "fp8":
        total += int(np.sum((np.asarray(lens) + 15) // 16)) * w.num_kv_heads * 2 * 4
    if w.kv_dtype == "fp8mx":                       # one exponent byte per 64 channels of every token
        total += toks * w.num_kv_heads * 2 * (w.head_dim // 64)
    return total


class Instance:
    """One copy of the workload: pool filled with every sequence's context."""

    def __init__(self, w, steps, torch, api, seed_offset):
        B, S = w.batch, 16
        self.w = w
        grow = steps * w.n_q
        pages = w.num_pages + B * (-(-grow // S) + 2)
        maxp = int(max(-(-int(n) // S) for n in w.seq_lens)) + -(-grow // S) + 4
        self.pool = api.Pool(pages, w.num_kv_heads, w.head_dim, w.kv_dtype, max_seqs=B,
                             max_pages_per_seq=maxp, free_order=np.random.default_rng(
                                 w.seed + seed_offset).permutation(pages), device="cuda")
        dt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
        if w.prefix_len:
            self.pool.alloc(0)
            pk, pv = w.prefix_kv()
            self.pool.append([0], [w.prefix_len], torch.from_numpy(pk).to(dt).cuda(),
                             torch.from_numpy(pv).to(dt).cuda())
            for b in range(1, B):
                self.pool.alloc(b, 0, w.prefix_len)
        else:
            for b in range(B):
                self.pool.alloc(b)
        for b in range(B):
            k, v = w.private_kv(b)
            ctx = int(w.cached_lens[b]) - w.prefix_len
            self.pool.append([b], [ctx], torch.from_numpy(np.ascontiguousarray(k[:ctx])).to(dt).cuda(),
                             torch.from_numpy(np.ascontiguousarray(v[:ctx])).to(dt).cuda())
        self.lens = np.asarray(w.cached_lens, dtype=np.int64).copy()
        # per-step inputs: new K/V of the n_q verification tokens, queries, logits
        g = torch.Generator(device="cuda")
        g.manual_seed(w.seed * 7 + seed_offset)
        n = B * w.n_q
        self.knew = torch.randn((n, w.num_kv_heads, w.head_dim), generator=g, device="cuda").to(dt)
        self.vnew = torch.randn((n, w.num_kv_heads, w.head_dim), generator=g, device="cuda").to(dt)
        self.q = torch.randn((B, w.n_q, w.num_q_heads, w.head_dim), generator=g,
                             device="cuda").to(torch.bfloat16)
        self.anc = None
        if w.tree_parents is not None:
            m = [api.tree_ancestor_masks(p) for p in w.tree_parents]
            self.anc = torch.tensor(np.array(m, dtype=np.uint64).view(np.int64), device="cuda")
        V, gam = w.accept_vocab, w.gamma
        self.accept = V > 0 and w.tree_parents is None
        self.tree_accept = V > 0 and w.tree_parents is not None
        if self.tree_accept:
            # logits at every tree node; node tokens drawn from the draft at
            # the parent (siblings independently)
            n = w.n_q
            par = torch.tensor(np.array(w.tree_parents, dtype=np.int32), device="cuda")
            self.parents = par
            self.T = torch.randn((B, n, V), generator=g, device="cuda") * w.accept_std
            self.D = torch.randn((B, n, V), generator=g, device="cuda") * w.accept_std
            tok = torch.full((B, n), -1, dtype=torch.int32, device="cuda")
            for c in range(1, n):
                rows = self.D[torch.arange(B, device="cuda"), par[:, c].long()]
                tok[:, c] = torch.multinomial(torch.softmax(rows, -1), 1, generator=g)[:, 0].to(torch.int32)
            self.tokens = tok
        if self.accept:
            self.T = torch.randn((B, gam + 1, V), generator=g, device="cuda") * w.accept_std
            self.D = torch.randn((B, gam, V), generator=g, device="cuda") * w.accept_std
            probs = torch.softmax(self.D.reshape(-1, V), -1)
            self.x = torch.multinomial(probs, 1, generator=g).reshape(B, gam).to(torch.int32)
            del probs
        self.verify = self.verify_append = self.accept_call = None
        self.step_t = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.graph_v = self.graph_a = self.accept_graph_call = None


def cascade_pages(args, w):
    """Whole pages of the shared prefix attended once for all sequences
    (bf16 and per-page-scale FP8 KV; off with --no-cascade)."""
    if args.no_cascade or not w.prefix_len or w.kv_dtype not in ("bf16", "fp8"):
        return 0
    return w.prefix_len // 16


def schedule_steps(first, last, launch, finish, serial=False):
    """Steps first..last-1 as launch(s) (append, verification, acceptance
    issued on the stream) and finish(s) (wait for the accepted lengths, then
    commit).  By default step s + 1 -- the next instance, an independent
    batch -- is issued before the host waits for step s, so the GPU has the
    next step queued while the host reads k and commits; with two or more
    instances used round-robin, each instance's commit is still issued before
    its next append.  serial=True issues one step at a time."""
    for s in range(first, last):
        launch(s)
        if serial:
            finish(s)
        elif s > first:
            finish(s - 1)
    if not serial and last > first:
        finish(last - 1)


def run_gpu(args, w, torch, api):
    B, nq, gam = w.batch, w.n_q, w.gamma
    total_steps = args.steps + args.warmup
    one = kv_bytes(w.seq_lens, w)
    R = args.instances or max(2, int(np.ceil(1.2e9 / max(one, 1))))
    R = min(R, 8)
    insts = [Instance(w, -(-total_steps // R) + 1, torch, api, r) for r in range(R)]
    # the accepted lengths (and tree nodes) of a step land in one of two pinned
    # host buffers: the chain acceptance writes its lengths there itself
    # (one prepared call per buffer), the tree acceptance's are copied
    k_host = [torch.empty(B, dtype=torch.int32, pin_memory=True) for _ in range(2)]
    nodes_host = [torch.empty((B, nq), dtype=torch.int32, pin_memory=True) for _ in range(2)]
    for I in insts:
        I.verify = I.pool.prepare_verify(I.q, nq, anc_mask=I.anc, sm_scale=w.sm_scale,
                                         shared_prefix_pages=cascade_pages(args, w))
        if args.fused:
            shp = (B, nq, w.num_kv_heads, w.head_dim)
            I.verify_append = I.pool.prepare_verify_append(
                np.arange(B), I.q, I.knew.view(shp), I.vnew.view(shp), anc_mask=I.anc, sm_scale=w.sm_scale,
                buffers=I.verify.buffers, shared_prefix_pages=cascade_pages(args, w))
        if I.accept:
            I.accept_calls = [api.PreparedAccept(I.T, I.D, I.x, seed=12345, accepted_len_out=k_host[j])
                              for j in range(2)]
            if args.graph:       # the captured launch reads its step counter from device memory
                I.accept_graph_call = api.PreparedAccept(I.T, I.D, I.x, seed=12345, step_tensor=I.step_t)
        if I.tree_accept:
            I.accept_call = api.PreparedTreeAccept(I.T, I.D, I.parents, I.tokens, seed=12345)
    seq_ids = np.arange(B, dtype=np.int64)
    n_new = np.full(B, nq, dtype=np.int32)
    for I in insts:                    # arguments marshalled once, as a serving loop would
        I.append_call = I.pool.prepare_append(seq_ids, n_new, I.knew, I.vnew)
        I.rollback_call = I.pool.prepare_rollback(seq_ids)
    cur = torch.cuda.current_stream()  # the launch stream, looked up once (each lookup costs ~3 us of host time)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(total_steps)]
    acc_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(total_steps)]
    step_lens, accepted = [], []
    # `done` marks the end of a step's work on the stream
    done = [torch.cuda.Event() for _ in range(2)]

    # HIP events around the verification and the acceptance on every
    # SAMPLE_EVERY-th timed step (each record holds the launch stream ~5 us and
    # costs host time, which would otherwise be counted in every step): the
    # verification on steps 0, 4, 8, ... after the warmup, the acceptance two
    # steps later (on the first step when there are fewer than three)
    acc_phase = min(SAMPLE_EVERY // 2, args.steps - 1)

    def sampled_verify(s):
        return s >= args.warmup and (s - args.warmup) % SAMPLE_EVERY == 0

    def sampled_accept(s):
        return s >= args.warmup and (s - args.warmup) % SAMPLE_EVERY == acc_phase

    def launch(s):
        """Steps 1-3 of step s (its instance's append, verification and
        acceptance) issued on the stream, ending with the accepted lengths'
        copy to the host."""
        I = insts[s % R]
        if not args.fused:
            I.append_call()
        I.lens += nq
        step_lens.append(I.lens.copy())
        timed_v = sampled_verify(s)                   # sampled: each record holds the stream ~5 us
        if timed_v:
            ev[s][0].record(cur)
        if args.fused:
            I.verify_append()
        elif I.graph_v is not None:
            I.graph_v.replay()
        else:
            I.verify()
        if timed_v:
            ev[s][1].record(cur)
        if I.accept or I.tree_accept:
            timed_acc = sampled_accept(s)
            if timed_acc:
                acc_ev[s][0].record(cur)
            k = None                                  # set where the lengths stay on the device
            if I.tree_accept:
                k, nodes, _ = I.accept_call(step=s)
                nodes_host[s % 2].copy_(nodes, non_blocking=True)
            elif I.graph_a is not None:
                I.graph_a.replay()                    # increments the step counter, then accepts
                k = I.accept_graph_call.buffers.accepted_len
            else:
                I.accept_calls[s % 2](step=s)         # writes the lengths into k_host[s % 2]
            if timed_acc:
                acc_ev[s][1].record(cur)
            if k is not None:
                k_host[s % 2].copy_(k, non_blocking=True)  # host needs k every step
        done[s % 2].record(cur)

    def finish(s):
        """Step 4 of step s once its accepted lengths are on the host: commit
        1 + k tokens per sequence (rollback of the rest, or the tree path)."""
        I = insts[s % R]
        done[s % 2].synchronize()
        if I.tree_accept:
            k = k_host[s % 2].numpy().copy()
            nd = nodes_host[s % 2].numpy()
            accepted.append(k)
            # keep each accepted branch, drop the rest of the tree
            I.pool.commit_path(seq_ids, n_new, [nd[b, :k[b]] for b in range(B)])
            I.lens -= (nq - 1) - k
            return
        k = k_host[s % 2].numpy().copy() if I.accept else np.full(B, gam, dtype=np.int32)
        accepted.append(k)
        drop = (nq - 1) - k
        I.rollback_call(drop)
        I.lens -= drop

    def run_steps(first, last):
        schedule_steps(first, last, launch, finish, args.serial)

    run_steps(0, args.warmup)
    torch.cuda.synchronize()
    if args.graph:
        # verification and acceptance of each instance captured once and
        # replayed every step (their arguments are fixed; the block tables,
        # lengths and the acceptance step counter are read from device memory)
        for I in insts:
            I.graph_v = torch.cuda.CUDAGraph()
            with torch.cuda.graph(I.graph_v):
                I.verify()
            if I.accept:
                I.graph_a = torch.cuda.CUDAGraph()
                with torch.cuda.graph(I.graph_a):
                    I.step_t.add_(1)
                    I.accept_graph_call(step=0)
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(args.warmup, total_steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timed = range(args.warmup, total_steps)
    attn_ms = np.array([ev[s][0].elapsed_time(ev[s][1]) for s in timed if sampled_verify(s)])
    attn_bytes = np.array([kv_bytes(step_lens[s], w) for s in timed if sampled_verify(s)],
                          dtype=np.float64)
    acc_ms = (np.array([acc_ev[s][0].elapsed_time(acc_ev[s][1]) for s in timed if sampled_accept(s)])
              if insts[0].accept or insts[0].tree_accept else None)
    res = {
        "wall_s": wall, "steps": args.steps, "instances": R,
        "attn_ms": attn_ms, "attn_bytes": attn_bytes, "acc_ms": acc_ms,
        "accept_direct": bool(insts[0].accept and not args.graph),
        "mean_k": float(np.mean([a.mean() for a in accepted[args.warmup:]])),
    }
    # a plain 1 GiB device-to-device copy, timed after the steps (outside the
    # timed region) as a measured reference for the verify rate
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(3)]
    for a, b in cev:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    copy_ms = min(a.elapsed_time(b) for a, b in cev)
    res["copy_gbps"] = 2.0 * (1 << 30) / (copy_ms / 1e3) / 1e9     # bytes read + written
    # the read-rate reference: a plain read of the same pages (every page of
    # every (sequence, KV head) the verification call reads, all 16 slots),
    # same partition over 1024 waves and the same loads, no arithmetic;
    # timed round-robin over the instances after the steps
    from paged_kv_speculative_amd import _lib
    sink = torch.empty(1024, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(4 * R)]
    for I in insts:                       # first launches (code object load) untimed
        _lib.check(_lib.lib.pkv_page_read_probe(C.byref(I.verify.args), sink.data_ptr(), 1024, stream))
    for j, (a, b) in enumerate(pev):
        I = insts[j % R]
        a.record()
        _lib.check(_lib.lib.pkv_page_read_probe(C.byref(I.verify.args), sink.data_ptr(), 1024, stream))
        b.record()
    torch.cuda.synchronize()
    probe_ms = np.array([a.elapsed_time(b) for a, b in pev])
    page_bytes = [int(np.sum((I.lens + 15) // 16)) * w.num_kv_heads * 2 * api.page_bytes(w.kv_dtype, w.head_dim)
                  for I in insts]
    res["probe_ms"] = probe_ms
    res["probe_bytes"] = np.array([page_bytes[j % R] for j in range(len(pev))], dtype=np.float64)
    del src, dst
    return res


_W_CACHE = {}


def _load_workloads():
    """The seeded input generators, loaded by file path so that a worker does
    not import the package (which loads the HIP library)."""
    import importlib.util
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "paged_kv_speculative_amd", "workloads.py")
    spec = importlib.util.spec_from_file_location("_pkv_workloads", path)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _oracle_worker_init():
    os.environ["OMP_NUM_THREADS"] = "1"
    os.environ["OPENBLAS_NUM_THREADS"] = "1"
    os.environ["MKL_NUM_THREADS"] = "1"


def _oracle_sequence(cfg, kv_dtype, b):
    """One sequence of the step on the oracle, as it stands: pool replay and
    gather, verification attention, acceptance.  Returns seconds spent."""
    from threadpoolctl import threadpool_limits

    from oracle import accept as oacc
    from oracle import attention as oatt
    from oracle import pool as opool
    key = (cfg, kv_dtype)
    if key not in _W_CACHE:
        wl = _load_workloads()
        w = wl.make(cfg)
        if kv_dtype:
            w.kv_dtype = kv_dtype
        acc = None
        if w.accept_vocab:
            acc = (w.accept_inputs(step=0, batch=min(w.batch, 8)) if w.tree_parents is None
                   else w.tree_accept_inputs(step=0, batch=min(w.batch, 4)))
        _W_CACHE[key] = (w, w.q_f32().astype(np.float64), acc)
    w, q, acc = _W_CACHE[key]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        n = int(w.seq_lens[b])
        pm = opool.PoolModel(-(-n // 16) + 2, 16, w.num_kv_heads, w.head_dim,
                             kv_dtype=w.kv_dtype if w.kv_dtype in ("fp8", "fp8mx") else "f64")
        pm.alloc(0)
        k, v = w.seq_kv(b)
        ctx = int(w.cached_lens[b])
        pm.append(0, k[:ctx], v[:ctx])
        pm.append(0, k[ctx:], v[ctx:])
        K, V = pm.gather(0)
        anc = None if w.tree_parents is None else [oatt.tree_masks(w.tree_parents[b])]
        oatt.verify_attention(q[b:b + 1], [K], [V], w.n_q, anc, float(w.sm_scale))
        if acc is not None:
            T, D, x = acc
            j = b % T.shape[0]
            if w.tree_parents is None:
                oacc.accept_one(T[j], D[j], x[j], 12345, 0, j)
            else:
                oacc.accept_tree_one(T[j], D[j], w.tree_parents[j], x[j], 12345, 0, j)
        return time.perf_counter() - t0


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(cfg, kv_dtype, budget_s, max_workers=16):
    """The oracle, as it stands, on a bounded sample of the same step: one
    worker process per host core this process may run on (at most
    max_workers, one BLAS thread each), sequences of the workload handed out
    in order, passes repeated until the wall-clock budget is reached.  Runs
    before anything touches the GPU (the workers are spawned fresh)."""
    import concurrent.futures as cf
    import multiprocessing as mp
    wl = _load_workloads()
    w = wl.make(cfg)
    B, nq = w.batch, w.n_q
    workers = max(1, min(len(os.sched_getaffinity(0)), max_workers))
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(workers, mp_context=ctx, initializer=_oracle_worker_init) as ex:
        # warm-up: every worker imports the oracle and builds the inputs once
        list(ex.map(_oracle_sequence, [cfg] * workers, [kv_dtype] * workers, [0] * workers))
        done, busy = 0, 0.0
        t0 = time.perf_counter()
        while True:
            futs = [ex.submit(_oracle_sequence, cfg, kv_dtype, b) for b in range(B)]
            busy += sum(f.result() for f in futs)
            done += B
            wall = time.perf_counter() - t0
            if wall >= budget_s or done >= 64 * B:
                break
    return {"value": done * nq / wall, "unit": "query-tokens/s", "cores": workers, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"{done} sequences ({done // B} pass(es) over all {B} sequences of the same "
                      f"workload: pool replay + gather, verification attention, acceptance over vocab "
                      f"{w.accept_vocab}), fp64 NumPy, {workers} worker processes with one BLAS "
                      f"thread each, {wall:.1f} s wall, {busy:.1f} s of worker time"}


def main():
    args = parse()
    if args.fused and args.graph:
        print("--fused does its pool bookkeeping on the host at every call: it is not replayed from a graph",
              file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the verification step would shard by sequence or KV head with no exchange)",
              file=sys.stderr)
        sys.exit(2)
    # the oracle's timing first: its worker processes start before this
    # process touches the GPU
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.config, args.kv_dtype, args.cpu_seconds)
    import torch

    import paged_kv_speculative_amd as api
    from paged_kv_speculative_amd import workloads
    w = workloads.make(args.config)
    if args.kv_dtype:
        w.kv_dtype = args.kv_dtype
    r = run_gpu(args, w, torch, api)
    B, nq = w.batch, w.n_q
    ms_step = 1e3 * r["wall_s"] / args.steps
    attn_s = r["attn_ms"] / 1e3
    gbps = r["attn_bytes"] / attn_s / 1e9
    achieved = float(np.sum(r["attn_bytes"]) / np.sum(attn_s) / 1e9)
    out = {
        "metric": METRIC,
        "value": B * nq / (r["wall_s"] / args.steps),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "launch": ("hip-graph (verification, acceptance)" if args.graph else "eager")
                  + (", append fused into verification" if args.fused else "")
                  + (", accepted lengths written to pinned host memory by the acceptance"
                     if r["accept_direct"] else "")
                  + ("; one step at a time" if args.serial
                     else "; next instance's step queued while the host reads accepted lengths"),
        "vs_baseline": None,
        "dtype": {"fp8": "fp8-kv/bf16", "fp8mx": "fp8-kv(mx64)/bf16"}.get(w.kv_dtype, "bf16"),
        "data": "synthetic",
        "config": {
            "workload": f"{workloads.CONFIG_NAMES[args.config]}: batch {B}, {w.num_q_heads} q / "
                        f"{w.num_kv_heads} KV heads, head_dim {w.head_dim}, {w.kv_dtype} KV, page 16, "
                        f"cached context {int(w.cached_lens.min())}..{int(w.cached_lens.max())}, "
                        f"n_q {nq} ({'tree' if w.tree_parents else 'chain'})"
                        + (f", acceptance over vocab {w.accept_vocab}" if w.accept_vocab else ""),
            "batch": B, "n_q": nq, "gamma": w.gamma, "instances": r["instances"],
            "shared_prefix_pages": cascade_pages(args, w),
        },
        "verify_attn": {
            "kv_gbps": achieved,
            "hbm_frac": achieved / HBM_PEAK_GBPS,
            "us_median": float(np.median(r["attn_ms"]) * 1e3),
            "us_p10": float(np.percentile(r["attn_ms"], 10) * 1e3),
            "us_p90": float(np.percentile(r["attn_ms"], 90) * 1e3),
            "kv_gbps_median": float(np.median(gbps)),
            "copy_gbps": r["copy_gbps"],
            "frac_of_copy": achieved / r["copy_gbps"],
            "kv_bytes_per_call": float(np.mean(r["attn_bytes"])),
            "query_tokens_per_s": float(B * nq / np.median(attn_s)),
        },
        "read_ceiling": {
            "what": "plain read of the same pages (all slots of every page of every sequence and KV head), "
                    "same wave partition and 16-byte non-temporal loads, no arithmetic; HIP events, "
                    "after the timed steps",
            "us_median": float(np.median(r["probe_ms"]) * 1e3),
            "bytes_per_call": float(np.mean(r["probe_bytes"])),
            "gbps": float(np.median(r["probe_bytes"] / (r["probe_ms"] / 1e3)) / 1e9),
            "frac_of_peak": float(np.median(r["probe_bytes"] / (r["probe_ms"] / 1e3)) / 1e9 / HBM_PEAK_GBPS),
            "verify_rate_frac": float(np.median(r["attn_bytes"] / (r["attn_ms"] / 1e3))
                                      / np.median(r["probe_bytes"] / (r["probe_ms"] / 1e3))),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": measured_traffic(args.config),
            "traffic_unit": "bytes per spec_verify_attention call (FETCH_SIZE + WRITE_SIZE)",
            "algorithmic_bytes": float(np.mean(r["attn_bytes"])),
        },
    }
    if r["acc_ms"] is not None and w.tree_parents is not None:
        # one pass over the target and draft rows of every internal node
        internal = sum(len(set(p[1:])) for p in w.tree_parents[:B])
        lb = 2 * internal * w.accept_vocab * 4
        out["spec_accept_tree"] = {"us_median": float(np.median(r["acc_ms"]) * 1e3),
                                   "logit_bytes": lb,
                                   "logit_gbps": lb / (np.median(r["acc_ms"]) / 1e3) / 1e9,
                                   "mean_accepted": r["mean_k"]}
    elif r["acc_ms"] is not None:
        lb = B * (2 * w.gamma + 1) * w.accept_vocab * 4
        out["spec_accept"] = {"us_median": float(np.median(r["acc_ms"]) * 1e3),
                              "logit_gbps": lb / (np.median(r["acc_ms"]) / 1e3) / 1e9,
                              "mean_accepted": r["mean_k"]}
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
