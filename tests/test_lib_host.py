"""Host-side tests of libpkvspec.so (no GPU): exports, allocator bookkeeping
against the oracle pool model, error paths, tree masks."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from oracle.attention import tree_masks
from oracle.pool import OutOfPages as OracleOOP
from oracle.pool import PoolModel
from paged_kv_speculative_amd import OutOfPages, PkvError, Pool, tree_ancestor_masks
from paged_kv_speculative_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "pkv_spec.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"typedef struct \{.*?\}\s*\w+;", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names) - {"defined"})


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 17
    lib = C.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTS)


def test_status_strings_and_version():
    assert _lib.lib.pkv_status_string(0) == b"ok"
    assert _lib.lib.pkv_status_string(2) == b"out of pages"
    assert b"gfx950" in _lib.lib.pkv_version()
    assert _lib.lib.pkv_page_bytes(1, 16, 128) == 4096
    assert _lib.lib.pkv_page_bytes(2, 16, 128) == 2048
    assert _lib.lib.pkv_page_bytes(0, 16, 64) == 4096
    assert _lib.lib.pkv_page_bytes(1, 8, 128) == 0


def test_tree_masks_match_oracle():
    rng = np.random.default_rng(0)
    for _ in range(50):
        n = int(rng.integers(1, 65))
        parents = [-1] + [int(rng.integers(0, i)) for i in range(1, n)]
        assert tree_ancestor_masks(parents) == tree_masks(parents)
    with pytest.raises(PkvError):
        tree_ancestor_masks([0, 0])
    with pytest.raises(PkvError):
        tree_ancestor_masks([-1, 2, 0])


def _tables_equal(lib_pool, model):
    for seq in model.tables:
        pages, length, _ = lib_pool.table(seq)
        assert pages == model.tables[seq] and length == model.lens[seq], seq
    st = lib_pool.stats()
    assert st["free_pages"] == len(model.free)
    assert st["num_seqs"] == len(model.tables)
    assert st["cow_copies"] == model.cow_copies
    for p in range(model.P):
        assert lib_pool.refcount(p) == model.refcount[p]


def test_random_ops_match_oracle_pool():
    rng = np.random.default_rng(1)
    P, S = 48, 16
    order = rng.permutation(P)
    lib_pool = Pool(P, 1, 64, "bf16", max_seqs=64, max_pages_per_seq=64, free_order=order)
    model = PoolModel(P, S, 1, 1, free_order=order)
    live, nid = [], 0
    for step in range(1500):
        op = int(rng.integers(0, 6))
        if op == 0 or not live:
            src = live[int(rng.integers(len(live)))] if live and rng.random() < 0.6 else None
            n_sh = int(rng.integers(0, model.lens[src] + 1)) if src is not None else 0
            model.alloc(nid, src, n_sh)
            lib_pool.alloc(nid, -1 if src is None else src, n_sh)
            live.append(nid)
            nid += 1
        elif op in (1, 2, 3):
            k = int(rng.integers(1, min(4, len(live)) + 1))
            seqs = list(rng.choice(live, size=k, replace=False))
            ns = [int(rng.integers(0, 40)) for _ in seqs]
            # the library call is atomic over the batch; mirror it on a copy
            import copy
            trial = copy.deepcopy(model)
            try:
                for s, n in zip(seqs, ns):
                    trial.append(s, np.zeros((n, 1, 1)), np.zeros((n, 1, 1)))
                ok = True
            except OracleOOP:
                ok = False
            if ok:
                lib_pool.append(seqs, ns)
                model = trial
            else:
                with pytest.raises(OutOfPages):
                    lib_pool.append(seqs, ns)
        elif op == 4:
            s = live[int(rng.integers(len(live)))]
            n = int(rng.integers(0, model.lens[s] + 1))
            model.rollback(s, n)
            lib_pool.rollback([s], [n])
        else:
            s = live.pop(int(rng.integers(len(live))))
            model.release(s)
            lib_pool.release(s)
        if step % 10 == 0:
            _tables_equal(lib_pool, model)
    _tables_equal(lib_pool, model)


def test_rollback_restores_free_set_and_tables():
    order = np.random.default_rng(2).permutation(40)
    p = Pool(40, 2, 128, "bf16", free_order=order)
    p.alloc(7)
    p.append([7], [37])
    before = (p.table(7), p.stats())
    for m in (1, 5, 11, 27):
        p.append([7], [m])
        p.rollback([7], [m])
        assert (p.table(7), p.stats()) == before


def test_errors_leave_state_unchanged():
    p = Pool(4, 1, 64, "bf16", max_seqs=2, max_pages_per_seq=3)
    p.alloc(1)
    p.append([1], [20])
    before = (p.table(1), p.stats())
    with pytest.raises(OutOfPages):
        p.alloc(2)
        p.append([2], [40])           # needs 3 pages, 2 free
    after_alloc = p.stats()
    with pytest.raises(PkvError) as e:
        p.append([1], [40])           # 60 tokens > 3 pages of capacity
    assert e.value.status == 9
    with pytest.raises(PkvError) as e:
        p.append([99], [1])
    assert e.value.status == 3
    with pytest.raises(PkvError) as e:
        p.append([1, 1], [1, 1])
    assert e.value.status == 1
    with pytest.raises(PkvError) as e:
        p.rollback([1], [21])
    assert e.value.status == 1
    with pytest.raises(PkvError) as e:
        p.alloc(1)
    assert e.value.status == 4
    with pytest.raises(PkvError) as e:
        p.alloc(3)                    # both block-table rows in use
    assert e.value.status == 8
    with pytest.raises(PkvError) as e:
        p.alloc(4, 1, 21)             # shared prefix longer than the source
    assert p.table(1) == before[0]
    assert p.stats() == after_alloc
    # a whole-call failure (second sequence does not fit) changes nothing
    p.release(2)
    p.alloc(2)
    snap = (p.table(1), p.table(2), p.stats())
    with pytest.raises(OutOfPages):
        p.append([1, 2], [10, 40])
    assert (p.table(1), p.table(2), p.stats()) == snap


def test_shared_prefix_cow_accounting():
    p = Pool(64, 8, 128, "bf16")
    p.alloc(0)
    p.append([0], [800])
    for s in range(1, 6):
        p.alloc(s, 0, 800)
    st = p.stats()
    assert st["used_pages"] == 50 and st["shared_pages"] == 50
    # partial shared page -> copy on first append
    q = Pool(8, 1, 64, "bf16")
    q.alloc(0)
    q.append([0], [24])
    q.alloc(1, 0, 20)
    q.append([1], [3])
    assert q.stats()["cow_copies"] == 1
    assert q.table(1)[0][0] == q.table(0)[0][0] and q.table(1)[0][1] != q.table(0)[0][1]


def test_layout_maps_are_bijections():
    """The documented page layouts place every (token, channel) at a distinct
    offset inside one slab."""
    from layout_ref import k_index, v_index
    for D in (64, 128):
        t = np.arange(16)[:, None]
        c = np.arange(D)[None, :]
        for dt in ("bf16", "fp8"):
            for f in (lambda: k_index(t, c, dt, D), lambda: v_index(t, c, dt)):
                idx = f().reshape(-1)
                assert sorted(idx.tolist()) == list(range(16 * D))


def test_commit_path_bookkeeping_matches_oracle():
    """paged_kv_commit_path on a metadata-only pool keeps the same pages,
    lengths and free set as the oracle's commit (moves need a GPU)."""
    rng = np.random.default_rng(12)
    order = rng.permutation(120).astype(np.int32)
    lp = Pool(120, 1, 64, "bf16", max_seqs=8, max_pages_per_seq=32, free_order=order)
    model = PoolModel(120, 16, 1, 1, free_order=order)
    parents = [-1, 0, 0, 0, 1, 1, 2, 3, 4, 4, 6, 8]
    kids = [[c for c in range(len(parents)) if parents[c] == u] for u in range(len(parents))]
    z = lambda n: np.zeros((n, 1, 1))
    for s in range(6):
        lp.alloc(s)
        model.alloc(s)
        ctx = int(rng.integers(0, 50))
        lp.append([s], [ctx + len(parents)])
        model.append(s, z(ctx + len(parents)), z(ctx + len(parents)))
    for rnd in range(3):
        paths = []
        for s in range(6):
            path, u = [], 0
            while kids[u] and rng.random() < 0.7:
                u = int(rng.choice(kids[u]))
                path.append(u)
            paths.append(path)
        lp.commit_path(range(6), [len(parents)] * 6, paths)
        for s in range(6):
            model.commit_path(s, len(parents), paths[s])
        _tables_equal(lp, model)
        assert lp.stats()["free_pages"] == len(model.free)
        for s in range(6):
            lp.append([s], [len(parents)])
            model.append(s, z(len(parents)), z(len(parents)))
    model.check_invariants()


def test_commit_path_errors_change_nothing():
    lp = Pool(40, 1, 64, "bf16", max_seqs=4, max_pages_per_seq=8)
    lp.alloc(0)
    lp.append([0], [30])
    before = lp.table(0)
    for n_tree, path in [(6, [2, 1]), (6, [6]), (6, [0]), (31, []), (0, []), (6, [1, 2, 3, 4, 5, 6])]:
        with pytest.raises(PkvError):
            lp.commit_path([0], [n_tree], [path])
        assert lp.table(0) == before
    with pytest.raises(PkvError):                  # listed twice
        lp.commit_path([0, 0], [6, 6], [[1], [1]])
    lp.alloc(1, 0, 30)                             # every page now shared
    with pytest.raises(PkvError):
        lp.commit_path([0], [6], [[3]])
    assert lp.table(0) == before
    lp.commit_path([0], [6], [[1, 2]])             # in place: no move, truncation only
    assert lp.table(0)[1] == 27


def test_argument_checks_of_newer_fields():
    """Host-side validation (no device work): FP8 tile pools, the cascade
    and tree-acceptance shapes."""
    lib = _lib.lib
    assert lib.pkv_page_bytes(3, 16, 128) == 2048 and lib.pkv_page_bytes(3, 16, 64) == 1024
    pool = Pool(32, 2, 128, "fp8mx", max_seqs=2, max_pages_per_seq=8)
    pool.alloc(0)
    pool.append([0], [40])
    assert pool.table(0)[1] == 40
    a = _lib.VerifyArgs()
    a.batch, a.n_q, a.num_q_heads, a.num_kv_heads, a.head_dim, a.page_size = 2, 5, 8, 2, 128, 16
    a.q_dtype, a.kv_dtype = _lib.BF16, _lib.FP8_E4M3
    a.sm_scale = 0.125
    a.q = a.k_pages = a.v_pages = a.block_table = a.seq_lens = a.k_scale = a.v_scale = 16
    a.block_table_stride = 8
    n = C.c_size_t()
    a.shared_prefix_pages = 1
    assert lib.spec_verify_workspace_size(C.byref(a), C.byref(n)) == 0       # per-page FP8 scales: accepted
    a.kv_dtype = _lib.FP8_E4M3_MX64
    assert lib.spec_verify_workspace_size(C.byref(a), C.byref(n)) == 5       # per-64-channel scales: not
    a.kv_dtype, a.shared_prefix_pages = _lib.BF16, -1
    assert lib.spec_verify_workspace_size(C.byref(a), C.byref(n)) == 1
    a.shared_prefix_pages, a.sm_scale = 0, 0.125
    assert lib.spec_verify_workspace_size(C.byref(a), C.byref(n)) == 0
    for bad in (0.0, -0.125, float("inf"), float("nan")):   # the softmax scale must be positive
        a.sm_scale = bad
        assert lib.spec_verify_workspace_size(C.byref(a), C.byref(n)) == 1, bad
    t = _lib.TreeAcceptArgs()
    t.batch, t.n_nodes, t.max_children, t.vocab = 2, 16, 4, 1000
    assert lib.spec_accept_tree_workspace_size(C.byref(t), C.byref(n)) == 0 and n.value > 0
    for field, bad in (("n_nodes", 1), ("n_nodes", 65), ("max_children", 0), ("max_children", 16),
                       ("vocab", 0)):
        t2 = _lib.TreeAcceptArgs()
        t2.batch, t2.n_nodes, t2.max_children, t2.vocab = 2, 16, 4, 1000
        setattr(t2, field, bad)
        assert lib.spec_accept_tree_workspace_size(C.byref(t2), C.byref(n)) == 1, field


def test_fused_append_needs_device_pool():
    """spec_verify_attention_append on a pool without device memory is refused
    (PKV_ERR_INVALID_ARG) and changes nothing; a null pool likewise."""
    p = Pool(8, 1, 64, "bf16")
    p.alloc(0)
    p.append([0], [5])
    snap = (p.table(0), p.stats())
    a = _lib.VerifyArgs()
    a.batch, a.n_q = 1, 1
    seqs = _lib.i64_array([0])
    assert _lib.lib.spec_verify_attention_append(p._h, 1, seqs, None, None, C.byref(a), None) == 1
    assert _lib.lib.spec_verify_attention_append(None, 1, seqs, None, None, C.byref(a), None) == 1
    assert (p.table(0), p.stats()) == snap


def test_prepared_rollback_matches_rollback_on_host_pool():
    """Pool.prepare_rollback marshals the sequences once; each call drops the
    given counts exactly as Pool.rollback does (tables, lengths, free set).  A
    prepared append needs device memory and is refused on a host-only pool."""
    order = np.random.default_rng(7).permutation(48)
    a = Pool(48, 2, 64, "bf16", max_seqs=4, max_pages_per_seq=16, free_order=order)
    b = Pool(48, 2, 64, "bf16", max_seqs=4, max_pages_per_seq=16, free_order=order)
    seqs = [0, 1, 2]
    for p in (a, b):
        for s in seqs:
            p.alloc(s)
        p.append(seqs, [37, 16, 5])
    rb = b.prepare_rollback(seqs)
    for drop in ([5, 0, 3], [16, 16, 2], [0, 0, 0]):
        a.rollback(seqs, drop)
        rb(np.asarray(drop, dtype=np.int32))
        assert [a.table(s) for s in seqs] == [b.table(s) for s in seqs]
        assert a.stats() == b.stats()
        a.append(seqs, [1, 2, 3])
        b.append(seqs, [1, 2, 3])
    with pytest.raises(ValueError):
        rb([1, 2])                     # one count per sequence
    with pytest.raises(ValueError):
        b.prepare_append(seqs, [1, 1, 1], None, None)
