"""Python front end over the C ABI (marshalling only)."""
import ctypes as C

import numpy as np
import torch

from ._lib import (AcceptArgs, DTYPES, F32, BF16, FP8_E4M3, PoolDesc, PoolStats, TreeAcceptArgs,
                   VerifyArgs, check, i32_array, i64_array, lib)

PAGE_SIZE = 16
_TORCH_SRC = {torch.float32: F32, torch.bfloat16: BF16}


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream):
    """hipStream_t of `stream` (None: torch's current stream) as an address."""
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(torch.cuda.current_device())
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _ints(values, dtype):
    """(array, address) of a sequence of integers (list, range or ndarray) as
    a contiguous C array of `dtype`; the array keeps the memory alive."""
    if not (type(values) is np.ndarray and values.dtype == dtype and values.ndim == 1
            and values.flags.c_contiguous):
        values = np.ascontiguousarray(np.asarray(values, dtype=dtype).reshape(-1))
    return values, values.ctypes.data


def page_bytes(kv_dtype, head_dim, page_size=PAGE_SIZE):
    return int(lib.pkv_page_bytes(DTYPES[kv_dtype], page_size, head_dim))


def tree_ancestor_masks(parents):
    """Ancestor-or-self bitmask per node (host, via the library)."""
    n = len(parents)
    out = (C.c_uint64 * n)()
    check(lib.spec_tree_ancestor_masks(n, i32_array(parents), out))
    return [int(x) for x in out]


class Pool:
    """Page pool with device-resident block table and lengths.

    device=None gives a metadata-only pool (host bookkeeping, no kernels)."""

    def __init__(self, num_pages, num_kv_heads, head_dim, kv_dtype="bf16", max_seqs=64,
                 max_pages_per_seq=256, free_order=None, device=None):
        self.num_pages, self.num_kv_heads, self.head_dim = num_pages, num_kv_heads, head_dim
        self.kv_dtype, self.max_seqs, self.max_pages_per_seq = kv_dtype, max_seqs, max_pages_per_seq
        self.page_bytes = page_bytes(kv_dtype, head_dim)
        if self.page_bytes == 0:
            raise ValueError("unsupported kv_dtype/head_dim")
        self.device = device
        desc = PoolDesc()
        desc.num_pages, desc.page_size, desc.num_kv_heads = num_pages, PAGE_SIZE, num_kv_heads
        desc.head_dim, desc.kv_dtype = head_dim, DTYPES[kv_dtype]
        desc.max_seqs, desc.max_pages_per_seq = max_seqs, max_pages_per_seq
        self.k_pages = self.v_pages = self.k_scale = self.v_scale = None
        self.block_table = self.seq_lens = None
        if device is not None:
            shape = (num_pages, num_kv_heads, self.page_bytes)
            self.k_pages = torch.empty(shape, dtype=torch.uint8, device=device)
            self.v_pages = torch.empty(shape, dtype=torch.uint8, device=device)
            if kv_dtype == "fp8":
                self.k_scale = torch.ones((num_pages, num_kv_heads), dtype=torch.float32, device=device)
                self.v_scale = torch.ones((num_pages, num_kv_heads), dtype=torch.float32, device=device)
            elif kv_dtype == "fp8mx":
                # E8M0 exponent bytes per (page, head, token, 64-channel tile); 127 = scale 1
                shp = (num_pages, num_kv_heads, 16, head_dim // 64)
                self.k_scale = torch.full(shp, 127, dtype=torch.uint8, device=device)
                self.v_scale = torch.full(shp, 127, dtype=torch.uint8, device=device)
            self.block_table = torch.zeros((max_seqs, max_pages_per_seq), dtype=torch.int32, device=device)
            self.seq_lens = torch.zeros(max_seqs, dtype=torch.int32, device=device)
            desc.k_pages, desc.v_pages = self.k_pages.data_ptr(), self.v_pages.data_ptr()
            if self.k_scale is not None:
                desc.k_scale, desc.v_scale = self.k_scale.data_ptr(), self.v_scale.data_ptr()
            desc.block_table, desc.seq_lens = self.block_table.data_ptr(), self.seq_lens.data_ptr()
        order = None
        if free_order is not None:
            order = i32_array(np.asarray(free_order))
            desc.free_order = C.cast(order, C.POINTER(C.c_int32))
        self._h = C.c_void_p()
        check(lib.pkv_pool_create(C.byref(desc), C.byref(self._h)))
        self._slots = {}

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            lib.pkv_pool_destroy(h)
            self._h = None

    def fill_nan(self):
        """Fill every page with NaN patterns so reads of unwritten slots show."""
        if self.k_pages is None:
            return
        if self.kv_dtype in ("fp8", "fp8mx"):
            self.k_pages.fill_(0x7F)
            self.v_pages.fill_(0x7F)
        elif self.kv_dtype == "bf16":
            self.k_pages.view(torch.int16).fill_(0x7FC0)
            self.v_pages.view(torch.int16).fill_(0x7FC0)
        else:
            self.k_pages.view(torch.int32).fill_(0x7FC00000)
            self.v_pages.view(torch.int32).fill_(0x7FC00000)

    # -- sequence operations ---------------------------------------------------
    def alloc(self, seq, share_from=-1, n_shared=0, stream=None):
        slot = C.c_int32()
        st = _stream(stream) if self.device is not None else None
        check(lib.paged_kv_alloc(self._h, int(seq), int(share_from), int(n_shared), C.byref(slot), st))
        self._slots[int(seq)] = slot.value
        return slot.value

    def append(self, seqs, n_tokens, k_src=None, v_src=None, stream=None):
        sa, sp = _ints(seqs, np.int64)
        na, np_ = _ints(n_tokens, np.int32)
        assert sa.size == na.size
        # with nothing to write the source dtype only has to be a valid one
        src_dtype, kp, vp = (F32 if self.kv_dtype in ("fp8", "fp8mx") else DTYPES[self.kv_dtype]), None, None
        if self.device is not None and int(na.sum()) > 0:
            assert k_src.is_contiguous() and v_src.is_contiguous() and k_src.dtype == v_src.dtype
            assert k_src.numel() >= int(na.sum()) * self.num_kv_heads * self.head_dim
            src_dtype = _TORCH_SRC[k_src.dtype]
            if k_src.data_ptr() % 16:
                k_src = k_src.clone()
            if v_src.data_ptr() % 16:
                v_src = v_src.clone()
            kp, vp = _ptr(k_src), _ptr(v_src)
        st = _stream(stream) if self.device is not None else None
        check(lib.paged_kv_append(self._h, sa.size, sp, np_, kp, vp, src_dtype, st))

    def prepare_append(self, seqs, n_tokens, k_src, v_src):
        """paged_kv_append of fixed sequences, counts and source buffers with
        its arguments marshalled once (a serving loop refills k_src, v_src in
        place and calls it each step)."""
        return PreparedAppend(self, seqs, n_tokens, k_src, v_src)

    def prepare_rollback(self, seqs):
        """paged_kv_rollback of fixed sequences; each call takes the counts."""
        return PreparedRollback(self, seqs)

    def rollback(self, seqs, n_tokens, stream=None):
        sa, sp = _ints(seqs, np.int64)
        na, np_ = _ints(n_tokens, np.int32)
        assert sa.size == na.size
        st = _stream(stream) if self.device is not None else None
        check(lib.paged_kv_rollback(self._h, sa.size, sp, np_, st))

    def commit_path(self, seqs, n_tree, paths, stream=None):
        """Keep each sequence's accepted tree branch (paths[i]: node ids in
        depth order, root excluded) and drop the other tree nodes."""
        sa, sp = _ints(seqs, np.int64)
        ta, tp = _ints(n_tree, np.int32)
        paths = [list(map(int, p)) for p in paths]
        la, lp = _ints([len(p) for p in paths], np.int32)
        flat = [c for p in paths for c in p]
        fa, fp = _ints(flat if flat else [0], np.int32)
        assert sa.size == ta.size == la.size
        st = _stream(stream) if self.device is not None else None
        check(lib.paged_kv_commit_path(self._h, sa.size, sp, tp, lp, fp, st))

    def release(self, seq, stream=None):
        st = _stream(stream) if self.device is not None else None
        check(lib.paged_kv_release(self._h, int(seq), st))
        self._slots.pop(int(seq), None)

    def table(self, seq):
        """(pages, length, slot) of a sequence, from the host bookkeeping."""
        n, length, slot = C.c_int32(), C.c_int32(), C.c_int32()
        check(lib.paged_kv_block_table(self._h, int(seq), None, 0, C.byref(n), C.byref(length),
                                       C.byref(slot)))
        buf = (C.c_int32 * max(1, n.value))()
        check(lib.paged_kv_block_table(self._h, int(seq), buf, n.value, C.byref(n), C.byref(length),
                                       C.byref(slot)))
        return [buf[i] for i in range(n.value)], length.value, slot.value

    def stats(self):
        s = PoolStats()
        check(lib.paged_kv_stats(self._h, C.byref(s)))
        return {k: getattr(s, k) for k, _ in PoolStats._fields_}

    def refcount(self, page):
        r = C.c_int32()
        check(lib.paged_kv_page_refcount(self._h, int(page), C.byref(r)))
        return r.value

    def slot(self, seq):
        return self._slots[int(seq)]

    # -- verification over this pool --------------------------------------------
    def prepare_verify(self, q, n_q, slots=None, anc_mask=None, sm_scale=None, buffers=None,
                       num_splits=0, n_q_seq=None, shared_prefix_pages=0):
        return PreparedVerify(q, self.k_pages, self.v_pages, self.block_table, self.seq_lens,
                              n_q=n_q, num_kv_heads=self.num_kv_heads, kv_dtype=self.kv_dtype,
                              k_scale=self.k_scale, v_scale=self.v_scale, batch_slots=slots,
                              anc_mask=anc_mask, sm_scale=sm_scale, buffers=buffers,
                              num_splits=num_splits, n_q_seq=n_q_seq,
                              shared_prefix_pages=shared_prefix_pages)

    def verify_append(self, seqs, q, k_new, v_new, anc_mask=None, sm_scale=None, buffers=None,
                      num_splits=0, shared_prefix_pages=0, stream=None):
        """Append n_q = q.shape[1] tokens to every sequence of `seqs` (sequence
        i in block-table row i) and verify them, in one launch
        (spec_verify_attention_append).  k_new, v_new: [B, n_q, Hkv, d],
        bfloat16 for a bf16 pool, float32 for the FP8 kinds."""
        if k_new.data_ptr() % 16:
            k_new = k_new.clone()
        if v_new.data_ptr() % 16:
            v_new = v_new.clone()
        return self.prepare_verify_append(seqs, q, k_new, v_new, anc_mask, sm_scale, buffers, num_splits,
                                          shared_prefix_pages)(stream)

    def prepare_verify_append(self, seqs, q, k_new, v_new, anc_mask=None, sm_scale=None, buffers=None,
                              num_splits=0, shared_prefix_pages=0):
        return PreparedVerifyAppend(self, seqs, q, k_new, v_new, anc_mask=anc_mask, sm_scale=sm_scale,
                                    buffers=buffers, num_splits=num_splits,
                                    shared_prefix_pages=shared_prefix_pages)

    def verify(self, q, n_q, slots=None, anc_mask=None, sm_scale=None, buffers=None, num_splits=0,
               n_q_seq=None, shared_prefix_pages=0, stream=None):
        return spec_verify_attention(
            q, self.k_pages, self.v_pages, self.block_table, self.seq_lens, n_q=n_q,
            num_kv_heads=self.num_kv_heads, kv_dtype=self.kv_dtype, k_scale=self.k_scale,
            v_scale=self.v_scale, batch_slots=slots, anc_mask=anc_mask, sm_scale=sm_scale,
            buffers=buffers, num_splits=num_splits, n_q_seq=n_q_seq,
            shared_prefix_pages=shared_prefix_pages, stream=stream)


def _verify_args(q, k_pages, v_pages, block_table, seq_lens, n_q, num_kv_heads, kv_dtype, k_scale,
                 v_scale, batch_slots, anc_mask, sm_scale, num_splits, n_q_seq=None,
                 shared_prefix_pages=0):
    B, nq, Hq, d = q.shape
    assert nq == n_q and q.is_contiguous()
    if q.dtype not in _TORCH_SRC:
        raise TypeError(f"q must be float32 or bfloat16, not {q.dtype}")
    for name, t in (("k_pages", k_pages), ("v_pages", v_pages), ("block_table", block_table),
                    ("seq_lens", seq_lens), ("k_scale", k_scale), ("v_scale", v_scale),
                    ("batch_slots", batch_slots), ("anc_mask", anc_mask), ("n_q_seq", n_q_seq)):
        if t is not None and t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}: all tensors must be on one device")
    a = VerifyArgs()
    a.batch, a.n_q, a.num_q_heads, a.num_kv_heads, a.head_dim = B, n_q, Hq, num_kv_heads, d
    a.page_size = PAGE_SIZE
    a.q_dtype = _TORCH_SRC[q.dtype]
    a.kv_dtype = DTYPES[kv_dtype]
    a.q, a.k_pages, a.v_pages = q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr()
    if k_scale is not None:
        a.k_scale, a.v_scale = k_scale.data_ptr(), v_scale.data_ptr()
    assert block_table.dtype == torch.int32 and block_table.is_contiguous()
    a.block_table, a.block_table_stride = block_table.data_ptr(), block_table.shape[-1]
    assert seq_lens.dtype == torch.int32
    a.seq_lens = seq_lens.data_ptr()
    if batch_slots is not None:
        assert batch_slots.dtype == torch.int32 and batch_slots.numel() == B
        a.batch_slots = batch_slots.data_ptr()
    if anc_mask is not None:
        assert anc_mask.dtype == torch.int64 and anc_mask.shape == (B, n_q)
        a.anc_mask = anc_mask.data_ptr()
    a.sm_scale = float(np.float32(1.0 / np.sqrt(d)) if sm_scale is None else sm_scale)
    a.num_splits = num_splits
    if n_q_seq is not None:
        assert n_q_seq.dtype == torch.int32 and n_q_seq.numel() == B and n_q_seq.is_contiguous()
        a.n_q_seq = n_q_seq.data_ptr()
    a.shared_prefix_pages = int(shared_prefix_pages)
    return a


def verify_workspace_size(args):
    n = C.c_size_t()
    check(lib.spec_verify_workspace_size(C.byref(args), C.byref(n)))
    return n.value


class VerifyBuffers:
    """Preallocated outputs and workspace for repeated calls of one shape."""

    def __init__(self, batch, n_q, num_q_heads, head_dim, workspace_bytes, device):
        self.out = torch.empty((batch, n_q, num_q_heads, head_dim), dtype=torch.float32, device=device)
        self.lse = torch.empty((batch, n_q, num_q_heads), dtype=torch.float32, device=device)
        self.workspace = torch.empty(max(1, workspace_bytes), dtype=torch.uint8, device=device)


def spec_verify_attention(q, k_pages, v_pages, block_table, seq_lens, *, n_q, num_kv_heads,
                          kv_dtype, k_scale=None, v_scale=None, batch_slots=None, anc_mask=None,
                          sm_scale=None, buffers=None, num_splits=0, n_q_seq=None,
                          shared_prefix_pages=0, stream=None):
    a = _verify_args(q, k_pages, v_pages, block_table, seq_lens, n_q, num_kv_heads, kv_dtype,
                     k_scale, v_scale, batch_slots, anc_mask, sm_scale, num_splits, n_q_seq,
                     shared_prefix_pages)
    ws = verify_workspace_size(a)
    if buffers is None:
        B, _, Hq, d = q.shape
        buffers = VerifyBuffers(B, n_q, Hq, d, ws, q.device)
    assert buffers.workspace.numel() >= ws
    a.out, a.lse = buffers.out.data_ptr(), buffers.lse.data_ptr()
    a.workspace, a.workspace_bytes = buffers.workspace.data_ptr(), buffers.workspace.numel()
    check(lib.spec_verify_attention(C.byref(a), _stream(stream)))
    return buffers.out, buffers.lse


def spec_verify_attention_static(q, k_pages, v_pages, block_table, seq_lens, *, n_q, num_kv_heads,
                                 kv_dtype, out, lse, k_scale=None, v_scale=None, batch_slots=None,
                                 anc_mask=None, sm_scale=None, num_splits=0, n_q_seq=None,
                                 shared_prefix_pages=0, stream=None):
    """spec_verify_attention with the library's static scratch: nothing is
    allocated, the caller passes the outputs `out` [B, n_q, Hq, d] and `lse`
    [B, n_q, Hq] (float32, on q's device).  Calls that overlap in time on one
    GPU share the scratch and race."""
    a = _verify_args(q, k_pages, v_pages, block_table, seq_lens, n_q, num_kv_heads, kv_dtype,
                     k_scale, v_scale, batch_slots, anc_mask, sm_scale, num_splits, n_q_seq,
                     shared_prefix_pages)
    B, _, Hq, d = q.shape
    assert out.dtype == torch.float32 and out.shape == (B, n_q, Hq, d) and out.is_contiguous()
    assert lse.dtype == torch.float32 and lse.shape == (B, n_q, Hq) and lse.is_contiguous()
    assert out.device == q.device and lse.device == q.device
    a.out, a.lse = out.data_ptr(), lse.data_ptr()
    check(lib.spec_verify_attention_static(C.byref(a), _stream(stream)))
    return out, lse


class PreparedVerify:
    """spec_verify_attention with its arguments marshalled once.  The launch
    reads the tensors given here (queries, pages, block table, lengths) at
    call time, so a serving loop that updates them in place calls this once
    per step; returns (out, lse) from the buffers it owns."""

    def __init__(self, q, k_pages, v_pages, block_table, seq_lens, *, n_q, num_kv_heads, kv_dtype,
                 k_scale=None, v_scale=None, batch_slots=None, anc_mask=None, sm_scale=None,
                 buffers=None, num_splits=0, n_q_seq=None, shared_prefix_pages=0):
        a = _verify_args(q, k_pages, v_pages, block_table, seq_lens, n_q, num_kv_heads, kv_dtype,
                         k_scale, v_scale, batch_slots, anc_mask, sm_scale, num_splits, n_q_seq,
                         shared_prefix_pages)
        ws = verify_workspace_size(a)
        if buffers is None:
            B, _, Hq, d = q.shape
            buffers = VerifyBuffers(B, n_q, Hq, d, ws, q.device)
        assert buffers.workspace.numel() >= ws
        a.out, a.lse = buffers.out.data_ptr(), buffers.lse.data_ptr()
        a.workspace, a.workspace_bytes = buffers.workspace.data_ptr(), buffers.workspace.numel()
        self.args, self.buffers = a, buffers
        self._keep = (q, k_pages, v_pages, block_table, seq_lens, k_scale, v_scale, batch_slots,
                      anc_mask, n_q_seq)

    def __call__(self, stream=None):
        check(lib.spec_verify_attention(C.byref(self.args), _stream(stream)))
        return self.buffers.out, self.buffers.lse


class PreparedVerifyAppend:
    """Pool.verify_append with its arguments marshalled once: each call
    appends the tokens held in k_new, v_new (read at call time) to every
    listed sequence and verifies the queries in q; returns (out, lse) from
    the buffers it owns."""

    def __init__(self, pool, seqs, q, k_new, v_new, *, anc_mask=None, sm_scale=None, buffers=None,
                 num_splits=0, shared_prefix_pages=0):
        B, n_q, _, d = q.shape
        want = torch.bfloat16 if pool.kv_dtype == "bf16" else torch.float32
        for name, t in (("k_new", k_new), ("v_new", v_new)):
            if t.dtype != want or tuple(t.shape) != (B, n_q, pool.num_kv_heads, d) or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous {want} tensor of shape "
                                 f"{(B, n_q, pool.num_kv_heads, d)}")
            if t.device != q.device:
                raise ValueError(f"{name} is on {t.device}, q on {q.device}")
            if t.data_ptr() % 16:
                raise ValueError(f"{name} must be 16-byte aligned")
        self._seqs, self._seqs_p = _ints(seqs, np.int64)
        assert self._seqs.size == B
        a = _verify_args(q, pool.k_pages, pool.v_pages, pool.block_table, pool.seq_lens, n_q,
                         pool.num_kv_heads, pool.kv_dtype, pool.k_scale, pool.v_scale, None, anc_mask,
                         sm_scale, num_splits, None, shared_prefix_pages)
        ws = verify_workspace_size(a)
        if buffers is None:
            buffers = VerifyBuffers(B, n_q, q.shape[2], d, ws, q.device)
        assert buffers.workspace.numel() >= ws
        a.out, a.lse = buffers.out.data_ptr(), buffers.lse.data_ptr()
        a.workspace, a.workspace_bytes = buffers.workspace.data_ptr(), buffers.workspace.numel()
        self.args, self.buffers, self.pool = a, buffers, pool
        self._kp, self._vp = _ptr(k_new), _ptr(v_new)
        self._keep = (q, k_new, v_new, anc_mask)

    def __call__(self, stream=None):
        check(lib.spec_verify_attention_append(self.pool._h, self._seqs.size, self._seqs_p, self._kp, self._vp,
                                               C.byref(self.args), _stream(stream)))
        return self.buffers.out, self.buffers.lse


class PreparedAppend:
    """Pool.append with its arguments marshalled once: each call appends
    n_tokens[i] tokens to sequence seqs[i] from k_src, v_src (read at call
    time, laid out as for Pool.append)."""

    def __init__(self, pool, seqs, n_tokens, k_src, v_src):
        self._seqs, sp = _ints(seqs, np.int64)
        self._n, np_ = _ints(n_tokens, np.int32)
        assert self._seqs.size == self._n.size
        if pool.device is None:
            raise ValueError("a prepared append needs a pool with device memory")
        total = int(self._n.sum())
        for name, t in (("k_src", k_src), ("v_src", v_src)):
            if not t.is_contiguous() or t.data_ptr() % 16 or t.dtype != k_src.dtype:
                raise ValueError(f"{name} must be contiguous, 16-byte aligned and of k_src's dtype")
            if t.numel() < total * pool.num_kv_heads * pool.head_dim:
                raise ValueError(f"{name} holds fewer than the {total} tokens to append")
            if t.device != k_src.device:
                raise ValueError(f"{name} is on {t.device}, k_src on {k_src.device}")
        self._h = pool._h
        self._call = (C.c_int32(self._seqs.size), C.c_void_p(sp), C.c_void_p(np_), _ptr(k_src), _ptr(v_src),
                      C.c_int32(_TORCH_SRC[k_src.dtype]))
        self._keep = (pool, k_src, v_src)

    def __call__(self, stream=None):
        check(lib.paged_kv_append(self._h, *self._call, _stream(stream)))


class PreparedRollback:
    """Pool.rollback of fixed sequences: each call drops n_tokens[i] (int32
    array-like, one per sequence) tokens from sequence seqs[i]."""

    def __init__(self, pool, seqs):
        self._seqs, sp = _ints(seqs, np.int64)
        self._h, self._nseq, self._sp = pool._h, C.c_int32(self._seqs.size), C.c_void_p(sp)
        self._device = pool.device is not None
        self._keep = pool

    def __call__(self, n_tokens, stream=None):
        na, np_ = _ints(n_tokens, np.int32)
        if na.size != self._seqs.size:
            raise ValueError(f"{na.size} counts for {self._seqs.size} sequences")
        check(lib.paged_kv_rollback(self._h, self._nseq, self._sp, np_,
                                    _stream(stream) if self._device else None))


def _accept_args(target_logits, draft_logits, draft_tokens, seed, step, gammas=None):
    B, g1, V = target_logits.shape
    assert draft_logits.shape == (B, g1 - 1, V) and draft_tokens.shape == (B, g1 - 1)
    for name, t in (("draft_logits", draft_logits), ("draft_tokens", draft_tokens), ("gammas", gammas)):
        if t is not None and t.device != target_logits.device:
            raise ValueError(f"{name} is on {t.device}, target_logits on {target_logits.device}")
    assert target_logits.dtype == torch.float32 and draft_logits.dtype == torch.float32
    assert draft_tokens.dtype == torch.int32
    assert target_logits.is_contiguous() and draft_logits.is_contiguous() and draft_tokens.is_contiguous()
    a = AcceptArgs()
    a.batch, a.gamma, a.vocab = B, g1 - 1, V
    a.target_logits, a.draft_logits = target_logits.data_ptr(), draft_logits.data_ptr()
    a.draft_tokens = draft_tokens.data_ptr()
    a.seed, a.step = int(seed) & 0xFFFFFFFFFFFFFFFF, int(step) & 0xFFFFFFFF
    if gammas is not None:
        assert gammas.dtype == torch.int32 and gammas.numel() == B and gammas.is_contiguous()
        a.gammas = gammas.data_ptr()
    return a


def accept_workspace_size(args):
    n = C.c_size_t()
    check(lib.spec_accept_workspace_size(C.byref(args), C.byref(n)))
    return n.value


class AcceptBuffers:
    def __init__(self, batch, workspace_bytes, device):
        self.accepted_len = torch.empty(batch, dtype=torch.int32, device=device)
        self.next_token = torch.empty(batch, dtype=torch.int32, device=device)
        self.workspace = torch.empty(max(1, workspace_bytes), dtype=torch.uint8, device=device)


def spec_accept(target_logits, draft_logits, draft_tokens, seed, step, buffers=None, gammas=None,
                stream=None):
    a = _accept_args(target_logits, draft_logits, draft_tokens, seed, step, gammas)
    ws = accept_workspace_size(a)
    if buffers is None:
        buffers = AcceptBuffers(a.batch, ws, target_logits.device)
    a.accepted_len, a.next_token = buffers.accepted_len.data_ptr(), buffers.next_token.data_ptr()
    a.workspace, a.workspace_bytes = buffers.workspace.data_ptr(), buffers.workspace.numel()
    check(lib.spec_accept(C.byref(a), _stream(stream)))
    return buffers.accepted_len, buffers.next_token


class PreparedAccept:
    """spec_accept with its arguments marshalled once; each call takes the
    step counter (and optionally a new seed) and reads the logits and draft
    tokens in place.  Returns (accepted_len, next_token) buffers it owns.
    With step_tensor (a device uint32/int32 scalar tensor) the kernels read the
    step from it when they run, so the launch can be captured in a graph."""

    def __init__(self, target_logits, draft_logits, draft_tokens, seed, buffers=None, gammas=None,
                 step_tensor=None, accepted_len_out=None):
        """accepted_len_out: optional int32 [batch] tensor the accepted lengths
        are written to instead of buffers.accepted_len: device memory, or
        pinned host memory, which the kernel then writes directly (no copy to
        the host needed once the stream has passed the call)."""
        a = _accept_args(target_logits, draft_logits, draft_tokens, seed, 0, gammas)
        if step_tensor is not None:
            assert step_tensor.numel() == 1 and step_tensor.element_size() == 4
            a.step_ptr = step_tensor.data_ptr()
        ws = accept_workspace_size(a)
        if buffers is None:
            buffers = AcceptBuffers(a.batch, ws, target_logits.device)
        assert buffers.workspace.numel() >= ws
        if accepted_len_out is not None:
            if accepted_len_out.dtype != torch.int32 or accepted_len_out.numel() != a.batch:
                raise ValueError("accepted_len_out must be int32 with one entry per sequence")
            if not accepted_len_out.is_contiguous():
                raise ValueError("accepted_len_out must be contiguous")
            if not (accepted_len_out.is_cuda or accepted_len_out.is_pinned()):
                raise ValueError("accepted_len_out must be device memory or pinned host memory")
            buffers.accepted_len = accepted_len_out
        a.accepted_len, a.next_token = buffers.accepted_len.data_ptr(), buffers.next_token.data_ptr()
        a.workspace, a.workspace_bytes = buffers.workspace.data_ptr(), buffers.workspace.numel()
        self.args, self.buffers = a, buffers
        self._keep = (target_logits, draft_logits, draft_tokens, gammas, step_tensor)

    def __call__(self, step, seed=None, stream=None):
        self.args.step = int(step) & 0xFFFFFFFF
        if seed is not None:
            self.args.seed = int(seed) & 0xFFFFFFFFFFFFFFFF
        check(lib.spec_accept(C.byref(self.args), _stream(stream)))
        return self.buffers.accepted_len, self.buffers.next_token


def tree_accept_workspace_size(args):
    n = C.c_size_t()
    check(lib.spec_accept_tree_workspace_size(C.byref(args), C.byref(n)))
    return n.value


def _max_children(parents, n):
    m = 1
    for p in parents.cpu().numpy():
        q = p[1:][(p[1:] >= 0) & (p[1:] < n)]
        if q.size:
            m = max(m, int(np.bincount(q).max()))
    return min(m, n - 1)


class PreparedTreeAccept:
    """spec_accept_tree with its arguments marshalled once.  target_logits,
    draft_logits [B, n, V] fp32, parents and tokens [B, n] int32 (device),
    read in place at each call.  max_children bounds any node's child count
    (computed from the parents when not given: one host copy).  Each call
    takes the step counter and returns (accepted_len [B], accepted_nodes
    [B, n], next_token [B]) buffers it owns."""

    def __init__(self, target_logits, draft_logits, parents, tokens, seed, max_children=None):
        B, n, V = target_logits.shape
        assert draft_logits.shape == (B, n, V) and parents.shape == (B, n) and tokens.shape == (B, n)
        assert target_logits.dtype == torch.float32 and draft_logits.dtype == torch.float32
        assert parents.dtype == torch.int32 and tokens.dtype == torch.int32
        for t in (target_logits, draft_logits, parents, tokens):
            assert t.is_contiguous()
        if max_children is None:
            max_children = _max_children(parents, n)
        a = TreeAcceptArgs()
        a.batch, a.n_nodes, a.max_children, a.vocab = B, n, int(max_children), V
        a.target_logits, a.draft_logits = target_logits.data_ptr(), draft_logits.data_ptr()
        a.parents, a.tokens = parents.data_ptr(), tokens.data_ptr()
        a.seed = int(seed) & 0xFFFFFFFFFFFFFFFF
        dev = target_logits.device
        self.accepted_len = torch.empty(B, dtype=torch.int32, device=dev)
        self.accepted_nodes = torch.empty((B, n), dtype=torch.int32, device=dev)
        self.next_token = torch.empty(B, dtype=torch.int32, device=dev)
        self.workspace = torch.empty(max(1, tree_accept_workspace_size(a)), dtype=torch.uint8, device=dev)
        a.accepted_len, a.accepted_nodes = self.accepted_len.data_ptr(), self.accepted_nodes.data_ptr()
        a.next_token = self.next_token.data_ptr()
        a.workspace, a.workspace_bytes = self.workspace.data_ptr(), self.workspace.numel()
        self.args = a
        self._keep = (target_logits, draft_logits, parents, tokens)

    def __call__(self, step, seed=None, stream=None):
        self.args.step = int(step) & 0xFFFFFFFF
        if seed is not None:
            self.args.seed = int(seed) & 0xFFFFFFFFFFFFFFFF
        check(lib.spec_accept_tree(C.byref(self.args), _stream(stream)))
        return self.accepted_len, self.accepted_nodes, self.next_token


def spec_accept_tree(target_logits, draft_logits, parents, tokens, seed, step, max_children=None,
                     stream=None):
    """Draft-tree acceptance (one call).  Returns (accepted_len [B],
    accepted_nodes [B, n], next_token [B])."""
    return PreparedTreeAccept(target_logits, draft_logits, parents, tokens, seed,
                              max_children)(step, stream=stream)
