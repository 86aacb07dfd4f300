"""O-B: paged KV pool with block tables — oracle side.

Follows the paged KV managers on the pages:
  * paurushmuley.com, diagram "PagedAttention virtual memory manager" and the
    PagedKVCacheManager listing: logical blocks of 16 tokens map to
    non-contiguous physical blocks; a shared prefix maps the same physical
    blocks with reference count N; a block with reference count > 1 is copied
    before a write (copy-on-write); releasing a session drops a reference and
    frees a block at zero; exhaustion is an error.
  * innvotechnologies.co, TypeScript PagedKVCacheManager.allocateBlocks:
    first-fit over the block list; "Memory Exhausted" error.
  * innvotechnologies.co, pipeline diagram: accepted tokens are committed to
    the block table, rejected ones discarded (rollback).
  * futurestack.online, section 2.3 note: the bundle extension is atomic.

Readings where the pages are silent or disagree:
  * free pages are kept in a set ordered by a rank (the position of the page
    in a given free order, or its id when none is given); an allocation takes
    the free page of lowest rank ("first fit" generalised to a shuffled list);
  * an append is all-or-nothing: it first counts the pages it needs (CoW copy
    of a shared, partly filled tail page, then one page per new 16-token
    block) and fails without any change if the pool has fewer free pages;
  * a shared prefix of n tokens maps ceil(n / S) of the source's pages; a
    partly valid last shared page is CoW-copied on the first append;
  * rollback by n truncates the length; pages wholly past the new length lose
    a reference (freed at zero); no data moves;
  * FP8 pools quantise on append (see oracle.fp8 for the scale rule); the
    "fp8mx" pools quantise every token on its own with a power-of-two scale
    per 64 channels (oracle.fp8, per-64-element tile scales).

The model stores page contents in a plain [page][head][slot][dim] array (its
own layout), so gathering a sequence back to contiguous K/V is a loop over the
block table.
"""
import heapq

import numpy as np

from . import fp8


class OutOfPages(Exception):
    pass


class UnknownSeq(Exception):
    pass


class PoolModel:
    def __init__(self, num_pages, page_size, num_kv_heads, head_dim, kv_dtype="f64",
                 free_order=None):
        self.P, self.S, self.H, self.d = num_pages, page_size, num_kv_heads, head_dim
        self.fp8 = kv_dtype == "fp8"
        self.mx = kv_dtype == "fp8mx"
        if free_order is None:
            free_order = np.arange(num_pages)
        free_order = [int(p) for p in free_order]
        assert sorted(free_order) == list(range(num_pages)), "free order must be a permutation"
        self.rank = {p: r for r, p in enumerate(free_order)}
        self.free = set(range(num_pages))
        # the same free set as a heap on (rank, page): lowest rank first
        self._heap = sorted((r, p) for p, r in self.rank.items())
        self.refcount = [0] * num_pages
        self.tables = {}      # seq -> list of page ids
        self.lens = {}        # seq -> length in tokens
        self.scale_growths = 0
        self.cow_copies = 0
        if self.fp8:
            self.kc = np.zeros((num_pages, self.H, self.S, self.d), dtype=np.uint8)
            self.vc = np.zeros_like(self.kc)
            self.ks = np.ones((num_pages, self.H), dtype=np.float32)
            self.vs = np.ones((num_pages, self.H), dtype=np.float32)
        elif self.mx:
            self.kc = np.zeros((num_pages, self.H, self.S, self.d), dtype=np.uint8)
            self.vc = np.zeros_like(self.kc)
            self.kx = np.full((num_pages, self.H, self.S, self.d // 64), 127, dtype=np.uint8)
            self.vx = np.full_like(self.kx, 127)
        else:
            self.k = np.full((num_pages, self.H, self.S, self.d), np.nan)
            self.v = np.full((num_pages, self.H, self.S, self.d), np.nan)

    # -- free set --------------------------------------------------------------
    def _take(self):
        _, p = heapq.heappop(self._heap)
        assert p in self.free
        self.free.remove(p)
        self.refcount[p] = 1
        return p

    def _unref(self, p):
        self.refcount[p] -= 1
        assert self.refcount[p] >= 0
        if self.refcount[p] == 0:
            self.free.add(p)
            heapq.heappush(self._heap, (self.rank[p], p))

    # -- sequence operations ---------------------------------------------------
    def alloc(self, seq, share_from=None, n_shared=0):
        if seq in self.tables:
            raise ValueError("sequence exists")
        table = []
        if share_from is not None:
            if share_from not in self.tables:
                raise UnknownSeq(share_from)
            if n_shared > self.lens[share_from]:
                raise ValueError("shared prefix longer than source")
            for p in self.tables[share_from][: -(-n_shared // self.S)]:
                self.refcount[p] += 1
                table.append(p)
        else:
            n_shared = 0
        self.tables[seq] = table
        self.lens[seq] = n_shared

    def pages_needed(self, seq, n):
        L, table = self.lens[seq], self.tables[seq]
        need = 0
        if n > 0 and L % self.S and self.refcount[table[L // self.S]] > 1:
            need += 1                               # copy-on-write of the tail
        need += -(-(L + n) // self.S) - len(table)   # whole new blocks
        return need

    def append(self, seq, k_new, v_new):
        """k_new, v_new: [n, Hkv, d].  Float pools take fp64 values; FP8 pools
        take the fp32 values to quantise."""
        if seq not in self.tables:
            raise UnknownSeq(seq)
        n = len(k_new)
        if n == 0:
            return
        if self.pages_needed(seq, n) > len(self.free):
            raise OutOfPages(seq)
        L, table = self.lens[seq], self.tables[seq]
        fresh = set()
        if L % self.S and self.refcount[table[L // self.S]] > 1:
            old = table[L // self.S]
            new = self._take()
            self._copy_page(old, new)
            self._unref(old)
            table[L // self.S] = new
            self.cow_copies += 1
        while len(table) < -(-(L + n) // self.S):
            p = self._take()
            table.append(p)
            fresh.add(p)
        # write token by token, grouping per page for the FP8 scale rule
        for blk in range(L // self.S, -(-(L + n) // self.S)):
            p = table[blk]
            t0 = max(L, blk * self.S)
            t1 = min(L + n, (blk + 1) * self.S)
            slots = np.arange(t0, t1) - blk * self.S
            src = slice(t0 - L, t1 - L)
            if self.mx:
                kq, ke = fp8.quantise_tiles(np.asarray(k_new[src], dtype=np.float32))
                vq, ve = fp8.quantise_tiles(np.asarray(v_new[src], dtype=np.float32))
                for h in range(self.H):
                    self.kc[p, h, slots], self.kx[p, h, slots] = kq[:, h], ke[:, h]
                    self.vc[p, h, slots], self.vx[p, h, slots] = vq[:, h], ve[:, h]
            elif self.fp8:
                kx = np.asarray(k_new[src], dtype=np.float32)
                vx = np.asarray(v_new[src], dtype=np.float32)
                n_old = t0 - blk * self.S            # slots of the page already holding tokens
                for h in range(self.H):
                    for codes, scales, x in ((self.kc, self.ks, kx[:, h]), (self.vc, self.vs, vx[:, h])):
                        if p in fresh:
                            scales[p, h] = fp8.page_scale(x)
                        elif fp8.needs_growth(x, scales[p, h]):
                            # the new values do not fit the page's range: the
                            # page's scale doubles until they do and its codes
                            # are encoded again with it
                            new_scale = fp8.grown_scale(x, scales[p, h])
                            self.scale_growths += 1
                            codes[p, h, :n_old] = fp8.reencode(codes[p, h, :n_old], scales[p, h], new_scale)
                            scales[p, h] = new_scale
                        codes[p, h, slots] = fp8.quantise(x, scales[p, h])
            else:
                for h in range(self.H):
                    self.k[p, h, slots] = np.asarray(k_new[src, h], dtype=np.float64)
                    self.v[p, h, slots] = np.asarray(v_new[src, h], dtype=np.float64)
        self.lens[seq] = L + n

    def _copy_page(self, src, dst):
        if self.mx:
            for a in (self.kc, self.vc, self.kx, self.vx):
                a[dst] = a[src]
        elif self.fp8:
            self.kc[dst] = self.kc[src]
            self.vc[dst] = self.vc[src]
            self.ks[dst] = self.ks[src]
            self.vs[dst] = self.vs[src]
        else:
            self.k[dst] = self.k[src]
            self.v[dst] = self.v[src]

    def rollback(self, seq, n):
        if seq not in self.tables:
            raise UnknownSeq(seq)
        L = self.lens[seq]
        if n < 0 or n > L:
            raise ValueError("rollback beyond length")
        keep = -(-(L - n) // self.S)
        table = self.tables[seq]
        for p in table[keep:]:
            self._unref(p)
        del table[keep:]
        self.lens[seq] = L - n

    def commit_path(self, seq, n_tree, path):
        """Keep the accepted branch of a verified draft tree and drop the rest
        (atozofsoftwareengineering.blog, pipeline diagram: tree verification
        followed by "Dynamic KV Rollback/Commit").  The last n_tree tokens of
        the sequence are the tree's nodes in index order (node 0, the root,
        first); path lists the accepted nodes in depth order (root excluded,
        ids strictly increasing, so node path[d] >= d + 1).  Node path[d]'s
        K/V moves to position base + 1 + d (base = position of the root), in
        increasing d, and the sequence is then truncated to base + 1 + k.
        Reading: an FP8 token keeps its code when both positions share the
        page's scale bit for bit, and is otherwise decoded with the source
        scale (fp32 product) and quantised again with the destination scale
        (the append rule's encoder)."""
        if seq not in self.tables:
            raise UnknownSeq(seq)
        L, table = self.lens[seq], self.tables[seq]
        k = len(path)
        if not 1 <= n_tree <= L or k > n_tree - 1:
            raise ValueError("bad tree size or path length")
        if any(not 0 < c < n_tree for c in path) or any(a >= b for a, b in zip(path, path[1:])):
            raise ValueError("path nodes must be increasing ids in (0, n_tree)")
        base = L - n_tree
        for d, c in enumerate(path):
            src, dst = base + c, base + 1 + d
            if src == dst:
                continue
            ps, os_ = table[src // self.S], src % self.S
            pd, od = table[dst // self.S], dst % self.S
            if self.refcount[pd] > 1:
                raise ValueError("destination page is shared")
            if self.mx:
                # each token carries its own scales: codes and scales move as they are
                for a in (self.kc, self.vc, self.kx, self.vx):
                    a[pd, :, od] = a[ps, :, os_]
            elif self.fp8:
                for h in range(self.H):
                    for codes, sc in ((self.kc, self.ks), (self.vc, self.vs)):
                        if np.float32(sc[ps, h]).view(np.uint32) == np.float32(sc[pd, h]).view(np.uint32):
                            codes[pd, h, od] = codes[ps, h, os_]
                        else:
                            x = (fp8.decode(codes[ps, h, os_]).astype(np.float32) * np.float32(sc[ps, h])
                                 ).astype(np.float32)
                            codes[pd, h, od] = fp8.quantise(x, sc[pd, h])
            else:
                self.k[pd, :, od] = self.k[ps, :, os_]
                self.v[pd, :, od] = self.v[ps, :, os_]
        self.rollback(seq, n_tree - 1 - k)

    def release(self, seq):
        if seq not in self.tables:
            raise UnknownSeq(seq)
        for p in self.tables.pop(seq):
            self._unref(p)
        del self.lens[seq]

    # -- views -----------------------------------------------------------------
    def gather(self, seq):
        """Contiguous fp64 K, V [N, Hkv, d] of a sequence, read through its
        block table (with FP8 codes decoded and multiplied by their scale)."""
        L, table = self.lens[seq], self.tables[seq]
        K = np.empty((L, self.H, self.d))
        V = np.empty((L, self.H, self.d))
        for t in range(L):
            p, o = table[t // self.S], t % self.S
            if self.mx:
                K[t] = fp8.dequantise_tiles(self.kc[p, :, o], self.kx[p, :, o])
                V[t] = fp8.dequantise_tiles(self.vc[p, :, o], self.vx[p, :, o])
            elif self.fp8:
                K[t] = fp8.decode(self.kc[p, :, o]) * self.ks[p][:, None].astype(np.float64)
                V[t] = fp8.decode(self.vc[p, :, o]) * self.vs[p][:, None].astype(np.float64)
            else:
                K[t] = self.k[p, :, o]
                V[t] = self.v[p, :, o]
        return K, V

    def check_invariants(self):
        refs = [0] * self.P
        for table in self.tables.values():
            for p in table:
                refs[p] += 1
        assert refs == self.refcount, "refcount != number of references"
        used = {p for p in range(self.P) if refs[p] > 0}
        assert used.isdisjoint(self.free), "page both used and free"
        assert used | self.free == set(range(self.P)), "page lost"
        for seq, table in self.tables.items():
            assert len(table) == -(-self.lens[seq] // self.S), "table length"
