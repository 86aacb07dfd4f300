// Page pool bookkeeping of libpkvspec (host side).
//
// Semantics follow the paged KV managers on the pages
// (paurushmuley.com, PagedKVCacheManager: shared-prefix reference counts,
// allocation at block boundaries, copy-on-write of shared blocks, release at
// reference count zero, an error on exhaustion; innvotechnologies.co,
// TypeScript allocateBlocks: first fit; futurestack.online section 2.3: the
// bundle extension is atomic; innvotechnologies.co pipeline diagram: commit
// accepted drafts, discard the rest).  Free pages form a set ordered by a
// caller-given rank; allocation takes the lowest rank, so the free set alone
// decides future allocations (rollback restores it exactly).
//
// All device effects (scatter of new tokens, CoW copies, block-table entries,
// lengths) are expressed as PoolTask records and applied in-stream by the
// pool-update kernel; a metadata-only pool skips them.

#include <algorithm>
#include <cstring>
#include <mutex>
#include <set>
#include <unordered_map>
#include <vector>

#include "common.h"

namespace pkv {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

pkv_status fail(pkv_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

}  // namespace pkv

using namespace pkv;

struct Seq {
  int32_t row = -1;
  int32_t len = 0;
  uint64_t stamp = 0;                 // last call that listed this sequence
  std::vector<int32_t> pages;
};

struct pkv_pool {
  pkv_pool_desc desc{};
  bool device = false;
  int64_t page_bytes = 0;
  std::mutex mu;
  std::vector<int32_t> rank;          // page -> rank
  std::vector<int32_t> page_of_rank;  // rank -> page
  std::set<int32_t> free_ranks;       // ranks of free pages
  std::vector<int32_t> refcount;
  std::set<int32_t> free_rows;
  std::unordered_map<int64_t, Seq> seqs;
  int64_t cow_copies = 0;
  uint64_t calls = 0;                 // stamps of multi-sequence calls (duplicate check)

  int32_t take_page() {
    auto it = free_ranks.begin();
    int32_t p = page_of_rank[*it];
    free_ranks.erase(it);
    refcount[p] = 1;
    return p;
  }
  void unref(int32_t p) {
    if (--refcount[p] == 0) free_ranks.insert(rank[p]);
  }
};

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Collects tasks and flushes them to the device in launch-sized batches.
struct TaskSink {
  pkv_pool* pool;
  const void* k_src;
  const void* v_src;
  pkv_dtype src_dtype;
  void* stream;
  PoolUpdateBatch batch{};
  pkv_status status = PKV_OK;

  TaskSink(pkv_pool* p, const void* k, const void* v, pkv_dtype sd, void* s)
      : pool(p), k_src(k), v_src(v), src_dtype(sd), stream(s) {
    batch.num_kv_heads = p->desc.num_kv_heads;
    batch.head_dim = p->desc.head_dim;
    batch.kv_dtype = p->desc.kv_dtype;
    batch.src_dtype = sd;
    batch.bt_stride = p->desc.max_pages_per_seq;
    batch.page_bytes = p->page_bytes;
  }
  void add(const PoolTask& t) {
    if (!pool->device) return;
    batch.tasks[batch.n_tasks++] = t;
    if (batch.n_tasks == kTasksPerLaunch) flush();
  }
  void flush() {
    if (!pool->device || batch.n_tasks == 0) return;
    PoolDevice dev{pool->desc.k_pages, pool->desc.v_pages, pool->desc.k_scale,
                   pool->desc.v_scale, pool->desc.block_table, pool->desc.seq_lens,
                   k_src, v_src};
    pkv_status st = launch_pool_update(dev, batch, stream);
    if (st != PKV_OK && status == PKV_OK) status = st;
    batch.n_tasks = 0;
  }
};

PoolTask len_task(int32_t row, int32_t len) {
  PoolTask t{};
  t.row = row;
  t.page = -1;
  t.cow_src = -1;
  t.flags = kSetLen;
  t.new_len = len;
  return t;
}

}  // namespace

extern "C" {

int64_t pkv_page_bytes(pkv_dtype kv_dtype, int32_t page_size, int32_t head_dim) {
  if (page_size != kPageSize || (head_dim != 64 && head_dim != 128)) return 0;
  switch (kv_dtype) {
    case PKV_F32: return int64_t(page_size) * head_dim * 4;
    case PKV_BF16: return int64_t(page_size) * head_dim * 2;
    case PKV_FP8_E4M3:
    case PKV_FP8_E4M3_MX64: return int64_t(page_size) * head_dim;
    default: return 0;
  }
}

pkv_status pkv_pool_create(const pkv_pool_desc* desc, pkv_pool** out) {
  if (!desc || !out) return fail(PKV_ERR_INVALID_ARG, "null descriptor or output");
  *out = nullptr;
  const pkv_pool_desc& d = *desc;
  if (d.num_pages <= 0 || d.num_kv_heads <= 0 || d.max_seqs <= 0 || d.max_pages_per_seq <= 0)
    return fail(PKV_ERR_INVALID_ARG, "pool sizes must be positive");
  if (d.kv_dtype != PKV_F32 && d.kv_dtype != PKV_BF16 && d.kv_dtype != PKV_FP8_E4M3 &&
      d.kv_dtype != PKV_FP8_E4M3_MX64)
    return fail(PKV_ERR_INVALID_ARG, "unknown kv dtype");
  int64_t pb = pkv_page_bytes(d.kv_dtype, d.page_size, d.head_dim);
  if (pb == 0) return fail(PKV_ERR_UNSUPPORTED, "page_size must be 16 and head_dim 64 or 128");
  bool any_dev = d.k_pages || d.v_pages || d.k_scale || d.v_scale || d.block_table || d.seq_lens;
  if (any_dev) {
    if (!d.k_pages || !d.v_pages || !d.block_table || !d.seq_lens)
      return fail(PKV_ERR_INVALID_ARG, "device pool needs k_pages, v_pages, block_table, seq_lens");
    if ((d.kv_dtype == PKV_FP8_E4M3 || d.kv_dtype == PKV_FP8_E4M3_MX64) && (!d.k_scale || !d.v_scale))
      return fail(PKV_ERR_INVALID_ARG, "FP8 pool needs k_scale and v_scale");
  }
  std::vector<int32_t> order(d.num_pages);
  if (d.free_order) {
    std::vector<char> seen(d.num_pages, 0);
    for (int32_t r = 0; r < d.num_pages; ++r) {
      int32_t p = d.free_order[r];
      if (p < 0 || p >= d.num_pages || seen[p])
        return fail(PKV_ERR_INVALID_ARG, "free_order is not a permutation of [0, num_pages)");
      seen[p] = 1;
      order[r] = p;
    }
  } else {
    for (int32_t r = 0; r < d.num_pages; ++r) order[r] = r;
  }
  auto* pool = new pkv_pool();
  pool->desc = d;
  pool->desc.free_order = nullptr;
  pool->device = any_dev;
  pool->page_bytes = pb;
  pool->rank.resize(d.num_pages);
  pool->page_of_rank = order;
  pool->refcount.assign(d.num_pages, 0);
  for (int32_t r = 0; r < d.num_pages; ++r) {
    pool->rank[order[r]] = r;
    pool->free_ranks.insert(pool->free_ranks.end(), r);
  }
  for (int32_t r = 0; r < d.max_seqs; ++r) pool->free_rows.insert(pool->free_rows.end(), r);
  *out = pool;
  return PKV_OK;
}

void pkv_pool_destroy(pkv_pool* pool) { delete pool; }

pkv_status paged_kv_alloc(pkv_pool* pool, int64_t seq, int64_t share_from, int32_t n_shared,
                          int32_t* slot_out, void* stream) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "null pool");
  std::lock_guard<std::mutex> lock(pool->mu);
  if (pool->seqs.count(seq)) return fail(PKV_ERR_SEQ_EXISTS, "sequence already allocated");
  const Seq* src = nullptr;
  if (share_from >= 0) {
    auto it = pool->seqs.find(share_from);
    if (it == pool->seqs.end()) return fail(PKV_ERR_UNKNOWN_SEQ, "share_from not allocated");
    src = &it->second;
    if (n_shared < 0 || n_shared > src->len)
      return fail(PKV_ERR_INVALID_ARG, "n_shared outside [0, len(share_from)]");
  } else if (n_shared != 0) {
    return fail(PKV_ERR_INVALID_ARG, "n_shared without share_from");
  }
  if (pool->free_rows.empty()) return fail(PKV_ERR_NO_SLOT, "no free block-table row");
  Seq s;
  s.row = *pool->free_rows.begin();
  if (src) {
    int64_t np = ceil_div(n_shared, kPageSize);
    s.pages.assign(src->pages.begin(), src->pages.begin() + np);
    s.len = n_shared;
  }
  TaskSink sink(pool, nullptr, nullptr, pool->desc.kv_dtype, stream);
  for (size_t i = 0; i < s.pages.size(); ++i) {
    PoolTask t = len_task(s.row, s.len);
    t.flags = kWriteTable | (i + 1 == s.pages.size() ? kSetLen : 0);
    t.logical = int32_t(i);
    t.page = s.pages[i];
    sink.add(t);
  }
  if (s.pages.empty()) sink.add(len_task(s.row, 0));
  sink.flush();
  if (sink.status != PKV_OK) return sink.status;
  for (int32_t p : s.pages) pool->refcount[p]++;
  pool->free_rows.erase(pool->free_rows.begin());
  if (slot_out) *slot_out = s.row;
  pool->seqs.emplace(seq, std::move(s));
  return PKV_OK;
}

pkv_status paged_kv_append(pkv_pool* pool, int32_t n_seqs, const int64_t* seqs,
                           const int32_t* n_tokens, const void* k_src, const void* v_src,
                           pkv_dtype src_dtype, void* stream) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "null pool");
  if (n_seqs < 0 || (n_seqs > 0 && (!seqs || !n_tokens)))
    return fail(PKV_ERR_INVALID_ARG, "bad sequence list");
  std::lock_guard<std::mutex> lock(pool->mu);
  const pkv_pool_desc& d = pool->desc;
  if (pool->device) {
    bool ok = (d.kv_dtype == PKV_FP8_E4M3 || d.kv_dtype == PKV_FP8_E4M3_MX64) ? src_dtype == PKV_F32
                                                                                : src_dtype == d.kv_dtype;
    if (!ok) return fail(PKV_ERR_INVALID_ARG, "source dtype does not match the pool dtype");
  }
  // Validate and count pages by simulating the whole call on a copy of the
  // reference counts of the touched shared tail pages (few: a short list).
  thread_local std::vector<Seq*> touched;
  thread_local std::vector<std::pair<int32_t, int32_t>> sim_ref;
  touched.clear();
  sim_ref.clear();
  const uint64_t stamp = ++pool->calls;
  int64_t need = 0, total_tokens = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    auto it = pool->seqs.find(seqs[i]);
    if (it == pool->seqs.end()) return fail(PKV_ERR_UNKNOWN_SEQ, "append to unknown sequence");
    Seq& s = it->second;
    if (s.stamp == stamp) return fail(PKV_ERR_INVALID_ARG, "sequence listed twice");
    s.stamp = stamp;
    touched.push_back(&s);
    int32_t n = n_tokens[i];
    if (n < 0) return fail(PKV_ERR_INVALID_ARG, "negative token count");
    int64_t new_pages = ceil_div(int64_t(s.len) + n, kPageSize);
    if (new_pages > d.max_pages_per_seq) return fail(PKV_ERR_CAPACITY, "sequence exceeds max_pages_per_seq");
    if (int64_t(s.len) + n > INT32_MAX) return fail(PKV_ERR_CAPACITY, "sequence too long");
    total_tokens += n;
    if (n == 0) continue;
    if (s.len % kPageSize) {
      int32_t tail = s.pages[s.len / kPageSize];
      if (pool->refcount[tail] > 1) {
        size_t r = 0;
        while (r < sim_ref.size() && sim_ref[r].first != tail) ++r;
        if (r == sim_ref.size()) sim_ref.emplace_back(tail, pool->refcount[tail]);
        if (sim_ref[r].second > 1) {
          need += 1;
          sim_ref[r].second -= 1;
        }
      }
    }
    need += new_pages - int64_t(s.pages.size());
  }
  if (pool->device && total_tokens > 0 && (!k_src || !v_src))
    return fail(PKV_ERR_INVALID_ARG, "null source arrays");
  if (pool->device && total_tokens > 0 &&
      ((reinterpret_cast<uintptr_t>(k_src) | reinterpret_cast<uintptr_t>(v_src)) & 15))
    return fail(PKV_ERR_INVALID_ARG, "source arrays must be 16-byte aligned");
  if (need > int64_t(pool->free_ranks.size()))
    return fail(PKV_ERR_OUT_OF_PAGES, "page pool exhausted");

  // Copy-on-write copies go to the device before any token write of this
  // call: a write may land in a page that another sequence just stopped
  // sharing, and the copy must see that page's old contents.
  thread_local std::vector<PoolTask> copies, writes;
  copies.clear();
  writes.clear();
  int64_t src_row = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    Seq& s = *touched[i];
    int32_t n = n_tokens[i];
    if (n == 0) continue;
    int32_t L = s.len;
    int32_t cow_src = -1;
    if (L % kPageSize) {
      int32_t tail = s.pages[L / kPageSize];
      if (pool->refcount[tail] > 1) {
        int32_t np = pool->take_page();
        pool->unref(tail);
        s.pages[L / kPageSize] = np;
        cow_src = tail;
        pool->cow_copies++;
        PoolTask c{};
        c.row = s.row;
        c.page = np;
        c.cow_src = tail;
        copies.push_back(c);
      }
    }
    const int32_t first_fresh = int32_t(s.pages.size());     // pages taken by this call follow
    while (int64_t(s.pages.size()) < ceil_div(int64_t(L) + n, kPageSize)) s.pages.push_back(pool->take_page());
    int32_t first_blk = L / kPageSize;
    int32_t last_blk = int32_t(ceil_div(int64_t(L) + n, kPageSize)) - 1;
    for (int32_t blk = first_blk; blk <= last_blk; ++blk) {
      int32_t t0 = std::max(L, blk * kPageSize);
      int32_t t1 = std::min(L + n, (blk + 1) * kPageSize);
      PoolTask t{};
      t.row = s.row;
      t.logical = blk;
      t.page = s.pages[blk];
      t.cow_src = -1;
      t.src_row = int32_t(src_row + (t0 - L));
      t.slot_begin = t0 - blk * kPageSize;
      t.n = t1 - t0;
      const bool fresh = blk >= first_fresh;
      t.flags = (fresh ? kFresh : 0) |
                ((fresh || (blk == first_blk && cow_src >= 0)) ? kWriteTable : 0) |
                (blk == last_blk ? kSetLen : 0);
      t.new_len = L + n;
      writes.push_back(t);
    }
    s.len = L + n;
    src_row += n;
  }
  TaskSink sink(pool, k_src, v_src, src_dtype, stream);
  for (const PoolTask& t : copies) sink.add(t);
  sink.flush();
  for (const PoolTask& t : writes) sink.add(t);
  sink.flush();
  return sink.status;
}

pkv_status spec_verify_attention_append(pkv_pool* pool, int32_t n_seqs, const int64_t* seqs,
                                        const void* k_new, const void* v_new, const pkv_verify_args* args,
                                        void* stream) {
  if (!pool || !args) return fail(PKV_ERR_INVALID_ARG, "null pool or arguments");
  if (!pool->device) return fail(PKV_ERR_INVALID_ARG, "the fused call needs a pool with device memory");
  const pkv_pool_desc& d = pool->desc;
  if (d.kv_dtype == PKV_F32) return fail(PKV_ERR_UNSUPPORTED, "the fused call supports bf16 and FP8 pools");
  if (n_seqs < 1 || n_seqs > kFusedMaxBatch || n_seqs != args->batch)
    return fail(PKV_ERR_INVALID_ARG, "n_seqs must equal args->batch and be in [1, 768]");
  if (args->n_q < 1 || args->n_q > kFusedMaxTokens)
    return fail(PKV_ERR_UNSUPPORTED, "the fused call appends 1..16 tokens per sequence");
  if (args->n_q_seq || args->batch_slots)
    return fail(PKV_ERR_UNSUPPORTED, "the fused call takes no per-sequence counts or batch slots");
  if (!seqs || !k_new || !v_new) return fail(PKV_ERR_INVALID_ARG, "null sequence list or sources");
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15)
    return fail(PKV_ERR_INVALID_ARG, "source arrays must be 16-byte aligned");
  if (args->kv_dtype != d.kv_dtype || args->num_kv_heads != d.num_kv_heads || args->head_dim != d.head_dim ||
      args->page_size != d.page_size || args->k_pages != d.k_pages || args->v_pages != d.v_pages ||
      args->k_scale != d.k_scale || args->v_scale != d.v_scale || args->block_table != d.block_table ||
      args->seq_lens != d.seq_lens || args->block_table_stride != d.max_pages_per_seq)
    return fail(PKV_ERR_INVALID_ARG, "the verification arguments must describe this pool");
  size_t need = 0;
  pkv_status st = spec_verify_workspace_size(args, &need);
  if (st != PKV_OK) return st;
  if (!args->out) return fail(PKV_ERR_INVALID_ARG, "null output pointer");
  if (need > 0 && (!args->workspace || args->workspace_bytes < need))
    return fail(PKV_ERR_WORKSPACE, "workspace smaller than spec_verify_workspace_size");
  std::lock_guard<std::mutex> lock(pool->mu);
  // validate every sequence before anything changes (all-or-nothing)
  thread_local std::vector<Seq*> touched;
  touched.clear();
  const uint64_t stamp = ++pool->calls;
  const int32_t n = args->n_q;
  int64_t pages_needed = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    auto it = pool->seqs.find(seqs[i]);
    if (it == pool->seqs.end()) return fail(PKV_ERR_UNKNOWN_SEQ, "append to unknown sequence");
    Seq& s = it->second;
    if (s.stamp == stamp) return fail(PKV_ERR_INVALID_ARG, "sequence listed twice");
    s.stamp = stamp;
    if (s.row != i) return fail(PKV_ERR_INVALID_ARG, "sequence i of the fused call must use block-table row i");
    const int64_t total = ceil_div(int64_t(s.len) + n, kPageSize);
    if (total > d.max_pages_per_seq) return fail(PKV_ERR_CAPACITY, "sequence exceeds max_pages_per_seq");
    if (s.len % kPageSize && pool->refcount[s.pages[s.len / kPageSize]] > 1)
      return fail(PKV_ERR_UNSUPPORTED, "the fused call does not copy shared pages (use paged_kv_append)");
    pages_needed += total - int64_t(s.pages.size());
    touched.push_back(&s);
  }
  if (pages_needed > int64_t(pool->free_ranks.size())) return fail(PKV_ERR_OUT_OF_PAGES, "page pool exhausted");
  FusedAppend f;
  f.k_new = k_new;
  f.v_new = v_new;
  for (int32_t i = 0; i < n_seqs; ++i) {
    Seq& s = *touched[i];
    f.new_page[i] = -1;
    while (int64_t(s.pages.size()) < ceil_div(int64_t(s.len) + n, kPageSize)) {
      s.pages.push_back(pool->take_page());
      f.new_page[i] = s.pages.back();          // n <= 16: at most one new page
    }
    s.len += n;
  }
  return verify_fused_launch(args, f, stream);
}

pkv_status paged_kv_rollback(pkv_pool* pool, int32_t n_seqs, const int64_t* seqs,
                             const int32_t* n_tokens, void* stream) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "null pool");
  if (n_seqs < 0 || (n_seqs > 0 && (!seqs || !n_tokens)))
    return fail(PKV_ERR_INVALID_ARG, "bad sequence list");
  std::lock_guard<std::mutex> lock(pool->mu);
  thread_local std::vector<Seq*> touched;
  touched.clear();
  const uint64_t stamp = ++pool->calls;
  for (int32_t i = 0; i < n_seqs; ++i) {
    auto it = pool->seqs.find(seqs[i]);
    if (it == pool->seqs.end()) return fail(PKV_ERR_UNKNOWN_SEQ, "rollback of unknown sequence");
    if (it->second.stamp == stamp) return fail(PKV_ERR_INVALID_ARG, "sequence listed twice");
    it->second.stamp = stamp;
    if (n_tokens[i] < 0 || n_tokens[i] > it->second.len)
      return fail(PKV_ERR_INVALID_ARG, "rollback outside [0, len]");
    touched.push_back(&it->second);
  }
  TaskSink sink(pool, nullptr, nullptr, pool->desc.kv_dtype, stream);
  for (int32_t i = 0; i < n_seqs; ++i) {
    Seq& s = *touched[i];
    if (n_tokens[i] == 0) continue;
    s.len -= n_tokens[i];
    size_t keep = size_t(ceil_div(s.len, kPageSize));
    for (size_t j = keep; j < s.pages.size(); ++j) pool->unref(s.pages[j]);
    s.pages.resize(keep);
    sink.add(len_task(s.row, s.len));
  }
  sink.flush();
  return sink.status;
}

pkv_status paged_kv_commit_path(pkv_pool* pool, int32_t n_seqs, const int64_t* seqs,
                                const int32_t* n_tree, const int32_t* path_len,
                                const int32_t* path_nodes, void* stream) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "null pool");
  if (n_seqs < 0 || (n_seqs > 0 && (!seqs || !n_tree || !path_len)))
    return fail(PKV_ERR_INVALID_ARG, "bad sequence list");
  std::lock_guard<std::mutex> lock(pool->mu);
  thread_local std::vector<Seq*> touched;
  touched.clear();
  const uint64_t stamp = ++pool->calls;
  int64_t off = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    auto it = pool->seqs.find(seqs[i]);
    if (it == pool->seqs.end()) return fail(PKV_ERR_UNKNOWN_SEQ, "commit of unknown sequence");
    Seq& s = it->second;
    if (s.stamp == stamp) return fail(PKV_ERR_INVALID_ARG, "sequence listed twice");
    s.stamp = stamp;
    const int32_t nt = n_tree[i], k = path_len[i];
    if (nt < 1 || nt > 64 || nt > s.len) return fail(PKV_ERR_INVALID_ARG, "n_tree outside [1, min(64, len)]");
    if (k < 0 || k > nt - 1) return fail(PKV_ERR_INVALID_ARG, "path_len outside [0, n_tree - 1]");
    if (k > 0 && !path_nodes) return fail(PKV_ERR_INVALID_ARG, "null path_nodes");
    const int32_t base = s.len - nt;
    for (int32_t d = 0; d < k; ++d) {
      const int32_t c = path_nodes[off + d];
      if (c <= (d ? path_nodes[off + d - 1] : 0) || c >= nt)
        return fail(PKV_ERR_INVALID_ARG, "path nodes must be increasing ids in (0, n_tree)");
      if (c != d + 1 && pool->refcount[s.pages[(base + 1 + d) / kPageSize]] > 1)
        return fail(PKV_ERR_INVALID_ARG, "destination page is shared with another sequence");
    }
    off += k;
    touched.push_back(&s);
  }
  // the moves, one group per sequence (in call order), then the truncation
  PoolMoveBatch mb{};
  mb.num_kv_heads = pool->desc.num_kv_heads;
  mb.head_dim = pool->desc.head_dim;
  mb.kv_dtype = pool->desc.kv_dtype;
  mb.page_bytes = pool->page_bytes;
  pkv_status status = PKV_OK;
  int32_t n_moves = 0;
  auto flush = [&]() {
    if (mb.n_groups > 0 && pool->device) {
      pkv_status st = launch_pool_moves(PoolDevice{pool->desc.k_pages, pool->desc.v_pages, pool->desc.k_scale,
                                                   pool->desc.v_scale, pool->desc.block_table,
                                                   pool->desc.seq_lens, nullptr, nullptr},
                                        mb, stream);
      if (st != PKV_OK && status == PKV_OK) status = st;
    }
    mb.n_groups = 0;
    n_moves = 0;
    mb.first[0] = 0;
  };
  off = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    const Seq& s = *touched[i];
    const int32_t nt = n_tree[i], k = path_len[i], base = s.len - nt;
    bool open = false;
    for (int32_t d = 0; d < k; ++d) {
      const int32_t src = base + path_nodes[off + d], dst = base + 1 + d;
      if (src == dst) continue;
      if (n_moves == kMovesPerLaunch || (!open && mb.n_groups == kMoveGroups)) {
        if (open) mb.n_groups++;
        flush();
        open = false;
      }
      if (!open) {
        mb.first[mb.n_groups] = n_moves;
        open = true;
      }
      mb.moves[n_moves++] = PoolMove{s.pages[src / kPageSize], s.pages[dst / kPageSize],
                                     (src % kPageSize) | ((dst % kPageSize) << 8)};
      mb.first[mb.n_groups + 1] = n_moves;
    }
    if (open) mb.n_groups++;
    off += k;
  }
  flush();
  if (status != PKV_OK) return status;
  TaskSink sink(pool, nullptr, nullptr, pool->desc.kv_dtype, stream);
  for (int32_t i = 0; i < n_seqs; ++i) {
    Seq& s = *touched[i];
    const int32_t drop = n_tree[i] - 1 - path_len[i];
    if (drop == 0) continue;
    s.len -= drop;
    size_t keep = size_t(ceil_div(s.len, kPageSize));
    for (size_t j = keep; j < s.pages.size(); ++j) pool->unref(s.pages[j]);
    s.pages.resize(keep);
    sink.add(len_task(s.row, s.len));
  }
  sink.flush();
  return sink.status;
}

pkv_status paged_kv_release(pkv_pool* pool, int64_t seq, void* stream) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "null pool");
  std::lock_guard<std::mutex> lock(pool->mu);
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return fail(PKV_ERR_UNKNOWN_SEQ, "release of unknown sequence");
  TaskSink sink(pool, nullptr, nullptr, pool->desc.kv_dtype, stream);
  sink.add(len_task(it->second.row, 0));
  sink.flush();
  if (sink.status != PKV_OK) return sink.status;
  for (int32_t p : it->second.pages) pool->unref(p);
  pool->free_rows.insert(it->second.row);
  pool->seqs.erase(it);
  return PKV_OK;
}

pkv_status paged_kv_block_table(const pkv_pool* cpool, int64_t seq, int32_t* pages_out,
                                int32_t max_pages, int32_t* n_pages_out, int32_t* len_out,
                                int32_t* slot_out) {
  if (!cpool) return fail(PKV_ERR_INVALID_ARG, "null pool");
  auto* pool = const_cast<pkv_pool*>(cpool);
  std::lock_guard<std::mutex> lock(pool->mu);
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return fail(PKV_ERR_UNKNOWN_SEQ, "unknown sequence");
  const Seq& s = it->second;
  if (pages_out) {
    if (max_pages < 0) return fail(PKV_ERR_INVALID_ARG, "negative max_pages");
    const size_t n = std::min<size_t>(size_t(max_pages), s.pages.size());
    if (n > 0) std::memcpy(pages_out, s.pages.data(), n * sizeof(int32_t));   // an empty table may have no storage
  }
  if (n_pages_out) *n_pages_out = int32_t(s.pages.size());
  if (len_out) *len_out = s.len;
  if (slot_out) *slot_out = s.row;
  return PKV_OK;
}

pkv_status paged_kv_stats(const pkv_pool* cpool, pkv_pool_stats* out) {
  if (!cpool || !out) return fail(PKV_ERR_INVALID_ARG, "null argument");
  auto* pool = const_cast<pkv_pool*>(cpool);
  std::lock_guard<std::mutex> lock(pool->mu);
  pkv_pool_stats st{};
  for (int32_t r : pool->refcount) {
    if (r > 0) st.used_pages++;
    if (r > 1) st.shared_pages++;
  }
  st.free_pages = int32_t(pool->free_ranks.size());
  st.num_seqs = int32_t(pool->seqs.size());
  st.cow_copies = pool->cow_copies;
  for (auto& kv : pool->seqs) st.used_token_slots += kv.second.len;
  *out = st;
  return PKV_OK;
}

pkv_status paged_kv_page_refcount(const pkv_pool* cpool, int32_t page, int32_t* refcount_out) {
  if (!cpool || !refcount_out) return fail(PKV_ERR_INVALID_ARG, "null argument");
  auto* pool = const_cast<pkv_pool*>(cpool);
  std::lock_guard<std::mutex> lock(pool->mu);
  if (page < 0 || page >= pool->desc.num_pages) return fail(PKV_ERR_INVALID_ARG, "page out of range");
  *refcount_out = pool->refcount[page];
  return PKV_OK;
}

pkv_status spec_tree_ancestor_masks(int32_t n_nodes, const int32_t* parents, uint64_t* masks_out) {
  if (n_nodes < 1 || n_nodes > 64 || !parents || !masks_out)
    return fail(PKV_ERR_INVALID_ARG, "need 1..64 nodes and non-null arrays");
  if (parents[0] != -1) return fail(PKV_ERR_INVALID_ARG, "node 0 must be the root (parent -1)");
  for (int32_t i = 1; i < n_nodes; ++i)
    if (parents[i] < 0 || parents[i] >= i)
      return fail(PKV_ERR_INVALID_ARG, "parents[i] must lie in [0, i)");
  // parents precede children, so each node's mask extends its parent's
  for (int32_t i = 0; i < n_nodes; ++i)
    masks_out[i] = (uint64_t(1) << i) | (i ? masks_out[parents[i]] : 0);
  return PKV_OK;
}

const char* pkv_status_string(pkv_status s) {
  switch (s) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_OUT_OF_PAGES: return "out of pages";
    case PKV_ERR_UNKNOWN_SEQ: return "unknown sequence";
    case PKV_ERR_SEQ_EXISTS: return "sequence exists";
    case PKV_ERR_UNSUPPORTED: return "unsupported";
    case PKV_ERR_DEVICE: return "device error";
    case PKV_ERR_WORKSPACE: return "workspace too small";
    case PKV_ERR_NO_SLOT: return "no free block-table row";
    case PKV_ERR_CAPACITY: return "sequence exceeds block-table capacity";
  }
  return "unknown status";
}

const char* pkv_last_error(void) { return pkv::g_last_error.c_str(); }

const char* pkv_version(void) { return "pkvspec 0.1 (gfx950)"; }

}  // extern "C"
