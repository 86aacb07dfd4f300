// Host-only check of the page pool's bookkeeping (pool.cpp), built with g++
// under AddressSanitizer + UndefinedBehaviorSanitizer and, separately, under
// ThreadSanitizer (host_check/run.py).  No GPU code is involved: the two
// device entry points the pool calls (launch_pool_update, launch_pool_moves)
// are replaced here by host functions that apply the same task records to
// host arrays standing in for device memory, with every index checked.
//
// What is checked, through the C ABI only:
//   * random sequences of alloc (fresh and shared-prefix), multi-sequence
//     append, rollback, commit_path and release, plus calls that must fail
//     (unknown sequence, rollback past the length, pool exhaustion, a path
//     into a shared page): after every call the pages, lengths and block-table
//     rows the library reports equal a contiguous per-sequence model, the
//     stand-in device table and lengths equal the host bookkeeping, every
//     token read back through the stand-in pages equals the model's, and the
//     reference counts equal the number of table entries per page
//     (paurushmuley.com, PagedKVCacheManager: shared-prefix reference counts,
//     copy-on-write, release at zero; futurestack.online section 2.3: an
//     append is all-or-nothing);
//   * several threads driving one pool concurrently, each with its own
//     sequences that share a common prefix (the pages' listing mutates its
//     block table without a lock; this one serialises calls on the handle).
//
// Exit status 0 when every check holds; a failed check prints its reason and
// aborts.

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <random>
#include <thread>
#include <vector>

#include "../common.h"

namespace {

void require(bool ok, const char* what, long a = 0, long b = 0) {
  if (!ok) {
    std::fprintf(stderr, "host_check: %s (%ld, %ld)\n", what, a, b);
    std::abort();
  }
}

// Stand-in device memory of one pool: fp32 pages in the plain layout
// [page][head][slot][dim], the block table and the lengths.
struct Device {
  int P = 0, H = 0, D = 0, rows = 0, cols = 0;
  std::vector<float> k, v;
  std::vector<int32_t> table, lens;
  float* kp(int page, int h, int slot) {
    require(page >= 0 && page < P && h >= 0 && h < H && slot >= 0 && slot < pkv::kPageSize,
            "page access out of range", page, slot);
    return &k[((size_t(page) * H + h) * pkv::kPageSize + slot) * D];
  }
  float* vp(int page, int h, int slot) { return &v[kp(page, h, slot) - k.data()]; }
};

// The stand-in for every pool of the process, found by its k_pages pointer.
std::mutex g_dev_mu;
std::map<const void*, Device*> g_devices;

Device* device_of(const void* k_pages) {
  std::lock_guard<std::mutex> lock(g_dev_mu);
  auto it = g_devices.find(k_pages);
  require(it != g_devices.end(), "launch for an unknown pool");
  return it->second;
}

}  // namespace

namespace pkv {

// Host stand-in of the pool-update kernel: the task semantics of common.h,
// applied in order (CoW copy, token scatter, table entry, length).
pkv_status launch_pool_update(const PoolDevice& dev, const PoolUpdateBatch& batch, void*) {
  Device* d = device_of(dev.k_pages);
  require(batch.n_tasks >= 0 && batch.n_tasks <= kTasksPerLaunch, "task count", batch.n_tasks);
  require(batch.kv_dtype == PKV_F32 && batch.src_dtype == PKV_F32, "host check uses fp32 pools");
  const float* ks = static_cast<const float*>(dev.k_src);
  const float* vs = static_cast<const float*>(dev.v_src);
  for (int i = 0; i < batch.n_tasks; ++i) {
    const PoolTask& t = batch.tasks[i];
    if (t.cow_src >= 0)
      for (int h = 0; h < d->H; ++h)
        for (int s = 0; s < kPageSize; ++s) {
          std::memcpy(d->kp(t.page, h, s), d->kp(t.cow_src, h, s), sizeof(float) * d->D);
          std::memcpy(d->vp(t.page, h, s), d->vp(t.cow_src, h, s), sizeof(float) * d->D);
        }
    if (t.n > 0) {
      require(t.slot_begin >= 0 && t.slot_begin + t.n <= kPageSize, "token slots", t.slot_begin, t.n);
      require(ks && vs && t.src_row >= 0, "token source");
      for (int j = 0; j < t.n; ++j)
        for (int h = 0; h < d->H; ++h) {
          const size_t src = (size_t(t.src_row + j) * d->H + h) * d->D;
          std::memcpy(d->kp(t.page, h, t.slot_begin + j), ks + src, sizeof(float) * d->D);
          std::memcpy(d->vp(t.page, h, t.slot_begin + j), vs + src, sizeof(float) * d->D);
        }
    }
    if (t.flags & kWriteTable) {
      require(t.row >= 0 && t.row < d->rows && t.logical >= 0 && t.logical < d->cols, "table entry",
              t.row, t.logical);
      require(t.page >= 0 && t.page < d->P, "table page", t.page);
      d->table[size_t(t.row) * d->cols + t.logical] = t.page;
    }
    if (t.flags & kSetLen) {
      require(t.row >= 0 && t.row < d->rows && t.new_len >= 0, "length entry", t.row, t.new_len);
      d->lens[t.row] = t.new_len;
    }
  }
  return PKV_OK;
}

// Host stand-in of the token-move kernel of a path commit.
pkv_status launch_pool_moves(const PoolDevice& dev, const PoolMoveBatch& batch, void*) {
  Device* d = device_of(dev.k_pages);
  require(batch.n_groups >= 0 && batch.n_groups <= kMoveGroups, "move groups", batch.n_groups);
  for (int g = 0; g < batch.n_groups; ++g) {
    require(batch.first[g] >= 0 && batch.first[g] <= batch.first[g + 1] &&
                batch.first[g + 1] <= kMovesPerLaunch, "move group bounds", batch.first[g], batch.first[g + 1]);
    for (int m = batch.first[g]; m < batch.first[g + 1]; ++m) {
      const PoolMove& mv = batch.moves[m];
      const int so = mv.slots & 0xFF, dn = mv.slots >> 8;
      for (int h = 0; h < d->H; ++h) {
        std::memcpy(d->kp(mv.dst_page, h, dn), d->kp(mv.src_page, h, so), sizeof(float) * d->D);
        std::memcpy(d->vp(mv.dst_page, h, dn), d->vp(mv.src_page, h, so), sizeof(float) * d->D);
      }
    }
  }
  return PKV_OK;
}

// The fused append + verification call refuses fp32 pools (the only kind
// this check builds) before it sizes a workspace or launches: reaching either
// stand-in is a failure.
pkv_status verify_fused_launch(const pkv_verify_args*, const FusedAppend&, void*) {
  require(false, "fused launch reached for an fp32 pool");
  return PKV_ERR_DEVICE;
}

}  // namespace pkv

extern "C" pkv_status spec_verify_workspace_size(const pkv_verify_args*, size_t*) {
  require(false, "verification workspace query reached for an fp32 pool");
  return PKV_ERR_DEVICE;
}

namespace {

constexpr int kH = 2, kD = 64;

// A token's K values: channel 0 holds its id (exact in fp32 below 2^24), the
// other channels (h, c) -> h * 4096 + c + 0.5; V holds the negatives.  A
// token, head or channel out of place shows.
float kval(int id, int h, int c) { return c == 0 ? float(id) : float(h * 4096 + c) + 0.5f; }

struct Harness {
  pkv_pool* pool = nullptr;
  Device dev;
  std::map<int64_t, std::vector<int>> model;   // seq -> token ids in order
  int next_token = 1;

  Harness(int pages, int rows, int cols, uint64_t seed) {
    dev.P = pages;
    dev.H = kH;
    dev.D = kD;
    dev.rows = rows;
    dev.cols = cols;
    dev.k.assign(size_t(pages) * kH * pkv::kPageSize * kD, -1.0f);
    dev.v = dev.k;
    dev.table.assign(size_t(rows) * cols, -1);
    dev.lens.assign(rows, 0);
    std::vector<int32_t> order(pages);
    for (int i = 0; i < pages; ++i) order[i] = i;
    std::shuffle(order.begin(), order.end(), std::mt19937_64(seed));
    pkv_pool_desc d{};
    d.num_pages = pages;
    d.page_size = pkv::kPageSize;
    d.num_kv_heads = kH;
    d.head_dim = kD;
    d.kv_dtype = PKV_F32;
    d.max_seqs = rows;
    d.max_pages_per_seq = cols;
    d.k_pages = dev.k.data();
    d.v_pages = dev.v.data();
    d.block_table = dev.table.data();
    d.seq_lens = dev.lens.data();
    d.free_order = order.data();
    {
      std::lock_guard<std::mutex> lock(g_dev_mu);
      g_devices[dev.k.data()] = &dev;
    }
    require(pkv_pool_create(&d, &pool) == PKV_OK, "pool create");
  }
  ~Harness() {
    pkv_pool_destroy(pool);
    std::lock_guard<std::mutex> lock(g_dev_mu);
    g_devices.erase(dev.k.data());
  }

  std::vector<int32_t> table_of(int64_t seq, int32_t* len, int32_t* row) {
    int32_t n = 0;
    require(paged_kv_block_table(pool, seq, nullptr, 0, &n, len, row) == PKV_OK, "block table size");
    std::vector<int32_t> pages(std::max(1, n));
    require(paged_kv_block_table(pool, seq, pages.data(), n, &n, len, row) == PKV_OK, "block table");
    pages.resize(n);
    return pages;
  }

  // Every check of one sequence: table length, stand-in device row and
  // length, every token through the stand-in pages.
  void check_seq(int64_t seq, const std::vector<int>& toks) {
    int32_t len = 0, row = 0;
    std::vector<int32_t> pages = table_of(seq, &len, &row);
    require(len == int32_t(toks.size()), "length", len, long(toks.size()));
    require(int64_t(pages.size()) == (len + pkv::kPageSize - 1) / pkv::kPageSize, "page count", long(pages.size()), len);
    require(row >= 0 && row < dev.rows && dev.lens[row] == len, "device length", row, dev.lens[row]);
    for (size_t j = 0; j < pages.size(); ++j)
      require(dev.table[size_t(row) * dev.cols + j] == pages[j], "device table entry", long(j), pages[j]);
    for (int t = 0; t < len; ++t)
      for (int h = 0; h < kH; ++h) {
        const float* kr = dev.kp(pages[t / pkv::kPageSize], h, t % pkv::kPageSize);
        const float* vr = dev.vp(pages[t / pkv::kPageSize], h, t % pkv::kPageSize);
        for (int c = 0; c < kD; ++c) {
          require(kr[c] == kval(toks[t], h, c), "K value", t, long(seq));
          require(vr[c] == -kval(toks[t], h, c), "V value", t, long(seq));
        }
      }
  }

  void check_all() {
    std::vector<int> refs(dev.P, 0);
    int64_t slots = 0;
    for (auto& [seq, toks] : model) {
      check_seq(seq, toks);
      int32_t len = 0, row = 0;
      for (int32_t p : table_of(seq, &len, &row)) refs[p]++;
      slots += int64_t(toks.size());
    }
    int used = 0, shared = 0;
    for (int p = 0; p < dev.P; ++p) {
      int32_t rc = -1;
      require(paged_kv_page_refcount(pool, p, &rc) == PKV_OK, "refcount call");
      require(rc == refs[p], "refcount != references", p, rc);
      used += refs[p] > 0;
      shared += refs[p] > 1;
    }
    pkv_pool_stats st{};
    require(paged_kv_stats(pool, &st) == PKV_OK, "stats");
    require(st.used_pages == used && st.free_pages == dev.P - used && st.shared_pages == shared,
            "page counts", st.used_pages, used);
    require(st.num_seqs == int32_t(model.size()) && st.used_token_slots == slots, "sequence counts",
            st.num_seqs, long(model.size()));
  }

  // K/V sources for the given token ids, laid out [token][head][dim].
  void fill_src(const std::vector<int>& ids, std::vector<float>& ks, std::vector<float>& vs) {
    ks.resize(std::max<size_t>(1, ids.size()) * kH * kD);
    vs.resize(ks.size());
    for (size_t i = 0; i < ids.size(); ++i)
      for (int h = 0; h < kH; ++h)
        for (int c = 0; c < kD; ++c) {
          ks[(i * kH + h) * kD + c] = kval(ids[i], h, c);
          vs[(i * kH + h) * kD + c] = -kval(ids[i], h, c);
        }
  }

  pkv_status append(const std::vector<int64_t>& seqs, const std::vector<int32_t>& ns) {
    std::vector<int> ids;
    for (int32_t n : ns)
      for (int j = 0; j < n; ++j) ids.push_back(next_token + int(ids.size()));
    std::vector<float> ks, vs;
    fill_src(ids, ks, vs);
    const pkv_status st = paged_kv_append(pool, int32_t(seqs.size()), seqs.data(), ns.data(), ks.data(),
                                          vs.data(), PKV_F32, nullptr);
    if (st == PKV_OK) {
      size_t o = 0;
      for (size_t i = 0; i < seqs.size(); ++i)
        for (int j = 0; j < ns[i]; ++j) model[seqs[i]].push_back(ids[o++]);
      next_token += int(ids.size());
    }
    return st;
  }
};

// Serial phase: random calls, every check after each.
void serial_phase(uint64_t seed, int n_ops) {
  Harness hx(96, 16, 40, seed);
  std::mt19937_64 rng(seed);
  auto pick = [&](int n) { return int(rng() % uint64_t(n)); };
  auto live = [&]() {
    std::vector<int64_t> v;
    for (auto& kv : hx.model) v.push_back(kv.first);
    return v;
  };
  int ok_calls = 0, failed_calls = 0, cow_before = 0;
  for (int op = 0; op < n_ops; ++op) {
    const int r = pick(100);
    std::vector<int64_t> L = live();
    pkv_pool_stats before{};
    paged_kv_stats(hx.pool, &before);
    pkv_status st = PKV_OK;
    bool expect_fail = false;
    if (r < 15 || L.empty()) {                                   // fresh sequence
      int64_t s = pick(24);
      int32_t row = -1;
      st = paged_kv_alloc(hx.pool, s, -1, 0, &row, nullptr);
      if (st == PKV_OK) hx.model[s] = {};
      else expect_fail = true;
    } else if (r < 25) {                                         // shared prefix
      int64_t s = pick(24), src = L[pick(int(L.size()))];
      const int n = pick(int(hx.model[src].size()) + 1);
      int32_t row = -1;
      st = paged_kv_alloc(hx.pool, s, src, n, &row, nullptr);
      if (st == PKV_OK) hx.model[s] = std::vector<int>(hx.model[src].begin(), hx.model[src].begin() + n);
      else expect_fail = true;
    } else if (r < 60) {                                         // append to 1..3 sequences
      std::shuffle(L.begin(), L.end(), rng);
      L.resize(std::min<size_t>(L.size(), 1 + pick(3)));
      std::vector<int32_t> ns;
      for (size_t i = 0; i < L.size(); ++i) ns.push_back(pick(r < 57 ? 41 : 400));   // sometimes too many
      st = hx.append(L, ns);
      expect_fail = st != PKV_OK;
      require(st == PKV_OK || st == PKV_ERR_OUT_OF_PAGES || st == PKV_ERR_CAPACITY, "append status", st);
    } else if (r < 75) {                                         // rollback 1..3 sequences
      std::shuffle(L.begin(), L.end(), rng);
      L.resize(std::min<size_t>(L.size(), 1 + pick(3)));
      std::vector<int32_t> ns;
      for (int64_t s : L) ns.push_back(pick(int(hx.model[s].size()) + (r < 73 ? 1 : 5)));
      st = paged_kv_rollback(hx.pool, int32_t(L.size()), L.data(), ns.data(), nullptr);
      if (st == PKV_OK)
        for (size_t i = 0; i < L.size(); ++i) hx.model[L[i]].resize(hx.model[L[i]].size() - ns[i]);
      else expect_fail = true;
    } else if (r < 85) {                                         // commit an accepted tree path
      const int64_t s = L[pick(int(L.size()))];
      const int len = int(hx.model[s].size());
      if (len == 0) continue;
      const int nt = 1 + pick(std::min(64, len));
      std::vector<int32_t> path;
      for (int c = 1; c < nt; ++c)
        if (pick(3) == 0) path.push_back(c);
      const int32_t k = int32_t(path.size()), ntt = nt;
      st = paged_kv_commit_path(hx.pool, 1, &s, &ntt, &k, path.empty() ? nullptr : path.data(), nullptr);
      if (st == PKV_OK) {
        auto& m = hx.model[s];
        const int base = len - nt;
        for (int d = 0; d < k; ++d) m[base + 1 + d] = m[base + path[d]];
        m.resize(base + 1 + k);
      } else {
        require(st == PKV_ERR_INVALID_ARG, "commit status", st);   // a path into a shared page
        expect_fail = true;
      }
    } else if (r < 93) {                                         // release
      const int64_t s = L[pick(int(L.size()))];
      require(paged_kv_release(hx.pool, s, nullptr) == PKV_OK, "release");
      hx.model.erase(s);
    } else {                                                     // calls that must fail
      const int64_t unknown = 1000 + pick(5);
      const int32_t one = 1;
      float buf[kH * kD] = {};
      require(paged_kv_append(hx.pool, 1, &unknown, &one, buf, buf, PKV_F32, nullptr) == PKV_ERR_UNKNOWN_SEQ,
              "append to unknown");
      require(paged_kv_rollback(hx.pool, 1, &unknown, &one, nullptr) == PKV_ERR_UNKNOWN_SEQ, "rollback unknown");
      const int64_t s = L[pick(int(L.size()))];
      const int32_t too_many = int32_t(hx.model[s].size()) + 1;
      require(paged_kv_rollback(hx.pool, 1, &s, &too_many, nullptr) == PKV_ERR_INVALID_ARG, "rollback past length");
      const int64_t twice[2] = {s, s};
      const int32_t ones[2] = {1, 1};
      require(paged_kv_append(hx.pool, 2, twice, ones, buf, buf, PKV_F32, nullptr) == PKV_ERR_INVALID_ARG,
              "sequence listed twice");
      int32_t row = -1;
      require(paged_kv_alloc(hx.pool, s, -1, 0, &row, nullptr) == PKV_ERR_SEQ_EXISTS, "alloc existing");
      pkv_verify_args va{};
      va.batch = 1;
      va.n_q = 1;
      require(spec_verify_attention_append(hx.pool, 1, &s, buf, buf, &va, nullptr) == PKV_ERR_UNSUPPORTED,
              "fused append on an fp32 pool");
      expect_fail = true;
    }
    if (expect_fail) {
      // a failed call changes nothing
      pkv_pool_stats after{};
      paged_kv_stats(hx.pool, &after);
      require(std::memcmp(&before, &after, sizeof(before)) == 0, "failed call changed the pool", op, st);
      ++failed_calls;
    } else {
      ++ok_calls;
    }
    hx.check_all();
  }
  pkv_pool_stats st{};
  paged_kv_stats(hx.pool, &st);
  cow_before = int(st.cow_copies);
  std::printf("serial seed %llu: %d calls ok, %d refused as documented, %d copy-on-write copies\n",
              (unsigned long long)seed, ok_calls, failed_calls, cow_before);
  require(cow_before > 0 && failed_calls > 0, "the run exercised neither copy-on-write nor errors");
}

// Threaded phase: one pool, a shared prefix, each thread its own sequences.
void threaded_phase(int n_threads, int n_ops) {
  Harness hx(64 * n_threads + 8, 4 * n_threads + 1, 24, 7);
  int32_t row = -1;
  require(paged_kv_alloc(hx.pool, 100000, -1, 0, &row, nullptr) == PKV_OK, "prefix alloc");
  require(hx.append({100000}, {37}) == PKV_OK, "prefix append");
  const std::vector<int> prefix = hx.model[100000];
  std::atomic<int> ok{0};
  auto worker = [&](int tid) {
    std::mt19937_64 rng(1234 + tid);
    auto pick = [&](int n) { return int(rng() % uint64_t(n)); };
    std::map<int64_t, std::vector<int>> mine;
    int token = 1000000 * (tid + 1);
    for (int op = 0; op < n_ops; ++op) {
      const int64_t s = int64_t(tid) * 10 + pick(4);
      auto it = mine.find(s);
      if (it == mine.end()) {
        const int n = pick(38);
        int32_t r = -1;
        if (paged_kv_alloc(hx.pool, s, 100000, n, &r, nullptr) == PKV_OK)
          mine[s] = std::vector<int>(prefix.begin(), prefix.begin() + n);
        continue;
      }
      const int what = pick(10);
      if (what < 5) {
        const int32_t n = pick(20);
        std::vector<int> ids(n);
        for (int j = 0; j < n; ++j) ids[j] = token++;
        std::vector<float> ks, vs;
        hx.fill_src(ids, ks, vs);
        if (paged_kv_append(hx.pool, 1, &s, &n, ks.data(), vs.data(), PKV_F32, nullptr) == PKV_OK)
          it->second.insert(it->second.end(), ids.begin(), ids.end());
      } else if (what < 8) {
        const int32_t n = pick(int(it->second.size()) + 1);
        require(paged_kv_rollback(hx.pool, 1, &s, &n, nullptr) == PKV_OK, "threaded rollback");
        it->second.resize(it->second.size() - n);
      } else {
        require(paged_kv_release(hx.pool, s, nullptr) == PKV_OK, "threaded release");
        mine.erase(it);
        continue;
      }
      int32_t len = 0, r = 0;
      std::vector<int32_t> pages = hx.table_of(s, &len, &r);
      require(len == int32_t(mine[s].size()), "threaded length", len, long(mine[s].size()));
      ok.fetch_add(1);
    }
    for (auto& kv : mine) require(paged_kv_release(hx.pool, kv.first, nullptr) == PKV_OK, "final release");
  };
  std::vector<std::thread> ts;
  for (int t = 0; t < n_threads; ++t) ts.emplace_back(worker, t);
  for (auto& t : ts) t.join();
  // only the prefix sequence is left, with its pages referenced once
  hx.model = {{100000, prefix}};
  hx.check_all();
  std::printf("threaded: %d threads, %d checked calls\n", n_threads, ok.load());
}

}  // namespace

int main(int argc, char** argv) {
  const int ops = argc > 1 ? std::atoi(argv[1]) : 600;
  for (uint64_t seed : {1ull, 2ull, 3ull}) serial_phase(seed, ops);
  threaded_phase(4, ops);
  std::printf("host_check: all checks passed\n");
  return 0;
}
