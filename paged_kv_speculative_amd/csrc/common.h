// Shared host-side helpers of libpkvspec: status/error reporting and the
// device-update task format exchanged between the pool bookkeeping
// (pool.cpp) and the pool-update kernel (kernels/kv_append.hip).
#pragma once

#include <cstdint>
#include <string>

#include "../../include/pkv_spec.h"

namespace pkv {

// Thread-local message of the calling thread's last failure.
void set_error(const std::string& msg);
pkv_status fail(pkv_status st, const std::string& msg);

constexpr int kPageSize = 16;

// One unit of device work on the pool, applied by one workgroup:
//   - if cow_src >= 0: copy page cow_src (all heads, K and V, and the FP8
//     scales) to page `page` before anything else;
//   - if n > 0: write tokens src_row .. src_row+n-1 of the source arrays into
//     slots slot_begin .. slot_begin+n-1 of page `page` (FP8: fresh pages get
//     new scales from these tokens, other pages keep theirs);
//   - if flags & kWriteTable: block_table[row][logical] = page;
//   - if flags & kSetLen: seq_lens[row] = new_len.
enum : int32_t { kFresh = 1, kWriteTable = 2, kSetLen = 4 };

struct PoolTask {
  int32_t row;
  int32_t logical;
  int32_t page;
  int32_t cow_src;
  int32_t src_row;
  int32_t slot_begin;
  int32_t n;
  int32_t flags;
  int32_t new_len;
  int32_t pad;
};

constexpr int kTasksPerLaunch = 96;

struct PoolUpdateBatch {
  int32_t n_tasks;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t kv_dtype;      // pkv_dtype of the pool
  int32_t src_dtype;     // pkv_dtype of k_src/v_src
  int32_t bt_stride;     // max_pages_per_seq
  int64_t page_bytes;    // bytes of one (page, head) slab
  PoolTask tasks[kTasksPerLaunch];
};
static_assert(sizeof(PoolUpdateBatch) <= 4000, "kernel argument block too large");

struct PoolDevice {
  void* k_pages;
  void* v_pages;
  void* k_scale;         // FP8: fp32 [page][head]; MX64: E8M0 bytes [page][head][token][D/64]
  void* v_scale;
  int32_t* block_table;
  int32_t* seq_lens;
  const void* k_src;
  const void* v_src;
};

// Token moves of a path commit: the K/V of token slot src_slot of page
// src_page (all KV heads) go to slot dst_slot of page dst_page.  Moves of one
// sequence form a group applied in order by one workgroup per four heads;
// FP8 codes are re-encoded when the two pages' scales differ.
struct PoolMove {
  int32_t src_page;
  int32_t dst_page;
  int32_t slots;         // src_slot | dst_slot << 8
};

constexpr int kMoveGroups = 32;
constexpr int kMovesPerLaunch = 256;

struct PoolMoveBatch {
  int32_t n_groups;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t kv_dtype;
  int64_t page_bytes;
  int32_t first[kMoveGroups + 1];    // group g = moves[first[g] .. first[g+1])
  PoolMove moves[kMovesPerLaunch];
};
static_assert(sizeof(PoolMoveBatch) <= 4000, "kernel argument block too large");

// Implemented in kernels/kv_append.hip.
pkv_status launch_pool_update(const PoolDevice& dev, const PoolUpdateBatch& batch, void* stream);
pkv_status launch_pool_moves(const PoolDevice& dev, const PoolMoveBatch& batch, void* stream);

// Appended tokens of a fused append + verification launch
// (spec_verify_attention_append): the pool's bookkeeping is done on the
// host; the verification kernels quantise and write the n_q new tokens of
// every sequence, attend them from registers, and then write each sequence's
// new block-table entry and length.  new_page[b] is the page taken by the
// call for logical page ceil(old_len / 16) of sequence b (-1 when the new
// tokens fit in the sequence's last page); at most one per sequence (n_q <=
// 16).  Sources are [batch][n_q][Hkv][head_dim]: bf16 for bf16 pools, fp32
// for the FP8 kinds.
constexpr int kFusedMaxBatch = 768;
constexpr int kFusedMaxTokens = 16;

struct FusedAppend {
  const void* k_new;
  const void* v_new;
  int32_t new_page[kFusedMaxBatch];
};

// Implemented in kernels/verify_attn.hip: the verification launch of a
// fused call (arguments already checked by the pool).
pkv_status verify_fused_launch(const pkv_verify_args* args, const FusedAppend& fused, void* stream);

}  // namespace pkv
