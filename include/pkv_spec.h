/*
 * pkv_spec.h — C ABI of the paged-KV speculative verification library
 * (libpkvspec.so, HIP for AMD gfx950 / MI355X).
 *
 * The library implements one verification step of speculative decoding over a
 * paged KV cache:
 *
 *   paged_kv_alloc / paged_kv_append / paged_kv_rollback / paged_kv_release
 *       a page pool with block tables, reference-counted shared prefixes,
 *       copy-on-write and rollback of rejected drafts
 *       (paurushmuley.com/blog/speculative-decoding-pagedattention-llm-serving-dotnet-10,
 *        diagram "PagedAttention virtual memory manager" and the
 *        PagedKVCacheManager listing; innvotechnologies.co/en/blog/low-latency-inference-decoding,
 *        pipeline diagram "Commit to KV-cache block table / Discard invalid KV blocks");
 *   spec_verify_attention
 *       attention of the gamma+1 verification queries over the pages of each
 *       sequence, with a causal-chain or draft-tree mask, bf16/fp32 or FP8 KV
 *       (atozofsoftwareengineering.blog, eq. A_speculative and section
 *        "Custom FP8 Quantized Memory Block Layout");
 *   spec_accept
 *       the acceptance rule alpha_i = min(1, P(x_i)/Q(x_i)), the accepted
 *       length k and the next token (innvotechnologies.co, section
 *        "Verification Acceptance Probabilities and Speedup Math").
 *
 * Conventions for every call
 *   - Memory: every device buffer (pools, block table, lengths, queries,
 *     outputs, workspaces) is allocated and owned by the caller.  The library
 *     never allocates device memory; it owns only the host-side pool handle.
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 *     stream).  Device work is enqueued asynchronously on it; host metadata is
 *     updated synchronously before the call returns.
 *   - Errors: a call either succeeds or returns a non-zero pkv_status with no
 *     effect on host metadata and nothing enqueued.  Arguments are validated
 *     before any work is enqueued; a failed kernel launch returns
 *     PKV_ERR_DEVICE.  pkv_last_error() returns a message for the calling
 *     thread's last failure.
 *   - Threads: a pool handle serialises its calls with an internal mutex.
 *   - Layout: all arrays are dense row-major; int32 page ids and lengths,
 *     int64 sequence ids.
 */
#ifndef PKV_SPEC_H
#define PKV_SPEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,   /* bad pointer, size, shape or dtype combination   */
  PKV_ERR_OUT_OF_PAGES = 2,  /* pool exhausted (the pages' OutOfMemory error)    */
  PKV_ERR_UNKNOWN_SEQ = 3,   /* sequence id not allocated (KeyNotFound)          */
  PKV_ERR_SEQ_EXISTS = 4,    /* sequence id already allocated                    */
  PKV_ERR_UNSUPPORTED = 5,   /* valid but not implemented (e.g. head_dim 96)     */
  PKV_ERR_DEVICE = 6,        /* HIP runtime / launch failure                     */
  PKV_ERR_WORKSPACE = 7,     /* workspace missing or smaller than required       */
  PKV_ERR_NO_SLOT = 8,       /* more live sequences than block-table rows        */
  PKV_ERR_CAPACITY = 9       /* sequence longer than max_pages_per_seq pages     */
} pkv_status;

/* PKV_FP8_E4M3: OCP E4M3 codes with one fp32 scale per (page, KV head).
 * PKV_FP8_E4M3_MX64: OCP E4M3 codes with a power-of-two scale per 64 channels
 * of each token, stored as OCP E8M0 exponent bytes (value 2^(e - 127)); the
 * per-64-element tile scales of atozofsoftwareengineering.blog's closing
 * checklist ("Precision Benchmarking").  A token's codes depend on that token
 * alone: s = 2^k, k the smallest integer with amax(tile)/2^k <= 448 (k = 0 for
 * an all-zero tile), code = round-to-nearest-even(x * 2^-k), saturating. */
typedef enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2, PKV_FP8_E4M3_MX64 = 3 } pkv_dtype;

/* ------------------------------------------------------------------------ */
/* Page pool                                                                 */
/* ------------------------------------------------------------------------ */

/*
 * Physical page layout.  A page holds page_size (= 16) tokens of one KV head;
 * pools are [num_pages][num_kv_heads][page_bytes] for K and for V.  Inside a
 * page the elements are tiled for the verification kernel's 16-byte loads:
 *   K, bf16:  element (t, c) at  s*16*32 + t*32 + j*8 + i
 *             where c = (head_dim/4)*j + 8*s + i,  j<4, i<8
 *   K, fp8:   element (t, c) at  u*16*64 + t*64 + j*16 + r
 *             where c = (head_dim/4)*j + 16*u + r, r<16
 *   V, bf16:  element (t, c) at  ((c/2)*4 + t/4)*8 + (c%2)*4 + t%4
 *   V, fp8:   element (t, c) at  ((c/4)*4 + t/4)*16 + (c%4)*4 + t%4
 *   K, V fp32: element (t, c) at t*head_dim + c (plain)
 * (t = slot in page, c = channel).  pkv_page_bytes() gives page_bytes.
 * FP8 is OCP E4M3 ("e4m3fn") with one fp32 scale per (page, KV head) for K
 * and one for V: value = decode(byte) * scale.  FP8_E4M3_MX64 pages use the
 * FP8 layouts above; their scales are bytes [num_pages][Hkv][16 tokens]
 * [head_dim/64] for K and for V: value = decode(byte) * 2^(e - 127).
 */
typedef struct pkv_pool pkv_pool;

typedef struct {
  int32_t num_pages;          /* physical pages in the pool                      */
  int32_t page_size;          /* tokens per page; must be 16                     */
  int32_t num_kv_heads;       /* Hkv >= 1                                        */
  int32_t head_dim;           /* 64 or 128                                       */
  pkv_dtype kv_dtype;         /* PKV_F32, PKV_BF16, PKV_FP8_E4M3 or
                                 PKV_FP8_E4M3_MX64                               */
  int32_t max_seqs;           /* rows of the device block table (live sequences) */
  int32_t max_pages_per_seq;  /* columns of the device block table               */
  void* k_pages;              /* device [num_pages][Hkv][page_bytes]             */
  void* v_pages;              /* device, same shape                              */
  void* k_scale;              /* device: FP8 fp32 [num_pages][Hkv]; FP8_E4M3_MX64
                                 uint8 [num_pages][Hkv][16][head_dim/64];
                                 else NULL                                       */
  void* v_scale;              /* device, same shape as k_scale                   */
  int32_t* block_table;       /* device [max_seqs][max_pages_per_seq]            */
  int32_t* seq_lens;          /* device [max_seqs]; 0 for free rows              */
  const int32_t* free_order;  /* host [num_pages]: a permutation giving each
                                 page's allocation rank (first fit takes the free
                                 page of lowest rank); NULL = rank by page id.
                                 Copied at creation.                             */
} pkv_pool_desc;

/* Bytes of one (page, KV head) slab; 0 for unsupported combinations. */
int64_t pkv_page_bytes(pkv_dtype kv_dtype, int32_t page_size, int32_t head_dim);

/* Create a pool.  When every device pointer of the descriptor is NULL the
 * pool is metadata-only: all calls below update the host bookkeeping and
 * enqueue nothing (used for planning and for host-side tests).  Otherwise
 * k_pages, v_pages, block_table and seq_lens (and the scales for FP8) are
 * required; they must stay valid for the pool's lifetime and are not
 * initialised by the library (the library only writes block-table entries
 * and lengths of sequences it manages). */
pkv_status pkv_pool_create(const pkv_pool_desc* desc, pkv_pool** out);
void pkv_pool_destroy(pkv_pool* pool);

/* Register sequence `seq` and give it a block-table row (*slot_out).  If
 * share_from >= 0 the first n_shared tokens map to share_from's first
 * ceil(n_shared/16) pages, whose reference counts are incremented
 * (paurushmuley.com, PagedKVCacheManager.AllocateSessionBlocks: shared
 * prefix blocks).  The row and its length are written on `stream`. */
pkv_status paged_kv_alloc(pkv_pool* pool, int64_t seq, int64_t share_from, int32_t n_shared,
                          int32_t* slot_out, void* stream);

/* Append n_tokens[i] tokens to each of seqs[0..n_seqs) (all-or-nothing over
 * the whole call; futurestack.online, section 2.3: the bundle extension is
 * atomic).  Pages are taken at 16-token boundaries; a partly filled tail page
 * shared with another sequence is copied first (copy-on-write,
 * PagedKVCacheManager.EnsureCapacityAndAppendToken).  k_src/v_src are device
 * arrays [sum(n_tokens)][Hkv][head_dim] in src_dtype, sequences in call order,
 * 16-byte aligned.
 * Allowed src_dtype: the pool dtype for F32/BF16 pools; PKV_F32 for FP8
 * pools, which quantise with the page's scale (a fresh page gets
 * scale = amax/448 of the tokens this call writes into it, per KV head; a page
 * that already holds tokens keeps its scale and values saturate to +-448);
 * PKV_F32 for FP8_E4M3_MX64 pools, which quantise every token on its own.
 * The scatter, the block-table entries and the new lengths are written on
 * `stream`; the sources must stay valid until the stream reaches the work. */
pkv_status paged_kv_append(pkv_pool* pool, int32_t n_seqs, const int64_t* seqs,
                           const int32_t* n_tokens, const void* k_src, const void* v_src,
                           pkv_dtype src_dtype, void* stream);

/* Drop the last n_tokens[i] tokens of each sequence (rejected drafts).  Pages
 * wholly past the new length lose a reference and are freed at zero; no KV
 * data moves.  New lengths are written on `stream`. */
pkv_status paged_kv_rollback(pkv_pool* pool, int32_t n_seqs, const int64_t* seqs,
                             const int32_t* n_tokens, void* stream);

/* Commit the accepted branch of a verified draft tree and drop the rest
 * (atozofsoftwareengineering.blog, pipeline diagram: "Tree-Attention
 * Verification" followed by "Dynamic KV Rollback/Commit").  For sequence
 * seqs[i] the last n_tree[i] tokens are the tree's nodes in index order (node 0,
 * the root, at position base = len - n_tree[i]); its accepted nodes are the
 * next path_len[i] entries of path_nodes (all sequences' paths concatenated in
 * call order), in depth order, root excluded, strictly increasing ids in
 * (0, n_tree[i]) -- what spec_accept_tree returns.  Node path[d]'s K/V moves to
 * position base + 1 + d (increasing d), then the sequence is truncated to
 * base + 1 + path_len[i] tokens as by paged_kv_rollback.  FP8 pools keep a
 * token's codes when source and destination (page, head) scales are equal bit
 * for bit, and otherwise decode with the source scale and encode with the
 * destination's (fp32, round to nearest even, saturating); FP8_E4M3_MX64
 * tokens move with their own scales.  Requirements:
 * 1 <= n_tree[i] <= min(64, len), path_len[i] <= n_tree[i] - 1, and every page
 * holding a destination position referenced by this sequence only (else
 * PKV_ERR_INVALID_ARG).  All-or-nothing over the call; the moves and the new
 * lengths are written on `stream`. */
pkv_status paged_kv_commit_path(pkv_pool* pool, int32_t n_seqs, const int64_t* seqs,
                                const int32_t* n_tree, const int32_t* path_len,
                                const int32_t* path_nodes, void* stream);

/* Unregister a sequence: every page loses a reference
 * (PagedKVCacheManager.ReleaseSession); its row's length is set to 0. */
pkv_status paged_kv_release(pkv_pool* pool, int64_t seq, void* stream);

/* Host copy of one sequence's block table.  pages_out may be NULL to query
 * sizes; otherwise it receives min(n_pages, max_pages) page ids. */
pkv_status paged_kv_block_table(const pkv_pool* pool, int64_t seq, int32_t* pages_out,
                                int32_t max_pages, int32_t* n_pages_out, int32_t* len_out,
                                int32_t* slot_out);

typedef struct {
  int32_t free_pages;         /* pages with reference count 0                    */
  int32_t used_pages;         /* pages referenced at least once                  */
  int32_t shared_pages;       /* pages referenced more than once                 */
  int32_t num_seqs;           /* live sequences                                  */
  int64_t cow_copies;         /* copy-on-write page copies so far                */
  int64_t used_token_slots;   /* sum of sequence lengths (tokens stored once per
                                 reference)                                      */
} pkv_pool_stats;

pkv_status paged_kv_stats(const pkv_pool* pool, pkv_pool_stats* out);
pkv_status paged_kv_page_refcount(const pkv_pool* pool, int32_t page, int32_t* refcount_out);

/* ------------------------------------------------------------------------ */
/* Draft-tree masks                                                          */
/* ------------------------------------------------------------------------ */

/* Ancestor-or-self bitmasks of a draft tree given by parents[i] (parents[0] =
 * -1, parents[i] < i, n_nodes <= 64): bit j of masks_out[i] is set iff node j
 * lies on the path from the root to node i.  Host arrays.  The additive tree
 * mask M_tree of atozofsoftwareengineering.blog eq. A_speculative is 0 where
 * the bit is set and -inf elsewhere. */
pkv_status spec_tree_ancestor_masks(int32_t n_nodes, const int32_t* parents, uint64_t* masks_out);

/* ------------------------------------------------------------------------ */
/* Verification attention                                                    */
/* ------------------------------------------------------------------------ */

/*
 * For every sequence b (N = seq_lens[row], L = N - n_q), query slot i < n_q
 * and query head h (KV head g = h / (Hq/Hkv)):
 *   s_t   = sm_scale * <q[b,i,h,:], K[t,g,:]>      for visible t
 *   out   = sum_t softmax(s)_t V[t,g,:],  lse = log(sum_t exp(s_t))  (natural log)
 * where token t < L is always visible and verification slot t - L is visible
 * iff bit (t - L) of anc_mask[b*n_q + i] is set (anc_mask == NULL: the causal
 * chain, t - L <= i).  K/V of token t is slot t%16 of page
 * block_table[row*block_table_stride + t/16], row = batch_slots ? batch_slots[b] : b.
 * (atozofsoftwareengineering.blog, eq. A_speculative; the verification
 * tokens' K/V must already be appended, futurestack.online section 2.3.)
 *
 * Per-sequence draft counts (n_q_seq != NULL): sequence b has n_b =
 * n_q_seq[b] verification slots (clamped to [1, n_q]), L = N - n_b, and only
 * slots i < n_b are computed and written (q, anc_mask and out keep their
 * [batch][n_q] shapes; the other slots are padding, neither read for the
 * result nor written).  This serves policies that pick gamma per sequence
 * (paurushmuley.com, dynamic lookahead; atozofsoftwareengineering.blog).
 *
 * Supported: q_dtype F32 with kv_dtype F32; q_dtype BF16 with kv_dtype BF16,
 * FP8_E4M3 or FP8_E4M3_MX64; head_dim 64 or 128; page_size 16; n_q*Hq/Hkv <= 64 rows per KV
 * head; n_q <= 64; 0 <= L and N < 2^24 for every sequence.  Long contexts are split over
 * workgroups and merged by log-sum-exp in a second kernel (workspace below).
 */
typedef struct {
  int32_t batch;
  int32_t n_q;                /* gamma + 1 (chain) or tree nodes                 */
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  pkv_dtype q_dtype;
  pkv_dtype kv_dtype;
  const void* q;              /* device [batch][n_q][Hq][head_dim]               */
  const void* k_pages;        /* device pool (layout above)                      */
  const void* v_pages;
  const void* k_scale;        /* device, FP8 kinds only (layout at the pool)     */
  const void* v_scale;
  const int32_t* block_table; /* device                                          */
  int32_t block_table_stride; /* int32 entries per block-table row               */
  const int32_t* seq_lens;    /* device, total length N incl. the n_q tokens     */
  const int32_t* batch_slots; /* device [batch] rows to use, or NULL (row = b)   */
  const uint64_t* anc_mask;   /* device [batch][n_q] or NULL (chain)             */
  float sm_scale;             /* usually 1/sqrt(head_dim); positive and finite,
                                 else PKV_ERR_INVALID_ARG                        */
  float* out;                 /* device [batch][n_q][Hq][head_dim] fp32          */
  float* lse;                 /* device [batch][n_q][Hq] fp32, may be NULL       */
  void* workspace;            /* device, >= spec_verify_workspace_size bytes;
                                 scratch for partial results of contexts split
                                 over workgroups; calls that share a workspace
                                 must not overlap in time                        */
  size_t workspace_bytes;
  int32_t num_splits;         /* workgroups sharing the work; 0 = as many as the
                                 GPU keeps resident                              */
  const int32_t* n_q_seq;     /* device [batch] slots per sequence, or NULL (n_q) */
  int32_t shared_prefix_pages;/* cascade (bf16 KV, or FP8_E4M3 with per-page scales;
                                 FP8_E4M3_MX64 returns PKV_ERR_UNSUPPORTED): the first this-many block-table
                                 entries are the same physical pages for every
                                 sequence of the call (a prefix shared through
                                 paged_kv_alloc) and hold cached tokens only
                                 (16 * shared_prefix_pages <= L for every
                                 sequence); they are attended once for all
                                 sequences and merged with each sequence's own
                                 pages.  0 = off                                 */
} pkv_verify_args;

pkv_status spec_verify_workspace_size(const pkv_verify_args* args, size_t* bytes_out);
pkv_status spec_verify_attention(const pkv_verify_args* args, void* stream);

/* Append and verify in one launch (atozofsoftwareengineering.blog, diagram
 * "Speculative Decoding Memory Pipeline": FP8 pages flow straight into the
 * fused verification attention).  Equivalent to
 *   paged_kv_append(pool, n_seqs, seqs, {n_q, ..., n_q}, k_new, v_new, src, stream)
 *   spec_verify_attention(args, stream)
 * except that the verification kernels quantise and write the new tokens
 * themselves and attend them from registers, so the step runs one kernel
 * launch fewer.  The pool's bookkeeping happens on the host before the launch
 * as for paged_kv_append (same pages, same codes and scales, bit for bit).
 * k_new, v_new: device [n_seqs][n_q][Hkv][head_dim], 16-byte aligned; bf16 for
 * bf16 pools, fp32 for the FP8 kinds.  args must describe this pool (its
 * page, scale, block-table and length arrays, its dtype and shape) with
 * batch == n_seqs, sequence i in block-table row i, batch_slots and n_q_seq
 * NULL, 1 <= n_q <= 16 and n_seqs <= 768; its workspace is sized by
 * spec_verify_workspace_size.  A sequence whose partly filled tail page is
 * shared (copy-on-write) or an fp32 pool returns PKV_ERR_UNSUPPORTED; every
 * check happens before anything changes (PKV_ERR_DEVICE after a failed launch
 * leaves the host bookkeeping advanced, as paged_kv_append). */
pkv_status spec_verify_attention_append(pkv_pool* pool, int32_t n_seqs, const int64_t* seqs,
                                        const void* k_new, const void* v_new, const pkv_verify_args* args,
                                        void* stream);

/* spec_verify_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the scratch taken from a
 * static array the library holds on each GPU it runs on (80 MiB per GPU,
 * 83886080 bytes, kept until the process ends) instead of args->workspace,
 * which is ignored.  The call itself allocates nothing.  A call whose scratch
 * (spec_verify_workspace_size) exceeds 80 MiB returns PKV_ERR_WORKSPACE and
 * enqueues nothing; fewer num_splits need less.  Every call on one GPU shares
 * that GPU's array: calls that overlap in time on one GPU (other streams,
 * other threads) race and give wrong results; calls ordered on one stream are
 * safe.  Nothing in the array needs to start at zero. */
pkv_status spec_verify_attention_static(const pkv_verify_args* args, void* stream);

/* ------------------------------------------------------------------------ */
/* Acceptance                                                                */
/* ------------------------------------------------------------------------ */

/*
 * For every sequence b, with P_i = softmax(target_logits[b,i,:]) and
 * Q_i = softmax(draft_logits[b,i,:]):
 *   draft token x_i is accepted iff u_i < min(1, P_i(x_i)/Q_i(x_i)), stopping
 *   at the first rejection; accepted_len[b] = k (0..gamma);
 *   next_token[b] = if k < gamma: a draw from max(0, P_k - Q_k) normalised
 *                   (from P_k if that is zero everywhere);
 *                   else a draw from P_gamma (the bonus token).
 * Uniforms come from Philox4x32-10 (Salmon et al., SC'11) keyed by `seed`:
 * u_i uses counter (0, b, step, i | 1<<16), word 0; the draw at position i uses
 * u_x from counter (x/4, b, step, i | 2<<16), word x%4, and takes
 * argmax_x log w(x) - log(-log u_x) (Gumbel-max; ties to the smaller x).
 * u = (floor(word / 2^9) + 0.5) * 2^-23.
 * Per-sequence draft counts (gammas != NULL): sequence b uses drafts
 * i < g_b = gammas[b] (clamped to [1, gamma]), k <= g_b, and the bonus comes
 * from P_{g_b}; the arrays keep their [batch][gamma(+1)] shapes and rows past
 * g_b are not read for the result.
 * (innvotechnologies.co, eq. alpha_i and eq. E[K]; pipeline diagram
 *  "Rejection Recovery (Resample)".)
 */
typedef struct {
  int32_t batch;
  int32_t gamma;              /* drafts per sequence, 1..64                      */
  int32_t vocab;              /* 1..2^26                                         */
  const float* target_logits; /* device [batch][gamma+1][vocab]                  */
  const float* draft_logits;  /* device [batch][gamma][vocab]                    */
  const int32_t* draft_tokens;/* device [batch][gamma], values in [0, vocab)     */
  uint64_t seed;
  uint32_t step;
  int32_t* accepted_len;      /* [batch]: device memory, or pinned host memory
                                 (hipHostMalloc) that the kernels write directly;
                                 each entry is stored once and never read back  */
  int32_t* next_token;        /* device [batch]                                  */
  void* workspace;            /* device, >= spec_accept_workspace_size bytes,
                                 16-byte aligned; scratch for per-chunk partial
                                 results; calls that share a workspace must not
                                 overlap in time                                 */
  size_t workspace_bytes;
  const int32_t* gammas;      /* device [batch] drafts per sequence, or NULL     */
  const uint32_t* step_ptr;   /* device: when not NULL the step counter is read
                                 from here when the kernels run (a captured HIP
                                 graph can then be replayed with a new step)     */
} pkv_accept_args;

pkv_status spec_accept_workspace_size(const pkv_accept_args* args, size_t* bytes_out);
pkv_status spec_accept(const pkv_accept_args* args, void* stream);

/*
 * Draft-tree acceptance.  The pages verify a draft tree in one pass and commit
 * its accepted branch (atozofsoftwareengineering.blog, pipeline diagram) but
 * give no rule for several candidates at one position; the rule implemented
 * applies eq. alpha_i of innvotechnologies.co child by child with the residual
 * update between candidates (multi-candidate speculative sampling, SpecInfer,
 * Miao et al., ASPLOS 2024), which keeps the emitted tokens distributed as the
 * target when sibling candidates are drawn independently from the draft:
 *   at node u (starting at the root, node 0) with P = softmax(target_logits[b,u])
 *   and Q = softmax(draft_logits[b,u]), the children c_1 < c_2 < ... of u are
 *   tried in index order; c_j is accepted iff u_{c_j} < min(1, P_{j-1}(x_c)/Q(x_c)),
 *   P_0 = P, P_j = max(0, P_{j-1} - Q) normalised (P_j = P_{j-1} if that is
 *   zero everywhere); an accepted child becomes the new node.  If every child
 *   of u is rejected, next_token is drawn from P_m (m = u's child count); at a
 *   leaf it is drawn from the leaf's P (the bonus).
 * Outputs: accepted_len[b] = k (depth of the accepted node), accepted_nodes[b]
 * = the accepted node ids in depth order followed by -1s, next_token[b].  A
 * sequence whose parents are not a tree in index order (parents[0] = -1,
 * parents[c] in [0, c)) or whose nodes have more than max_children children
 * gets k = -1 and next_token = -1.  A node token outside [0, vocab) is
 * rejected.  Uniforms are those of spec_accept with draft i = node i + 1: the
 * test of node c uses counter (0, b, step, (c - 1) | 1<<16) word 0, the draw at
 * node u counters (x/4, b, step, u | 2<<16).  On a chain
 * (parents[c] = c - 1) the result equals spec_accept's.
 */
typedef struct {
  int32_t batch;
  int32_t n_nodes;            /* nodes per tree including the root, 2..64        */
  int32_t max_children;       /* bound on any node's child count, 1..n_nodes-1   */
  int32_t vocab;              /* 1..2^26                                         */
  const float* target_logits; /* device [batch][n_nodes][vocab]: at each node     */
  const float* draft_logits;  /* device [batch][n_nodes][vocab]: at each node     */
  const int32_t* parents;     /* device [batch][n_nodes]                          */
  const int32_t* tokens;      /* device [batch][n_nodes]; entry 0 is not read     */
  uint64_t seed;
  uint32_t step;
  int32_t* accepted_len;      /* device [batch]                                  */
  int32_t* accepted_nodes;    /* device [batch][n_nodes]                          */
  int32_t* next_token;        /* device [batch]                                  */
  void* workspace;            /* device, >= spec_accept_tree_workspace_size bytes,
                                 16-byte aligned; calls sharing it must not
                                 overlap in time                                 */
  size_t workspace_bytes;
  const uint32_t* step_ptr;   /* device step counter read at run time, or NULL   */
} pkv_tree_accept_args;

pkv_status spec_accept_tree_workspace_size(const pkv_tree_accept_args* args, size_t* bytes_out);
pkv_status spec_accept_tree(const pkv_tree_accept_args* args, void* stream);

/* ------------------------------------------------------------------------ */
/* Measurement aid (not a step of the path; futurestack.online, sections 1.1-1.2:
 * the roofline of a memory-bound kernel is the rate at which its bytes can be
 * read).  Reads, once each, the K and V slabs of every (sequence, KV head,
 * page) position that spec_verify_attention(args) reads -- the same bytes, the
 * same partition into equal contiguous ranges over n_waves waves, the same
 * 16-byte non-temporal loads with four pages in flight per wave -- and does no
 * arithmetic but folding them into one word per wave, written to
 * sink[n_waves] (device).  Uses args' k_pages, v_pages, block_table,
 * block_table_stride, seq_lens, batch (1..4096), num_kv_heads, head_dim,
 * page_size and kv_dtype; the slab must be 1, 2, 4 or 8 KiB.  n_waves: a
 * positive multiple of 4 (1024 = one wave per SIMD on MI355X).  Errors as for
 * the other calls; nothing is written but sink. */
pkv_status pkv_page_read_probe(const pkv_verify_args* args, uint32_t* sink, int32_t n_waves, void* stream);

/* ------------------------------------------------------------------------ */
const char* pkv_status_string(pkv_status status);
const char* pkv_last_error(void);
/* Library version string. */
const char* pkv_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PKV_SPEC_H */
