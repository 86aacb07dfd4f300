// Verification attention over a paged KV cache (gfx950 / CDNA4).
//
// Computes, for every sequence, query slot i < n_q and query head h,
//   out = softmax(sm_scale * q K^T + M) V,   lse = log sum exp(...)
// over the K/V of the sequence reached through its block table, with M the
// 0/-inf mask that shows every cached token and, among the n_q verification
// slots, the ancestors-or-self of slot i (a chain when no mask is given)
// (atozofsoftwareengineering.blog, eq. A_speculative; the K/V of the
// verification tokens are in the cache before the pass, futurestack.online
// section 2.3).
//
// Design for MI355X:
//  * Work is the list of (sequence, KV head, page) triples in that order.  A
//    fixed number of workgroups (what the GPU keeps resident) each take an
//    equal contiguous range of it ("stream-K"), so long and short contexts
//    balance exactly.  Each wave is one worker with its own range (with more
//    than 48 query rows per KV head, two waves take the same range, 32 rows
//    each).  A range covers whole (sequence, KV head) units, which are
//    finished in place, and at most two pieces of units, which are written
//    as partial (max, sum, unnormalised O) and merged by a second kernel
//    with a log-sum-exp combine.
//  * One (sequence, KV head) unit serves all n_q * G query rows that read the
//    same pages (G = Hq/Hkv): every KV byte is read once per call.
//  * A page of one KV head is one slab in a tiled layout (layout.h) so each
//    16-byte load instruction of a wave reads one contiguous kilobyte and
//    the lanes' registers are already MFMA operands: no LDS staging.
//  * Scores: S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = 16 tokens of K,
//    B = 16 query rows of Q).  Output: O^T = V^T P^T, with A = V^T (16
//    channels x 32 tokens of two pages) and B = P^T.  In these orientations
//    the score registers of a lane (its row, 4 tokens per page) are exactly
//    the P^T operand it needs, so P never crosses lanes, and the O registers
//    of a lane belong to its own row, so the softmax rescale is lane-local.
//  * P is split into a bf16 high part and a bf16 low part and both are
//    multiplied by the exact bf16 V, which keeps PV accurate to ~2^-16
//    (bf16-only P is ~2^-9, outside the accuracy target).  FP8 K/V are
//    decoded to bf16 exactly in registers; the K scale multiplies the scores
//    of its page and the V scale multiplies P of its page.
//  * Scores are kept in base 2 (scale * log2 e folded into one multiply) and
//    exponentiated with v_exp_f32.

#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <tuple>

#include "../common.h"
#include "fp8_codec.h"
#include "layout.h"

namespace pkv {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Scalar (SMEM) buffer load of one dword, bound to the LLVM intrinsic (clang
// has no builtin for it; declared with external linkage so the binding is an
// ordinary external declaration).  Block-table entries are read through the
// scalar unit so that waiting for them never waits for the vector loads of
// K/V in flight (vector-memory counters retire in order).
__device__ int s_buffer_load_dword(i32x4 rsrc, int offset, int cachepolicy)
    __asm("llvm.amdgcn.s.buffer.load.i32");

typedef int i32x8 __attribute__((ext_vector_type(8)));
// Eight consecutive dwords through the scalar unit (one request).
__device__ i32x8 s_buffer_load_dwordx8(i32x4 rsrc, int offset, int cachepolicy)
    __asm("llvm.amdgcn.s.buffer.load.v8i32");

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
// s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8) that waits until at most n vector memory operations are
// outstanding and leaves the other counters alone.
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int kVmcnt0 = vmcnt_imm(0);

struct VerifyParams {
  const void* q;
  const char* k_pages;
  const char* v_pages;
  const void* k_scale;   // FP8: fp32 per (page, KV head); MX: E8M0 bytes [page][head][token][D/64]
  const void* v_scale;
  const int* block_table;
  const int* seq_lens;
  const int* batch_slots;
  const unsigned long long* anc;
  const int* nq_seq;     // [batch] verification slots per sequence, or null (n_q for all)
  float* out;
  float* lse;
  float* part;           // [n_wg][2][slot_floats] partial (O, max, sum) of split units
  float* prefix_part;    // cascade: [batch][n_q][Hq][D + 2] (O, max, sum) over the shared prefix
  int* cum;              // [batch + 1] page prefix sums (written by workgroup 0)
  // fused append (spec_verify_attention_append): the pages hold the cached
  // tokens only, every one visible; the merge adds the new tokens; old_len
  // [batch] keeps the cached lengths
  int fused;
  int kv_kind;           // pkv_dtype of the pool
  // fused calls and the cascade: a unit finished by one wave writes its
  // normalised O to out and its log2-sum-exp to unit_lse [batch][n_q][Hq]
  // (not lse), and the merge combines it with the rest of the row
  int defer;
  float* unit_lse;
  int* old_len;
  long slab_bytes;       // bytes of one (page, KV head) slab
  int batch, n_q, Hq, Hkv, G, rows, bt_stride, n_wg;
  int pref;              // cascade: leading block-table pages shared by every sequence (0: none)
  int rg;                // row groups: waves that share a range, each taking rows_w rows
  int rows_w;            // rows per wave (rows when rg = 1)
  int min_range;         // fewest page-heads per workgroup range
  float scale_log2;      // sm_scale * log2(e)
};

__device__ inline f32x4 mfma_bf16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Two floats -> one dword of two bf16, upper halves taken (exact for values
// that fit bf16, truncation otherwise).
__device__ inline unsigned pack_hi16(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two finite floats -> two bf16 rounded to nearest even (one hardware
// conversion), a in the low half.
__device__ inline unsigned pack_rne_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Four fp8 (OCP E4M3) bytes -> four bf16 in two dwords, bytes 0,1 in the
// first.  Every E4M3 value is a bf16 value, so with a unit scale the
// conversion is exact.
struct Dw2 {
  unsigned lo, hi;
};
__device__ inline Dw2 fp8x4_to_bf16x4(unsigned w) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return Dw2{__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b)};
}

// The same with a per-lane scale multiplied in before the rounding to bf16
// (gfx950's scaled FP8 conversion).  With power-of-two scales the products
// are exact in bf16.
__device__ inline Dw2 fp8x4_to_bf16x4_scaled(unsigned w, float scale) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, true);
  return Dw2{__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b)};
}

// 2^(e - 127) of an OCP E8M0 exponent byte e (0..254).
__device__ inline float e8m0_value(unsigned e) {
  e = e < 254u ? e : 254u;                       // never written above 254; keeps stale bytes finite
  return __uint_as_float(e ? e << 23 : 0x00400000u);
}

__device__ inline u32x4 load16(const void* p) { return *static_cast<const u32x4*>(p); }

// global -> LDS copies through the load path (global_load_lds): lane l's
// 16 (or 4) bytes land at LDS address lds + 16 l (4 l).  Written as inline
// assembly so that the compiler tracks nothing for them: as a builtin, every
// later scalar load would wait for all vector memory operations (it treats
// the copy as a store that may alias them).  The caller orders the LDS reads
// of the data with an explicit vmcnt wait.  The LDS base goes in through an
// M0 operand ("{m0}"), so the compiler sets M0 itself and knows its value is
// only read here.
__device__ inline void copy16_to_lds(const void* src, unsigned lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(src), "{m0}"(lds) : "memory");
}
__device__ inline void copy4_to_lds(const void* src, unsigned lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" :: "v"(src), "{m0}"(lds) : "memory");
}
// LDS address (offset in the workgroup's LDS) of a pointer into __shared__
// memory: the low half of its flat address.
__device__ inline unsigned lds_addr(const void* p) {
  return unsigned(reinterpret_cast<unsigned long long>(p));
}

// Word 3 of a raw buffer resource on gfx9-family GPUs (32-bit data format,
// no swizzle): with stride 0, num_records counts bytes.
constexpr int kBufferFlags = 0x00020000;

// Cache-policy operand of the K/V page loads: the non-temporal bit.  Every
// page is read once per call, so the loads stream past the caches (measured
// on MI355X: ~15% more bandwidth for this kernel than default-policy loads).
constexpr int kStreamPolicy = 2;

__device__ inline i32x4 scalar_rsrc(const void* base, unsigned bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  return i32x4{int(unsigned(a)), int(unsigned(a >> 32) & 0xFFFFu), int(bytes), kBufferFlags};
}

// Maximum over the four lanes {l, l^16, l^32, l^48} of a wave: the lanes that
// hold one score row.  v_permlane32_swap / v_permlane16_swap exchange halves
// and 16-lane rows between two registers in the VALU.
__device__ inline float row_max4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ inline f32x4 mfma_bf16_k16(unsigned a0, unsigned a1, unsigned b0, unsigned b1, const f32x4& c) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, u32x2{a0, a1}),
                                                   __builtin_bit_cast(s16x4, u32x2{b0, b1}), c, 0, 0, 0);
}

// c + A (b_hi + b_lo) over the 16 tokens of a page, with the hi/lo split of
// P as the two halves of one K = 32 product: lane group j holds tokens
// 4j..4j+3 of A twice (elements 0-3 and 4-7) against the same tokens' hi
// parts (0-3) and lo parts (4-7).  One instruction instead of two K = 16
// ones, which on gfx950 take as many cycles each.
__device__ inline f32x4 mfma_bf16_split(unsigned a0, unsigned a1, unsigned h0, unsigned h1, unsigned l0, unsigned l1,
                                        const f32x4& c) {
  return mfma_bf16(u32x4{a0, a1, a0, a1}, u32x4{h0, h1, l0, l1}, c);
}

// Compile-time shape of the streaming kernel for one (head_dim, row tiles, KV type).
// W2: the variant that runs two waves per SIMD (at most 256 registers each),
// with two pages in flight per wave.
// MX: FP8 with a power-of-two scale per 64 channels of each token.
template <int D, int NT, bool FP8, bool W2 = false, bool MX = false>
struct Shape {
  static constexpr int KS = D / 32;                  // k-steps of the score MFMA (32 channels)
  static constexpr int DT = D / 16;                  // 16-channel tiles of the output
  static constexpr int KL = FP8 ? KS / 2 : KS;       // 16-byte K loads per page
  static constexpr int VL = FP8 ? D / 64 : D / 32;   // 16-byte V loads per page
  // vector loads per page (FP8: + two scales; MX: + one K and D/64 V scale words)
  static constexpr int LPP = KL + VL + (FP8 ? (MX ? 1 + D / 64 : 2) : 0);
  // Q of a unit staged in LDS: QS slots per wave of NT*16 rows x D bf16, plus
  // the unit's n_q ancestor masks
  static constexpr int QS = W2 ? 1 : 2;
  static constexpr int QSLOT = NT * 16 * D * 2;
  static constexpr int ASLOT = 64 * 8;
  // pages in flight per wave while one page is computed
  static constexpr int PF = W2 ? (FP8 ? 2 : 1)
                                : FP8 ? (NT <= 2 ? 8 : (NT == 3 ? 5 : 3)) : (NT <= 2 ? 4 : (NT == 3 ? 3 : 2));
  static constexpr int RS = PF + 1;                 // ring slots
};

template <int D, bool FP8>
struct PageRegs {
  static constexpr int KL = Shape<D, 1, FP8>::KL, VL = Shape<D, 1, FP8>::VL;
  u32x4 k[KL];
  u32x4 v[VL];
};

// Where a ring slot's page sits (all wave-uniform, kept to three scalars per
// slot): unit = sequence << 16 | KV head, page, and the sequence's length n
// (0 for a slot past the range).  The sequence's page count is (n + 15) / 16.
struct PageMeta {
  int unit, page, n;
  float ks, vs;          // FP8 scales of the page (per lane, all lanes alike)
  unsigned ksw, vsw[2];  // MX: the lane's words of E8M0 scale bytes (K: its token; V: its four tokens)
};

// A ring slot's length word: the sequence's length N in bits 0..23 and its
// number of verification slots in bits 24..30 (0 for a slot past the range).
constexpr int kNqShift = 24;
constexpr int kLenMask = (1 << kNqShift) - 1;

// Values every lane of the wave holds alike (read from LDS or computed from
// such reads): moved to scalar registers so addresses built from them stay
// scalar.
__device__ inline int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Verification slots of sequence b: n_q, or its own count clamped to [1, n_q].
__device__ inline int seq_slots(const VerifyParams& P, int b) {
  return P.nq_seq ? min(max(P.nq_seq[b], 1), P.n_q) : P.n_q;
}

// Exclusive prefix of pages per sequence into s_cum[0..batch], and per
// sequence its block-table row and length word (N | n_b << kNqShift) into
// s_seq[2b], s_seq[2b + 1], so that the streaming loop reads them from LDS.
__device__ void page_prefix(const VerifyParams& P, int* s_cum, int* s_tmp, int* s_seq) {
  const int tid = threadIdx.x;
  if (P.batch <= 64) {                         // one wave: a shuffle scan
    if (tid < 64) {
      int v = 0;
      if (tid < P.batch) {
        const int row = P.batch_slots ? P.batch_slots[tid] : tid;
        const int N = P.seq_lens[row];
        v = max(0, ((N + 15) >> 4) - P.pref);
        s_seq[2 * tid] = row;
        s_seq[2 * tid + 1] = N | ((P.fused ? 0 : seq_slots(P, tid)) << kNqShift);
      }
      int x = v;
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (tid >= off) x += y;
      }
      if (tid < P.batch) s_cum[tid] = x - v;
      if (tid == 63) s_cum[P.batch] = x;
    }
    __syncthreads();
    return;
  }
  const int per = (P.batch + kThreads - 1) / kThreads;
  const int b0 = min(P.batch, tid * per), b1 = min(P.batch, b0 + per);
  int local = 0;
  for (int b = b0; b < b1; ++b) {
    const int row = P.batch_slots ? P.batch_slots[b] : b;
    const int N = P.seq_lens[row];
    local += max(0, ((N + 15) >> 4) - P.pref);
    s_seq[2 * b] = row;
    s_seq[2 * b + 1] = N | ((P.fused ? 0 : seq_slots(P, b)) << kNqShift);
  }
  s_tmp[tid] = local;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    int add = tid >= off ? s_tmp[tid - off] : 0;
    __syncthreads();
    s_tmp[tid] += add;
    __syncthreads();
  }
  int run = s_tmp[tid] - local;
  for (int b = b0; b < b1; ++b) {
    s_cum[b] = run;
    run += max(0, (((s_seq[2 * b + 1] & kLenMask) + 15) >> 4) - P.pref);
  }
  if (tid == kThreads - 1) s_cum[P.batch] = s_tmp[tid];
  __syncthreads();
}

// Work range of worker w out of n over W positions: [lo(w), lo(w+1)).
__device__ inline long range_lo(long w, long W, long n) { return w * W / n; }

// Waves in use and ranges over W positions: every range is taken by rg waves
// (one per row group), and no range is empty.
__device__ inline int used_ranges(const VerifyParams& P, long W) {
  const long waves = min(long(P.n_wg) * kWaves, max(long(P.rg), W * P.rg / P.min_range));
  return int(max(1L, min(W, waves / P.rg)));
}

// Worker whose range holds position p (all ranges are non-empty: n <= W).
__device__ inline int owner_of(long p, long W, int n) {
  // range_lo(w) <= p  <=>  w * W < (p + 1) * n: integer products only (no
  // 64-bit division in the loop)
  int w = int((double(p) * n) / double(W));
  w = min(max(w, 0), n - 1);
  while (w + 1 < n && long(w + 1) * W < (p + 1) * n) ++w;
  while (w > 0 && long(w) * W >= (p + 1) * n) --w;
  return w;
}

// range_lo(w, W, n) == p without a division.
__device__ inline bool range_starts_at(long w, long W, long n, long p) {
  return p * n <= w * W && w * W < (p + 1) * n;
}
// The running maximum of a row is only moved when the block maximum exceeds
// it by more than this (log2 units), so P <= 2^8 and the O rescale is rare.
constexpr float kRescaleSlack = 8.0f;


// Floats of one partial slot: O [rows][D], then max [rows], then sum [rows].
__device__ __host__ inline long slot_floats(int rows, int D) { return long(rows) * (D + 2); }

// Cursor over work positions (sequence b, KV head g, page) in that order.
struct Cursor {
  int b, g, page, np, row, n;
};

// SHARED: two waves (row groups) read the same pages at about the same time;
// their loads keep the default cache policy so the second finds the first's
// lines in L2.  Otherwise pages stream with the non-temporal policy.
template <int D, int NT, bool FP8, bool TREE, bool SHARED, bool W2, bool MX>
__device__ void stream_range(const VerifyParams& P, const int* s_cum, const int* s_seq, int lo, int hi,
                             int worker, int q_lds_off, int row0) {
  using SH = Shape<D, NT, FP8, W2, MX>;
  constexpr int G = D / 64;                      // MX: scale tiles per token
  using Regs = PageRegs<D, FP8>;
  constexpr int KS = SH::KS, DT = SH::DT, PF = SH::PF;
  const int lane = threadIdx.x & 63;
  const int m16 = lane & 15, jg = lane >> 4;
  const unsigned lane_off = unsigned(m16 * 64 + jg * 16);
  const long page_stride = long(P.Hkv) * P.slab_bytes;
  // ---- cursor helpers (all scalar) -----------------------------------------
  // A sequence's page count, block-table row and length word come from LDS
  // (page_prefix), so moving to the next unit waits for no global load.
  auto seq_info = [&](Cursor& c) {
    c.np = uni(s_cum[c.b + 1]) - uni(s_cum[c.b]);
    c.row = uni(s_seq[2 * c.b]);
    c.n = uni(s_seq[2 * c.b + 1]);
  };
  auto locate = [&](int pos) {
    int a = 0, z = P.batch - 1;
    while (a < z) {
      const int mid = (a + z + 1) >> 1;
      if (P.Hkv * uni(s_cum[mid]) <= pos) a = mid;
      else z = mid - 1;
    }
    Cursor c;
    c.b = a;
    seq_info(c);
    const int off = pos - P.Hkv * uni(s_cum[a]);
    c.g = off / c.np;
    c.page = off - c.g * c.np;
    return c;
  };
  auto advance = [&](Cursor& c) {
    if (++c.page < c.np) return;
    c.page = 0;
    if (++c.g < P.Hkv) return;
    c.g = 0;
    do {
      ++c.b;
    } while (c.b < P.batch - 1 && uni(s_cum[c.b + 1]) == uni(s_cum[c.b]));
    if (c.b >= P.batch) c.b = P.batch - 1;    // past the end: only null loads follow
    seq_info(c);
  };
  auto bt_rsrc = [&](const Cursor& c) {
    return scalar_rsrc(P.block_table + long(c.row) * P.bt_stride + P.pref, unsigned(c.np) * 4u);
  };

  // ---- loads ---------------------------------------------------------------
  // Bounds-checked buffer loads of one page: a position outside the range
  // gets num_records = 0, which returns zeros without touching memory.
  auto load_page = [&](Regs& R, PageMeta& M, const Cursor& c, int id, bool valid) {
    const int nrec = valid ? int(P.slab_bytes) : 0;
    const char* kb = P.k_pages + long(id) * page_stride + long(c.g) * P.slab_bytes;
    const char* vb = P.v_pages + long(id) * page_stride + long(c.g) * P.slab_bytes;
    const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kb), 0, nrec, kBufferFlags);
    const auto rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vb), 0, nrec, kBufferFlags);
#pragma unroll
    for (int u = 0; u < SH::KL; ++u)
      R.k[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, lane_off + u * 1024, 0, SHARED ? 0 : kStreamPolicy));
#pragma unroll
    for (int cc = 0; cc < SH::VL; ++cc)
      R.v[cc] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, lane_off + cc * 1024, 0, SHARED ? 0 : kStreamPolicy));
    M.unit = (c.b << 16) | c.g;
    M.page = c.page;
    M.n = valid ? c.n : 0;
    if (MX) {
      // the page-head's E8M0 bytes, [token][tile], K then V: this lane's K
      // token and tile, and the four tokens of its V operand
      const long sb = (long(id) * P.Hkv + c.g) * 16 * G;
      const auto rks = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<unsigned char*>(static_cast<const unsigned char*>(P.k_scale) + sb), 0, valid ? 16 * G : 0,
          kBufferFlags);
      const auto rvs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<unsigned char*>(static_cast<const unsigned char*>(P.v_scale) + sb), 0, valid ? 16 * G : 0,
          kBufferFlags);
      const int kbyte = m16 * G + ((D / 4) * jg) / 64;
      M.ksw = unsigned(__builtin_amdgcn_raw_buffer_load_b32(rks, kbyte & ~3, 0, 0));
#pragma unroll
      for (int g = 0; g < G; ++g)
        M.vsw[g] = unsigned(__builtin_amdgcn_raw_buffer_load_b32(rvs, 4 * jg * G + 4 * g, 0, 0));
    } else if (FP8) {
      // the scales come through the vector path, issued after the page's
      // loads: they complete with the page, whereas a scalar load here
      // (a random line of the scale arrays) would be waited for at the
      // next scalar wait, one page later
      const int so = (id * P.Hkv + c.g) * 4;
      const auto rks = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(P.k_scale), 0, valid ? 0x7FFFFFFF : 0,
                                                         kBufferFlags);
      const auto rvs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(P.v_scale), 0, valid ? 0x7FFFFFFF : 0,
                                                         kBufferFlags);
      M.ks = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rks, 0, so, 0));
      M.vs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rvs, 0, so, 0));
    }
  };
  // This wave's rows are row0 .. row0 + rows_here - 1 of the unit's n_q*G
  // rows; lane row 16nt+m16 is local.  Rows past them read row row0 (never
  // output).
  const int rows_here = min(P.rows_w, P.rows - row0);
  auto local_ok = [&](int nt) { return nt * 16 + m16 < rows_here; };
  // Q fragments (B operand of S^T = K Q^T) of unit (b, g): local row 16nt+m16,
  // channels (D/4)jg + 8s .. +7.
  auto load_q = [&](u32x4 (&q)[NT][KS], unsigned long long (&an)[NT], int b, int g) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = row0 + (local_ok(nt) ? nt * 16 + m16 : 0);
      const int i = r / P.G, h = g * P.G + r % P.G;
      const unsigned short* qp = static_cast<const unsigned short*>(P.q) +
                                 (long(b * P.n_q + i) * P.Hq + h) * D + (D / 4) * jg;
#pragma unroll
      for (int s = 0; s < KS; ++s) q[nt][s] = load16(qp + 8 * s);
      if (TREE) an[nt] = P.anc[long(b) * P.n_q + i];
    }
  };

  // ---- per-unit state --------------------------------------------------------
  int qi[NT];                     // verification slot of the row (padding rows: 64)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) qi[nt] = local_ok(nt) ? (row0 + nt * 16 + m16) / P.G : 64;
  u32x4 qf[NT][KS];
  unsigned long long anc[NT];

  // ---- Q staging ---------------------------------------------------------------
  // When a unit enters the prefetch window its Q rows (and ancestor masks)
  // are copied global -> LDS (copy16_to_lds), issued
  // just before the unit's first page loads.  Those page loads, and the
  // pages prefetched after them, complete after the copy (vector memory
  // operations complete in order), so once the unit's first page may be
  // computed an explicit vmcnt wait for that many operations covers the
  // copy too; the compiler tracks no register for it, so no other wait is
  // widened by it.  A slot is reused only after the unit that held it has
  // started (and read its Q into registers); otherwise the unit's Q is
  // loaded when it starts (rare: several very short units in one window).
  extern __shared__ __align__(16) unsigned char s_dyn[];
  constexpr int QS = SH::QS, QSLOT = SH::QSLOT, ASLOT = SH::ASLOT;
  const int wave = uni(threadIdx.x >> 6);
  unsigned char* q_lds = s_dyn + q_lds_off + wave * QS * QSLOT;
  unsigned char* a_lds = s_dyn + q_lds_off + kWaves * QS * QSLOT + wave * QS * ASLOT;
  int pf_units = 0, cm_units = 0;   // units entered in the window / started
  unsigned staged = 0;              // bit u % 32: unit u's Q is in its LDS slot
  auto stage_q = [&](int slot, int b, int g) {
    constexpr int LANES_PER_ROW = D / 8, RPI = 64 / LANES_PER_ROW;
    const int rr = lane / LANES_PER_ROW, ch = lane % LANES_PER_ROW;
#pragma unroll
    for (int k = 0; k < NT * 16 / RPI; ++k) {
      if (k * RPI < rows_here) {
        const int r = row0 + (k * RPI + rr < rows_here ? k * RPI + rr : 0);
        const int i = r / P.G, h = g * P.G + r % P.G;
        const unsigned short* src = static_cast<const unsigned short*>(P.q) +
                                    (long(b * P.n_q + i) * P.Hq + h) * D + ch * 8;
        copy16_to_lds(src, uni(lds_addr(q_lds + slot * QSLOT + k * 1024)));
      }
    }
    if (TREE) {
      const int dw = lane < 2 * P.n_q ? lane : 0;
      const unsigned* src = reinterpret_cast<const unsigned*>(P.anc + long(b) * P.n_q) + dw;
      copy4_to_lds(src, uni(lds_addr(a_lds + slot * ASLOT)));
    }
  };
  auto read_q = [&](int slot) {
    const unsigned char* qs = q_lds + slot * QSLOT;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = local_ok(nt) ? nt * 16 + m16 : 0;     // LDS row (local)
#pragma unroll
      for (int s = 0; s < KS; ++s)
        qf[nt][s] = *reinterpret_cast<const u32x4*>(qs + (r * D + (D / 4) * jg + 8 * s) * 2);
      if (TREE)
        anc[nt] = *reinterpret_cast<const unsigned long long*>(a_lds + slot * ASLOT + ((row0 + r) / P.G) * 8);
    }
  };
  float m_run[NT], l_run[NT];
  f32x4 acc[DT][NT];
  int u_b = -1, u_g = 0, u_first = 0, u_last = 0, u_np = 0, u_nq = 0, units_done = 0;

  auto finalize = [&]() {
    const bool full = u_first == 0 && u_last == u_np - 1;
    const int slot = units_done == 0 ? 0 : 1;
    float* part = P.part + (long(worker) * 2 + slot) * slot_floats(P.rows_w, D);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float l = l_run[nt];
      l += __shfl_xor(l, 16, 64);
      l += __shfl_xor(l, 32, 64);
      const int rl = nt * 16 + m16, r = row0 + rl;
      // rows of slots past the sequence's count are not written (fused
      // calls have no per-sequence counts: every row)
      if (local_ok(nt) && (P.fused || r / P.G < u_nq)) {
        const int i = r / P.G, h = u_g * P.G + r % P.G;
        const long oi = long(u_b * P.n_q + i) * P.Hq + h;
        const float inv = full ? 1.0f / l : 1.0f;
        float* dst = full ? P.out + oi * D : part + long(rl) * D;
        if (FP8) {
#pragma unroll
          for (int c = 0; c < D / 64; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int ch = c * 64 + 16 * jg + 4 * e;
              *reinterpret_cast<float4*>(dst + ch) =
                  make_float4(acc[4 * c][nt][e] * inv, acc[4 * c + 1][nt][e] * inv,
                              acc[4 * c + 2][nt][e] * inv, acc[4 * c + 3][nt][e] * inv);
            }
        } else {
#pragma unroll
          for (int c = 0; c < D / 32; ++c) {
            const int ch = c * 32 + 8 * jg;
            *reinterpret_cast<float4*>(dst + ch) =
                make_float4(acc[2 * c][nt][0] * inv, acc[2 * c + 1][nt][0] * inv,
                            acc[2 * c][nt][1] * inv, acc[2 * c + 1][nt][1] * inv);
            *reinterpret_cast<float4*>(dst + ch + 4) =
                make_float4(acc[2 * c][nt][2] * inv, acc[2 * c + 1][nt][2] * inv,
                            acc[2 * c][nt][3] * inv, acc[2 * c + 1][nt][3] * inv);
          }
        }
        if (jg == 0) {
          if (full) {
            if (P.defer) P.unit_lse[oi] = m_run[nt] + __log2f(l);
            else if (P.lse) P.lse[oi] = (m_run[nt] + __log2f(l)) * kLn2;
          } else {
            part[long(P.rows_w) * D + rl] = m_run[nt];
            part[long(P.rows_w) * D + P.rows_w + rl] = l;
          }
        }
      }
    }
    ++units_done;
  };

  // P is split into bf16 high and low parts, the two halves of one K = 32
  // MFMA, so PV is fp32-accurate: for bf16 KV (target 2e-3 of rms(O)) and for
  // FP8 KV too, where P rounded once to bf16 (relative error <= 2^-9 per
  // weight) reached 2.8e-2 of rms(O) against a 2e-2 target on pages with a
  // wide range of magnitudes.
#ifndef PKV_FP8_SPLIT_P
#define PKV_FP8_SPLIT_P 1
#endif
  constexpr bool kSplitP = !FP8 || PKV_FP8_SPLIT_P;
  auto compute_page = [&](Regs& R, const PageMeta& M) {
    const int tok0 = (M.page + P.pref) * 16;       // positions past the shared prefix (cascade)
    const int L = (M.n & kLenMask) - (M.n >> kNqShift);
    // scores S^T (lane: row 16nt+m16, tokens tok0 + 4jg .. +3)
    float kx = 1.0f;                             // MX: this lane's K scale (its token, its tile)
    if (MX) kx = e8m0_value((M.ksw >> (8 * ((m16 * G + ((D / 4) * jg) / 64) & 3))) & 0xFFu);
    f32x4 sc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 a = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        u32x4 kf;
        if (FP8) {
          const u32x4 w = R.k[s >> 1];
          const int o = (s & 1) * 2;
          const Dw2 a0 = MX ? fp8x4_to_bf16x4_scaled(w[o], kx) : fp8x4_to_bf16x4(w[o]);
          const Dw2 a1 = MX ? fp8x4_to_bf16x4_scaled(w[o + 1], kx) : fp8x4_to_bf16x4(w[o + 1]);
          kf = u32x4{a0.lo, a0.hi, a1.lo, a1.hi};
        } else {
          kf = R.k[s];
        }
        a = mfma_bf16(kf, qf[nt][s], a);
      }
      sc[nt] = a;
    }
    float ksc = P.scale_log2, vsc = 1.0f;
    if (FP8 && !MX) {
      ksc *= M.ks;
      vsc = M.vs;
    }
    // the scores stay unscaled: ksc > 0, so the row maximum is taken on them
    // and scaled once, and each weight is exp2(fma(score, ksc, -m))

    if (tok0 + 16 > L) {                         // page reaches the verification slots or the end
      const int N = M.n & kLenMask;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = tok0 + 4 * jg + e;
        const int j = t - L;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          bool vis;
          if (TREE) vis = (t < L) || (t < N && ((anc[nt] >> (j & 63)) & 1ull));
          else vis = (t < L) || (t < N && j <= qi[nt]);
          sc[nt][e] = vis ? sc[nt][e] : kNegInf;
        }
      }
      // zero V of tokens at or past N (stale slots may hold anything)
      const int valid = min(4, max(0, N - (tok0 + 4 * jg)));
      if (FP8) {
        const unsigned keep = valid >= 4 ? 0xFFFFFFFFu : ((1u << (8 * valid)) - 1u);
#pragma unroll
        for (int c = 0; c < SH::VL; ++c)
#pragma unroll
          for (int w = 0; w < 4; ++w) R.v[c][w] &= keep;
      } else {
        const unsigned keep0 = valid >= 2 ? 0xFFFFFFFFu : (valid == 1 ? 0xFFFFu : 0u);
        const unsigned keep1 = valid >= 4 ? 0xFFFFFFFFu : (valid == 3 ? 0xFFFFu : 0u);
#pragma unroll
        for (int c = 0; c < SH::VL; ++c) {
          R.v[c][0] &= keep0;
          R.v[c][1] &= keep1;
          R.v[c][2] &= keep0;
          R.v[c][3] &= keep1;
        }
      }
    }

    // MX: the V scales of this lane's four tokens, per tile of channels
    float vx[G][4];
    if (MX) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int byte = e * G + g;                  // token 4jg+e, tile g
          vx[g][e] = e8m0_value((M.vsw[byte >> 2] >> (8 * (byte & 3))) & 0xFFu);
        }
    }
    // online softmax (base 2, lazy rescale) and the P^T operands (MX: one
    // hi/lo pair per tile of channels, P times the tokens' V scales)
    constexpr int PG = MX ? G : 1;
    unsigned ph[NT][2], pl[NT][2], pm[PG][NT][2], pml[PG][NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float mx = row_max4(fmaxf(fmaxf(sc[nt][0], sc[nt][1]), fmaxf(sc[nt][2], sc[nt][3]))) * ksc;
      const bool grow = mx > m_run[nt] + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? mx : m_run[nt];
        const float alpha = grow ? exp2_fast(m_run[nt] - m_new) : 1.0f;
        l_run[nt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt][nt] *= alpha;
        m_run[nt] = m_new;
      }
      const float m_ref = m_run[nt] == kNegInf ? 0.0f : m_run[nt];
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = exp2_fast(fmaf(sc[nt][e], ksc, -m_ref));
      l_run[nt] += (p[0] + p[1]) + (p[2] + p[3]);
      if (MX) {
        // P = hi + lo as for bf16 KV; scaling by a power of two is exact, so
        // the pair of (P x scale) is the scaled pair of P
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          r[e] = p[e] - __uint_as_float(__float_as_uint(p[e]) & 0xFFFF0000u);
#pragma unroll
        for (int g = 0; g < PG; ++g) {
          pm[g][nt][0] = pack_hi16(p[0] * vx[g][0], p[1] * vx[g][1]);
          pm[g][nt][1] = pack_hi16(p[2] * vx[g][2], p[3] * vx[g][3]);
          pml[g][nt][0] = pack_rne_bf16(r[0] * vx[g][0], r[1] * vx[g][1]);
          pml[g][nt][1] = pack_rne_bf16(r[2] * vx[g][2], r[3] * vx[g][3]);
        }
      } else if (FP8) {
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] *= vsc;
      }
      if (MX) {
        ph[nt][0] = ph[nt][1] = pl[nt][0] = pl[nt][1] = 0u;
      } else if (kSplitP) {
        // P = hi + lo: hi the truncated upper half, lo the rounded rest
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          r[e] = p[e] - __uint_as_float(__float_as_uint(p[e]) & 0xFFFF0000u);
        ph[nt][0] = pack_hi16(p[0], p[1]);
        ph[nt][1] = pack_hi16(p[2], p[3]);
        pl[nt][0] = pack_rne_bf16(r[0], r[1]);
        pl[nt][1] = pack_rne_bf16(r[2], r[3]);
      } else {
        ph[nt][0] = pack_rne_bf16(p[0], p[1]);
        ph[nt][1] = pack_rne_bf16(p[2], p[3]);
        pl[nt][0] = pl[nt][1] = 0u;
      }
    }

    // O^T += V^T P^T  (16 tokens of the page per MFMA)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      unsigned v0, v1;
      if (FP8) {
        const Dw2 a = fp8x4_to_bf16x4(R.v[dt >> 2][dt & 3]);
        v0 = a.lo;
        v1 = a.hi;
      } else {
        const int w = (dt & 1) * 2;
        v0 = R.v[dt >> 1][w];
        v1 = R.v[dt >> 1][w + 1];
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (MX) {
          // channels of tile dt lie in 64-channel tile dt / 4
          const int g = (dt >> 2) % PG;
          acc[dt][nt] = mfma_bf16_split(v0, v1, pm[g][nt][0], pm[g][nt][1], pml[g][nt][0], pml[g][nt][1], acc[dt][nt]);
          continue;
        }
        if (kSplitP) acc[dt][nt] = mfma_bf16_split(v0, v1, ph[nt][0], ph[nt][1], pl[nt][0], pl[nt][1], acc[dt][nt]);
        else acc[dt][nt] = mfma_bf16_k16(v0, v1, ph[nt][0], ph[nt][1], acc[dt][nt]);
      }
    }
  };

  // ---- the stream ---------------------------------------------------------------
  // Positions lo..hi-1 are computed in order; the loads of position i + PF are
  // issued while position i is computed, continuing across unit and sequence
  // boundaries, and the page id of position i + PF + 1 is fetched one step
  // ahead through the scalar unit.  The loop body is straight-line (positions
  // past hi are null loads, and their compute is skipped by a uniform branch),
  // so the compiler's wait counts keep all PF pages in flight.
  constexpr int RS = SH::RS;
  Regs ring[RS];
  PageMeta meta[RS];
  Cursor c = locate(lo);
  const int len = hi - lo;
  // The page ids of the first positions come from one scalar load of eight
  // consecutive block-table entries of the starting unit (inside the unit's
  // row, so never past its valid entries); later ids are fetched one
  // position ahead.  Without this the prologue waited for PF dependent loads.
  const bool win = c.np >= 8;
  const int wb = win ? min(c.page, c.np - 8) : 0;
  const i32x8 ids8 = win ? s_buffer_load_dwordx8(bt_rsrc(c), wb * 4, 0) : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  const int b_start = c.b, g_start = c.g;
  auto next_id = [&](const Cursor& cc, bool prologue) {
    if (prologue && win && cc.b == b_start && cc.g == g_start && cc.page - wb < 8) return ids8[cc.page - wb];
    return s_buffer_load_dword(bt_rsrc(cc), cc.page * 4, 0);
  };
  int id_pend = next_id(c, true);
  auto prefetch = [&](Regs& R, PageMeta& M, int rel, bool prologue = false) {
    const bool valid = rel < len;
    if (valid && (c.page == 0 || rel == 0)) {  // a new unit enters the window: stage its Q
      if (pf_units - cm_units < QS) {
        stage_q(pf_units % QS, c.b, c.g);
        staged |= 1u << (pf_units & 31);
      } else {
        staged &= ~(1u << (pf_units & 31));
      }
      ++pf_units;
    }
    load_page(R, M, c, id_pend, valid);
    if (rel + 1 < len) {
      advance(c);
      id_pend = next_id(c, prologue);
    }
  };
#pragma unroll
  for (int r = 0; r < PF; ++r) prefetch(ring[r], meta[r], r, true);
  for (int i0 = 0; i0 < len; i0 += RS) {
#pragma unroll
    for (int r = 0; r < RS; ++r) {
      const int i = i0 + r;
      prefetch(ring[(r + PF) % RS], meta[(r + PF) % RS], i + PF);
      const PageMeta& M = meta[r];
      if (M.n != 0) {
        const int mb = M.unit >> 16, mg = M.unit & 0xFFFF;
        if (mb != u_b || mg != u_g) {            // a new unit starts at this position
          if (u_b >= 0) finalize();
          if ((staged >> (cm_units & 31)) & 1u) {
            // the copy was issued before this page's loads, and the loads
            // of this page and of the PF pages after it since
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(SH::LPP * (PF + 1)));
            asm volatile("" ::: "memory");
            read_q(cm_units % QS);
          } else {
            load_q(qf, anc, mb, mg);
            // wait here, on this rare path, so that the common path's MFMAs
            // never inherit a wait for these loads (which would also drain
            // every prefetched page)
            __builtin_amdgcn_s_waitcnt(kVmcnt0);
          }
          ++cm_units;
          u_b = mb;
          u_g = mg;
          u_first = M.page;
          u_np = (((M.n & kLenMask) + 15) >> 4) - P.pref;
          u_nq = M.n >> kNqShift;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            m_run[nt] = kNegInf;
            l_run[nt] = 0.0f;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[dt][nt] = f32x4{0, 0, 0, 0};
          }
        }
        u_last = M.page;
        compute_page(ring[r], M);
      }
    }
  }
  if (u_b >= 0) finalize();
}

// Adds (max, sum, O) of one piece to a running log-sum-exp combine (base 2).
__device__ inline void lse_combine(float& M, float& Ls, float4& o, float m, float l, const float4& v) {
  const float mn = fmaxf(M, m);
  const float ref = mn == kNegInf ? 0.0f : mn;
  const float a = exp2_fast(M - ref), c = exp2_fast(m - ref);
  Ls = Ls * a + l * c;
  o.x = o.x * a + v.x * c;
  o.y = o.y * a + v.y * c;
  o.z = o.z * a + v.z * c;
  o.w = o.w * a + v.w * c;
  M = mn;
}

// The streamed pieces of unit (b, g), row r (output row oi), channels
// 4 c4 .. 4 c4 + 3, combined into (M, Ls, o).  Returns false when the unit
// was finished in place by one worker (nothing to merge; in a fused call
// or with the cascade that worker left its normalised O in out and its
// log2-sum-exp in unit_lse, which are then combined and true returned).
// The pieces of a split unit are the slots of the workers whose ranges
// overlap it, found in closed form; each thread issues the loads of up to
// eight pieces (their maxima, sums and its float4 of O) before combining
// them.
template <int D>
__device__ bool merge_stream_pieces(const VerifyParams& P, int b, int g, int r, long oi, int c4, float& M,
                                    float& Ls, float4& o) {
  const int* __restrict__ cum = P.cum;
  const long W = long(P.Hkv) * cum[P.batch];
  const int np = cum[b + 1] - cum[b];
  if (np == 0) return true;                       // no pages past the prefix: nothing streamed
  const int n_rng = used_ranges(P, W);
  const long u0 = long(P.Hkv) * cum[b] + long(g) * np, u1 = u0 + np;
  const int wf = owner_of(u0, W, n_rng), wl = owner_of(u1 - 1, W, n_rng);
  if (wf == wl) {                                 // finished in place
    if (!P.defer) return false;
    lse_combine(M, Ls, o, P.unit_lse[oi], 1.0f, *reinterpret_cast<const float4*>(P.out + oi * D + 4 * c4));
    return true;
  }
  // row r is row rl of row group rgi, held by wave (range * rg + rgi)
  const int rgi = r / P.rows_w, rl = r % P.rows_w, RW = P.rows_w;
  const long sf = slot_floats(RW, D);
  // the first range's piece is its second slot when the range began in an
  // earlier unit; for the others the unit is their first
  const long first_base = (2L * (long(wf) * P.rg + rgi) + (range_starts_at(wf, W, n_rng, u0) ? 0 : 1)) * sf;
  const float* __restrict__ part = P.part;
  constexpr int KB = 8;
  for (int w0 = wf; w0 <= wl; w0 += KB) {
    float mk[KB], lk[KB];
    float4 v[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int w = min(w0 + u, wl);
      const long base = w == wf ? first_base : 2L * (long(w) * P.rg + rgi) * sf;
      mk[u] = part[base + long(RW) * D + rl];
      lk[u] = part[base + long(RW) * D + RW + rl];
      v[u] = *reinterpret_cast<const float4*>(part + base + long(rl) * D + 4 * c4);
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (w0 + u > wl) break;
      lse_combine(M, Ls, o, mk[u], lk[u], v[u]);
    }
  }
  return true;
}

// Merge of the units split over workers.  Block (unit, y) owns 256
// consecutive float4s of the unit's [rows][D] output; a unit finished in
// place by one worker is skipped.
template <int D>
__global__ __launch_bounds__(kThreads) void verify_merge_kernel(VerifyParams P) {
  const int b = blockIdx.x / P.Hkv, g = blockIdx.x % P.Hkv;
  const int R = P.rows;
  const int x = blockIdx.y * kThreads + threadIdx.x;
  if (x >= R * (D / 4)) return;
  const int r = x / (D / 4), c4 = x % (D / 4);
  if (r / P.G >= seq_slots(P, b)) return;
  const int i = r / P.G, h = g * P.G + r % P.G;
  const long oi = long(b * P.n_q + i) * P.Hq + h;
  // cascade: the shared prefix's partial is the first piece of every row
  float M = kNegInf, Ls = 0.0f;
  float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (P.pref > 0) {
    const float* pp = P.prefix_part + oi * (D + 2);
    M = pp[D];
    Ls = pp[D + 1];
    o = *reinterpret_cast<const float4*>(pp + 4 * c4);
  }
  const bool split = merge_stream_pieces<D>(P, b, g, r, oi, c4, M, Ls, o);
  // without a prefix, a unit finished in place (or a unit with no pages at
  // all) was written by the streaming kernel
  if (!split || (P.pref == 0 && P.cum[b + 1] == P.cum[b])) return;
  const float inv = 1.0f / Ls;
  *reinterpret_cast<float4*>(P.out + oi * D + 4 * c4) = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
  if (c4 == 0 && P.lse) P.lse[oi] = (M + __log2f(Ls)) * kLn2;
}

// Fused append (spec_verify_attention_append), after the streaming kernel.
// Block (unit (b, g), y) owns the same 256 float4s of the unit's [rows][D]
// output as the plain merge.  Every block of the unit encodes the unit's n_q
// new tokens exactly as the pool-update kernel encodes an append (same page
// scales and codes; fp8_codec.h), keeps their values as attended (decoded)
// in LDS, and computes its rows' attention piece over them (the chain or tree
// mask among the new tokens) in fp32; that piece is combined with the
// streamed pieces of the cached tokens and the cascade's prefix piece.  Block
// y = 0 writes the codes and scales into the pool, and for head 0 the
// sequence's new block-table entry and length (nothing in this launch reads
// them after the streaming kernel, which used the cached lengths).  The
// blocks of a unit compute the same scales from the same values, so the
// copies agree bit for bit.
template <int D>
__global__ __launch_bounds__(kThreads) void verify_fused_merge_kernel(VerifyParams P, FusedAppend F) {
  constexpr int NT = kFusedMaxTokens, IT = D / 8;     // new tokens; 8-channel items per token
  constexpr int NRB = kThreads / (D / 4);             // output rows per block
  constexpr int KP = D + 4;                           // LDS row pitch (16-byte rows, banks staggered)
  __shared__ __align__(16) float s_k[NT][KP];        // new K, V as attended (decoded), fp32
  __shared__ __align__(16) float s_v[NT][KP];
  __shared__ __align__(16) float s_q[NRB][KP];
  __shared__ float s_w[NRB][NT];                      // scores, then weights
  __shared__ float s_m[NRB], s_l[NRB];
  __shared__ float s_amax[2][2][kWaves];              // [page of the call][K, V][wave]
  const int b = blockIdx.x / P.Hkv, g = blockIdx.x % P.Hkv, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int nq = P.n_q, G = P.G, R = P.rows, row = b;
  const int r0 = blockIdx.y * NRB, nrb = min(NRB, R - r0);
  const bool writer = blockIdx.y == 0;
  const int N0 = P.old_len[b], N = N0 + nq;
  const int np_old = (N0 + 15) >> 4, pa = N0 >> 4;    // pages pa and pa + 1 can take new tokens
  const bool fp8 = P.kv_kind == PKV_FP8_E4M3, mx = P.kv_kind == PKV_FP8_E4M3_MX64;
  auto page_id = [&](int p) { return p < np_old ? P.block_table[long(row) * P.bt_stride + p] : F.new_page[b]; };

  // ---- loads: the new tokens' items (token j, channels c0 .. c0 + 7) and
  // this block's query rows, issued before the streamed pieces are read ----
  const int j = tid / IT, c0 = (tid % IT) * 8;
  const bool ok = j < nq;
  float kx[8], vx[8];
  const long src = (long(b * nq + (ok ? j : 0)) * P.Hkv + g) * D + c0;
  if (fp8 || mx) {
    const float4* ks = static_cast<const float4*>(F.k_new) + src / 4;
    const float4* vs = static_cast<const float4*>(F.v_new) + src / 4;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const float4 a = ok ? ks[h2] : make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 c = ok ? vs[h2] : make_float4(0.f, 0.f, 0.f, 0.f);
      kx[4 * h2] = a.x; kx[4 * h2 + 1] = a.y; kx[4 * h2 + 2] = a.z; kx[4 * h2 + 3] = a.w;
      vx[4 * h2] = c.x; vx[4 * h2 + 1] = c.y; vx[4 * h2 + 2] = c.z; vx[4 * h2 + 3] = c.w;
    }
  } else {
    const uint4 a = ok ? *reinterpret_cast<const uint4*>(static_cast<const unsigned short*>(F.k_new) + src)
                       : make_uint4(0, 0, 0, 0);
    const uint4 c = ok ? *reinterpret_cast<const uint4*>(static_cast<const unsigned short*>(F.v_new) + src)
                       : make_uint4(0, 0, 0, 0);
    const unsigned wa[4] = {a.x, a.y, a.z, a.w}, wc[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kx[e] = __uint_as_float((wa[e / 2] >> (16 * (e % 2))) << 16);
      vx[e] = __uint_as_float((wc[e / 2] >> (16 * (e % 2))) << 16);
    }
  }
  // query rows r0 .. r0 + nrb - 1: thread -> (row, 8 channels)
  const int qr = tid / IT, qc = (tid % IT) * 8;
  uint4 qbits = make_uint4(0, 0, 0, 0);
  if (qr < nrb) {
    const int rr = r0 + qr, i = rr / G, h = g * G + rr % G;
    qbits = *reinterpret_cast<const uint4*>(static_cast<const unsigned short*>(P.q) +
                                            (long(b * nq + i) * P.Hq + h) * D + qc);
  }
  // ---- streamed pieces and the prefix piece of this thread's float4 ------------
  const int x = blockIdx.y * kThreads + tid;
  const bool out_ok = x < R * (D / 4);
  const int rr = out_ok ? x / (D / 4) : r0, c4 = x % (D / 4), rl = rr - r0;
  const int oi_i = rr / G, oi_h = g * G + rr % G;
  const long oi = long(b * nq + oi_i) * P.Hq + oi_h;
  float M = kNegInf, Ls = 0.0f;
  float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (out_ok) {
    if (P.pref > 0) {
      const float* pp = P.prefix_part + oi * (D + 2);
      M = pp[D];
      Ls = pp[D + 1];
      o = *reinterpret_cast<const float4*>(pp + 4 * c4);
    }
    merge_stream_pieces<D>(P, b, g, rr, oi, c4, M, Ls, o);
  }
  // ---- encode the new tokens ---------------------------------------------------
  const int t = N0 + (ok ? j : 0), pj = t >> 4, slot = t & 15;
  // page-head scales: a page first written by this call takes amax / 448 of
  // the values written into it (per K and V); the partly filled page pa
  // keeps its scale unless the new values exceed its range, in which case
  // the scale doubles until they fit and the page's cached slots are encoded
  // again.  Its old scales are read before this block's barrier, so before
  // its writer (this block when y = 0) replaces them; a block y > 0 may read
  // the replaced value, which yields the same grown scale.
  float sk_pg = 1.0f, sv_pg = 1.0f;
  float sk_old = 1.0f, sv_old = 1.0f;
  if (fp8 && (N0 & 15) != 0) {
    const long sidx = long(page_id(pa)) * P.Hkv + g;
    sk_old = static_cast<const float*>(P.k_scale)[sidx];
    sv_old = static_cast<const float*>(P.v_scale)[sidx];
  }
  if (fp8) {
    float ak = 0.0f, av = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ak = fmaxf(ak, fabsf(kx[e]));
      av = fmaxf(av, fabsf(vx[e]));
    }
    float red[2][2];
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      red[q2][0] = ok && pj == pa + q2 ? ak : 0.0f;
      red[q2][1] = ok && pj == pa + q2 ? av : 0.0f;
#pragma unroll
      for (int kv = 0; kv < 2; ++kv)
        for (int o2 = 32; o2 > 0; o2 >>= 1) red[q2][kv] = fmaxf(red[q2][kv], __shfl_xor(red[q2][kv], o2, 64));
    }
    if (lane == 0)
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        s_amax[q2][0][wave] = red[q2][0];
        s_amax[q2][1][wave] = red[q2][1];
      }
    __syncthreads();
    const int q2 = pj - pa;
    const bool fresh = (pj << 4) >= N0;
    const int id = page_id(pj);
    float mk = 0.0f, mv = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mk = fmaxf(mk, s_amax[q2][0][w]);
      mv = fmaxf(mv, s_amax[q2][1][w]);
    }
    if (fresh) {
      sk_pg = fresh_page_scale(mk);
      sv_pg = fresh_page_scale(mv);
    } else {
      sk_pg = grown_page_scale(mk, sk_old);
      sv_pg = grown_page_scale(mv, sv_old);
    }
    // the item holding the call's first token of each page writes its scales
    if (writer && ok && (slot == 0 || t == N0) && c0 == 0) {
      const_cast<float*>(static_cast<const float*>(P.k_scale))[long(id) * P.Hkv + g] = sk_pg;
      const_cast<float*>(static_cast<const float*>(P.v_scale))[long(id) * P.Hkv + g] = sv_pg;
    }
    if (writer && (N0 & 15) != 0) {
      // the cached slots 0 .. N0 % 16 - 1 of page pa under a grown scale
      float mk0 = 0.0f, mv0 = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        mk0 = fmaxf(mk0, s_amax[0][0][w]);
        mv0 = fmaxf(mv0, s_amax[0][1][w]);
      }
      const float skn = grown_page_scale(mk0, sk_old), svn = grown_page_scale(mv0, sv_old);
      const long sidx = long(page_id(pa)) * P.Hkv + g;
      unsigned char* kp = reinterpret_cast<unsigned char*>(const_cast<char*>(P.k_pages) + sidx * P.slab_bytes);
      unsigned char* vp = reinterpret_cast<unsigned char*>(const_cast<char*>(P.v_pages) + sidx * P.slab_bytes);
      const int n_old = (N0 & 15) * D;
      if (skn != sk_old) {
        const float inv = 1.0f / skn;
        for (int e = tid; e < n_old; e += kThreads) {
          unsigned char& c = kp[k_index_fp8(e / D, e % D, D)];
          c = reencode_e4m3(c, sk_old, inv);
        }
      }
      if (svn != sv_old) {
        const float inv = 1.0f / svn;
        for (int e = tid; e < n_old; e += kThreads) {
          unsigned char& c = vp[v_index_fp8(e / D, e % D)];
          c = reencode_e4m3(c, sv_old, inv);
        }
      }
    }
  }
  if (ok) {
    const int id = page_id(pj);
    char* kslab = const_cast<char*>(P.k_pages) + (long(id) * P.Hkv + g) * P.slab_bytes;
    char* vslab = const_cast<char*>(P.v_pages) + (long(id) * P.Hkv + g) * P.slab_bytes;
    float kd[8], vd[8];
    if (fp8 || mx) {
      float ik = 1.0f / sk_pg, iv = 1.0f / sv_pg, dk = sk_pg, dv = sv_pg;
      if (mx) {
        // one power-of-two scale per 64 channels of the token: the tile's
        // eight items are eight consecutive threads
        float ak = 0.0f, av = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ak = fmaxf(ak, fabsf(kx[e]));
          av = fmaxf(av, fabsf(vx[e]));
        }
#pragma unroll
        for (int o2 = 1; o2 < 8; o2 <<= 1) {
          ak = fmaxf(ak, __shfl_xor(ak, o2, 64));
          av = fmaxf(av, __shfl_xor(av, o2, 64));
        }
        const int ek = tile_exponent_byte(ak), ev = tile_exponent_byte(av);
        ik = ldexpf(1.0f, 127 - ek);
        iv = ldexpf(1.0f, 127 - ev);
        dk = ldexpf(1.0f, ek - 127);
        dv = ldexpf(1.0f, ev - 127);
        if (writer && (c0 & 63) == 0) {
          const long eo = ((long(id) * P.Hkv + g) * 16 + slot) * (D / 64) + c0 / 64;
          const_cast<unsigned char*>(static_cast<const unsigned char*>(P.k_scale))[eo] = static_cast<unsigned char>(ek);
          const_cast<unsigned char*>(static_cast<const unsigned char*>(P.v_scale))[eo] = static_cast<unsigned char>(ev);
        }
      }
      unsigned lo = 0, hi = 0;
      unsigned char cv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const unsigned char ck = quant_e4m3(kx[e], ik);
        cv[e] = quant_e4m3(vx[e], iv);
        if (e < 4) lo |= unsigned(ck) << (8 * e);
        else hi |= unsigned(ck) << (8 * (e - 4));
        kd[e] = dequant_e4m3(ck) * dk;
        vd[e] = dequant_e4m3(cv[e]) * dv;
      }
      if (writer) {
        *reinterpret_cast<uint2*>(kslab + k_index_fp8(slot, c0, D)) = make_uint2(lo, hi);
#pragma unroll
        for (int e = 0; e < 8; ++e) reinterpret_cast<unsigned char*>(vslab)[v_index_fp8(slot, c0 + e)] = cv[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kd[e] = kx[e];
        vd[e] = vx[e];
      }
      if (writer) {
        unsigned kw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          kw[e] = (__float_as_uint(kx[2 * e]) >> 16) | (__float_as_uint(kx[2 * e + 1]) & 0xFFFF0000u);
        *reinterpret_cast<uint4*>(kslab + 2 * k_index_bf16(slot, c0, D)) = make_uint4(kw[0], kw[1], kw[2], kw[3]);
        unsigned short* vs16 = reinterpret_cast<unsigned short*>(vslab);
#pragma unroll
        for (int e = 0; e < 8; ++e) vs16[v_index_bf16(slot, c0 + e)] = static_cast<unsigned short>(__float_as_uint(vx[e]) >> 16);
      }
    }
    *reinterpret_cast<float4*>(&s_k[j][c0]) = make_float4(kd[0], kd[1], kd[2], kd[3]);
    *reinterpret_cast<float4*>(&s_k[j][c0 + 4]) = make_float4(kd[4], kd[5], kd[6], kd[7]);
    *reinterpret_cast<float4*>(&s_v[j][c0]) = make_float4(vd[0], vd[1], vd[2], vd[3]);
    *reinterpret_cast<float4*>(&s_v[j][c0 + 4]) = make_float4(vd[4], vd[5], vd[6], vd[7]);
  }
  if (qr < nrb) {
    const unsigned wq[4] = {qbits.x, qbits.y, qbits.z, qbits.w};
    float qf[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[e] = __uint_as_float((wq[e / 2] >> (16 * (e % 2))) << 16);
    *reinterpret_cast<float4*>(&s_q[qr][qc]) = make_float4(qf[0], qf[1], qf[2], qf[3]);
    *reinterpret_cast<float4*>(&s_q[qr][qc + 4]) = make_float4(qf[4], qf[5], qf[6], qf[7]);
  }
  __syncthreads();
  // ---- scores of this block's rows over the new tokens -------------------------
  for (int y = tid; y < nrb * nq; y += kThreads) {
    const int ql = y / nq, jj = y % nq, i = (r0 + ql) / G;
    const bool vis = P.anc ? ((P.anc[long(b) * nq + i] >> jj) & 1ull) != 0 : jj <= i;
    float d0 = 0.0f, d1 = 0.0f;
#pragma unroll 8
    for (int c = 0; c < D; c += 4) {
      const float4 a = *reinterpret_cast<const float4*>(&s_q[ql][c]);
      const float4 k = *reinterpret_cast<const float4*>(&s_k[jj][c]);
      d0 = fmaf(a.x, k.x, d0);
      d1 = fmaf(a.y, k.y, d1);
      d0 = fmaf(a.z, k.z, d0);
      d1 = fmaf(a.w, k.w, d1);
    }
    s_w[ql][jj] = vis ? (d0 + d1) * P.scale_log2 : kNegInf;
  }
  __syncthreads();
  if (tid < nrb) {
    float m = kNegInf;
    for (int jj = 0; jj < nq; ++jj) m = fmaxf(m, s_w[tid][jj]);
    const float ref = m == kNegInf ? 0.0f : m;
    float l = 0.0f;
    for (int jj = 0; jj < nq; ++jj) {
      const float w = exp2_fast(s_w[tid][jj] - ref);
      s_w[tid][jj] = w;
      l += w;
    }
    s_m[tid] = m;
    s_l[tid] = l;
  }
  __syncthreads();
  // ---- combine and write -----------------------------------------------------------
  if (out_ok) {
    float4 on = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int jj = 0; jj < nq; ++jj) {
      const float w = s_w[rl][jj];
      const float4 v = *reinterpret_cast<const float4*>(&s_v[jj][4 * c4]);
      on.x = fmaf(w, v.x, on.x);
      on.y = fmaf(w, v.y, on.y);
      on.z = fmaf(w, v.z, on.z);
      on.w = fmaf(w, v.w, on.w);
    }
    lse_combine(M, Ls, o, s_m[rl], s_l[rl], on);
    const float inv = 1.0f / Ls;
    *reinterpret_cast<float4*>(P.out + oi * D + 4 * c4) = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
    if (c4 == 0 && P.lse) P.lse[oi] = (M + __log2f(Ls)) * kLn2;
  }
  // ---- the sequence's new length and block-table entry ---------------------------
  if (writer && g == 0 && tid == 0) {
    const_cast<int*>(P.seq_lens)[row] = N;
    if (F.new_page[b] >= 0) const_cast<int*>(P.block_table)[long(row) * P.bt_stride + np_old] = F.new_page[b];
  }
}

// Shared-prefix pass of the cascade (bf16 or FP8 KV with per-page scales):
// the first P.pref pages are the same physical pages for every sequence of
// the call, and every query sees all of their tokens, so they are attended
// once for all sequences.  A
// workgroup takes 64 query rows of one KV head from the flattened (sequence,
// slot, head) rows (any mix of sequences), 16 per wave.  The four waves walk
// every prefix page together: each page is read once per workgroup into LDS
// (double-buffered; the loads of the next kPrefixAhead pages are in flight in
// registers) and every wave reads its MFMA operands from there, so the prefix
// is read from L2 once per 64 rows.  The walk has no data-dependent branch
// around its loads and LDS traffic: it runs over whole groups of kPrefixAhead
// pages, pages past the prefix (read from the first page's address) enter
// with scores of -inf, and the Q fragments have landed before the first page
// load, so the load queue is waited on only as deep as each page needs.  Each
// wave leaves one unnormalised (O, max, sum) per row, which the merge (plain
// or fused) combines with the row's streamed pieces.  Same tiled layout, MFMA
// orientation and split-P arithmetic as the streaming kernel, without masks.
constexpr int kPrefixRows = kWaves * 16;
constexpr int kPrefixAhead = 4;

// A page slab in LDS holds each 1 KB MFMA tile with its 16-byte chunks in
// (quarter, token) order instead of the pool's (token, quarter) order, so
// that lane l of a wave reads its operand at byte 16 l of the tile: the
// linear pattern is the one gfx950 serves at the full LDS rate for 16-byte
// reads (the pool's order runs at half of it).  Pool chunk of LDS chunk q,
// and LDS chunk of pool chunk x:
__device__ inline int prefix_pool_chunk(int q) {
  return (q & ~63) | ((q & 15) << 2) | ((q >> 4) & 3);
}
__device__ inline int prefix_lds_chunk(int x) {
  return (x & ~63) | ((x & 3) << 4) | ((x >> 2) & 15);
}

// FP8 pages (per-page scales): each 16-byte group of the pool's FP8 slab is
// decoded while it is staged, into the two bf16 chunks it makes (in byte
// order: K group x = 64 s2 + 4 t + j gives bf16 chunks x + 64 s2 and that
// + 64, V group x = 4 qc + quad gives x + 4 qc and that + 4), so the waves
// read the same bf16 operand layout as for bf16 pages.  The page's K scale
// multiplies its scores and its V scale its P, as in the streaming kernel.
template <int D, bool FP8>
__global__ __launch_bounds__(kThreads) void verify_prefix_kernel(VerifyParams P) {
  constexpr int KS = D / 32, DT = D / 16, VL = D / 32;
  constexpr int PB = 64 * D;                     // bf16 bytes of one (page, head) in LDS: K slab then V slab
  constexpr int SB = FP8 ? 32 * D : PB;          // pool bytes of one (page, head)
  constexpr int NCH = (SB / 16 + kThreads - 1) / kThreads;   // 16-byte pool chunks of a page per thread
  constexpr int F = kPrefixAhead;
  static_assert((F & (F - 1)) == 0 && F <= 64, "one id per lane for a group of pages");
  __shared__ __align__(16) unsigned char s_pg[2][PB];
  __shared__ float s_sc[2][2];                   // FP8: the staged page's K and V scales
  const int g = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m16 = lane & 15, jg = lane >> 4;
  const unsigned lane_off = unsigned(lane * 16);
  const int rows_seq = P.n_q * P.G;
  const long R = long(P.batch) * rows_seq;
  const long r_lane = long(blockIdx.y) * kPrefixRows + wave * 16 + m16;   // this lane's query row
  const int row_b0 = P.batch_slots ? P.batch_slots[0] : 0;
  const int* bt = P.block_table + long(row_b0) * P.bt_stride;
  // whole pages of the first sequence only (its table has no other entries)
  const int n_pref = min(P.pref, P.seq_lens[row_b0] >> 4);
  const long rq = r_lane < R ? r_lane : 0;       // rows past the batch read row 0 and are not written
  const int qb = int(rq / rows_seq), qrem = int(rq % rows_seq);
  const int qi = qrem / P.G, qh = g * P.G + qrem % P.G;
  const long oi = long(qb * P.n_q + qi) * P.Hq + qh;
  u32x4 qf[KS];
  {
    const unsigned short* qp = static_cast<const unsigned short*>(P.q) + oi * D + (D / 4) * jg;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = load16(qp + 8 * s);
  }
  float m_run = kNegInf, l_run = 0.0f;
  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0, 0, 0, 0};
  const long page_stride = long(P.Hkv) * P.slab_bytes;
  // page ids a group of F pages at a time: lane i of `ids` holds the id of
  // page p + (i mod F) (past the prefix: the first page's), read with
  // readlane.  Each group loads the ids of the group after the next one with
  // a vector load issued before its page loads, so no wait in the walk is
  // deeper than the page it needs (a scalar load of the table would make
  // every LDS wait a full one: its returns are out of order)
  auto group_ids = [&](int p) {
    const int q = p + (lane & (F - 1));
    return bt[q < n_pref ? q : 0];
  };
  const int ids0 = group_ids(0);
  int ids_ahead = group_ids(F);
  // the Q and id loads stay ahead of every page load (the fences of the
  // barrier keep them there), so waiting for the first page covers them
  __syncthreads();
  u32x4 stg[F][NCH];
  float sc_k[F], sc_v[F];                        // FP8: ring slot's scales (thread 0)
  // bf16: this thread's LDS chunks q = tid + j * kThreads of the page with id
  // `id` into ring slot u (the K slab's chunks, then the V slab's); each
  // wave's load covers one whole 1 KB tile.  FP8: pool group q of the page
  // (K slab, then V slab), and thread 0 the page's two scales.
  auto fetch = [&](int u, int id) {
    const char* kb = P.k_pages + long(id) * page_stride + long(g) * P.slab_bytes;
    const char* vb = P.v_pages + long(id) * page_stride + long(g) * P.slab_bytes;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int q = tid + j * kThreads;
      if (FP8) {
        if (q < SB / 16) stg[u][j] = load16(q < SB / 32 ? kb + q * 16 : vb + (q - SB / 32) * 16);
      } else {
        stg[u][j] = load16(q < PB / 32 ? kb + prefix_pool_chunk(q) * 16 : vb + prefix_pool_chunk(q - PB / 32) * 16);
      }
    }
    if (FP8 && tid == 0) {
      sc_k[u] = static_cast<const float*>(P.k_scale)[long(id) * P.Hkv + g];
      sc_v[u] = static_cast<const float*>(P.v_scale)[long(id) * P.Hkv + g];
    }
  };
  auto stage = [&](int u, int buf) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int q = tid + j * kThreads;
      if (FP8) {
        if (q < SB / 16) {
          const u32x4 w = stg[u][j];
          const Dw2 a0 = fp8x4_to_bf16x4(w[0]), a1 = fp8x4_to_bf16x4(w[1]);
          const Dw2 a2 = fp8x4_to_bf16x4(w[2]), a3 = fp8x4_to_bf16x4(w[3]);
          const bool isk = q < SB / 32;
          const int x = isk ? q : q - SB / 32;                  // group within its slab
          const int lo = isk ? x + (x >> 6) * 64 : x + (x >> 2) * 4;
          const int hi = lo + (isk ? 64 : 4);
          unsigned char* base = &s_pg[buf][isk ? 0 : PB / 2];
          *reinterpret_cast<u32x4*>(base + prefix_lds_chunk(lo) * 16) = u32x4{a0.lo, a0.hi, a1.lo, a1.hi};
          *reinterpret_cast<u32x4*>(base + prefix_lds_chunk(hi) * 16) = u32x4{a2.lo, a2.hi, a3.lo, a3.hi};
        }
      } else {
        *reinterpret_cast<u32x4*>(&s_pg[buf][q * 16]) = stg[u][j];
      }
    }
    if (FP8 && tid == 0) {
      s_sc[buf][0] = sc_k[u];
      s_sc[buf][1] = sc_v[u];
    }
  };
  // (n_pref is the same for the whole workgroup; the walk is entered only
  // through the prologue, so no path reaches it with the Q loads in flight)
  if (n_pref > 0) {
#pragma unroll
    for (int u = 0; u < F; ++u) fetch(u, __builtin_amdgcn_readlane(ids0, u));
    stage(0, 0);
    __syncthreads();
    for (int p0 = 0; p0 < n_pref; p0 += F) {
      const int ids_next = group_ids(p0 + 2 * F);
#pragma unroll
      for (int u = 0; u < F; ++u) {
        const int p = p0 + u;
        const float bias = p < n_pref ? 0.0f : kNegInf;
        const unsigned char* kl = s_pg[p & 1];
        const unsigned char* vl = kl + PB / 2;
        u32x4 kc[KS], vc[VL];
#pragma unroll
        for (int s = 0; s < KS; ++s) kc[s] = *reinterpret_cast<const u32x4*>(kl + lane_off + s * 1024);
#pragma unroll
        for (int c = 0; c < VL; ++c) vc[c] = *reinterpret_cast<const u32x4*>(vl + lane_off + c * 1024);
        f32x4 sc = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < KS; ++s) sc = mfma_bf16(kc[s], qf[s], sc);
        const float ksc = FP8 ? P.scale_log2 * s_sc[p & 1][0] : P.scale_log2;
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[e] = fmaf(sc[e], ksc, bias);
        const float mx = row_max4(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
        const bool grow = mx > m_run + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(grow)) {
          const float m_new = grow ? mx : m_run;
          const float alpha = grow ? exp2_fast(m_run - m_new) : 1.0f;
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
          m_run = m_new;
        }
        float pv[4], rv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = exp2_fast(sc[e] - m_run);
        l_run += (pv[0] + pv[1]) + (pv[2] + pv[3]);
        if (FP8) {
          const float vsc = s_sc[p & 1][1];
#pragma unroll
          for (int e = 0; e < 4; ++e) pv[e] *= vsc;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) rv[e] = pv[e] - __uint_as_float(__float_as_uint(pv[e]) & 0xFFFF0000u);
        const unsigned ph0 = pack_hi16(pv[0], pv[1]), ph1 = pack_hi16(pv[2], pv[3]);
        const unsigned pl0 = pack_rne_bf16(rv[0], rv[1]), pl1 = pack_rne_bf16(rv[2], rv[3]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int w = (dt & 1) * 2;
          acc[dt] = mfma_bf16_split(vc[dt >> 1][w], vc[dt >> 1][w + 1], ph0, ph1, pl0, pl1, acc[dt]);
        }
        // page p + 1 (fetched F - 1 pages ago) into the other buffer, whose
        // last readers passed the previous barrier; page p + F into the slot
        // page p used
        stage((u + 1) % F, (p + 1) & 1);
        fetch(u, __builtin_amdgcn_readlane(ids_ahead, u));
        __syncthreads();
      }
      ids_ahead = ids_next;
    }
  }
  // this lane's row: unnormalised O over channels c*32 + 8jg .. +7, max, sum
  float l = l_run;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (r_lane >= R || qi >= seq_slots(P, qb)) return;
  float* dst = P.prefix_part + oi * (D + 2);
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    const int ch = c * 32 + 8 * jg;
    *reinterpret_cast<float4*>(dst + ch) =
        make_float4(acc[2 * c][0], acc[2 * c + 1][0], acc[2 * c][1], acc[2 * c + 1][1]);
    *reinterpret_cast<float4*>(dst + ch + 4) =
        make_float4(acc[2 * c][2], acc[2 * c + 1][2], acc[2 * c][3], acc[2 * c + 1][3]);
  }
  if (jg == 0) {
    dst[D] = m_run;
    dst[D + 1] = l;
  }
}

// Dynamic LDS of the streaming kernel: page prefix sums, scan scratch and
// per-sequence (row, length word) pairs, then every wave's Q slots, then
// their ancestor-mask slots.
__host__ __device__ inline int cum_lds_bytes(int batch) {
  const int cum_words = (batch + 1 + 3) & ~3;
  const int seq_words = (2 * batch + 3) & ~3;
  return (cum_words + kThreads + seq_words) * 4;
}

template <int D, int NT, bool W2 = false>
size_t split_smem(int batch) {
  using SH = Shape<D, NT, false, W2>;
  return size_t(cum_lds_bytes(batch)) + size_t(kWaves) * SH::QS * (SH::QSLOT + SH::ASLOT);
}

// Each wave is one worker streaming an equal contiguous range of the
// (sequence, KV head, page) positions.
template <int D, int NT, bool FP8, bool TREE, bool SHARED, bool W2, bool MX>
__device__ inline void stream_kernel_body(VerifyParams P) {
  extern __shared__ int s_cum[];
  const int cum_words = (P.batch + 1 + 3) & ~3;
  int* s_seq = s_cum + cum_words + kThreads;
  page_prefix(P, s_cum, s_cum + cum_words, s_seq);
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i <= P.batch; i += kThreads) P.cum[i] = s_cum[i];
    if (P.fused)
      for (int i = threadIdx.x; i < P.batch; i += kThreads) P.old_len[i] = s_seq[2 * i + 1] & kLenMask;
  }
  const int W = P.Hkv * uni(s_cum[P.batch]);
  if (W == 0) return;
  const int worker = blockIdx.x * kWaves + uni(threadIdx.x >> 6);
  const int n_rng = used_ranges(P, W);
  const int range = worker / P.rg, rgi = worker % P.rg;
  if (range >= n_rng) return;
  const int lo = int(range_lo(range, W, n_rng)), hi = int(range_lo(range + 1, W, n_rng));
  stream_range<D, NT, FP8, TREE, SHARED, W2, MX>(P, s_cum, s_seq, lo, hi, worker, cum_lds_bytes(P.batch),
                                                 rgi * P.rows_w);
}

template <int D, int NT, bool FP8, bool TREE, bool SHARED, bool MX = false>
__global__ __launch_bounds__(kThreads) void verify_stream_kernel(VerifyParams P) {
  stream_kernel_body<D, NT, FP8, TREE, SHARED, false, MX>(P);
}

// Two waves per SIMD: each kept within 256 registers.
template <int D, int NT, bool FP8, bool TREE, bool SHARED, bool MX = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void verify_stream_kernel_w2(VerifyParams P) {
  stream_kernel_body<D, NT, FP8, TREE, SHARED, true, MX>(P);
}

// fp32 K/V (plain [token][channel] pages): one workgroup per (query head,
// sequence), VALU arithmetic, no split.  Meant for small fp32 problems.
template <int D>
__global__ __launch_bounds__(128) void verify_f32_kernel(VerifyParams P) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int g = h / P.G;
  const int row_b = P.batch_slots ? P.batch_slots[b] : b;
  const int nq_b = seq_slots(P, b);
  const int N = P.seq_lens[row_b], L = N - nq_b;
  const int* bt = P.block_table + long(row_b) * P.bt_stride;
  __shared__ float s_q[D];
  __shared__ float s_p[128];
  __shared__ float s_red[2];
  const float scale = P.scale_log2;
  for (int i = 0; i < nq_b; ++i) {
    const long oi = long(b * P.n_q + i) * P.Hq + h;
    __syncthreads();
    for (int c = tid; c < D; c += 128) s_q[c] = static_cast<const float*>(P.q)[oi * D + c];
    const unsigned long long anc = P.anc ? P.anc[long(b) * P.n_q + i] : 0ull;
    __syncthreads();
    float m_run = kNegInf, l_run = 0.0f, acc = 0.0f;     // acc: channel tid (if < D)
    for (int t0 = 0; t0 < N; t0 += 128) {
      const int t = t0 + tid;
      float s = kNegInf;
      bool vis = false;
      if (t < N) {
        const int j = t - L;
        vis = (t < L) || (P.anc ? ((anc >> (j & 63)) & 1ull) != 0 : j <= i);
      }
      if (vis) {
        const float* kp = reinterpret_cast<const float*>(
            P.k_pages + (long(bt[t >> 4]) * P.Hkv + g) * P.slab_bytes) + (t & 15) * D;
        float d = 0.0f;
        for (int c = 0; c < D; ++c) d = fmaf(s_q[c], kp[c], d);
        s = d * scale;
      }
      // block max
      float mx = s;
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      __syncthreads();
      if ((tid & 63) == 0) s_red[tid >> 6] = mx;
      __syncthreads();
      mx = fmaxf(s_red[0], s_red[1]);
      const float m_new = fmaxf(m_run, mx);
      const float m_ref = m_new == kNegInf ? 0.0f : m_new;
      const float alpha = exp2f(m_run - m_ref);
      const float p = exp2f(s - m_ref);
      s_p[tid] = p;
      float ps = p;
      for (int o = 32; o > 0; o >>= 1) ps += __shfl_xor(ps, o, 64);
      __syncthreads();
      if ((tid & 63) == 0) s_red[tid >> 6] = ps;
      __syncthreads();
      l_run = l_run * alpha + s_red[0] + s_red[1];
      m_run = m_new;
      acc *= alpha;
      if (tid < D) {
        const int tn = min(128, N - t0);
        for (int u = 0; u < tn; ++u) {
          const float pu = s_p[u];
          if (pu != 0.0f) {
            const int tt = t0 + u;
            const float* vp = reinterpret_cast<const float*>(
                P.v_pages + (long(bt[tt >> 4]) * P.Hkv + g) * P.slab_bytes) + (tt & 15) * D;
            acc = fmaf(pu, vp[tid], acc);
          }
        }
      }
      __syncthreads();
    }
    if (tid < D) P.out[oi * D + tid] = acc / l_run;
    if (tid == 0 && P.lse) P.lse[oi] = (m_run + log2f(l_run)) * kLn2;
  }
}

struct Plan {
  int D, NT, rows, n_wg, rg, rows_w;
  bool fp8, mx, tree, f32;
  size_t cum_bytes, part_bytes, prefix_bytes, fused_bytes;
  size_t bytes() const { return cum_bytes + part_bytes + prefix_bytes + fused_bytes; }
};

pkv_status check_args(const pkv_verify_args* a, Plan* pl) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "null args");
  if (a->batch < 1 || a->batch > 4096) return fail(PKV_ERR_INVALID_ARG, "batch must be in [1, 4096]");
  if (a->n_q < 1 || a->n_q > 64) return fail(PKV_ERR_INVALID_ARG, "n_q must be in [1, 64]");
  if (a->num_kv_heads < 1 || a->num_kv_heads > 65535 || a->num_q_heads < a->num_kv_heads ||
      a->num_q_heads % a->num_kv_heads)
    return fail(PKV_ERR_INVALID_ARG, "num_kv_heads must be in [1, 65535] and divide num_q_heads");
  if (a->page_size != kPageSize) return fail(PKV_ERR_UNSUPPORTED, "page_size must be 16");
  if (a->head_dim != 64 && a->head_dim != 128) return fail(PKV_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (a->block_table_stride < 1) return fail(PKV_ERR_INVALID_ARG, "block_table_stride must be >= 1");
  if (!(a->sm_scale > 0.0f) || !(a->sm_scale < INFINITY))
    return fail(PKV_ERR_INVALID_ARG, "sm_scale must be positive and finite");
  if (!a->q || !a->k_pages || !a->v_pages || !a->block_table || !a->seq_lens)
    return fail(PKV_ERR_INVALID_ARG, "null device pointer");
  if (a->shared_prefix_pages < 0) return fail(PKV_ERR_INVALID_ARG, "shared_prefix_pages must be >= 0");
  if (a->shared_prefix_pages > 0 && a->kv_dtype != PKV_BF16 && a->kv_dtype != PKV_FP8_E4M3)
    return fail(PKV_ERR_UNSUPPORTED, "the shared-prefix pass supports bf16 and per-page-scale FP8 KV");
  if (a->num_splits < 0 || a->num_splits > 1024)
    return fail(PKV_ERR_INVALID_ARG, "num_splits must be in [0, 1024]");
  const int G = a->num_q_heads / a->num_kv_heads;
  pl->D = a->head_dim;
  pl->rows = a->n_q * G;
  pl->tree = a->anc_mask != nullptr;
  pl->f32 = false;
  pl->fp8 = false;
  pl->mx = false;
  if (a->kv_dtype == PKV_F32) {
    if (a->q_dtype != PKV_F32) return fail(PKV_ERR_INVALID_ARG, "fp32 KV needs fp32 queries");
    pl->f32 = true;
  } else if (a->kv_dtype == PKV_BF16 || a->kv_dtype == PKV_FP8_E4M3 || a->kv_dtype == PKV_FP8_E4M3_MX64) {
    if (a->q_dtype != PKV_BF16) return fail(PKV_ERR_INVALID_ARG, "bf16/fp8 KV needs bf16 queries");
    pl->fp8 = a->kv_dtype != PKV_BF16;
    pl->mx = a->kv_dtype == PKV_FP8_E4M3_MX64;
    if (pl->fp8 && (!a->k_scale || !a->v_scale)) return fail(PKV_ERR_INVALID_ARG, "FP8 KV needs scales");
    if (pl->rows > 64) return fail(PKV_ERR_UNSUPPORTED, "n_q * Hq/Hkv must be <= 64");
  } else {
    return fail(PKV_ERR_INVALID_ARG, "unknown dtype");
  }
  // More than 48 rows: two waves share each range, 32 rows each (the same
  // pages reach both from one fetch, and each keeps a 32-row register set).
  pl->rg = pl->rows > 48 ? 2 : 1;
  pl->rows_w = pl->rg == 1 ? pl->rows : 32;
  pl->NT = (pl->rows_w + 15) / 16;
  return PKV_OK;
}

// Resident workgroups of one kernel instance per GPU (cached per device,
// instance and LDS size).
int resident_workgroups(const void* fn, size_t smem) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, size_t>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  std::lock_guard<std::mutex> lock(mu);
  auto key = std::make_tuple(dev, fn, smem);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per_cu = 0;
  if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, smem) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  (void)hipGetLastError();
  const int n = cus * per_cu;
  cache[key] = n;
  return n;
}

size_t split_smem_rt(int D, int NT, int batch) {
  switch ((D == 64 ? 0 : 4) + NT - 1) {
    case 0: return split_smem<64, 1>(batch);
    case 1: return split_smem<64, 2>(batch);
    case 2: return split_smem<64, 3>(batch);
    case 3: return split_smem<64, 4>(batch);
    case 4: return split_smem<128, 1>(batch);
    case 5: return split_smem<128, 2>(batch);
    case 6: return split_smem<128, 3>(batch);
    default: return split_smem<128, 4>(batch);
  }
}

#ifndef PKV_TWO_WAVES
#define PKV_TWO_WAVES 1
#endif
// FP8 KV with up to 32 rows per wave runs the two-waves-per-SIMD kernel: its
// per-page instruction stream (decoding) leaves the SIMD idle between one
// wave's loads otherwise (measured: 96.6 -> 65.3 us for 16 x 8192 tokens,
// 20 rows); for bf16 KV the one-wave kernel with its deeper prefetch is as
// fast or faster.
inline bool two_waves(int NT, bool fp8) { return PKV_TWO_WAVES && fp8 && NT <= 2; }

template <int D, int NT, bool FP8, bool TREE, bool SHARED = false, bool MX = false>
const void* split_fn() {
  return reinterpret_cast<const void*>(&verify_stream_kernel<D, NT, FP8, TREE, SHARED, MX>);
}
template <int D, int NT, bool FP8, bool TREE, bool SHARED, bool MX = false>
const void* split_fn_w2() {
  return reinterpret_cast<const void*>(&verify_stream_kernel_w2<D, NT, FP8, TREE, SHARED, MX>);
}

template <int D, int NT>
const void* pick_fn(bool fp8, bool tree) {
  if (fp8) return tree ? split_fn<D, NT, true, true>() : split_fn<D, NT, true, false>();
  return tree ? split_fn<D, NT, false, true>() : split_fn<D, NT, false, false>();
}

template <int D>
const void* pick_fn(int NT, bool shared, bool fp8, bool tree) {
  if (two_waves(NT, fp8)) {
    if (shared) return tree ? split_fn_w2<D, 2, true, true, true>() : split_fn_w2<D, 2, true, false, true>();
    if (NT == 1) return tree ? split_fn_w2<D, 1, true, true, false>() : split_fn_w2<D, 1, true, false, false>();
    return tree ? split_fn_w2<D, 2, true, true, false>() : split_fn_w2<D, 2, true, false, false>();
  }
  if (shared) {
    if (fp8) return tree ? split_fn<D, 2, true, true, true>() : split_fn<D, 2, true, false, true>();
    return tree ? split_fn<D, 2, false, true, true>() : split_fn<D, 2, false, false, true>();
  }
  switch (NT) {
    case 1: return pick_fn<D, 1>(fp8, tree);
    case 2: return pick_fn<D, 2>(fp8, tree);
    default: return pick_fn<D, 3>(fp8, tree);
  }
}

// Per-64-channel scales (MX): the two-waves kernels for up to 32 rows per
// wave, the one-wave kernel for 33..48.
template <int D>
const void* pick_fn_mx(int NT, bool shared, bool tree) {
  if (shared) return tree ? split_fn_w2<D, 2, true, true, true, true>() : split_fn_w2<D, 2, true, false, true, true>();
  if (NT == 1) return tree ? split_fn_w2<D, 1, true, true, false, true>() : split_fn_w2<D, 1, true, false, false, true>();
  if (NT == 2) return tree ? split_fn_w2<D, 2, true, true, false, true>() : split_fn_w2<D, 2, true, false, false, true>();
  return tree ? split_fn<D, 3, true, true, false, true>() : split_fn<D, 3, true, false, false, true>();
}

pkv_status make_plan(const pkv_verify_args* a, Plan* pl) {
  pkv_status st = check_args(a, pl);
  if (st != PKV_OK) return st;
  pl->cum_bytes = 0;
  pl->part_bytes = 0;
  // cascade: the prefix partials, then the log2-sum-exp of units finished in place
  pl->prefix_bytes = a->shared_prefix_pages > 0
                         ? ((size_t(a->batch) * a->n_q * a->num_q_heads * (a->head_dim + 2) * sizeof(float) + 255) &
                            ~size_t(255)) +
                               ((size_t(a->batch) * a->n_q * a->num_q_heads * sizeof(float) + 255) & ~size_t(255))
                         : 0;
  pl->n_wg = 0;
  // a call that spec_verify_attention_append can take also sizes its
  // per-row log2-sum-exp of units finished in place and the cached lengths
  const bool fusable = !pl->f32 && a->n_q <= kFusedMaxTokens && a->batch <= kFusedMaxBatch && !a->n_q_seq &&
                       !a->batch_slots;
  pl->fused_bytes = fusable ? ((size_t(a->batch) * a->n_q * a->num_q_heads * sizeof(float) + 255) & ~size_t(255)) +
                                  ((size_t(a->batch) * sizeof(int) + 255) & ~size_t(255))
                            : 0;
  if (!pl->f32) {
    int n = a->num_splits;
    if (n == 0) {
      const size_t smem = two_waves(pl->NT, pl->fp8)
                              ? (pl->D == 64 ? (pl->NT == 1 ? split_smem<64, 1, true>(a->batch) : split_smem<64, 2, true>(a->batch))
                                             : (pl->NT == 1 ? split_smem<128, 1, true>(a->batch) : split_smem<128, 2, true>(a->batch)))
                              : split_smem_rt(pl->D, pl->NT, a->batch);
      const void* fn = pl->mx ? (pl->D == 64 ? pick_fn_mx<64>(pl->NT, pl->rg > 1, pl->tree)
                                             : pick_fn_mx<128>(pl->NT, pl->rg > 1, pl->tree))
                     : pl->D == 64 ? pick_fn<64>(pl->NT, pl->rg > 1, pl->fp8, pl->tree)
                                   : pick_fn<128>(pl->NT, pl->rg > 1, pl->fp8, pl->tree);
      n = resident_workgroups(fn, smem);
    }
    pl->n_wg = n;
    pl->cum_bytes = ((size_t(a->batch) + 1) * sizeof(int) + 255) & ~size_t(255);
    pl->part_bytes = (size_t(n) * kWaves * 2 * size_t(pl->rows_w) * (pl->D + 2) * sizeof(float) + 255) & ~size_t(255);
  }
  return PKV_OK;
}

template <int D, int NT, bool FP8, bool TREE, bool SHARED, bool MX = false>
hipError_t launch_split_w2(const VerifyParams& p, hipStream_t st) {
  const size_t smem = split_smem<D, NT, true>(p.batch);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&verify_stream_kernel_w2<D, NT, FP8, TREE, SHARED, MX>),
      hipFuncAttributeMaxDynamicSharedMemorySize, int(split_smem<D, NT, true>(4096)));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((verify_stream_kernel_w2<D, NT, FP8, TREE, SHARED, MX>), dim3(p.n_wg), dim3(kThreads), smem, st, p);
  return hipGetLastError();
}

template <int D, int NT, bool FP8, bool TREE, bool SHARED = false, bool MX = false>
hipError_t launch_split(const VerifyParams& p, hipStream_t st) {
  const size_t smem = split_smem<D, NT>(p.batch);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&verify_stream_kernel<D, NT, FP8, TREE, SHARED, MX>),
      hipFuncAttributeMaxDynamicSharedMemorySize, int(split_smem<D, NT>(4096)));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((verify_stream_kernel<D, NT, FP8, TREE, SHARED, MX>), dim3(p.n_wg), dim3(kThreads), smem, st, p);
  return hipGetLastError();
}

// The merge after the streaming kernel: of the split units, or, in a fused
// call, of every unit with its new tokens (which it also writes).
template <int D>
hipError_t launch_merge(const VerifyParams& p, const FusedAppend* f, hipStream_t st) {
  const dim3 grid(p.batch * p.Hkv, (p.rows * (D / 4) + kThreads - 1) / kThreads);
  if (f) hipLaunchKernelGGL((verify_fused_merge_kernel<D>), grid, dim3(kThreads), 0, st, p, *f);
  else hipLaunchKernelGGL((verify_merge_kernel<D>), grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

template <int D, int NT>
hipError_t dispatch_kv(const VerifyParams& p, bool fp8, bool tree, hipStream_t st) {
  if (fp8) return tree ? launch_split<D, NT, true, true>(p, st) : launch_split<D, NT, true, false>(p, st);
  return tree ? launch_split<D, NT, false, true>(p, st) : launch_split<D, NT, false, false>(p, st);
}

template <int D>
hipError_t dispatch_mx(const VerifyParams& p, int NT, bool tree, hipStream_t st) {
  if (p.rg > 1)
    return tree ? launch_split_w2<D, 2, true, true, true, true>(p, st) : launch_split_w2<D, 2, true, false, true, true>(p, st);
  if (NT == 1) return tree ? launch_split_w2<D, 1, true, true, false, true>(p, st) : launch_split_w2<D, 1, true, false, false, true>(p, st);
  if (NT == 2) return tree ? launch_split_w2<D, 2, true, true, false, true>(p, st) : launch_split_w2<D, 2, true, false, false, true>(p, st);
  return tree ? launch_split<D, 3, true, true, false, true>(p, st) : launch_split<D, 3, true, false, false, true>(p, st);
}

template <int D>
hipError_t dispatch_nt(const VerifyParams& p, int NT, bool fp8, bool tree, hipStream_t st) {
  if (two_waves(NT, fp8)) {
    if (p.rg > 1)
      return tree ? launch_split_w2<D, 2, true, true, true>(p, st) : launch_split_w2<D, 2, true, false, true>(p, st);
    if (NT == 1) return tree ? launch_split_w2<D, 1, true, true, false>(p, st) : launch_split_w2<D, 1, true, false, false>(p, st);
    return tree ? launch_split_w2<D, 2, true, true, false>(p, st) : launch_split_w2<D, 2, true, false, false>(p, st);
  }
  if (p.rg > 1) {
    if (fp8) return tree ? launch_split<D, 2, true, true, true>(p, st) : launch_split<D, 2, true, false, true>(p, st);
    return tree ? launch_split<D, 2, false, true, true>(p, st) : launch_split<D, 2, false, false, true>(p, st);
  }
  switch (NT) {
    case 1: return dispatch_kv<D, 1>(p, fp8, tree, st);
    case 2: return dispatch_kv<D, 2>(p, fp8, tree, st);
    default: return dispatch_kv<D, 3>(p, fp8, tree, st);
  }
}

}  // namespace

}  // namespace pkv

using namespace pkv;

extern "C" pkv_status spec_verify_workspace_size(const pkv_verify_args* args, size_t* bytes_out) {
  if (!bytes_out) return fail(PKV_ERR_INVALID_ARG, "null output");
  Plan pl;
  pkv_status st = make_plan(args, &pl);
  if (st != PKV_OK) return st;
  *bytes_out = pl.bytes();
  return PKV_OK;
}

namespace pkv {
namespace {

// Launches a planned call with its scratch at `ws` (at least the plan's
// bytes): the page prefix sums, the partial results of split units, the
// cascade's prefix partials and log2-sum-exp of units finished in place and,
// for a fused call (f not null), its own log2-sum-exp of units finished in
// place and the cached lengths.  None of
// it has to start at zero: every word the merge reads is written earlier in
// the same call.
pkv_status verify_launch(const pkv_verify_args* a, const Plan& pl, void* ws, void* stream,
                         const FusedAppend* f = nullptr) {
  VerifyParams p{};
  char* w = static_cast<char*>(ws);
  p.q = a->q;
  p.k_pages = static_cast<const char*>(a->k_pages);
  p.v_pages = static_cast<const char*>(a->v_pages);
  p.k_scale = a->k_scale;
  p.v_scale = a->v_scale;
  p.block_table = a->block_table;
  p.seq_lens = a->seq_lens;
  p.batch_slots = a->batch_slots;
  p.anc = reinterpret_cast<const unsigned long long*>(a->anc_mask);
  p.nq_seq = a->n_q_seq;
  p.out = a->out;
  p.lse = a->lse;
  p.cum = reinterpret_cast<int*>(w);
  p.part = reinterpret_cast<float*>(w + pl.cum_bytes);
  p.prefix_part = pl.prefix_bytes ? reinterpret_cast<float*>(w + pl.cum_bytes + pl.part_bytes) : nullptr;
  if (pl.prefix_bytes) {
    p.defer = 1;
    p.unit_lse = reinterpret_cast<float*>(
        w + pl.cum_bytes + pl.part_bytes +
        ((size_t(a->batch) * a->n_q * a->num_q_heads * (a->head_dim + 2) * sizeof(float) + 255) & ~size_t(255)));
  }
  if (f) {
    char* fw = w + pl.cum_bytes + pl.part_bytes + pl.prefix_bytes;
    p.fused = 1;
    p.defer = 1;
    p.unit_lse = reinterpret_cast<float*>(fw);
    p.old_len = reinterpret_cast<int*>(fw + ((size_t(a->batch) * a->n_q * a->num_q_heads * sizeof(float) + 255) &
                                             ~size_t(255)));
  }
  p.kv_kind = a->kv_dtype;
  p.pref = a->shared_prefix_pages;
  p.min_range = a->num_splits == 0 ? 8 : 1;
  p.slab_bytes = pkv_page_bytes(a->kv_dtype, a->page_size, a->head_dim);
  p.batch = a->batch;
  p.n_q = a->n_q;
  p.Hq = a->num_q_heads;
  p.Hkv = a->num_kv_heads;
  p.G = a->num_q_heads / a->num_kv_heads;
  p.rows = pl.rows;
  p.rg = pl.rg;
  p.rows_w = pl.rows_w;
  p.bt_stride = a->block_table_stride;
  p.n_wg = pl.n_wg;
  p.scale_log2 = a->sm_scale * kLog2e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (pl.f32) {
    if (pl.D == 64)
      hipLaunchKernelGGL(verify_f32_kernel<64>, dim3(p.Hq, p.batch), dim3(128), 0, s, p);
    else
      hipLaunchKernelGGL(verify_f32_kernel<128>, dim3(p.Hq, p.batch), dim3(128), 0, s, p);
    e = hipGetLastError();
  } else if (pl.mx) {
    e = pl.D == 64 ? dispatch_mx<64>(p, pl.NT, pl.tree, s) : dispatch_mx<128>(p, pl.NT, pl.tree, s);
  } else {
    e = pl.D == 64 ? dispatch_nt<64>(p, pl.NT, pl.fp8, pl.tree, s) : dispatch_nt<128>(p, pl.NT, pl.fp8, pl.tree, s);
    if (e == hipSuccess && p.pref > 0) {
      // cascade: the shared prefix once for all sequences.  Neither kernel
      // reads what the other writes: the streaming kernel leaves the units it
      // finishes as (normalised O, log2-sum-exp) and the merge combines every
      // row with its prefix partial, so no wave of the streaming kernel waits
      // on prefix results.
      const long rows = long(p.batch) * p.n_q * p.G;
      const dim3 grid(p.Hkv, unsigned((rows + kPrefixRows - 1) / kPrefixRows));
      if (pl.D == 64) {
        if (pl.fp8) hipLaunchKernelGGL((verify_prefix_kernel<64, true>), grid, dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL((verify_prefix_kernel<64, false>), grid, dim3(kThreads), 0, s, p);
      } else {
        if (pl.fp8) hipLaunchKernelGGL((verify_prefix_kernel<128, true>), grid, dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL((verify_prefix_kernel<128, false>), grid, dim3(kThreads), 0, s, p);
      }
      e = hipGetLastError();
    }
  }
  if (e == hipSuccess && !pl.f32) e = pl.D == 64 ? launch_merge<64>(p, f, s) : launch_merge<128>(p, f, s);
  if (e != hipSuccess) return fail(PKV_ERR_DEVICE, std::string("verify launch: ") + hipGetErrorString(e));
  return PKV_OK;
}

// Scratch of spec_verify_attention_static: one array per GPU, held by the
// library until the process ends (uninitialised device data, so the shared
// library's file does not grow with it).  Host code never uses the array's
// name as an address: each device's address comes from hipGetSymbolAddress,
// taken once per device with that device current.
constexpr size_t kStaticScratchBytes = size_t(80) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, or null with the status.
pkv_status static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return fail(PKV_ERR_DEVICE, "no current HIP device for the static scratch");
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return fail(PKV_ERR_DEVICE, std::string("static scratch address: ") + hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace
}  // namespace pkv

extern "C" pkv_status spec_verify_attention(const pkv_verify_args* a, void* stream) {
  Plan pl;
  pkv_status st = make_plan(a, &pl);
  if (st != PKV_OK) return st;
  if (!a->out) return fail(PKV_ERR_INVALID_ARG, "null output pointer");
  const size_t need = pl.bytes();
  if (need > 0 && (!a->workspace || a->workspace_bytes < need))
    return fail(PKV_ERR_WORKSPACE, "workspace smaller than spec_verify_workspace_size");
  return verify_launch(a, pl, a->workspace, stream);
}

extern "C" pkv_status spec_verify_attention_static(const pkv_verify_args* a, void* stream) {
  Plan pl;
  pkv_status st = make_plan(a, &pl);
  if (st != PKV_OK) return st;
  if (!a->out) return fail(PKV_ERR_INVALID_ARG, "null output pointer");
  const size_t need = pl.bytes();
  if (need > kStaticScratchBytes)
    return fail(PKV_ERR_WORKSPACE, "call needs " + std::to_string(need) + " bytes of scratch; the static scratch holds " +
                                       std::to_string(kStaticScratchBytes) + " (fewer num_splits need less)");
  void* ws = nullptr;
  if (need > 0 && (st = static_scratch(&ws)) != PKV_OK) return st;
  return verify_launch(a, pl, ws, stream);
}

pkv_status pkv::verify_fused_launch(const pkv_verify_args* a, const FusedAppend& f, void* stream) {
  Plan pl;
  pkv_status st = make_plan(a, &pl);
  if (st != PKV_OK) return st;
  if (pl.f32 || pl.fused_bytes == 0) return fail(PKV_ERR_UNSUPPORTED, "call cannot be fused");
  return verify_launch(a, pl, a->workspace, stream, &f);
}
