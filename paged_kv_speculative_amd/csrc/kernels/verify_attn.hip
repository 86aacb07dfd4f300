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
//    balance exactly.  A range covers whole (sequence, KV head) units, which
//    are finished in place, and at most two pieces of units, which are
//    written as partial (max, sum, unnormalised O) and merged by a second
//    kernel with a log-sum-exp combine.
//  * One (sequence, KV head) unit serves all n_q * G query rows that read the
//    same pages (G = Hq/Hkv): every KV byte is read once per call.
//  * Four waves of a workgroup share a range's page pairs; each keeps its
//    own online-softmax state and the four are combined through LDS.
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

#include "../common.h"

namespace pkv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

struct VerifyParams {
  const void* q;
  const char* k_pages;
  const char* v_pages;
  const float* k_scale;
  const float* v_scale;
  const int* block_table;
  const int* seq_lens;
  const int* batch_slots;
  const unsigned long long* anc;
  float* out;
  float* lse;
  float* part;           // [n_wg][2][slot_floats]
  int* cum_ws;           // [batch + 1] page prefix sums, written by workgroup 0
  long slab_bytes;       // bytes of one (page, KV head) slab
  int batch, n_q, Hq, Hkv, G, rows, bt_stride, n_wg;
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

// bf16 round-to-nearest-even bits of a finite float, in the upper half.
__device__ inline unsigned rne_bf16_bits(float x) {
  unsigned u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
}

// Four fp8 (OCP E4M3) bytes -> four bf16 (exact) in two dwords.
struct Dw2 {
  unsigned lo, hi;
};
__device__ inline Dw2 fp8x4_to_bf16x4(unsigned w) {
  auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  return Dw2{pack_hi16(f01[0], f01[1]), pack_hi16(f23[0], f23[1])};
}

__device__ inline u32x4 load16(const void* p) { return *static_cast<const u32x4*>(p); }

template <int D, bool FP8>
struct PageRegs {
  static constexpr int KS = D / 32;                    // k-steps of the score MFMA
  static constexpr int KL = FP8 ? KS / 2 : KS;         // 16-byte K loads per page
  static constexpr int VL = FP8 ? D / 64 : D / 32;     // 16-byte V loads per page
  u32x4 k[2][KL];
  u32x4 v[2][VL];
  int id[2];
  bool has_y;
};

// Inclusive-exclusive prefix of pages per sequence into s_cum[0..batch].
__device__ void page_prefix(const VerifyParams& P, int* s_cum, int* s_tmp) {
  const int tid = threadIdx.x;
  const int per = (P.batch + kThreads - 1) / kThreads;
  const int b0 = min(P.batch, tid * per), b1 = min(P.batch, b0 + per);
  int local = 0;
  for (int b = b0; b < b1; ++b) {
    const int row = P.batch_slots ? P.batch_slots[b] : b;
    local += (P.seq_lens[row] + 15) >> 4;
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
    const int row = P.batch_slots ? P.batch_slots[b] : b;
    run += (P.seq_lens[row] + 15) >> 4;
  }
  if (tid == kThreads - 1) s_cum[P.batch] = s_tmp[tid];
  __syncthreads();
}

__device__ inline long range_lo(long w, long W, long n) { return w * W / n; }

template <int D, int NT, bool FP8, bool TREE>
__device__ void process_segment(const VerifyParams& P, int b, int g, int p0, int p1, bool full,
                                int slot, float* s_red, float* s_m, float* s_l) {
  using Regs = PageRegs<D, FP8>;
  constexpr int KS = Regs::KS;
  constexpr int DT = D / 16;
  constexpr int RP = D + 4;                       // padded LDS row
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m16 = lane & 15, jg = lane >> 4;
  const int row_b = P.batch_slots ? P.batch_slots[b] : b;
  const int N = P.seq_lens[row_b];
  const int L = N - P.n_q;
  const int* bt = P.block_table + long(row_b) * P.bt_stride;
  const unsigned lane_off = unsigned(m16 * 64 + jg * 16);

  // Q fragments (B operand of S^T = K Q^T): row 16nt+m16, channels (D/4)jg + 8s .. +7.
  u32x4 qf[NT][KS];
  int qi[NT];                      // verification slot of the row (padding rows: 64)
  unsigned long long anc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + m16;
    qi[nt] = 64;
    anc[nt] = ~0ull;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[nt][s] = u32x4{0, 0, 0, 0};
    if (r < P.rows) {
      const int i = r / P.G, h = g * P.G + r % P.G;
      qi[nt] = i;
      const unsigned short* qp = static_cast<const unsigned short*>(P.q) +
                                 (long(b * P.n_q + i) * P.Hq + h) * D + (D / 4) * jg;
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[nt][s] = load16(qp + 8 * s);
      if (TREE) anc[nt] = P.anc[long(b) * P.n_q + i];
    }
  }

  float m_run[NT], l_run[NT];
  f32x4 acc[DT][NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = kNegInf;
    l_run[nt] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt][nt] = f32x4{0, 0, 0, 0};
  }

  const char* kbase = P.k_pages + long(g) * P.slab_bytes;
  const char* vbase = P.v_pages + long(g) * P.slab_bytes;
  const long page_stride = long(P.Hkv) * P.slab_bytes;
  const int npairs = (p1 - p0 + 1) >> 1;

  auto load_pair = [&](Regs& R, int q) {
    const int px = p0 + 2 * q;
    R.has_y = px + 1 < p1;
    R.id[0] = bt[px];
    R.id[1] = R.has_y ? bt[px + 1] : R.id[0];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const char* kp = kbase + R.id[x] * page_stride + lane_off;
      const char* vp = vbase + R.id[x] * page_stride + lane_off;
      if (x == 1 && !R.has_y) {
#pragma unroll
        for (int u = 0; u < Regs::KL; ++u) R.k[1][u] = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < Regs::VL; ++c) R.v[1][c] = u32x4{0, 0, 0, 0};
      } else {
#pragma unroll
        for (int u = 0; u < Regs::KL; ++u) R.k[x][u] = load16(kp + u * 1024);
#pragma unroll
        for (int c = 0; c < Regs::VL; ++c) R.v[x][c] = load16(vp + c * 1024);
      }
    }
  };

  auto compute_pair = [&](Regs& R, int q) {
    const int px = p0 + 2 * q;
    const int tok0 = px * 16;                   // first token of page X
    const bool need_mask = tok0 + 32 > L;       // pair reaches the verification slots or the end

    // scores S^T (lane: row 16nt+m16, tokens 4jg..4jg+3 of each page)
    f32x4 sc[2][NT];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4 a = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          u32x4 kf;
          if (FP8) {
            const u32x4 w = R.k[x][s >> 1];
            const int o = (s & 1) * 2;
            const Dw2 a0 = fp8x4_to_bf16x4(w[o]), a1 = fp8x4_to_bf16x4(w[o + 1]);
            kf = u32x4{a0.lo, a0.hi, a1.lo, a1.hi};
          } else {
            kf = R.k[x][s];
          }
          a = mfma_bf16(kf, qf[nt][s], a);
        }
        sc[x][nt] = a;
      }
    }
    float ksc[2] = {P.scale_log2, P.scale_log2};
    float vsc[2] = {1.0f, 1.0f};
    if (FP8) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        ksc[x] *= P.k_scale[long(R.id[x]) * P.Hkv + g];
        vsc[x] = P.v_scale[long(R.id[x]) * P.Hkv + g];
      }
    }
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[x][nt][e] *= ksc[x];

    if (need_mask || !R.has_y) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = tok0 + 16 * x + 4 * jg + e;
          const int j = t - L;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            bool vis;
            if (TREE) vis = (t < L) || (t < N && ((anc[nt] >> (j & 63)) & 1ull));
            else vis = (t < L) || (t < N && j <= qi[nt]);
            if (x == 1 && !R.has_y) vis = false;
            sc[x][nt][e] = vis ? sc[x][nt][e] : kNegInf;
          }
        }
      }
      // zero V of tokens at or past N (stale slots may hold anything)
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int valid = (x == 1 && !R.has_y) ? 0 : min(4, max(0, N - (tok0 + 16 * x + 4 * jg)));
        if (FP8) {
          const unsigned keep = valid >= 4 ? 0xFFFFFFFFu : ((1u << (8 * valid)) - 1u);
#pragma unroll
          for (int c = 0; c < Regs::VL; ++c)
#pragma unroll
            for (int w = 0; w < 4; ++w) R.v[x][c][w] &= keep;
        } else {
          const unsigned keep0 = valid >= 2 ? 0xFFFFFFFFu : (valid == 1 ? 0xFFFFu : 0u);
          const unsigned keep1 = valid >= 4 ? 0xFFFFFFFFu : (valid == 3 ? 0xFFFFu : 0u);
#pragma unroll
          for (int c = 0; c < Regs::VL; ++c) {
            R.v[x][c][0] &= keep0;
            R.v[x][c][1] &= keep1;
            R.v[x][c][2] &= keep0;
            R.v[x][c][3] &= keep1;
          }
        }
      }
    }

    // online softmax (base 2) and P^T operands
    u32x4 phi[NT], plo[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float mx = fmaxf(fmaxf(fmaxf(sc[0][nt][0], sc[0][nt][1]), fmaxf(sc[0][nt][2], sc[0][nt][3])),
                       fmaxf(fmaxf(sc[1][nt][0], sc[1][nt][1]), fmaxf(sc[1][nt][2], sc[1][nt][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[nt], mx);
      const float m_ref = m_new == kNegInf ? 0.0f : m_new;
      const float alpha = exp2_fast(m_run[nt] - m_ref);
      m_run[nt] = m_new;
      float p[2][4];
      float psum = 0.0f;
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[x][e] = exp2_fast(sc[x][nt][e] - m_ref);
          psum += p[x][e];
        }
      l_run[nt] = l_run[nt] * alpha + psum;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt][nt] *= alpha;
      if (FP8) {
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int e = 0; e < 4; ++e) p[x][e] *= vsc[x];
      }
      float hi[2][4], lo[2][4];
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hi[x][e] = __uint_as_float(__float_as_uint(p[x][e]) & 0xFFFF0000u);
          lo[x][e] = __uint_as_float(rne_bf16_bits(p[x][e] - hi[x][e]));
        }
      phi[nt] = u32x4{pack_hi16(hi[0][0], hi[0][1]), pack_hi16(hi[0][2], hi[0][3]),
                      pack_hi16(hi[1][0], hi[1][1]), pack_hi16(hi[1][2], hi[1][3])};
      plo[nt] = u32x4{pack_hi16(lo[0][0], lo[0][1]), pack_hi16(lo[0][2], lo[0][3]),
                      pack_hi16(lo[1][0], lo[1][1]), pack_hi16(lo[1][2], lo[1][3])};
    }

    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      u32x4 vf;
      if (FP8) {
        const int c = dt >> 2, w = dt & 3;
        const Dw2 a0 = fp8x4_to_bf16x4(R.v[0][c][w]), a1 = fp8x4_to_bf16x4(R.v[1][c][w]);
        vf = u32x4{a0.lo, a0.hi, a1.lo, a1.hi};
      } else {
        const int c = dt >> 1, w = (dt & 1) * 2;
        vf = u32x4{R.v[0][c][w], R.v[0][c][w + 1], R.v[1][c][w], R.v[1][c][w + 1]};
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        acc[dt][nt] = mfma_bf16(vf, phi[nt], acc[dt][nt]);
        acc[dt][nt] = mfma_bf16(vf, plo[nt], acc[dt][nt]);
      }
    }
  };

  // software pipeline: the next pair's loads are in flight while a pair is
  // computed; two register sets alternate so nothing is copied
  int q = wave;
  Regs ra, rb;
  if (q < npairs) load_pair(ra, q);
  while (q < npairs) {
    if (q + kWaves < npairs) load_pair(rb, q + kWaves);
    compute_pair(ra, q);
    q += kWaves;
    if (q >= npairs) break;
    if (q + kWaves < npairs) load_pair(ra, q + kWaves);
    compute_pair(rb, q);
    q += kWaves;
  }

  // ---- combine the four waves ---------------------------------------------
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    l_run[nt] += __shfl_xor(l_run[nt], 16, 64);
    l_run[nt] += __shfl_xor(l_run[nt], 32, 64);
  }
  __syncthreads();                              // previous segment's LDS readers are done
  if (jg == 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      s_m[wave * 64 + nt * 16 + m16] = m_run[nt];
      s_l[wave * 64 + nt * 16 + m16] = l_run[nt];
    }
  }
  __syncthreads();
  const long slot_floats = long(NT) * 16 * (D + 2);
  float* part = P.part + (long(blockIdx.x) * 2 + slot) * slot_floats;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + m16;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w * 64 + r]);
    const float Mref = M == kNegInf ? 0.0f : M;
    const float f = exp2_fast(m_run[nt] - Mref);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ch = FP8 ? (dt >> 2) * 64 + 16 * jg + 4 * e + (dt & 3)
                           : (dt >> 1) * 32 + 8 * jg + 2 * e + (dt & 1);
        s_red[(wave * 16 + m16) * RP + ch] = acc[dt][nt][e] * f;
      }
    __syncthreads();
    for (int idx = tid; idx < 16 * D; idx += kThreads) {
      const int rr = idx / D, ch = idx % D, rw = nt * 16 + rr;
      if (rw < P.rows) {
        float Mr = kNegInf;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) Mr = fmaxf(Mr, s_m[w * 64 + rw]);
        const float Mrr = Mr == kNegInf ? 0.0f : Mr;
        float Lr = 0.0f, o = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          Lr += s_l[w * 64 + rw] * exp2_fast(s_m[w * 64 + rw] - Mrr);
          o += s_red[(w * 16 + rr) * RP + ch];
        }
        if (full) {
          const int i = rw / P.G, h = g * P.G + rw % P.G;
          const long oi = long(b * P.n_q + i) * P.Hq + h;
          P.out[oi * D + ch] = o / Lr;
          if (ch == 0 && P.lse) P.lse[oi] = (Mr + __log2f(Lr)) * kLn2;
        } else {
          part[rw * D + ch] = o;
          if (ch == 0) {
            part[NT * 16 * D + rw] = Mr;
            part[NT * 16 * D + NT * 16 + rw] = Lr;
          }
        }
      }
    }
    __syncthreads();
  }
}

template <int D, int NT, bool FP8, bool TREE>
__global__ __launch_bounds__(kThreads) void verify_partial_kernel(VerifyParams P) {
  extern __shared__ float smem[];
  int* s_cum = reinterpret_cast<int*>(smem);
  const int cum_words = (P.batch + 1 + 3) & ~3;
  float* s_red = smem + cum_words;
  float* s_m = s_red + kWaves * 16 * (D + 4);
  float* s_l = s_m + kWaves * 64;

  page_prefix(P, s_cum, reinterpret_cast<int*>(s_red));
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= P.batch; i += kThreads) P.cum_ws[i] = s_cum[i];

  const long W = long(P.Hkv) * s_cum[P.batch];
  const long lo = range_lo(blockIdx.x, W, P.n_wg), hi = range_lo(blockIdx.x + 1, W, P.n_wg);
  long pos = lo;
  while (pos < hi) {
    // sequence b: last b with Hkv * cum[b] <= pos
    int a = 0, z = P.batch - 1;
    while (a < z) {
      const int mid = (a + z + 1) >> 1;
      if (long(P.Hkv) * s_cum[mid] <= pos) a = mid;
      else z = mid - 1;
    }
    const int b = a;
    const int np = s_cum[b + 1] - s_cum[b];
    const long base = long(P.Hkv) * s_cum[b];
    const int g = int((pos - base) / np);
    const int p0 = int((pos - base) % np);
    const long seg_end = min(hi, base + long(g + 1) * np);
    const int p1 = p0 + int(seg_end - pos);
    process_segment<D, NT, FP8, TREE>(P, b, g, p0, p1, p0 == 0 && p1 == np, pos == lo ? 0 : 1,
                                      s_red, s_m, s_l);
    pos = seg_end;
  }
}

// Workgroup whose range holds work position p (lo(w) <= p < lo(w+1)).
__device__ inline int owner_of(long p, long W, int n) {
  int w = int(p * n / W);
  while (w + 1 < n && range_lo(w + 1, W, n) <= p) ++w;
  while (w > 0 && range_lo(w, W, n) > p) --w;
  return w;
}

template <int D, int NT>
__global__ __launch_bounds__(256) void verify_merge_kernel(VerifyParams P) {
  const int b = blockIdx.x / P.Hkv, g = blockIdx.x % P.Hkv;
  const int* cum = P.cum_ws;
  const long W = long(P.Hkv) * cum[P.batch];
  const int np = cum[b + 1] - cum[b];
  if (np == 0 || W == 0) return;
  const long u0 = long(P.Hkv) * cum[b] + long(g) * np, u1 = u0 + np;
  const int wf = owner_of(u0, W, P.n_wg), wl = owner_of(u1 - 1, W, P.n_wg);
  if (wf == wl) return;                       // finished in place by one workgroup
  const long slot_floats = long(NT) * 16 * (D + 2);
  const int RW = NT * 16;
  for (int idx = threadIdx.x; idx < P.rows * D; idx += blockDim.x) {
    const int r = idx / D, ch = idx % D;
    float M = kNegInf;
    for (int w = wf; w <= wl; ++w) {
      if (range_lo(w + 1, W, P.n_wg) == range_lo(w, W, P.n_wg)) continue;   // empty range
      const int slot = (w == wf && range_lo(w, W, P.n_wg) != u0) ? 1 : 0;
      const float* pt = P.part + (long(w) * 2 + slot) * slot_floats;
      M = fmaxf(M, pt[RW * D + r]);
    }
    const float Mref = M == kNegInf ? 0.0f : M;
    float Ls = 0.0f, o = 0.0f;
    for (int w = wf; w <= wl; ++w) {
      if (range_lo(w + 1, W, P.n_wg) == range_lo(w, W, P.n_wg)) continue;
      const int slot = (w == wf && range_lo(w, W, P.n_wg) != u0) ? 1 : 0;
      const float* pt = P.part + (long(w) * 2 + slot) * slot_floats;
      const float f = exp2_fast(pt[RW * D + r] - Mref);
      Ls += pt[RW * D + RW + r] * f;
      o += pt[r * D + ch] * f;
    }
    const int i = r / P.G, h = g * P.G + r % P.G;
    const long oi = long(b * P.n_q + i) * P.Hq + h;
    P.out[oi * D + ch] = o / Ls;
    if (ch == 0 && P.lse) P.lse[oi] = (M + __log2f(Ls)) * kLn2;
  }
}

// fp32 K/V (plain [token][channel] pages): one workgroup per (query head,
// sequence), VALU arithmetic, no split.  Meant for small fp32 problems.
template <int D>
__global__ __launch_bounds__(128) void verify_f32_kernel(VerifyParams P) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int g = h / P.G;
  const int row_b = P.batch_slots ? P.batch_slots[b] : b;
  const int N = P.seq_lens[row_b], L = N - P.n_q;
  const int* bt = P.block_table + long(row_b) * P.bt_stride;
  __shared__ float s_q[D];
  __shared__ float s_p[128];
  __shared__ float s_red[2];
  const float scale = P.scale_log2;
  for (int i = 0; i < P.n_q; ++i) {
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

struct DeviceInfo {
  int cus = 0;
};

DeviceInfo device_info() {
  static thread_local int cached_dev = -1;
  static thread_local DeviceInfo info;
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev != cached_dev) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    info.cus = cus;
    cached_dev = dev;
  }
  return info;
}

template <int D, int NT>
size_t partial_smem(int batch) {
  const int cum_words = (batch + 1 + 3) & ~3;
  return size_t(cum_words + kWaves * 16 * (D + 4) + 2 * kWaves * 64) * sizeof(float);
}

struct Plan {
  int D, NT, rows, n_wg;
  bool fp8, tree, f32;
  size_t cum_bytes, part_bytes;
};

pkv_status make_plan(const pkv_verify_args* a, Plan* pl) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "null args");
  if (a->batch < 1 || a->batch > 4096) return fail(PKV_ERR_INVALID_ARG, "batch must be in [1, 4096]");
  if (a->n_q < 1 || a->n_q > 64) return fail(PKV_ERR_INVALID_ARG, "n_q must be in [1, 64]");
  if (a->num_kv_heads < 1 || a->num_q_heads < a->num_kv_heads || a->num_q_heads % a->num_kv_heads)
    return fail(PKV_ERR_INVALID_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
  if (a->page_size != kPageSize) return fail(PKV_ERR_UNSUPPORTED, "page_size must be 16");
  if (a->head_dim != 64 && a->head_dim != 128) return fail(PKV_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (a->block_table_stride < 1) return fail(PKV_ERR_INVALID_ARG, "block_table_stride must be >= 1");
  if (!a->q || !a->k_pages || !a->v_pages || !a->block_table || !a->seq_lens)
    return fail(PKV_ERR_INVALID_ARG, "null device pointer");
  const int G = a->num_q_heads / a->num_kv_heads;
  pl->D = a->head_dim;
  pl->rows = a->n_q * G;
  pl->tree = a->anc_mask != nullptr;
  pl->f32 = false;
  pl->fp8 = false;
  if (a->kv_dtype == PKV_F32) {
    if (a->q_dtype != PKV_F32) return fail(PKV_ERR_INVALID_ARG, "fp32 KV needs fp32 queries");
    pl->f32 = true;
  } else if (a->kv_dtype == PKV_BF16 || a->kv_dtype == PKV_FP8_E4M3) {
    if (a->q_dtype != PKV_BF16) return fail(PKV_ERR_INVALID_ARG, "bf16/fp8 KV needs bf16 queries");
    pl->fp8 = a->kv_dtype == PKV_FP8_E4M3;
    if (pl->fp8 && (!a->k_scale || !a->v_scale)) return fail(PKV_ERR_INVALID_ARG, "FP8 KV needs scales");
    if (pl->rows > 64) return fail(PKV_ERR_UNSUPPORTED, "n_q * Hq/Hkv must be <= 64");
  } else {
    return fail(PKV_ERR_INVALID_ARG, "unknown dtype");
  }
  pl->NT = (pl->rows + 15) / 16;
  if (a->num_splits < 0) return fail(PKV_ERR_INVALID_ARG, "num_splits must be >= 0");
  pl->cum_bytes = 0;
  pl->part_bytes = 0;
  pl->n_wg = 0;
  if (!pl->f32) {
    int n = a->num_splits;
    if (n == 0) n = device_info().cus * 2;
    pl->n_wg = n;
    pl->cum_bytes = ((size_t(a->batch) + 1) * sizeof(int) + 255) & ~size_t(255);
    pl->part_bytes = size_t(n) * 2 * pl->NT * 16 * (pl->D + 2) * sizeof(float);
  }
  return PKV_OK;
}

template <int D, int NT, bool FP8, bool TREE>
hipError_t launch_split(const VerifyParams& p, hipStream_t st) {
  const size_t smem = partial_smem<D, NT>(p.batch);
  hipLaunchKernelGGL((verify_partial_kernel<D, NT, FP8, TREE>), dim3(p.n_wg), dim3(kThreads), smem, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((verify_merge_kernel<D, NT>), dim3(p.batch * p.Hkv), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <int D, int NT>
hipError_t dispatch_kv(const VerifyParams& p, bool fp8, bool tree, hipStream_t st) {
  if (fp8) return tree ? launch_split<D, NT, true, true>(p, st) : launch_split<D, NT, true, false>(p, st);
  return tree ? launch_split<D, NT, false, true>(p, st) : launch_split<D, NT, false, false>(p, st);
}

template <int D>
hipError_t dispatch_nt(const VerifyParams& p, int NT, bool fp8, bool tree, hipStream_t st) {
  switch (NT) {
    case 1: return dispatch_kv<D, 1>(p, fp8, tree, st);
    case 2: return dispatch_kv<D, 2>(p, fp8, tree, st);
    case 3: return dispatch_kv<D, 3>(p, fp8, tree, st);
    default: return dispatch_kv<D, 4>(p, fp8, tree, st);
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
  *bytes_out = pl.cum_bytes + pl.part_bytes;
  return PKV_OK;
}

extern "C" pkv_status spec_verify_attention(const pkv_verify_args* a, void* stream) {
  Plan pl;
  pkv_status st = make_plan(a, &pl);
  if (st != PKV_OK) return st;
  if (!a->out) return fail(PKV_ERR_INVALID_ARG, "null output pointer");
  const size_t need = pl.cum_bytes + pl.part_bytes;
  if (need > 0 && (!a->workspace || a->workspace_bytes < need))
    return fail(PKV_ERR_WORKSPACE, "workspace smaller than spec_verify_workspace_size");
  VerifyParams p{};
  p.q = a->q;
  p.k_pages = static_cast<const char*>(a->k_pages);
  p.v_pages = static_cast<const char*>(a->v_pages);
  p.k_scale = a->k_scale;
  p.v_scale = a->v_scale;
  p.block_table = a->block_table;
  p.seq_lens = a->seq_lens;
  p.batch_slots = a->batch_slots;
  p.anc = reinterpret_cast<const unsigned long long*>(a->anc_mask);
  p.out = a->out;
  p.lse = a->lse;
  p.cum_ws = static_cast<int*>(a->workspace);
  p.part = reinterpret_cast<float*>(static_cast<char*>(a->workspace) + pl.cum_bytes);
  p.slab_bytes = pkv_page_bytes(a->kv_dtype, a->page_size, a->head_dim);
  p.batch = a->batch;
  p.n_q = a->n_q;
  p.Hq = a->num_q_heads;
  p.Hkv = a->num_kv_heads;
  p.G = a->num_q_heads / a->num_kv_heads;
  p.rows = pl.rows;
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
  } else if (pl.D == 64) {
    e = dispatch_nt<64>(p, pl.NT, pl.fp8, pl.tree, s);
  } else {
    e = dispatch_nt<128>(p, pl.NT, pl.fp8, pl.tree, s);
  }
  if (e != hipSuccess) return fail(PKV_ERR_DEVICE, std::string("verify launch: ") + hipGetErrorString(e));
  return PKV_OK;
}
