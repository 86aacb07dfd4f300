// Speculative acceptance: accepted length and next token (gfx950).
//
// Rule (innvotechnologies.co, section "Verification Acceptance
// Probabilities and Speedup Math", eq. alpha_i): draft token x_i is accepted
// with probability min(1, P_i(x_i) / Q_i(x_i)); the accepted length k is the
// number of leading accepts.  On a rejection at position k the next token is
// drawn from max(0, P_k - Q_k) (the resample of the pipeline diagram, which
// keeps the target distribution exact); after gamma accepts it is drawn from
// P_gamma (the bonus token).
//
// The work is one pass over every logit row (the normalisers) and one pass
// over the row pair the draw needs, each cut into chunks of logits so
// that a launch holds thousands of workgroups with every load of a thread in
// flight at once:
//  1. stats: workgroup (row, chunk) reduces max and sum(exp) of its chunk
//     (8192 logits, eight 16-byte loads per thread, all in flight);
//  2. draw: workgroup (sequence, chunk of 2048) combines the row partials into log
//     normalisers, runs the gamma acceptance tests in one wave (lane i tests
//     draft i), and computes its chunk's Gumbel-max candidate for the token
//     drawn at position k (residual, or bonus when k = gamma);
//  3. finish: one wave per sequence takes the best candidate.
// Uniforms are Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) keyed by the
// 64-bit seed; counters are documented in pkv_spec.h.  Drawing by argmax of
// Gumbel-perturbed log weights needs no prefix sum over the vocabulary and its
// outcome is an argmax, stable under rounding differences.  Keys are kept in
// base-2 units (every key of one draw scaled by 1/ln 2 and shifted by one
// constant), which leaves the argmax unchanged.

#include <hip/hip_runtime.h>

#include "../common.h"
#include "sampling.h"

namespace pkv {

namespace {

using namespace sampling;

constexpr int kWaves = kThreads / 64;
constexpr int kStatsQuads = 8;                            // 16-byte loads per thread
constexpr int kStatsChunk = kThreads * kStatsQuads * 4;   // logits per stats workgroup
constexpr int kDrawQuads = 2;
constexpr int kDrawChunk = kThreads * kDrawQuads * 4;     // logits per draw workgroup
constexpr int kMaxVocab = 1 << 26;
constexpr int kMaxBatch = 1 << 20;

struct AcceptParams {
  const float* T;
  const float* Dl;
  const int* tokens;
  const int* gammas;   // [batch] drafts per sequence, or null (gamma for all)
  const unsigned* step_ptr;  // device step counter, or null (step below)
  int* accepted_len;
  int* next_token;
  float2* stats;       // [batch][2*gamma+1][schunks] (max, sum exp) in base 2
  int4* cand;          // [batch][dchunks] (residual key bits, index, fallback key bits, index)
  int batch, gamma, vocab, schunks, dchunks;
  unsigned k0, k1, step;
};

__device__ inline const float* row_ptr(const AcceptParams& P, int b, int j) {
  return j <= P.gamma ? P.T + (long(b) * (P.gamma + 1) + j) * P.vocab
                      : P.Dl + (long(b) * P.gamma + (j - P.gamma - 1)) * P.vocab;
}

template <bool kAligned>
__global__ __launch_bounds__(kThreads) void accept_stats_kernel(AcceptParams P) {
  const int chunk = blockIdx.x % P.schunks;
  const int r = blockIdx.x / P.schunks;  // b * (2 gamma + 1) + j
  const int rows_per_seq = 2 * P.gamma + 1;
  const int b = r / rows_per_seq, j = r % rows_per_seq;
  if (P.gammas) {                                // rows past the sequence's drafts are never used
    const int gb = min(max(P.gammas[b], 1), P.gamma);
    if (j <= P.gamma ? j > gb : j - P.gamma - 1 >= gb) return;
  }
  const float* row = row_ptr(P, b, j);
  float v[kStatsQuads][4];
  load_chunk<kAligned, kStatsQuads, true>(row, P.vocab, chunk * (kStatsChunk / 4), v);
  float m = kNegInf;
#pragma unroll
  for (int u = 0; u < kStatsQuads; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) m = fmaxf(m, v[u][e]);
  m *= kLog2e;
  float s = 0.0f;
  if (m > kNegInf) {
#pragma unroll
    for (int u = 0; u < kStatsQuads; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) s += exp2_hw(__builtin_fmaf(v[u][e], kLog2e, -m));
  }
  for (int o = 32; o > 0; o >>= 1) combine_ms(m, s, __shfl_xor(m, o, 64), __shfl_xor(s, o, 64));
  __shared__ float sm[kWaves], ss[kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sm[wave] = m;
    ss[wave] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kWaves; ++w) combine_ms(m, s, sm[w], ss[w]);
    P.stats[long(r) * P.schunks + chunk] = make_float2(m, s);
  }
}

// Gumbel-max candidate of this thread over its quads of row k: the fallback
// (bonus) key log2 P_k(x) + g(x) and, with kResidual, the residual key
// log2 max(0, P_k - Q_k)(x) + g(x).  Branch-free per logit.
template <bool kResidual>
__device__ inline void draw_quads(const float (&tv)[kDrawQuads][4], const float (&dv)[kDrawQuads][4],
                                  int q0, int b, unsigned step, unsigned c3, float lt, float ld,
                                  const AcceptParams& P,
                                  float& rk, int& ri, float& fk, int& fi) {
#pragma unroll
  for (int u = 0; u < kDrawQuads; ++u) {
    const int q = q0 + u * kThreads + int(threadIdx.x);
    const Philox4 r = philox4x32_10(unsigned(q), unsigned(b), step, c3, P.k0, P.k1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int x = q * 4 + e;
      const float g = gumbel2(uniform01(r.x[e]));
      const float a = __builtin_fmaf(tv[u][e], kLog2e, -lt);  // log2 P_k(x); -inf past the row
      better(fk, fi, a + g, x);
      if (kResidual) {
        const float c = __builtin_fmaf(dv[u][e], kLog2e, -ld);  // log2 Q_k(x)
        // log2 max(0, P - Q) = a + log2(1 - 2^(c - a)) where P > Q
        const float key = a > c ? a + log2_one_minus_exp2(c - a) + g : kNegInf;
        better(rk, ri, key, x);
      }
    }
  }
}

template <bool kAligned>
__global__ __launch_bounds__(kThreads) void accept_draw_kernel(AcceptParams P) {
  const unsigned step = P.step_ptr ? *P.step_ptr : P.step;
  const int chunk = blockIdx.x % P.dchunks;
  const int b = blockIdx.x / P.dchunks;
  const int rows_per_seq = 2 * P.gamma + 1;
  __shared__ float s_lse[2 * 64 + 1];  // base-2 log normaliser per row
  __shared__ int s_k;
  __shared__ float sk[2][kWaves];
  __shared__ int si[2][kWaves];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int gb = P.gammas ? min(max(P.gammas[b], 1), P.gamma) : P.gamma;
  // wave 0, lane i < gamma: the logits of draft token x_i (independent of the
  // normalisers, so issued first)
  int x = -1;
  float tx = 0.0f, dx = 0.0f;
  if (t < P.gamma) {
    x = P.tokens[long(b) * P.gamma + t];
    if (x >= 0 && x < P.vocab) {
      tx = P.T[(long(b) * (P.gamma + 1) + t) * P.vocab + x];
      dx = P.Dl[(long(b) * P.gamma + t) * P.vocab + x];
    }
  }
  // log normalisers of the sequence's rows from the chunk partials.  Up to
  // 16 partials per row (vocabularies up to 16 stats chunks): each 16-lane
  // group of a wave reduces one row, lane l16 holding chunk l16, so a wave
  // covers four rows in four shuffle steps (waves 0.. take rows 4w .. 4w+3).
  // Otherwise wave w takes rows w, w + 4, ... four at a time, lane c chunks
  // c, c + 64, ...
  const float2* st = P.stats + long(b) * rows_per_seq * P.schunks;
  if (P.schunks <= 16) {
    const int r = 4 * wave + (lane >> 4), c = lane & 15;
    float2 v = r < rows_per_seq && c < P.schunks ? st[long(r) * P.schunks + c] : make_float2(kNegInf, 0.0f);
    for (int o = 8; o > 0; o >>= 1) combine_ms(v.x, v.y, __shfl_xor(v.x, o, 64), __shfl_xor(v.y, o, 64));
    if (c == 0 && r < rows_per_seq) s_lse[r] = v.x + log2_hw(v.y);
    for (int r1 = 4 * kWaves + wave; r1 < rows_per_seq; r1 += kWaves) {   // rows past 4 per wave
      float m = kNegInf, sm = 0.0f;
      if (lane < P.schunks) {
        const float2 w = st[long(r1) * P.schunks + lane];
        m = w.x;
        sm = w.y;
      }
      for (int o = 8; o > 0; o >>= 1) combine_ms(m, sm, __shfl_xor(m, o, 64), __shfl_xor(sm, o, 64));
      if (lane == 0) s_lse[r1] = m + log2_hw(sm);
    }
  } else
  for (int r0 = wave; r0 < rows_per_seq; r0 += 4 * kWaves) {
    float m[4], sm[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m[j] = kNegInf;
      sm[j] = 0.0f;
    }
    for (int c = lane; c < P.schunks; c += 64) {
      float2 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = r0 + j * kWaves;
        v[j] = r < rows_per_seq ? st[long(r) * P.schunks + c] : make_float2(kNegInf, 0.0f);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) combine_ms(m[j], sm[j], v[j].x, v[j].y);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      for (int o = 32; o > 0; o >>= 1)
        combine_ms(m[j], sm[j], __shfl_xor(m[j], o, 64), __shfl_xor(sm[j], o, 64));
      const int r = r0 + j * kWaves;
      if (lane == 0 && r < rows_per_seq) s_lse[r] = m[j] + log2_hw(sm[j]);
    }
  }
  __syncthreads();
  if (wave == 0) {
    // lane i tests draft i: accept iff u_i < min(1, P_i(x_i) / Q_i(x_i)); an
    // out-of-range token is rejected
    bool reject = false;
    if (t < P.gamma) {
      if (x < 0 || x >= P.vocab) {
        reject = true;
      } else {
        const float lp = tx * kLog2e - s_lse[t];
        const float lq = dx * kLog2e - s_lse[P.gamma + 1 + t];
        const float d = lp - lq;
        const float acc = d >= 0.0f ? 1.0f : exp2_hw(d);
        const Philox4 r = philox4x32_10(0u, unsigned(b), step, unsigned(t) | (kPurposeAccept << 16),
                                        P.k0, P.k1);
        reject = !(uniform01(r.x[0]) < acc);
      }
    }
    // a sequence with fewer drafts stops at its count
    const unsigned long long rej = __ballot(reject || (t >= gb && t < P.gamma));
    if (t == 0) s_k = rej ? __builtin_ctzll(rej) : P.gamma;
  }
  __syncthreads();
  const int k = s_k;
  if (chunk == 0 && t == 0) P.accepted_len[b] = k;
  const bool residual = k < gb;
  const float lt = s_lse[k], ld = residual ? s_lse[P.gamma + 1 + k] : 0.0f;
  const int q0 = chunk * (kDrawChunk / 4);
  float tv[kDrawQuads][4], dv[kDrawQuads][4];
  float rk = kNegInf, fk = kNegInf;
  int ri = 0x7FFFFFFF, fi = 0x7FFFFFFF;
  const unsigned c3 = unsigned(k) | (kPurposeSample << 16);
  load_chunk<kAligned, kDrawQuads>(row_ptr(P, b, k), P.vocab, q0, tv);
  if (residual) {
    load_chunk<kAligned, kDrawQuads>(row_ptr(P, b, P.gamma + 1 + k), P.vocab, q0, dv);
    draw_quads<true>(tv, dv, q0, b, step, c3, lt, ld, P, rk, ri, fk, fi);
  } else {
    draw_quads<false>(tv, dv, q0, b, step, c3, lt, ld, P, rk, ri, fk, fi);
  }
  for (int o = 32; o > 0; o >>= 1) {
    better(rk, ri, __shfl_xor(rk, o, 64), __shfl_xor(ri, o, 64));
    better(fk, fi, __shfl_xor(fk, o, 64), __shfl_xor(fi, o, 64));
  }
  if (lane == 0) {
    sk[0][wave] = rk;
    si[0][wave] = ri;
    sk[1][wave] = fk;
    si[1][wave] = fi;
  }
  __syncthreads();
  if (t == 0) {
    for (int w = 1; w < kWaves; ++w) {
      better(rk, ri, sk[0][w], si[0][w]);
      better(fk, fi, sk[1][w], si[1][w]);
    }
    P.cand[long(b) * P.dchunks + chunk] = make_int4(__float_as_int(rk), ri, __float_as_int(fk), fi);
  }
}

// One wave per sequence: the best candidate over the chunks.
__global__ __launch_bounds__(64) void accept_finish_kernel(AcceptParams P) {
  const int b = blockIdx.x, lane = threadIdx.x;
  float rk = kNegInf, fk = kNegInf;
  int ri = 0x7FFFFFFF, fi = 0x7FFFFFFF;
  for (int c = lane; c < P.dchunks; c += 64) {
    const int4 v = P.cand[long(b) * P.dchunks + c];
    better(rk, ri, __int_as_float(v.x), v.y);
    better(fk, fi, __int_as_float(v.z), v.w);
  }
  for (int o = 32; o > 0; o >>= 1) {
    better(rk, ri, __shfl_xor(rk, o, 64), __shfl_xor(ri, o, 64));
    better(fk, fi, __shfl_xor(fk, o, 64), __shfl_xor(fi, o, 64));
  }
  // residual zero everywhere (or k = gamma): the draw from P_k
  if (lane == 0) P.next_token[b] = rk > kNegInf ? ri : fi;
}

struct WsLayout {
  size_t stats, cand, total;
};

WsLayout ws_layout(const pkv_accept_args* a) {
  const size_t sch = (size_t(a->vocab) + kStatsChunk - 1) / kStatsChunk;
  const size_t dch = (size_t(a->vocab) + kDrawChunk - 1) / kDrawChunk;
  WsLayout w;
  w.stats = 0;
  const size_t stats_bytes = size_t(a->batch) * (2 * a->gamma + 1) * sch * sizeof(float2);
  w.cand = (stats_bytes + 255) & ~size_t(255);
  w.total = w.cand + size_t(a->batch) * dch * sizeof(int4);
  return w;
}

pkv_status check_shape(const pkv_accept_args* a) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "null args");
  if (a->batch < 1 || a->batch > kMaxBatch) return fail(PKV_ERR_INVALID_ARG, "batch must be in [1, 2^20]");
  if (a->gamma < 1 || a->gamma > 64) return fail(PKV_ERR_INVALID_ARG, "gamma must be in [1, 64]");
  if (a->vocab < 1 || a->vocab > kMaxVocab) return fail(PKV_ERR_INVALID_ARG, "vocab must be in [1, 2^26]");
  const long long sch = (a->vocab + kStatsChunk - 1) / kStatsChunk;
  const long long dch = (a->vocab + kDrawChunk - 1) / kDrawChunk;
  if (sch * a->batch * (2 * a->gamma + 1) > 0x7FFFFFFFll || dch * a->batch > 0x7FFFFFFFll)
    return fail(PKV_ERR_INVALID_ARG, "batch * (2 gamma + 1) * vocab too large for one launch");
  return PKV_OK;
}

pkv_status check(const pkv_accept_args* a) {
  pkv_status st = check_shape(a);
  if (st != PKV_OK) return st;
  if (!a->target_logits || !a->draft_logits || !a->draft_tokens || !a->accepted_len || !a->next_token)
    return fail(PKV_ERR_INVALID_ARG, "null device pointer");
  if ((reinterpret_cast<uintptr_t>(a->target_logits) | reinterpret_cast<uintptr_t>(a->draft_logits)) & 15)
    return fail(PKV_ERR_INVALID_ARG, "logit arrays must be 16-byte aligned");
  return PKV_OK;
}

}  // namespace

}  // namespace pkv

using namespace pkv;

extern "C" pkv_status spec_accept_workspace_size(const pkv_accept_args* a, size_t* bytes_out) {
  if (!bytes_out) return fail(PKV_ERR_INVALID_ARG, "null output");
  pkv_status st = check_shape(a);
  if (st != PKV_OK) return st;
  *bytes_out = ws_layout(a).total;
  return PKV_OK;
}

extern "C" pkv_status spec_accept(const pkv_accept_args* a, void* stream) {
  pkv_status st = check(a);
  if (st != PKV_OK) return st;
  const WsLayout w = ws_layout(a);
  if (!a->workspace || a->workspace_bytes < w.total)
    return fail(PKV_ERR_WORKSPACE, "workspace smaller than spec_accept_workspace_size");
  if (reinterpret_cast<uintptr_t>(a->workspace) & 15)
    return fail(PKV_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  AcceptParams p{};
  p.T = a->target_logits;
  p.Dl = a->draft_logits;
  p.tokens = a->draft_tokens;
  p.gammas = a->gammas;
  p.step_ptr = a->step_ptr;
  p.accepted_len = a->accepted_len;
  p.next_token = a->next_token;
  char* ws = static_cast<char*>(a->workspace);
  p.stats = reinterpret_cast<float2*>(ws + w.stats);
  p.cand = reinterpret_cast<int4*>(ws + w.cand);
  p.batch = a->batch;
  p.gamma = a->gamma;
  p.vocab = a->vocab;
  p.schunks = (a->vocab + kStatsChunk - 1) / kStatsChunk;
  p.dchunks = (a->vocab + kDrawChunk - 1) / kDrawChunk;
  p.k0 = unsigned(a->seed & 0xFFFFFFFFu);
  p.k1 = unsigned(a->seed >> 32);
  p.step = a->step;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool aligned = (a->vocab & 3) == 0;
  const unsigned n_stats = unsigned(a->batch) * (2 * a->gamma + 1) * p.schunks;
  const unsigned n_draw = unsigned(a->batch) * p.dchunks;
  if (aligned) hipLaunchKernelGGL(accept_stats_kernel<true>, dim3(n_stats), dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL(accept_stats_kernel<false>, dim3(n_stats), dim3(kThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) {
    if (aligned) hipLaunchKernelGGL(accept_draw_kernel<true>, dim3(n_draw), dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL(accept_draw_kernel<false>, dim3(n_draw), dim3(kThreads), 0, s, p);
    e = hipGetLastError();
  }
  if (e == hipSuccess) {
    hipLaunchKernelGGL(accept_finish_kernel, dim3(a->batch), dim3(64), 0, s, p);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return fail(PKV_ERR_DEVICE, std::string("accept launch: ") + hipGetErrorString(e));
  return PKV_OK;
}
