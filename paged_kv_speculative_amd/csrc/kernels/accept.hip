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
// Two kernels:
//  1. row statistics: one workgroup per logit row (gamma+1 target rows and
//     gamma draft rows per sequence) streams the row once with 16-byte loads
//     and reduces max and sum(exp) to the log-normaliser; the workgroup of
//     target row gamma also draws the bonus token by Gumbel-max;
//  2. decision: one workgroup per sequence computes all gamma acceptance
//     tests, finds k, and if k < gamma streams rows k of target and draft to
//     draw the residual token by Gumbel-max.
// Uniforms are Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) keyed by the
// 64-bit seed; counters are documented in pkv_spec.h.  Drawing by argmax of
// Gumbel-perturbed log weights needs no prefix sum over the vocabulary and its
// outcome is an argmax, stable under rounding differences.

#include <hip/hip_runtime.h>

#include "../common.h"

namespace pkv {

namespace {

constexpr int kThreads = 256;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr unsigned kPurposeAccept = 1u, kPurposeSample = 2u;

struct Philox4 {
  unsigned x[4];
};

__device__ inline Philox4 philox4x32_10(unsigned c0, unsigned c1, unsigned c2, unsigned c3,
                                        unsigned k0, unsigned k1) {
  for (int r = 0; r < 10; ++r) {
    const unsigned lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    const unsigned lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    const unsigned n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return Philox4{{c0, c1, c2, c3}};
}

// u = (floor(w / 2^9) + 1/2) * 2^-23, exact in fp32, in (0, 1).
__device__ inline float uniform01(unsigned w) {
  return (float(w >> 9) + 0.5f) * 1.1920928955078125e-7f;
}

__device__ inline float gumbel(float u) { return -logf(-logf(u)); }

struct AcceptParams {
  const float* T;
  const float* Dl;
  const int* tokens;
  int* accepted_len;
  int* next_token;
  float* lse;          // [batch][2*gamma+1]: target rows 0..gamma, then draft rows
  float* bonus_key;    // [batch]
  int* bonus_tok;      // [batch]
  int batch, gamma, vocab;
  unsigned k0, k1, step;
};

// Block-wide combine of (max, sum) pairs; result valid in all threads.
__device__ inline void combine_ms(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == kNegInf) return;
  s = s * expf(m - mn) + s2 * expf(m2 - mn);
  m = mn;
}

// Block-wide argmax of (key, index): larger key wins, ties to smaller index.
__device__ inline void better(float& k, int& i, float k2, int i2) {
  if (k2 > k || (k2 == k && i2 < i)) {
    k = k2;
    i = i2;
  }
}

__device__ void block_argmax(float& key, int& idx, float* sk, int* si) {
  for (int o = 32; o > 0; o >>= 1) {
    const float k2 = __shfl_xor(key, o, 64);
    const int i2 = __shfl_xor(idx, o, 64);
    better(key, idx, k2, i2);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) {
    sk[wave] = key;
    si[wave] = idx;
  }
  __syncthreads();
  key = sk[0];
  idx = si[0];
  for (int w = 1; w < kThreads / 64; ++w) better(key, idx, sk[w], si[w]);
}

__global__ __launch_bounds__(kThreads) void accept_rowstats_kernel(AcceptParams P) {
  const int rows_per_seq = 2 * P.gamma + 1;
  const int b = blockIdx.x / rows_per_seq, j = blockIdx.x % rows_per_seq;
  const float* row = j <= P.gamma ? P.T + (long(b) * (P.gamma + 1) + j) * P.vocab
                                  : P.Dl + (long(b) * P.gamma + (j - P.gamma - 1)) * P.vocab;
  const bool bonus = j == P.gamma;
  const bool aligned = (P.vocab & 3) == 0;
  float m = kNegInf, s = 0.0f, bk = kNegInf;
  int bi = 0x7FFFFFFF;
  const int nq = (P.vocab + 3) >> 2;
  for (int qd = threadIdx.x; qd < nq; qd += kThreads) {
    float v[4];
    const int x0 = qd * 4;
    if (aligned) {
      const float4 f = reinterpret_cast<const float4*>(row)[qd];
      v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = x0 + e < P.vocab ? row[x0 + e] : kNegInf;
    }
    const float mv = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
    if (mv > m) {
      s *= expf(m - mv);
      m = mv;
    }
    if (m > kNegInf) {
#pragma unroll
      for (int e = 0; e < 4; ++e) s += expf(v[e] - m);
    }
    if (bonus) {
      const Philox4 r = philox4x32_10(unsigned(qd), unsigned(b), P.step,
                                      unsigned(P.gamma) | (kPurposeSample << 16), P.k0, P.k1);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (x0 + e < P.vocab) better(bk, bi, v[e] + gumbel(uniform01(r.x[e])), x0 + e);
    }
  }
  // combine (m, s) across the block
  for (int o = 32; o > 0; o >>= 1) combine_ms(m, s, __shfl_xor(m, o, 64), __shfl_xor(s, o, 64));
  __shared__ float sm[kThreads / 64], ss[kThreads / 64];
  __shared__ float sk[kThreads / 64];
  __shared__ int si[kThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sm[wave] = m;
    ss[wave] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = sm[0], S = ss[0];
    for (int w = 1; w < kThreads / 64; ++w) combine_ms(M, S, sm[w], ss[w]);
    P.lse[long(b) * rows_per_seq + j] = M + logf(S);
  }
  if (bonus) {
    block_argmax(bk, bi, sk, si);
    if (threadIdx.x == 0) {
      P.bonus_key[b] = bk;
      P.bonus_tok[b] = bi;
    }
  }
}

__global__ __launch_bounds__(kThreads) void accept_decide_kernel(AcceptParams P) {
  const int b = blockIdx.x;
  const int rows_per_seq = 2 * P.gamma + 1;
  const float* lse = P.lse + long(b) * rows_per_seq;
  __shared__ int s_k;
  __shared__ float sk[kThreads / 64];
  __shared__ int si[kThreads / 64];
  if (threadIdx.x == 0) {
    int k = P.gamma;
    for (int i = 0; i < P.gamma; ++i) {
      const int x = P.tokens[long(b) * P.gamma + i];
      if (x < 0 || x >= P.vocab) {       // invalid draft token: reject
        k = i;
        break;
      }
      const float lt = P.T[(long(b) * (P.gamma + 1) + i) * P.vocab + x] - lse[i];
      const float ld = P.Dl[(long(b) * P.gamma + i) * P.vocab + x] - lse[P.gamma + 1 + i];
      const float lr = lt - ld;
      const float a = lr >= 0.0f ? 1.0f : expf(lr);
      const Philox4 r = philox4x32_10(0u, unsigned(b), P.step, unsigned(i) | (kPurposeAccept << 16),
                                      P.k0, P.k1);
      if (!(uniform01(r.x[0]) < a)) {
        k = i;
        break;
      }
    }
    s_k = k;
  }
  __syncthreads();
  const int k = s_k;
  if (k == P.gamma) {
    if (threadIdx.x == 0) {
      P.accepted_len[b] = k;
      P.next_token[b] = P.bonus_tok[b];
    }
    return;
  }
  // residual max(0, P_k - Q_k): argmax of log(residual) + Gumbel; fall back to
  // log P_k + Gumbel when the residual is zero everywhere
  const float* trow = P.T + (long(b) * (P.gamma + 1) + k) * P.vocab;
  const float* drow = P.Dl + (long(b) * P.gamma + k) * P.vocab;
  const float lt = lse[k], ld = lse[P.gamma + 1 + k];
  float rk = kNegInf, fk = kNegInf;
  int ri = 0x7FFFFFFF, fi = 0x7FFFFFFF;
  const bool aligned = (P.vocab & 3) == 0;
  const int nq = (P.vocab + 3) >> 2;
  for (int qd = threadIdx.x; qd < nq; qd += kThreads) {
    float tv[4], dv[4];
    const int x0 = qd * 4;
    if (aligned) {
      const float4 a = reinterpret_cast<const float4*>(trow)[qd];
      const float4 c = reinterpret_cast<const float4*>(drow)[qd];
      tv[0] = a.x; tv[1] = a.y; tv[2] = a.z; tv[3] = a.w;
      dv[0] = c.x; dv[1] = c.y; dv[2] = c.z; dv[3] = c.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        tv[e] = x0 + e < P.vocab ? trow[x0 + e] : kNegInf;
        dv[e] = x0 + e < P.vocab ? drow[x0 + e] : kNegInf;
      }
    }
    const Philox4 r = philox4x32_10(unsigned(qd), unsigned(b), P.step,
                                    unsigned(k) | (kPurposeSample << 16), P.k0, P.k1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (x0 + e >= P.vocab) continue;
      const float g = gumbel(uniform01(r.x[e]));
      const float res = expf(tv[e] - lt) - expf(dv[e] - ld);
      if (res > 0.0f) better(rk, ri, logf(res) + g, x0 + e);
      better(fk, fi, tv[e] + g, x0 + e);
    }
  }
  block_argmax(rk, ri, sk, si);
  __syncthreads();
  block_argmax(fk, fi, sk, si);
  if (threadIdx.x == 0) {
    P.accepted_len[b] = k;
    P.next_token[b] = rk > kNegInf ? ri : fi;
  }
}

size_t ws_layout(const pkv_accept_args* a, size_t* off_key, size_t* off_tok) {
  const size_t lse = size_t(a->batch) * (2 * a->gamma + 1) * sizeof(float);
  *off_key = (lse + 255) & ~size_t(255);
  *off_tok = *off_key + ((size_t(a->batch) * sizeof(float) + 255) & ~size_t(255));
  return *off_tok + size_t(a->batch) * sizeof(int);
}

pkv_status check_shape(const pkv_accept_args* a) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "null args");
  if (a->batch < 1) return fail(PKV_ERR_INVALID_ARG, "batch must be >= 1");
  if (a->gamma < 1 || a->gamma > 64) return fail(PKV_ERR_INVALID_ARG, "gamma must be in [1, 64]");
  if (a->vocab < 1) return fail(PKV_ERR_INVALID_ARG, "vocab must be >= 1");
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
  size_t ok, ot;
  *bytes_out = ws_layout(a, &ok, &ot);
  return PKV_OK;
}

extern "C" pkv_status spec_accept(const pkv_accept_args* a, void* stream) {
  pkv_status st = check(a);
  if (st != PKV_OK) return st;
  size_t off_key, off_tok;
  const size_t need = ws_layout(a, &off_key, &off_tok);
  if (!a->workspace || a->workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "workspace smaller than spec_accept_workspace_size");
  AcceptParams p{};
  p.T = a->target_logits;
  p.Dl = a->draft_logits;
  p.tokens = a->draft_tokens;
  p.accepted_len = a->accepted_len;
  p.next_token = a->next_token;
  char* ws = static_cast<char*>(a->workspace);
  p.lse = reinterpret_cast<float*>(ws);
  p.bonus_key = reinterpret_cast<float*>(ws + off_key);
  p.bonus_tok = reinterpret_cast<int*>(ws + off_tok);
  p.batch = a->batch;
  p.gamma = a->gamma;
  p.vocab = a->vocab;
  p.k0 = unsigned(a->seed & 0xFFFFFFFFu);
  p.k1 = unsigned(a->seed >> 32);
  p.step = a->step;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(accept_rowstats_kernel, dim3(a->batch * (2 * a->gamma + 1)), dim3(kThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) {
    hipLaunchKernelGGL(accept_decide_kernel, dim3(a->batch), dim3(kThreads), 0, s, p);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return fail(PKV_ERR_DEVICE, std::string("accept launch: ") + hipGetErrorString(e));
  return PKV_OK;
}
