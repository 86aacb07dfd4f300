// Device helpers shared by the acceptance kernels (chain and draft tree):
// the Philox4x32-10 counter-based generator (Salmon, Moraes, Dror, Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC'11), uniforms and Gumbel
// noise in base-2 units, log-domain helpers, argmax and (max, sum) combines,
// and the chunked logit loads.
#pragma once

#include <hip/hip_runtime.h>

namespace pkv {
namespace sampling {

constexpr int kThreads = 256;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr unsigned kPurposeAccept = 1u, kPurposeSample = 2u;

struct Philox4 {
  unsigned x[4];
};

__device__ inline Philox4 philox4x32_10(unsigned c0, unsigned c1, unsigned c2, unsigned c3,
                                        unsigned k0, unsigned k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const unsigned long long p0 = 0xD2511F53ull * c0, p1 = 0xCD9E8D57ull * c2;
    const unsigned lo0 = unsigned(p0), hi0 = unsigned(p0 >> 32);
    const unsigned lo1 = unsigned(p1), hi1 = unsigned(p1 >> 32);
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

__device__ inline float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// Gumbel noise -ln(-ln u) in base-2 units, less the constant log2(ln 2):
// -log2(-log2 u).  u is at least 2^-24 and at most 1 - 2^-24, so both
// logarithms see normal arguments.
__device__ inline float gumbel2(float u) { return -log2_hw(-log2_hw(u)); }

// log2(1 - 2^d) for d < 0.  Near 0 the difference 1 - 2^d cancels, so it is
// taken from the Taylor series of 1 - e^t (t = d ln 2), whose truncation error
// for |t| <= 0.35 is below 1e-7 relative.
__device__ inline float log2_one_minus_exp2(float d) {
  const float t = d * kLn2;
  // 1 - e^t = -t (1 + t/2 + t^2/6 + t^3/24 + t^4/120 + t^5/720)
  const float p = 1.0f + t * (0.5f + t * (1.0f / 6 + t * (1.0f / 24 + t * (1.0f / 120 + t * (1.0f / 720)))));
  return log2_hw(t > -0.35f ? -t * p : 1.0f - exp2_hw(d));
}

// Argmax of (key, index): larger key wins, ties to the smaller index.
__device__ inline void better(float& k, int& i, float k2, int i2) {
  if (k2 > k || (k2 == k && i2 < i)) {
    k = k2;
    i = i2;
  }
}

// (max, sum 2^(v - max)) pairs in base 2.
__device__ inline void combine_ms(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == kNegInf) return;
  s = s * exp2_hw(m - mn) + s2 * exp2_hw(m2 - mn);
  m = mn;
}

// Loads NQ quads per thread of one row, quad q at logits 4q..4q+3, thread t
// taking quads q0 + u * TH + t (TH threads per workgroup).  Past the row's end: -inf.  kStream:
// non-temporal loads for data read once.
template <bool kAligned, int NQ, bool kStream = false, int TH = kThreads>
__device__ inline void load_chunk(const float* row, int vocab, int q0, float (&v)[NQ][4]) {
  if (kAligned) {
    const int nq = vocab >> 2;
    float4 f[NQ];
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int q = q0 + u * TH + int(threadIdx.x);
      typedef float f32x4 __attribute__((ext_vector_type(4)));
      const f32x4* src = reinterpret_cast<const f32x4*>(row) + q;
      f32x4 x = f32x4{kNegInf, kNegInf, kNegInf, kNegInf};
      if (q < nq) x = kStream ? __builtin_nontemporal_load(src) : *src;
      f[u] = make_float4(x[0], x[1], x[2], x[3]);
    }
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      v[u][0] = f[u].x;
      v[u][1] = f[u].y;
      v[u][2] = f[u].z;
      v[u][3] = f[u].w;
    }
  } else {
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int x0 = (q0 + u * TH + int(threadIdx.x)) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[u][e] = x0 + e < vocab ? row[x0 + e] : kNegInf;
    }
  }
}

}  // namespace sampling
}  // namespace pkv
