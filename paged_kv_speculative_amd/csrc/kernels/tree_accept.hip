// Draft-tree acceptance: accepted branch and next token (gfx950).
//
// Rule (the per-token test of innvotechnologies.co, section "Verification
// Acceptance Probabilities and Speedup Math", eq. alpha_i, applied to the
// candidates of a draft tree child by child with the residual update between
// them, as in multi-candidate speculative sampling; the pages verify and
// commit trees, atozofsoftwareengineering.blog pipeline diagram, without
// stating a rule):
//   at node u with P = softmax(target at u), Q = softmax(draft at u), the
//   children c_1 < c_2 < ... are tried in index order; c_j is accepted iff
//   u_{c_j} < min(1, P_{j-1}(x) / Q(x)), P_0 = P, P_j = max(0, P_{j-1} - Q)
//   normalised (P_{j-1} again if that is zero everywhere).  Accepting moves to
//   the child; rejecting every child ends with a draw from P_m; a leaf ends
//   with a draw from its P (the bonus).
//
// The residual after j rejections depends on the node only, not on the draws,
// so every candidate's test can be evaluated up front, in parallel:
//  1. stats: workgroup (sequence, node, T|D row, chunk) reduces (max, sum 2^x)
//     of its 8192 logits (internal nodes only);
//  2. levels 1 .. max_children-1, one launch each: workgroup (sequence, node,
//     chunk) sums 2^lr_j over its chunk, lr_j = log2 max(0, P_{j-1} - Q), with
//     P_{j-1} rebuilt per logit from the row normalisers and the earlier
//     levels' masses Z_1..Z_{j-1};
//  3. decide: one workgroup per sequence tests every candidate (lane c tests
//     node c against its sibling rank's residual) and walks the tree by
//     ballots to the stopping node;
//  4. draw: workgroup (sequence, chunk of 2048) computes its chunk's
//     Gumbel-max candidates for the token drawn there;
//  5. finish: one wave per sequence takes the best candidate.
// Everything is kept in base-2 logs; P_{j-1} - Q is formed as
// lp + log2(1 - 2^(lq - lp)), accurate where the two nearly cancel.

#include <hip/hip_runtime.h>

#include "../common.h"
#include "sampling.h"

namespace pkv {

namespace {

using namespace sampling;

constexpr int kWaves = kThreads / 64;
constexpr int kQuads = 8;                                 // 16-byte loads per thread (stats, levels)
constexpr int kChunk = kThreads * kQuads * 4;             // logits per stats workgroup
// Level kernels: small chunks (2048 logits) so that the few rows a level
// needs are spread over many workgroups.
constexpr int kLevelThreads = kThreads;
constexpr int kLevelWaves = kLevelThreads / 64;
constexpr int kLevelQuads = 2;
constexpr int kLevelChunk = kLevelThreads * kLevelQuads * 4;
constexpr int kDrawQuads = 2;
constexpr int kDrawChunk = kThreads * kDrawQuads * 4;     // logits per draw workgroup
constexpr int kMaxVocab = 1 << 26;
constexpr int kMaxBatch = 1 << 20;
constexpr int kMaxNodes = 64;

struct TreeParams {
  const float* T;
  const float* Dl;
  const int* parents;
  const int* tokens;
  int* accepted_len;
  int* accepted_nodes;
  int* next_token;
  float2* stats;       // [batch][n][2][chunks] (max, sum 2^x) in base 2
  float* zpart;        // [batch][n][levels][zchunks] residual masses per level chunk
  int4* cand;          // [batch][dchunks] (residual key bits, index, fallback key bits, index)
  int* decision;       // [batch][4]: stopping node (-1: rejected tree), its child count
  float* decision_f;   // [batch][64 + 2]: the stopping node's lse of T, D and log2 Z_1..Z_{m-1}
  int batch, n, levels, max_children, vocab, chunks, zchunks, dchunks;
  unsigned k0, k1, step;
  const unsigned* step_ptr;  // device step counter, or null (step above)
};

__device__ inline const float* trow(const TreeParams& P, int b, int u) {
  return P.T + (long(b) * P.n + u) * P.vocab;
}
__device__ inline const float* drow(const TreeParams& P, int b, int u) {
  return P.Dl + (long(b) * P.n + u) * P.vocab;
}

// Children of node u in sequence b: one parent per lane, counted by a ballot
// (every lane of the calling wave takes part; the result is wave-uniform).
__device__ inline int child_count(const TreeParams& P, int b, int u) {
  const int lane = threadIdx.x & 63;
  const int par = lane > 0 && lane < P.n ? P.parents[long(b) * P.n + lane] : -1;
  return __popcll(__ballot(par == u));
}

// Block-wide (max, sum) combine of one value pair per thread; thread 0 gets it.
__device__ inline void block_ms(float& m, float& s) {
  for (int o = 32; o > 0; o >>= 1) combine_ms(m, s, __shfl_xor(m, o, 64), __shfl_xor(s, o, 64));
  __shared__ float sm[kWaves], ss[kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) {
    sm[wave] = m;
    ss[wave] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0)
    for (int w = 1; w < kWaves; ++w) combine_ms(m, s, sm[w], ss[w]);
}

template <int NW>
__device__ inline float block_sum(float s) {
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  __shared__ float sp[NW];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sp[wave] = s;
  __syncthreads();
  if (threadIdx.x == 0)
    for (int w = 1; w < NW; ++w) s += sp[w];
  return s;
}

template <bool kAligned>
__global__ __launch_bounds__(kThreads) void tree_stats_kernel(TreeParams P) {
  const int chunk = blockIdx.x % P.chunks;
  const int r = blockIdx.x / P.chunks;           // (b * n + u) * 2 + which
  const int which = r & 1, u = (r >> 1) % P.n, b = (r >> 1) / P.n;
  if (child_count(P, b, u) == 0) return;         // a leaf's normalisers are never used
  const float* row = which ? drow(P, b, u) : trow(P, b, u);
  float v[kQuads][4];
  load_chunk<kAligned, kQuads, true>(row, P.vocab, chunk * (kChunk / 4), v);
  float m = kNegInf;
#pragma unroll
  for (int q = 0; q < kQuads; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) m = fmaxf(m, v[q][e]);
  m *= kLog2e;
  float s = 0.0f;
  if (m > kNegInf) {
#pragma unroll
    for (int q = 0; q < kQuads; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) s += exp2_hw(__builtin_fmaf(v[q][e], kLog2e, -m));
  }
  block_ms(m, s);
  if (threadIdx.x == 0) P.stats[long(r) * P.chunks + chunk] = make_float2(m, s);
}

// Base-2 log normaliser of row (b, u, which) from its chunk partials: lanes
// take chunks c, c + 64, ... and the wave combines them (every lane calls).
__device__ inline float row_lse(const TreeParams& P, int b, int u, int which) {
  const int lane = threadIdx.x & 63;
  const float2* st = P.stats + (long(b * P.n + u) * 2 + which) * P.chunks;
  float m = kNegInf, s = 0.0f;
  for (int c = lane; c < P.chunks; c += 64) combine_ms(m, s, st[c].x, st[c].y);
  for (int o = 32; o > 0; o >>= 1) combine_ms(m, s, __shfl_xor(m, o, 64), __shfl_xor(s, o, 64));
  return m + log2_hw(s);
}

// log2 of the residual mass Z_j of node u (j >= 1; -inf when it is zero),
// summed over the chunk partials by the calling wave.
__device__ inline float level_lz(const TreeParams& P, int b, int u, int j) {
  const int lane = threadIdx.x & 63;
  const float* z = P.zpart + (long(b * P.n + u) * P.levels + (j - 1)) * P.zchunks;
  float s = 0.0f;
  for (int c = lane; c < P.zchunks; c += 64) s += z[c];
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  return s > 0.0f ? log2_hw(s) : kNegInf;
}

// One residual step in base-2 logs: lr = log2 max(0, 2^lp - 2^lq).
__device__ inline float residual_log(float lp, float lq) {
  return lp > lq ? lp + log2_one_minus_exp2(lq - lp) : kNegInf;
}

// lp_{j} from lp_0 through the node's first j levels (lz[i-1] = log2 Z_i).
__device__ inline float advance_levels(float lp, float lq, const float* lz, int j) {
  for (int i = 0; i < j; ++i) {
    const float lr = residual_log(lp, lq);
    lp = lz[i] > kNegInf ? lr - lz[i] : lp;
  }
  return lp;
}

// Level j (1-based): residual mass of P_{j-1} - Q per chunk, for nodes with
// more than j children (their (j+1)-th candidate is tested against P_j).  A
// tree of n nodes has at most (n-1)/(j+1) such nodes; workgroup (sequence,
// slot, chunk) takes the slot-th of them in index order, if it exists.
template <bool kAligned>
__global__ __launch_bounds__(kLevelThreads) void tree_level_kernel(TreeParams P, int j, int slots) {
  const int chunk = blockIdx.x % P.zchunks;
  const int slot = (blockIdx.x / P.zchunks) % slots;
  const int b = blockIdx.x / P.zchunks / slots;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // lane u counts node u's children; the node of this slot is the slot-th
  // lane (in index order) with more than j
  const int par = lane > 0 && lane < P.n ? P.parents[long(b) * P.n + lane] : -1;
  int kids = 0;
  for (int c = 1; c < P.n; ++c) kids += __shfl(par, c, 64) == lane;
  const unsigned long long q = __ballot(lane < P.n && kids > j);
  if (__popcll(q) <= slot) return;
  unsigned long long rest = q;
  for (int i = 0; i < slot; ++i) rest &= rest - 1;
  const int u = __builtin_ctzll(rest);
  const int r = b * P.n + u;
  __shared__ float s_lz[kMaxNodes];
  __shared__ float s_iz[kMaxNodes];              // 1 / Z_i of the earlier levels
  __shared__ float s_l[2];
  // the chunk's logits do not depend on the normalisers: their loads go out
  // first and are in flight while the normalisers are gathered
  float tv[kLevelQuads][4], dv[kLevelQuads][4];
  const int q0 = chunk * (kLevelChunk / 4);
  load_chunk<kAligned, kLevelQuads, false, kLevelThreads>(trow(P, b, u), P.vocab, q0, tv);
  load_chunk<kAligned, kLevelQuads, false, kLevelThreads>(drow(P, b, u), P.vocab, q0, dv);
  // waves 0 and 1: the row normalisers; the others: the earlier levels' masses
  if (wave < 2) {
    const float l = row_lse(P, b, u, wave);
    if (lane == 0) s_l[wave] = l;
  } else {
    for (int i = wave - 2; i < j - 1; i += kLevelWaves - 2) {
      const float l = level_lz(P, b, u, i + 1);
      if (lane == 0) {
        s_lz[i] = l;
        s_iz[i] = l > kNegInf ? exp2_hw(-l) : 1.0f;
      }
    }
  }
  __syncthreads();
  const float lt = s_l[0], ld = s_l[1];
  float s = 0.0f;
#pragma unroll
  for (int qq = 0; qq < kLevelQuads; ++qq)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // in linear terms: P_0 and Q, P_i = max(0, P_{i-1} - Q) / Z_i through
      // the earlier levels (unchanged where Z_i = 0), then this level's term
      // max(0, P_{j-1} - Q); past the row both are 0
      const float qv = exp2_hw(__builtin_fmaf(dv[qq][e], kLog2e, -ld));
      float pv = exp2_hw(__builtin_fmaf(tv[qq][e], kLog2e, -lt));
      for (int i = 0; i < j - 1; ++i) pv = s_lz[i] > kNegInf ? fmaxf(pv - qv, 0.0f) * s_iz[i] : pv;
      s += fmaxf(pv - qv, 0.0f);
    }
  s = block_sum<kLevelWaves>(s);
  if (t == 0) P.zpart[(long(r) * P.levels + (j - 1)) * P.zchunks + chunk] = s;
}

// One workgroup per sequence: checks the tree, gathers the normalisers and
// residual masses of its internal nodes, tests every candidate (lane c tests
// node c against the residual of its sibling rank), and walks from the root
// by ballots to the stopping node.  Writes the accepted branch and, for the
// draw, the stopping node, its child count and its normalisers.
__global__ __launch_bounds__(kThreads) void tree_decide_kernel(TreeParams P) {
  const unsigned step = P.step_ptr ? *P.step_ptr : P.step;
  const int b = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  __shared__ int s_par[kMaxNodes];
  __shared__ int s_nkids[kMaxNodes];
  __shared__ float s_lt[kMaxNodes], s_ld[kMaxNodes];
  __shared__ float s_lz[kMaxNodes][kMaxNodes];   // [node][level - 1]
  __shared__ int s_bad;
  __shared__ int s_items[2 * kMaxNodes];
  __shared__ int s_nitems;
  // tree shape: parents and child counts; wave 0 also loads lane c's draft
  // token with its parent (independent loads, one round trip)
  int x = -1;
  if (wave == 0) {
    x = lane >= 1 && lane < P.n ? P.tokens[long(b) * P.n + lane] : -1;
    const int par = lane < P.n ? (lane == 0 ? -1 : P.parents[long(b) * P.n + lane]) : -2;
    const bool bad_par = lane < P.n && (lane == 0 ? P.parents[long(b) * P.n] != -1 : (par < 0 || par >= lane));
    s_par[lane] = par;
    int kids = 0;
    for (int c = 0; c < P.n; ++c) kids += __shfl(par, c, 64) == lane;
    s_nkids[lane] = lane < P.n ? kids : 0;
    const unsigned long long bad = __ballot(bad_par || kids > P.max_children);
    if (lane == 0) s_bad = bad != 0;
  }
  __syncthreads();
  int* dec = P.decision + long(b) * 4;
  if (s_bad) {
    for (int i = t; i < P.n; i += kThreads) P.accepted_nodes[long(b) * P.n + i] = -1;
    if (t == 0) {
      P.accepted_len[b] = -1;
      dec[0] = -1;
    }
    return;
  }
  // wave 0, lane c: candidate c's parent, sibling rank and the two logits of
  // its token, loaded before the normalisers are gathered (they depend on
  // nothing else)
  int u_c = 0, rank = 0;
  float tx = 0.0f, dx = 0.0f;
  const bool cand = wave == 0 && lane >= 1 && lane < P.n;
  if (cand) {
    u_c = s_par[lane];
    for (int c = 1; c < lane; ++c) rank += s_par[c] == u_c;
    if (x >= 0 && x < P.vocab) {
      dx = drow(P, b, u_c)[x];
      tx = trow(P, b, u_c)[x];
    }
  }
  // normalisers of internal nodes and their residual masses: item
  // (u, 0) and (u, 1) are the target and draft rows, (u, 1 + j) level j;
  // wave w takes items w, w + 4, ... (each a wave reduction)
  const int per = P.levels + 2, items = P.n * per;
  // an item is needed for internal nodes only, and a level only below the
  // node's child count
  auto needed = [&](int i) {
    const int u = i / per, q = i % per;
    return i < items && (q < 2 ? s_nkids[u] > 0 : q - 1 < s_nkids[u]);
  };
  // the first 64 partials of an item, every lane one: (max, sum) of a row's
  // chunk or the mass of a level's chunk.  Loaded for two items before
  // either is reduced, without branches (a loaded value copied at a branch
  // merge was waited for there): lanes past the chunk count read a valid
  // element and drop it afterwards.
  auto raw_part = [&](int i) {
    const int u = i / per, q = i % per;
    const bool row = q < 2;
    const int c = lane < (row ? P.chunks : P.zchunks) ? lane : 0;
    const float* src = row ? reinterpret_cast<const float*>(P.stats + (long(b * P.n + u) * 2 + q) * P.chunks + c)
                           : P.zpart + (long(b * P.n + u) * P.levels + (q - 2)) * P.zchunks + c;
    return make_float2(src[0], src[row ? 1 : 0]);
  };
  auto finish_item = [&](int i, float2 r) {
    const int u = i / per, q = i % per;
    if (q < 2) {
      const bool has = lane < P.chunks;
      float m = has ? r.x : kNegInf, sm = has ? r.y : 0.0f;
      const float2* st = P.stats + (long(b * P.n + u) * 2 + q) * P.chunks;
      for (int c = lane + 64; c < P.chunks; c += 64) combine_ms(m, sm, st[c].x, st[c].y);
      for (int o = 32; o > 0; o >>= 1) combine_ms(m, sm, __shfl_xor(m, o, 64), __shfl_xor(sm, o, 64));
      if (lane == 0) (q ? s_ld : s_lt)[u] = m + log2_hw(sm);
    } else {
      float z = lane < P.zchunks ? r.x : 0.0f;
      const float* zp = P.zpart + (long(b * P.n + u) * P.levels + (q - 2)) * P.zchunks;
      for (int c = lane + 64; c < P.zchunks; c += 64) z += zp[c];
      for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o, 64);
      if (lane == 0) s_lz[u][q - 2] = z > 0.0f ? log2_hw(z) : kNegInf;
    }
  };
  // wave 0 lists the needed items (at most 2n - 2: two rows per internal
  // node and one level per extra child), then the waves take them two at a time
  if (wave == 0) {
    int cnt = 0;
    for (int base = 0; base < items; base += 64) {
      const bool pred = needed(base + lane);
      const unsigned long long mask = __ballot(pred);
      if (pred) s_items[cnt + __popcll(mask & ((1ull << lane) - 1ull))] = base + lane;
      cnt += __popcll(mask);
    }
    if (lane == 0) s_nitems = cnt;
  }
  __syncthreads();
  const int nit = s_nitems;
  for (int k = wave; k < nit; k += 2 * kWaves) {
    const int k2 = k + kWaves;
    const int i1 = s_items[k], i2 = s_items[min(k2, nit - 1)];
    const float2 r1 = raw_part(i1), r2 = raw_part(i2);
    finish_item(i1, r1);
    if (k2 < nit) finish_item(i2, r2);
  }
  __syncthreads();
  if (wave != 0) return;
  bool acc = false;
  if (cand) {
    const int u = u_c;
    if (x >= 0 && x < P.vocab) {
      const float lq = __builtin_fmaf(dx, kLog2e, -s_ld[u]);
      const float lp = advance_levels(__builtin_fmaf(tx, kLog2e, -s_lt[u]), lq, s_lz[u], rank);
      const float d = lp - lq;
      const float a = d >= 0.0f ? 1.0f : exp2_hw(d);
      const Philox4 r = philox4x32_10(0u, unsigned(b), step, unsigned(lane - 1) | (kPurposeAccept << 16),
                                      P.k0, P.k1);
      acc = uniform01(r.x[0]) < a;
    }
  }
  const unsigned long long accepted = __ballot(acc);
  // walk from the root: the first accepted child (in index order) is taken
  int node = 0, depth = 0;
  unsigned long long kids;
  while (true) {
    kids = __ballot(lane < P.n && s_par[lane] == node);
    const unsigned long long take = kids & accepted;
    if (!take) break;
    node = __builtin_ctzll(take);
    if (lane == 0) P.accepted_nodes[long(b) * P.n + depth] = node;
    ++depth;
  }
  for (int i = depth + lane; i < P.n; i += 64) P.accepted_nodes[long(b) * P.n + i] = -1;
  const int m = __builtin_popcountll(kids);
  float* decf = P.decision_f + long(b) * (kMaxNodes + 2);
  if (m > 0) {
    if (lane == 0) {
      decf[0] = s_lt[node];
      decf[1] = s_ld[node];
    }
    if (lane < m - 1) decf[2 + lane] = s_lz[node][lane];
  }
  if (lane == 0) {
    P.accepted_len[b] = depth;
    dec[0] = node;
    dec[1] = m;
  }
}

// Workgroup (sequence, chunk of 2048 logits): the chunk's Gumbel-max
// candidates for the token drawn at the stopping node: from the residual
// P_{m-1} - Q after m rejections (falling back to P_{m-1}), or from the
// target at a leaf (the bonus).
template <bool kAligned>
__global__ __launch_bounds__(kThreads) void tree_draw_kernel(TreeParams P) {
  const unsigned step = P.step_ptr ? *P.step_ptr : P.step;
  const int chunk = blockIdx.x % P.dchunks;
  const int b = blockIdx.x / P.dchunks;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  __shared__ float s_f[kMaxNodes + 2];
  __shared__ float sk[2][kWaves];
  __shared__ int si[2][kWaves];
  const int u = P.decision[long(b) * 4], m = P.decision[long(b) * 4 + 1];
  if (u < 0) return;                             // rejected tree: no draw
  if (t < m + 1) s_f[t] = P.decision_f[long(b) * (kMaxNodes + 2) + t];
  const int q0 = chunk * (kDrawChunk / 4);
  float tv[kDrawQuads][4], dv[kDrawQuads][4];
  load_chunk<kAligned, kDrawQuads>(trow(P, b, u), P.vocab, q0, tv);
  if (m > 0) load_chunk<kAligned, kDrawQuads>(drow(P, b, u), P.vocab, q0, dv);
  __syncthreads();
  float rk = kNegInf, fk = kNegInf;
  int ri = 0x7FFFFFFF, fi = 0x7FFFFFFF;
  const unsigned c3 = unsigned(u) | (kPurposeSample << 16);
  if (m > 0) {
    const float lt = s_f[0], ld = s_f[1];
#pragma unroll
    for (int qq = 0; qq < kDrawQuads; ++qq) {
      const int q = q0 + qq * kThreads + t;
      const Philox4 r = philox4x32_10(unsigned(q), unsigned(b), step, c3, P.k0, P.k1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int x = q * 4 + e;
        const float g = gumbel2(uniform01(r.x[e]));
        const float lq = __builtin_fmaf(dv[qq][e], kLog2e, -ld);
        const float lp = advance_levels(__builtin_fmaf(tv[qq][e], kLog2e, -lt), lq, s_f + 2, m - 1);
        better(fk, fi, lp + g, x);
        better(rk, ri, residual_log(lp, lq) + g, x);
      }
    }
  } else {
#pragma unroll
    for (int qq = 0; qq < kDrawQuads; ++qq) {
      const int q = q0 + qq * kThreads + t;
      const Philox4 r = philox4x32_10(unsigned(q), unsigned(b), step, c3, P.k0, P.k1);
#pragma unroll
      for (int e = 0; e < 4; ++e) better(fk, fi, tv[qq][e] * kLog2e + gumbel2(uniform01(r.x[e])), q * 4 + e);
    }
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

// One wave per sequence: the best candidate over the chunks (-1 for a
// sequence whose tree was rejected).
__global__ __launch_bounds__(64) void tree_finish_kernel(TreeParams P) {
  const int b = blockIdx.x, lane = threadIdx.x;
  if (P.accepted_len[b] < 0) {
    if (lane == 0) P.next_token[b] = -1;
    return;
  }
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
  if (lane == 0) P.next_token[b] = rk > kNegInf ? ri : fi;
}

struct WsLayout {
  size_t stats, zpart, cand, decision, decision_f, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

WsLayout ws_layout(const pkv_tree_accept_args* a) {
  const size_t ch = (size_t(a->vocab) + kChunk - 1) / kChunk;
  const size_t zch = (size_t(a->vocab) + kLevelChunk - 1) / kLevelChunk;
  const size_t dch = (size_t(a->vocab) + kDrawChunk - 1) / kDrawChunk;
  const size_t levels = size_t(a->max_children > 1 ? a->max_children - 1 : 1);
  const size_t rows = size_t(a->batch) * a->n_nodes;
  WsLayout w;
  w.stats = 0;
  w.zpart = align256(rows * 2 * ch * sizeof(float2));
  w.cand = w.zpart + align256(rows * levels * zch * sizeof(float));
  w.decision = w.cand + align256(size_t(a->batch) * dch * sizeof(int4));
  w.decision_f = w.decision + align256(size_t(a->batch) * 4 * sizeof(int));
  w.total = w.decision_f + size_t(a->batch) * (kMaxNodes + 2) * sizeof(float);
  return w;
}

pkv_status check_shape(const pkv_tree_accept_args* a) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "null args");
  if (a->batch < 1 || a->batch > kMaxBatch) return fail(PKV_ERR_INVALID_ARG, "batch must be in [1, 2^20]");
  if (a->n_nodes < 2 || a->n_nodes > kMaxNodes) return fail(PKV_ERR_INVALID_ARG, "n_nodes must be in [2, 64]");
  if (a->max_children < 1 || a->max_children > a->n_nodes - 1)
    return fail(PKV_ERR_INVALID_ARG, "max_children must be in [1, n_nodes - 1]");
  if (a->vocab < 1 || a->vocab > kMaxVocab) return fail(PKV_ERR_INVALID_ARG, "vocab must be in [1, 2^26]");
  const long long ch = (a->vocab + kChunk - 1) / kChunk;
  const long long dch = (a->vocab + kDrawChunk - 1) / kDrawChunk;
  const long long zch = (a->vocab + kLevelChunk - 1) / kLevelChunk;
  if (ch * a->batch * a->n_nodes * 2 > 0x7FFFFFFFll || dch * a->batch > 0x7FFFFFFFll ||
      zch * a->batch * (a->n_nodes / 2) > 0x7FFFFFFFll)
    return fail(PKV_ERR_INVALID_ARG, "batch * n_nodes * vocab too large for one launch");
  return PKV_OK;
}

}  // namespace

}  // namespace pkv

using namespace pkv;

extern "C" pkv_status spec_accept_tree_workspace_size(const pkv_tree_accept_args* a, size_t* bytes_out) {
  if (!bytes_out) return fail(PKV_ERR_INVALID_ARG, "null output");
  pkv_status st = check_shape(a);
  if (st != PKV_OK) return st;
  *bytes_out = ws_layout(a).total;
  return PKV_OK;
}

extern "C" pkv_status spec_accept_tree(const pkv_tree_accept_args* a, void* stream) {
  pkv_status st = check_shape(a);
  if (st != PKV_OK) return st;
  if (!a->target_logits || !a->draft_logits || !a->parents || !a->tokens || !a->accepted_len ||
      !a->accepted_nodes || !a->next_token)
    return fail(PKV_ERR_INVALID_ARG, "null device pointer");
  if ((reinterpret_cast<uintptr_t>(a->target_logits) | reinterpret_cast<uintptr_t>(a->draft_logits)) & 15)
    return fail(PKV_ERR_INVALID_ARG, "logit arrays must be 16-byte aligned");
  const WsLayout w = ws_layout(a);
  if (!a->workspace || a->workspace_bytes < w.total)
    return fail(PKV_ERR_WORKSPACE, "workspace smaller than spec_accept_tree_workspace_size");
  if (reinterpret_cast<uintptr_t>(a->workspace) & 15)
    return fail(PKV_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  TreeParams p{};
  p.T = a->target_logits;
  p.Dl = a->draft_logits;
  p.parents = a->parents;
  p.tokens = a->tokens;
  p.accepted_len = a->accepted_len;
  p.accepted_nodes = a->accepted_nodes;
  p.next_token = a->next_token;
  char* ws = static_cast<char*>(a->workspace);
  p.stats = reinterpret_cast<float2*>(ws + w.stats);
  p.zpart = reinterpret_cast<float*>(ws + w.zpart);
  p.cand = reinterpret_cast<int4*>(ws + w.cand);
  p.decision = reinterpret_cast<int*>(ws + w.decision);
  p.decision_f = reinterpret_cast<float*>(ws + w.decision_f);
  p.batch = a->batch;
  p.n = a->n_nodes;
  p.max_children = a->max_children;
  p.levels = a->max_children > 1 ? a->max_children - 1 : 1;
  p.vocab = a->vocab;
  p.chunks = (a->vocab + kChunk - 1) / kChunk;
  p.zchunks = (a->vocab + kLevelChunk - 1) / kLevelChunk;
  p.dchunks = (a->vocab + kDrawChunk - 1) / kDrawChunk;
  p.k0 = unsigned(a->seed & 0xFFFFFFFFu);
  p.k1 = unsigned(a->seed >> 32);
  p.step = a->step;
  p.step_ptr = a->step_ptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool aligned = (a->vocab & 3) == 0;
  const unsigned rows = unsigned(a->batch) * a->n_nodes;
  if (aligned) hipLaunchKernelGGL(tree_stats_kernel<true>, dim3(rows * 2 * p.chunks), dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL(tree_stats_kernel<false>, dim3(rows * 2 * p.chunks), dim3(kThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  for (int j = 1; e == hipSuccess && j < a->max_children; ++j) {
    const int slots = (a->n_nodes - 1) / (j + 1);
    const dim3 grid(unsigned(a->batch) * slots * p.zchunks);
    if (aligned) hipLaunchKernelGGL(tree_level_kernel<true>, grid, dim3(kLevelThreads), 0, s, p, j, slots);
    else hipLaunchKernelGGL(tree_level_kernel<false>, grid, dim3(kLevelThreads), 0, s, p, j, slots);
    e = hipGetLastError();
  }
  if (e == hipSuccess) {
    hipLaunchKernelGGL(tree_decide_kernel, dim3(a->batch), dim3(kThreads), 0, s, p);
    e = hipGetLastError();
  }
  if (e == hipSuccess) {
    const unsigned n_draw = unsigned(a->batch) * p.dchunks;
    if (aligned) hipLaunchKernelGGL(tree_draw_kernel<true>, dim3(n_draw), dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL(tree_draw_kernel<false>, dim3(n_draw), dim3(kThreads), 0, s, p);
    e = hipGetLastError();
  }
  if (e == hipSuccess) {
    hipLaunchKernelGGL(tree_finish_kernel, dim3(a->batch), dim3(64), 0, s, p);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return fail(PKV_ERR_DEVICE, std::string("tree accept launch: ") + hipGetErrorString(e));
  return PKV_OK;
}
