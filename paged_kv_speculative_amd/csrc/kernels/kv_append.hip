// Pool-update kernel: applies PoolTask records (copy-on-write page copies,
// token scatter into the tiled page layout with optional FP8 quantisation,
// block-table entries and sequence lengths) in stream order.  A workgroup
// takes one task and four KV heads; each wave moves one head's tokens in
// groups of 8 channels, all loads of a lane issued before its stores.
//
// FP8 quantisation (reading of atozofsoftwareengineering.blog, section
// "Custom FP8 Quantized Memory Block Layout", per-block scales S_K, S_V):
// a fresh page gets, per KV head, scale = amax/448 over the tokens written
// into it by this call (1 when amax is 0); values are x * (1/scale) in fp32,
// clamped to +-448 and rounded to nearest-even OCP E4M3.

#include <hip/hip_runtime.h>

#include "../common.h"
#include "fp8_codec.h"
#include "layout.h"

namespace pkv {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// 8-channel groups of one head in one task: at most 16 tokens x 128/8 groups,
// i.e. four per lane of the head's wave.
constexpr int kItemsPerLane = 4;

__device__ inline float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}


// Item it of a task (token it / G, channel group it % G) for the calling lane.
// An item past the task's tokens reads the task's first source row instead
// (valid whenever the task has tokens) and stores nothing, so every source
// load is unconditional and a lane's loads can all be in flight at once.
struct Item {
  bool ok;
  int slot, c0;
  long src;  // element offset of channel c0 of head h in the source row
};

__device__ inline Item item(const PoolTask& t, int u, int h, int H, int D) {
  const int G = D / 8;
  const int it = u * 64 + int(threadIdx.x & 63);
  Item r;
  r.ok = it < t.n * G;
  const int tok = r.ok ? it / G : 0;
  r.c0 = (it % G) * 8;
  r.slot = t.slot_begin + tok;
  r.src = (long(t.src_row) + tok) * H * D + long(h) * D + r.c0;
  return r;
}

// bf16 pool, bf16 source: 16-byte loads; K groups of 8 channels are
// contiguous in the tiled layout (D/4 is a multiple of 8), V is scattered.
// The items are named values, not arrays: arrays indexed in these loops were
// placed in LDS by the compiler (before the loops are unrolled), and every
// source load then waited for its LDS copy.
__device__ void write_bf16(const PoolDevice& dev, const PoolTask& t, int h, int H, int D, long pb) {
  static_assert(kItemsPerLane == 4, "four named items per lane");
  const uint4* ks = static_cast<const uint4*>(dev.k_src);
  const uint4* vs = static_cast<const uint4*>(dev.v_src);
  const Item i0 = item(t, 0, h, H, D), i1 = item(t, 1, h, H, D), i2 = item(t, 2, h, H, D),
             i3 = item(t, 3, h, H, D);
  const uint4 k0 = ks[i0.src / 8], k1 = ks[i1.src / 8], k2 = ks[i2.src / 8], k3 = ks[i3.src / 8];
  const uint4 v0 = vs[i0.src / 8], v1 = vs[i1.src / 8], v2 = vs[i2.src / 8], v3 = vs[i3.src / 8];
  char* kslab = static_cast<char*>(dev.k_pages) + (long(t.page) * H + h) * pb;
  unsigned short* vslab = reinterpret_cast<unsigned short*>(static_cast<char*>(dev.v_pages) + (long(t.page) * H + h) * pb);
  auto put = [&](const Item& im, const uint4& kx, const uint4& vx) {
    if (!im.ok) return;
    *reinterpret_cast<uint4*>(kslab + 2 * k_index_bf16(im.slot, im.c0, D)) = kx;
    auto put_pair = [&](int i, unsigned w) {     // channels c0 + i, c0 + i + 1
      vslab[v_index_bf16(im.slot, im.c0 + i)] = static_cast<unsigned short>(w);
      vslab[v_index_bf16(im.slot, im.c0 + i + 1)] = static_cast<unsigned short>(w >> 16);
    };
    put_pair(0, vx.x);
    put_pair(2, vx.y);
    put_pair(4, vx.z);
    put_pair(6, vx.w);
  };
  put(i0, k0, v0);
  put(i1, k1, v1);
  put(i2, k2, v2);
  put(i3, k3, v3);
}

// fp32 pool, fp32 source: row-major slab, two 16-byte moves per group (named
// values, as for bf16).
__device__ void write_f32(const PoolDevice& dev, const PoolTask& t, int h, int H, int D, long pb) {
  static_assert(kItemsPerLane == 4, "four named items per lane");
  const float4* ks = static_cast<const float4*>(dev.k_src);
  const float4* vs = static_cast<const float4*>(dev.v_src);
  const Item i0 = item(t, 0, h, H, D), i1 = item(t, 1, h, H, D), i2 = item(t, 2, h, H, D),
             i3 = item(t, 3, h, H, D);
  const float4 k0a = ks[i0.src / 4], k0b = ks[i0.src / 4 + 1], k1a = ks[i1.src / 4], k1b = ks[i1.src / 4 + 1];
  const float4 k2a = ks[i2.src / 4], k2b = ks[i2.src / 4 + 1], k3a = ks[i3.src / 4], k3b = ks[i3.src / 4 + 1];
  const float4 v0a = vs[i0.src / 4], v0b = vs[i0.src / 4 + 1], v1a = vs[i1.src / 4], v1b = vs[i1.src / 4 + 1];
  const float4 v2a = vs[i2.src / 4], v2b = vs[i2.src / 4 + 1], v3a = vs[i3.src / 4], v3b = vs[i3.src / 4 + 1];
  float4* kslab = reinterpret_cast<float4*>(static_cast<char*>(dev.k_pages) + (long(t.page) * H + h) * pb);
  float4* vslab = reinterpret_cast<float4*>(static_cast<char*>(dev.v_pages) + (long(t.page) * H + h) * pb);
  auto put = [&](const Item& im, const float4& ka, const float4& kb, const float4& va, const float4& vb) {
    if (!im.ok) return;
    const long o = index_f32(im.slot, im.c0, D) / 4;
    kslab[o] = ka;
    kslab[o + 1] = kb;
    vslab[o] = va;
    vslab[o + 1] = vb;
  };
  put(i0, k0a, k0b, v0a, v0b);
  put(i1, k1a, k1b, v1a, v1b);
  put(i2, k2a, k2b, v2a, v2b);
  put(i3, k3a, k3b, v3a, v3b);
}

// FP8 pool, fp32 source: the head's values stay in registers while the wave
// reduces their amax for the page's scale; K groups of 8 channels are 8 contiguous
// bytes of the tiled layout (D/4 is a multiple of 16), V is scattered.
__device__ void write_fp8(const PoolDevice& dev, const PoolTask& t, int h, int H, int D, long pb) {
  const float4* ks = static_cast<const float4*>(dev.k_src);
  const float4* vs = static_cast<const float4*>(dev.v_src);
  float kx[kItemsPerLane][8], vx[kItemsPerLane][8];
  Item im[kItemsPerLane];
  float ak = 0.0f, av = 0.0f;
#pragma unroll
  for (int u = 0; u < kItemsPerLane; ++u) {
    im[u] = item(t, u, h, H, D);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const float4 a = ks[im[u].src / 4 + p];
      const float4 b = vs[im[u].src / 4 + p];
      kx[u][4 * p + 0] = a.x; kx[u][4 * p + 1] = a.y; kx[u][4 * p + 2] = a.z; kx[u][4 * p + 3] = a.w;
      vx[u][4 * p + 0] = b.x; vx[u][4 * p + 1] = b.y; vx[u][4 * p + 2] = b.z; vx[u][4 * p + 3] = b.w;
    }
    // items past the task's tokens hold another item's values: not in the amax
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ak = fmaxf(ak, im[u].ok ? fabsf(kx[u][i]) : 0.0f);
      av = fmaxf(av, im[u].ok ? fabsf(vx[u][i]) : 0.0f);
    }
  }
  const long sidx = long(t.page) * H + h;
  unsigned char* kslab = static_cast<unsigned char*>(dev.k_pages) + sidx * pb;
  unsigned char* vslab = static_cast<unsigned char*>(dev.v_pages) + sidx * pb;
  ak = wave_max(ak);
  av = wave_max(av);
  float sk, sv;
  if (t.flags & kFresh) {
    sk = fresh_page_scale(ak);
    sv = fresh_page_scale(av);
  } else {
    // a page written before keeps its scale unless the new values exceed
    // its range: then the scale doubles until they fit and the slots
    // already written (0 .. slot_begin - 1) are encoded again
    const float sk0 = static_cast<const float*>(dev.k_scale)[sidx];
    const float sv0 = static_cast<const float*>(dev.v_scale)[sidx];
    sk = grown_page_scale(ak, sk0);
    sv = grown_page_scale(av, sv0);
    const int lane = threadIdx.x & 63, n_old = t.slot_begin * D;
    if (sk != sk0) {
      const float inv = 1.0f / sk;
      for (int e = lane; e < n_old; e += 64) {
        unsigned char& c = kslab[k_index_fp8(e / D, e % D, D)];
        c = reencode_e4m3(c, sk0, inv);
      }
    }
    if (sv != sv0) {
      const float inv = 1.0f / sv;
      for (int e = lane; e < n_old; e += 64) {
        unsigned char& c = vslab[v_index_fp8(e / D, e % D)];
        c = reencode_e4m3(c, sv0, inv);
      }
    }
  }
  if ((threadIdx.x & 63) == 0) {
    static_cast<float*>(dev.k_scale)[sidx] = sk;
    static_cast<float*>(dev.v_scale)[sidx] = sv;
  }
  const float ik = 1.0f / sk, iv = 1.0f / sv;
#pragma unroll
  for (int u = 0; u < kItemsPerLane; ++u) {
    if (!im[u].ok) continue;
    unsigned lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= unsigned(quant_e4m3(kx[u][i], ik)) << (8 * i);
      hi |= unsigned(quant_e4m3(kx[u][4 + i], ik)) << (8 * i);
    }
    *reinterpret_cast<uint2*>(kslab + k_index_fp8(im[u].slot, im[u].c0, D)) = make_uint2(lo, hi);
#pragma unroll
    for (int i = 0; i < 8; ++i) vslab[v_index_fp8(im[u].slot, im[u].c0 + i)] = quant_e4m3(vx[u][i], iv);
  }
}

// FP8 pool with per-64-channel scales, fp32 source: every token is quantised
// on its own.  A lane holds 8 channels of one token; the 8 lanes of a
// 64-channel tile (consecutive items, 8-aligned) reduce its amax by
// shuffles, and the tile's first lane writes the exponent byte.
__device__ void write_fp8mx(const PoolDevice& dev, const PoolTask& t, int h, int H, int D, long pb) {
  static_assert(kItemsPerLane == 4, "four named items per lane");
  const float4* ks = static_cast<const float4*>(dev.k_src);
  const float4* vs = static_cast<const float4*>(dev.v_src);
  const int G = D / 64;
  unsigned char* kslab = static_cast<unsigned char*>(dev.k_pages) + (long(t.page) * H + h) * pb;
  unsigned char* vslab = static_cast<unsigned char*>(dev.v_pages) + (long(t.page) * H + h) * pb;
  unsigned char* kexp = static_cast<unsigned char*>(dev.k_scale) + (long(t.page) * H + h) * 16 * G;
  unsigned char* vexp = static_cast<unsigned char*>(dev.v_scale) + (long(t.page) * H + h) * 16 * G;
  // every item's source values are loaded before the first one is encoded
  // (encoding an item before the next item's loads issued made each lane's
  // loads wait for one another)
  const Item i0 = item(t, 0, h, H, D), i1 = item(t, 1, h, H, D), i2 = item(t, 2, h, H, D),
             i3 = item(t, 3, h, H, D);
  const float4 k0a = ks[i0.src / 4], k0b = ks[i0.src / 4 + 1], k1a = ks[i1.src / 4], k1b = ks[i1.src / 4 + 1];
  const float4 k2a = ks[i2.src / 4], k2b = ks[i2.src / 4 + 1], k3a = ks[i3.src / 4], k3b = ks[i3.src / 4 + 1];
  const float4 v0a = vs[i0.src / 4], v0b = vs[i0.src / 4 + 1], v1a = vs[i1.src / 4], v1b = vs[i1.src / 4 + 1];
  const float4 v2a = vs[i2.src / 4], v2b = vs[i2.src / 4 + 1], v3a = vs[i3.src / 4], v3b = vs[i3.src / 4 + 1];
  auto put = [&](const Item& im, const float4& ka, const float4& kb, const float4& va, const float4& vb) {
    const float kx[8] = {ka.x, ka.y, ka.z, ka.w, kb.x, kb.y, kb.z, kb.w};
    const float vx[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
    float ak = 0.0f, av = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ak = fmaxf(ak, im.ok ? fabsf(kx[i]) : 0.0f);
      av = fmaxf(av, im.ok ? fabsf(vx[i]) : 0.0f);
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      ak = fmaxf(ak, __shfl_xor(ak, o, 64));
      av = fmaxf(av, __shfl_xor(av, o, 64));
    }
    if (!im.ok) return;
    const int ek = tile_exponent_byte(ak), ev = tile_exponent_byte(av);
    const float ik = ldexpf(1.0f, 127 - ek), iv = ldexpf(1.0f, 127 - ev);
    unsigned lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= unsigned(quant_e4m3(kx[i], ik)) << (8 * i);
      hi |= unsigned(quant_e4m3(kx[4 + i], ik)) << (8 * i);
    }
    *reinterpret_cast<uint2*>(kslab + k_index_fp8(im.slot, im.c0, D)) = make_uint2(lo, hi);
#pragma unroll
    for (int i = 0; i < 8; ++i) vslab[v_index_fp8(im.slot, im.c0 + i)] = quant_e4m3(vx[i], iv);
    if ((im.c0 & 63) == 0) {
      kexp[im.slot * G + im.c0 / 64] = static_cast<unsigned char>(ek);
      vexp[im.slot * G + im.c0 / 64] = static_cast<unsigned char>(ev);
    }
  };
  put(i0, k0a, k0b, v0a, v0b);
  put(i1, k1a, k1b, v1a, v1b);
  put(i2, k2a, k2b, v2a, v2b);
  put(i3, k3a, k3b, v3a, v3b);
}

// Block (task, y) handles KV heads 4y .. 4y+3 of its task, one wave per head.
__global__ __launch_bounds__(kThreads) void pool_update_kernel(PoolDevice dev, PoolUpdateBatch batch) {
  const PoolTask t = batch.tasks[blockIdx.x];
  const int H = batch.num_kv_heads, D = batch.head_dim;
  const long pb = batch.page_bytes;
  const int h0 = blockIdx.y * kWaves;
  const int nh = min(kWaves, H - h0);

  if (t.cow_src >= 0) {
    const long n16 = nh * pb / 16;
    const long so = (long(t.cow_src) * H + h0) * pb, dO = (long(t.page) * H + h0) * pb;
    const uint4* sk = reinterpret_cast<const uint4*>(static_cast<const char*>(dev.k_pages) + so);
    const uint4* sv = reinterpret_cast<const uint4*>(static_cast<const char*>(dev.v_pages) + so);
    uint4* dk = reinterpret_cast<uint4*>(static_cast<char*>(dev.k_pages) + dO);
    uint4* dv = reinterpret_cast<uint4*>(static_cast<char*>(dev.v_pages) + dO);
    // four 16-byte chunks of K and of V per thread per round, all loaded
    // before any is stored (named values: see write_bf16)
    for (long i0 = threadIdx.x; i0 < n16; i0 += 4 * kThreads) {
      const long i1 = i0 + kThreads, i2 = i0 + 2 * kThreads, i3 = i0 + 3 * kThreads, last = n16 - 1;
      const uint4 k0 = sk[i0], k1 = sk[min(i1, last)], k2 = sk[min(i2, last)], k3 = sk[min(i3, last)];
      const uint4 v0 = sv[i0], v1 = sv[min(i1, last)], v2 = sv[min(i2, last)], v3 = sv[min(i3, last)];
      dk[i0] = k0;
      dv[i0] = v0;
      if (i1 < n16) {
        dk[i1] = k1;
        dv[i1] = v1;
      }
      if (i2 < n16) {
        dk[i2] = k2;
        dv[i2] = v2;
      }
      if (i3 < n16) {
        dk[i3] = k3;
        dv[i3] = v3;
      }
    }
    if (batch.kv_dtype == PKV_FP8_E4M3 && int(threadIdx.x) < nh) {
      const int h = h0 + threadIdx.x;
      float* ksc = static_cast<float*>(dev.k_scale);
      float* vsc = static_cast<float*>(dev.v_scale);
      ksc[long(t.page) * H + h] = ksc[long(t.cow_src) * H + h];
      vsc[long(t.page) * H + h] = vsc[long(t.cow_src) * H + h];
    }
    if (batch.kv_dtype == PKV_FP8_E4M3_MX64) {
      // the exponent bytes of the copied heads: 16 tokens x D/64 each
      const int nb = nh * 16 * (D / 64);
      unsigned char* ke = static_cast<unsigned char*>(dev.k_scale);
      unsigned char* ve = static_cast<unsigned char*>(dev.v_scale);
      const long so8 = (long(t.cow_src) * H + h0) * 16 * (D / 64), do8 = (long(t.page) * H + h0) * 16 * (D / 64);
      for (int i = threadIdx.x; i < nb; i += kThreads) {
        ke[do8 + i] = ke[so8 + i];
        ve[do8 + i] = ve[so8 + i];
      }
    }
    __syncthreads();
  }

  const int h = h0 + int(threadIdx.x >> 6);
  if (t.n > 0 && h < H) {
    if (batch.kv_dtype == PKV_BF16) write_bf16(dev, t, h, H, D, pb);
    else if (batch.kv_dtype == PKV_F32) write_f32(dev, t, h, H, D, pb);
    else if (batch.kv_dtype == PKV_FP8_E4M3_MX64) write_fp8mx(dev, t, h, H, D, pb);
    else write_fp8(dev, t, h, H, D, pb);
  }

  if (blockIdx.y == 0 && threadIdx.x == 0) {
    if (t.flags & kWriteTable) dev.block_table[long(t.row) * batch.bt_stride + t.logical] = t.page;
    if (t.flags & kSetLen) dev.seq_lens[t.row] = t.new_len;
  }
}

// Element e of channel c, token slot t of a (page, head) slab, in the pool's
// layout, as raw bits (bf16/fp8) or a float (fp32).
template <typename E>
__device__ inline E& k_elem(char* slab, int t, int c, int D, int dtype) {
  if (dtype == PKV_BF16) return *reinterpret_cast<E*>(slab + 2 * k_index_bf16(t, c, D));
  if (dtype == PKV_F32) return *reinterpret_cast<E*>(slab + 4 * index_f32(t, c, D));
  return *reinterpret_cast<E*>(slab + k_index_fp8(t, c, D));
}
template <typename E>
__device__ inline E& v_elem(char* slab, int t, int c, int D, int dtype) {
  if (dtype == PKV_BF16) return *reinterpret_cast<E*>(slab + 2 * v_index_bf16(t, c));
  if (dtype == PKV_F32) return *reinterpret_cast<E*>(slab + 4 * index_f32(t, c, D));
  return *reinterpret_cast<E*>(slab + v_index_fp8(t, c));
}

// One FP8 code moved between pages: kept when the scales are equal bit for
// bit, else decoded with the source scale (fp32 product) and encoded again
// with the destination's.
__device__ inline unsigned char move_fp8(unsigned char code, float s_src, float s_dst) {
  if (__float_as_uint(s_src) == __float_as_uint(s_dst)) return code;
  const float x = __builtin_amdgcn_cvt_f32_fp8(int(code), 0) * s_src;
  return quant_e4m3(x, 1.0f / s_dst);
}

// Block (group, y): heads 4y .. 4y+3 of one sequence's moves, one wave per
// head, lane l moving channels l and l + 64.  The moves of a group run in
// order; a later move never reads a slot an earlier one wrote (path nodes
// lie at or after their destinations), and each lane touches only its own
// channels, so program order is the only ordering needed.
__global__ __launch_bounds__(kThreads) void pool_move_kernel(PoolDevice dev, PoolMoveBatch batch) {
  const int H = batch.num_kv_heads, D = batch.head_dim, dt = batch.kv_dtype;
  const long pb = batch.page_bytes;
  const int h = blockIdx.y * kWaves + int(threadIdx.x >> 6);
  if (h >= H) return;
  const int lane = threadIdx.x & 63;
  char* K = static_cast<char*>(dev.k_pages);
  char* V = static_cast<char*>(dev.v_pages);
  for (int i = batch.first[blockIdx.x]; i < batch.first[blockIdx.x + 1]; ++i) {
    const PoolMove m = batch.moves[i];
    const int ts = m.slots & 0xFF, td = (m.slots >> 8) & 0xFF;
    const long so = (long(m.src_page) * H + h) * pb, dO = (long(m.dst_page) * H + h) * pb;
    if (dt == PKV_FP8_E4M3_MX64) {
      // codes and the token's own exponent bytes move unchanged
      for (int c = lane; c < D; c += 64) {
        const unsigned char kc = k_elem<unsigned char>(K + so, ts, c, D, PKV_FP8_E4M3);
        const unsigned char vc = v_elem<unsigned char>(V + so, ts, c, D, PKV_FP8_E4M3);
        k_elem<unsigned char>(K + dO, td, c, D, PKV_FP8_E4M3) = kc;
        v_elem<unsigned char>(V + dO, td, c, D, PKV_FP8_E4M3) = vc;
      }
      const int G = D / 64;
      if (lane < G) {
        unsigned char* ke = static_cast<unsigned char*>(dev.k_scale);
        unsigned char* ve = static_cast<unsigned char*>(dev.v_scale);
        const long s8 = ((long(m.src_page) * H + h) * 16 + ts) * G + lane;
        const long d8 = ((long(m.dst_page) * H + h) * 16 + td) * G + lane;
        const unsigned char kx = ke[s8], vx = ve[s8];
        ke[d8] = kx;
        ve[d8] = vx;
      }
    } else if (dt == PKV_FP8_E4M3) {
      const float* ksc = static_cast<const float*>(dev.k_scale);
      const float* vsc = static_cast<const float*>(dev.v_scale);
      const float ks = ksc[long(m.src_page) * H + h], kd = ksc[long(m.dst_page) * H + h];
      const float vs = vsc[long(m.src_page) * H + h], vd = vsc[long(m.dst_page) * H + h];
      for (int c = lane; c < D; c += 64) {
        const unsigned char kc = k_elem<unsigned char>(K + so, ts, c, D, dt);
        const unsigned char vc = v_elem<unsigned char>(V + so, ts, c, D, dt);
        k_elem<unsigned char>(K + dO, td, c, D, dt) = move_fp8(kc, ks, kd);
        v_elem<unsigned char>(V + dO, td, c, D, dt) = move_fp8(vc, vs, vd);
      }
    } else if (dt == PKV_BF16) {
      for (int c = lane; c < D; c += 64) {
        const unsigned short kc = k_elem<unsigned short>(K + so, ts, c, D, dt);
        const unsigned short vc = v_elem<unsigned short>(V + so, ts, c, D, dt);
        k_elem<unsigned short>(K + dO, td, c, D, dt) = kc;
        v_elem<unsigned short>(V + dO, td, c, D, dt) = vc;
      }
    } else {
      for (int c = lane; c < D; c += 64) {
        const float kc = k_elem<float>(K + so, ts, c, D, dt);
        const float vc = v_elem<float>(V + so, ts, c, D, dt);
        k_elem<float>(K + dO, td, c, D, dt) = kc;
        v_elem<float>(V + dO, td, c, D, dt) = vc;
      }
    }
  }
}

}  // namespace

pkv_status launch_pool_moves(const PoolDevice& dev, const PoolMoveBatch& batch, void* stream) {
  if (batch.n_groups <= 0) return PKV_OK;
  const unsigned gy = unsigned((batch.num_kv_heads + kWaves - 1) / kWaves);
  hipLaunchKernelGGL(pool_move_kernel, dim3(batch.n_groups, gy), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), dev, batch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_DEVICE, std::string("pool move launch: ") + hipGetErrorString(e));
  return PKV_OK;
}

pkv_status launch_pool_update(const PoolDevice& dev, const PoolUpdateBatch& batch, void* stream) {
  if (batch.n_tasks <= 0) return PKV_OK;
  const unsigned gy = unsigned((batch.num_kv_heads + kWaves - 1) / kWaves);
  hipLaunchKernelGGL(pool_update_kernel, dim3(batch.n_tasks, gy), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), dev, batch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_DEVICE, std::string("pool update launch: ") + hipGetErrorString(e));
  return PKV_OK;
}

}  // namespace pkv
