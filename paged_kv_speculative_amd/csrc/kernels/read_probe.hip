// Read-rate reference for the verification kernel (a measurement aid, not a
// step of the path): one launch reads the K and V slabs of every (sequence,
// KV head, page) position that spec_verify_attention reads for the same
// arguments, with the same partition over waves (equal contiguous ranges of
// positions, one wave per SIMD), the same 16-byte non-temporal buffer loads
// and four pages in flight per wave, and no arithmetic beyond folding the
// bytes into one word per wave.  Its duration is what this access pattern
// costs on the device; the verification kernel's duration over the same
// bytes is compared with it.

#include <hip/hip_runtime.h>

#include <string>

#include "../common.h"

namespace pkv {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRing = 4;          // pages in flight per wave
constexpr int kIdsPerFill = 256;  // block-table entries staged in LDS per refill
constexpr int kBufferFlags = 0x00020000;
constexpr int kStreamPolicy = 2;  // non-temporal

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct ProbeParams {
  const char* k_pages;
  const char* v_pages;
  const int* block_table;
  const int* seq_lens;
  unsigned* sink;     // [waves] folded words
  long slab_bytes;
  int batch, Hkv, bt_stride, n_waves;
};

// Page prefix of the batch (pages per sequence) into s_cum[0..batch].
__device__ void page_prefix(const ProbeParams& P, int* s_cum, int* s_part) {
  const int t = threadIdx.x;
  const int per = (P.batch + kThreads - 1) / kThreads;
  const int b0 = min(P.batch, t * per), b1 = min(P.batch, b0 + per);
  int local = 0;
  for (int b = b0; b < b1; ++b) local += (P.seq_lens[b] + 15) >> 4;
  s_part[t] = local;
  __syncthreads();
  for (int o = 1; o < kThreads; o <<= 1) {
    const int v = t >= o ? s_part[t - o] : 0;
    __syncthreads();
    s_part[t] += v;
    __syncthreads();
  }
  int run = s_part[t] - local;
  for (int b = b0; b < b1; ++b) {
    s_cum[b] = run;
    run += (P.seq_lens[b] + 15) >> 4;
  }
  if (t == kThreads - 1) s_cum[P.batch] = s_part[t];
  __syncthreads();
}

template <int L>  // 1 KiB loads per slab
__global__ __launch_bounds__(kThreads) void page_read_kernel(ProbeParams P) {
  extern __shared__ int s_dyn[];
  int* s_cum = s_dyn;
  int* s_part = s_cum + P.batch + 1;
  // this wave's staged page ids and heads
  int* s_ids = s_part + kThreads + (threadIdx.x >> 6) * 2 * kIdsPerFill;
  int* s_gs = s_ids + kIdsPerFill;
  page_prefix(P, s_cum, s_part);
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const long W = long(P.Hkv) * s_cum[P.batch];
  if (wave >= P.n_waves || W == 0) return;
  const int lo = int(wave * W / P.n_waves), hi = int((wave + 1) * W / P.n_waves);
  // page id of position p: sequence by binary search over the prefix
  auto id_of = [&](int p) {
    int a = 0, z = P.batch - 1;
    while (a < z) {
      const int mid = (a + z + 1) >> 1;
      if (long(P.Hkv) * s_cum[mid] <= p) a = mid;
      else z = mid - 1;
    }
    const int np = s_cum[a + 1] - s_cum[a];
    const int off = p - P.Hkv * s_cum[a];
    const int g = off / np, page = off - g * np;
    return make_int2(P.block_table[long(a) * P.bt_stride + page], g);
  };
  const long page_stride = long(P.Hkv) * P.slab_bytes;
  u32x4 ring[kRing][2 * L];
  int gs[kRing];
  u32x4 acc = {0u, 0u, 0u, 0u};
  auto issue = [&](int r, int id, int g, bool valid) {
    const char* kb = P.k_pages + long(id) * page_stride + long(g) * P.slab_bytes;
    const char* vb = P.v_pages + long(id) * page_stride + long(g) * P.slab_bytes;
    const int nrec = valid ? int(P.slab_bytes) : 0;
    const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kb), 0, nrec, kBufferFlags);
    const auto rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vb), 0, nrec, kBufferFlags);
#pragma unroll
    for (int u = 0; u < L; ++u) {
      ring[r][u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, lane * 16 + u * 1024, 0, kStreamPolicy));
      ring[r][L + u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, lane * 16 + u * 1024, 0, kStreamPolicy));
    }
    gs[r] = g;
  };
  // Per fill of up to kIdsPerFill positions: the page ids and heads go to
  // this wave's LDS slice first (their loads drain the wave once per fill;
  // LDS is private to the wave, so no workgroup barrier), then the pages
  // stream with kRing in flight.
  for (int base = lo; base < hi; base += kIdsPerFill) {
    const int n = min(kIdsPerFill, hi - base);
    for (int j = lane; j < n; j += 64) {
      const int2 v = id_of(base + j);
      s_ids[j] = v.x;
      s_gs[j] = v.y;
    }
#pragma unroll
    for (int r = 0; r < kRing; ++r) {
      const bool v = r < n;
      issue(r, v ? s_ids[r] : 0, v ? s_gs[r] : 0, v);
    }
    for (int i0 = 0; i0 < n; i0 += kRing) {
#pragma unroll
      for (int r = 0; r < kRing; ++r) {
#pragma unroll
        for (int u = 0; u < 2 * L; ++u) acc ^= ring[r][u];
        const int nx = i0 + r + kRing;
        const bool v = nx < n;
        issue(r, v ? s_ids[nx] : 0, v ? s_gs[nx] : 0, v);
      }
    }
  }
  const unsigned f = acc.x ^ acc.y ^ acc.z ^ acc.w ^ unsigned(gs[0]);
  if (lane == 0) P.sink[wave] = f;
}

}  // namespace

}  // namespace pkv

using namespace pkv;

extern "C" pkv_status pkv_page_read_probe(const pkv_verify_args* a, uint32_t* sink, int32_t n_waves, void* stream) {
  if (!a || !sink) return fail(PKV_ERR_INVALID_ARG, "null argument");
  if (a->batch < 1 || a->batch > 4096 || a->num_kv_heads < 1 || a->page_size != kPageSize)
    return fail(PKV_ERR_INVALID_ARG, "batch in [1, 4096], num_kv_heads >= 1 and page size 16 required");
  if (!a->k_pages || !a->v_pages || !a->block_table || !a->seq_lens)
    return fail(PKV_ERR_INVALID_ARG, "null device pointer");
  if (n_waves < kWaves || n_waves % kWaves) return fail(PKV_ERR_INVALID_ARG, "n_waves must be a positive multiple of 4");
  ProbeParams p{};
  p.k_pages = static_cast<const char*>(a->k_pages);
  p.v_pages = static_cast<const char*>(a->v_pages);
  p.block_table = a->block_table;
  p.seq_lens = a->seq_lens;
  p.sink = sink;
  p.slab_bytes = pkv_page_bytes(a->kv_dtype, a->page_size, a->head_dim);
  p.batch = a->batch;
  p.Hkv = a->num_kv_heads;
  p.bt_stride = a->block_table_stride;
  p.n_waves = n_waves;
  if (p.slab_bytes <= 0 || p.slab_bytes % 1024) return fail(PKV_ERR_UNSUPPORTED, "slab size must be a multiple of 1 KiB");
  const size_t smem = (size_t(a->batch) + 1 + kThreads + size_t(kWaves) * 2 * kIdsPerFill) * sizeof(int);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(unsigned(n_waves / kWaves));
  switch (p.slab_bytes / 1024) {
    case 1: hipLaunchKernelGGL(page_read_kernel<1>, grid, dim3(kThreads), smem, s, p); break;
    case 2: hipLaunchKernelGGL(page_read_kernel<2>, grid, dim3(kThreads), smem, s, p); break;
    case 4: hipLaunchKernelGGL(page_read_kernel<4>, grid, dim3(kThreads), smem, s, p); break;
    case 8: hipLaunchKernelGGL(page_read_kernel<8>, grid, dim3(kThreads), smem, s, p); break;
    default: return fail(PKV_ERR_UNSUPPORTED, "slab size must be 1, 2, 4 or 8 KiB");
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_DEVICE, std::string("read probe launch: ") + hipGetErrorString(e));
  return PKV_OK;
}
