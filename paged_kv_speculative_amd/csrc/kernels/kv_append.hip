// Pool-update kernel: applies PoolTask records (copy-on-write page copies,
// token scatter into the tiled page layout with optional FP8 quantisation,
// block-table entries and sequence lengths) in stream order.
//
// FP8 quantisation (reading of atozofsoftwareengineering.blog, section
// "Custom FP8 Quantized Memory Block Layout", per-block scales S_K, S_V):
// a fresh page gets, per KV head, scale = amax/448 over the tokens written
// into it by this call (1 when amax is 0); values are x * (1/scale) in fp32,
// clamped to +-448 and rounded to nearest-even OCP E4M3.

#include <hip/hip_runtime.h>

#include "../common.h"
#include "layout.h"

namespace pkv {

namespace {

constexpr int kThreads = 256;

__device__ inline float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ inline float block_max(float v, float* red) {
  v = wave_max(v);
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < kThreads / 64; ++w) r = fmaxf(r, red[w]);
  return r;
}

__device__ inline float load_src(const void* src, int dtype, long idx) {
  if (dtype == PKV_BF16) {
    unsigned short b = static_cast<const unsigned short*>(src)[idx];
    return __uint_as_float(unsigned(b) << 16);
  }
  return static_cast<const float*>(src)[idx];
}

__device__ inline unsigned char quant_e4m3(float x, float inv) {
  float y = x * inv;
  y = fminf(fmaxf(y, -448.0f), 448.0f);
  // hardware OCP E4M3 conversion, round to nearest even
  unsigned packed = __builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false);
  return static_cast<unsigned char>(packed & 0xFF);
}

__global__ __launch_bounds__(kThreads) void pool_update_kernel(PoolDevice dev, PoolUpdateBatch batch) {
  const PoolTask t = batch.tasks[blockIdx.x];
  const int H = batch.num_kv_heads, D = batch.head_dim;
  const long pb = batch.page_bytes;
  const bool fp8 = batch.kv_dtype == PKV_FP8_E4M3;
  __shared__ float red[kThreads / 64];
  __shared__ float s_scale[2];

  if (t.cow_src >= 0) {
    const long n16 = H * pb / 16;
    const uint4* sk = reinterpret_cast<const uint4*>(static_cast<const char*>(dev.k_pages) + t.cow_src * H * pb);
    const uint4* sv = reinterpret_cast<const uint4*>(static_cast<const char*>(dev.v_pages) + t.cow_src * H * pb);
    uint4* dk = reinterpret_cast<uint4*>(static_cast<char*>(dev.k_pages) + long(t.page) * H * pb);
    uint4* dv = reinterpret_cast<uint4*>(static_cast<char*>(dev.v_pages) + long(t.page) * H * pb);
    for (long i = threadIdx.x; i < n16; i += kThreads) {
      dk[i] = sk[i];
      dv[i] = sv[i];
    }
    if (fp8) {
      for (int h = threadIdx.x; h < H; h += kThreads) {
        dev.k_scale[long(t.page) * H + h] = dev.k_scale[long(t.cow_src) * H + h];
        dev.v_scale[long(t.page) * H + h] = dev.v_scale[long(t.cow_src) * H + h];
      }
    }
  }
  __syncthreads();

  if (t.n > 0) {
    const int per_tok = H * D;
    for (int h = 0; h < H; ++h) {
      float inv_k = 1.0f, inv_v = 1.0f;
      if (fp8) {
        if (t.flags & kFresh) {
          float ak = 0.0f, av = 0.0f;
          for (int e = threadIdx.x; e < t.n * D; e += kThreads) {
            long idx = long(t.src_row + e / D) * per_tok + h * D + (e % D);
            ak = fmaxf(ak, fabsf(load_src(dev.k_src, batch.src_dtype, idx)));
            av = fmaxf(av, fabsf(load_src(dev.v_src, batch.src_dtype, idx)));
          }
          ak = block_max(ak, red);
          av = block_max(av, red);
          if (threadIdx.x == 0) {
            float sk = ak == 0.0f ? 1.0f : ak / 448.0f;
            float sv = av == 0.0f ? 1.0f : av / 448.0f;
            dev.k_scale[long(t.page) * H + h] = sk;
            dev.v_scale[long(t.page) * H + h] = sv;
            s_scale[0] = sk;
            s_scale[1] = sv;
          }
        } else if (threadIdx.x == 0) {
          s_scale[0] = dev.k_scale[long(t.page) * H + h];
          s_scale[1] = dev.v_scale[long(t.page) * H + h];
        }
        __syncthreads();
        inv_k = 1.0f / s_scale[0];
        inv_v = 1.0f / s_scale[1];
      }
      char* kslab = static_cast<char*>(dev.k_pages) + (long(t.page) * H + h) * pb;
      char* vslab = static_cast<char*>(dev.v_pages) + (long(t.page) * H + h) * pb;
      for (int e = threadIdx.x; e < t.n * D; e += kThreads) {
        const int tok = e / D, c = e % D, slot = t.slot_begin + tok;
        const long idx = long(t.src_row + tok) * per_tok + h * D + c;
        if (batch.kv_dtype == PKV_F32) {
          reinterpret_cast<float*>(kslab)[index_f32(slot, c, D)] = load_src(dev.k_src, PKV_F32, idx);
          reinterpret_cast<float*>(vslab)[index_f32(slot, c, D)] = load_src(dev.v_src, PKV_F32, idx);
        } else if (batch.kv_dtype == PKV_BF16) {
          reinterpret_cast<unsigned short*>(kslab)[k_index_bf16(slot, c, D)] =
              static_cast<const unsigned short*>(dev.k_src)[idx];
          reinterpret_cast<unsigned short*>(vslab)[v_index_bf16(slot, c)] =
              static_cast<const unsigned short*>(dev.v_src)[idx];
        } else {
          reinterpret_cast<unsigned char*>(kslab)[k_index_fp8(slot, c, D)] =
              quant_e4m3(load_src(dev.k_src, batch.src_dtype, idx), inv_k);
          reinterpret_cast<unsigned char*>(vslab)[v_index_fp8(slot, c)] =
              quant_e4m3(load_src(dev.v_src, batch.src_dtype, idx), inv_v);
        }
      }
      __syncthreads();
    }
  }

  if (threadIdx.x == 0) {
    if (t.flags & kWriteTable) dev.block_table[long(t.row) * batch.bt_stride + t.logical] = t.page;
    if (t.flags & kSetLen) dev.seq_lens[t.row] = t.new_len;
  }
}

}  // namespace

pkv_status launch_pool_update(const PoolDevice& dev, const PoolUpdateBatch& batch, void* stream) {
  if (batch.n_tasks <= 0) return PKV_OK;
  hipLaunchKernelGGL(pool_update_kernel, dim3(batch.n_tasks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), dev, batch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_DEVICE, std::string("pool update launch: ") + hipGetErrorString(e));
  return PKV_OK;
}

}  // namespace pkv
