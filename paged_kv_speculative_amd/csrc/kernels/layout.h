// Tiled layout of one (page, KV head) slab of 16 tokens x head_dim channels.
//
// The verification kernel reads a page with 16-byte loads whose lanes land
// directly in the operand registers of the gfx950 16x16x32 bf16 MFMA:
//   K is the A operand of S^T = K Q^T: lane (t = lane%16, j = lane/16) holds
//     token t, channels (D/4)*j + 8*s .. +7 for k-step s;
//   V is the A operand of O^T = V^T P^T: lane (m = lane%16, j = lane/16)
//     holds 4 consecutive tokens 4j..4j+3 of one channel, for two (bf16) or
//     four (fp8) neighbouring channels per 16-byte load.
// With the layouts below every such load instruction of a wave reads one
// contiguous kilobyte.  The pool-update kernel writes through the same maps.
#pragma once

namespace pkv {

__host__ __device__ inline int k_index_bf16(int t, int c, int D) {
  int q = D / 4, j = c / q, r = c % q;
  return (r / 8) * 512 + t * 32 + j * 8 + (r % 8);
}

__host__ __device__ inline int k_index_fp8(int t, int c, int D) {
  int q = D / 4, j = c / q, r = c % q;
  return (r / 16) * 1024 + t * 64 + j * 16 + (r % 16);
}

__host__ __device__ inline int v_index_bf16(int t, int c) {
  return ((c / 2) * 4 + t / 4) * 8 + (c % 2) * 4 + (t % 4);
}

__host__ __device__ inline int v_index_fp8(int t, int c) {
  return ((c / 4) * 4 + t / 4) * 16 + (c % 4) * 4 + (t % 4);
}

__host__ __device__ inline int index_f32(int t, int c, int D) { return t * D + c; }

}  // namespace pkv
