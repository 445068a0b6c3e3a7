// Layout kernels: packing of bf16 weights into MFMA-operand blocks (once per
// model load) and forming the state-update input x = E[tok] + h_t as packed
// hi/lo planes (once per depth).
#include "common.hpp"
#include "launch.hpp"

namespace dt {

// One thread per 16 bytes of the packed output.  Rows are grouped by 128
// (8 tiles of 16); block (g, kb, t) holds rows 128 g + 16 t .. + 15 and K
// 32 kb .. + 31, and inside it lane l holds row 128 g + 16 t + l % 16, K
// 32 kb + 8 (l / 16) .. + 8.  Rows >= N are zero.
__global__ __launch_bounds__(256) void k_pack_weight(const uint16_t* __restrict__ src,
                                                     uint16_t* __restrict__ dst, int N, int K) {
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int kblocks = K / 32;
  const long nchunks = (long)((N + PACK_ROWS - 1) / PACK_ROWS) * (PACK_ROWS / 16) * kblocks * 64;
  if (gid >= nchunks) return;
  const int lane = gid & 63;
  const long blk = gid >> 6;
  const int t = blk % (PACK_ROWS / 16);
  const long rest = blk / (PACK_ROWS / 16);
  const int kb = rest % kblocks;
  const long g = rest / kblocks;
  const long n = g * PACK_ROWS + t * 16 + (lane & 15);
  const int k = kb * 32 + (lane >> 4) * 8;
  u32x4 v = u32x4{0u, 0u, 0u, 0u};
  if (n < N) v = *(const u32x4*)(src + n * K + k);
  *(u32x4*)(dst + gid * 8) = v;
}

hipError_t launch_pack_weight(const uint16_t* src, uint16_t* dst, int N, int K, hipStream_t st) {
  const long n = (long)((N + PACK_ROWS - 1) / PACK_ROWS) * (PACK_ROWS / 16) * (K / 32) * 64;
  hipLaunchKernelGGL(k_pack_weight, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src, dst,
                     N, K);
  return hipGetLastError();
}

// One thread per (row m < Mp, 8 consecutive columns k).
__global__ __launch_bounds__(256) void k_prep_x(PrepArgs p) {
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int d8 = p.d / 8;
  if (gid >= (long)p.Mp * d8) return;
  const int m = gid / d8, k = (gid % d8) * 8;
  const int tok = m < p.rows ? p.tok[m] : -1;
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = 0.f;
  if (tok >= 0) {
    const u32x4 e = *(const u32x4*)(p.E + (long)tok * p.d + k);
    const float* h = p.h + (long)(m / p.rpr) * p.h_req_stride + k;
    const float4 h0 = *(const float4*)h, h1 = *(const float4*)(h + 4);
    y[0] = bf16_to_f32(e[0] & 0xffffu) + h0.x;
    y[1] = bf16_to_f32(e[0] >> 16) + h0.y;
    y[2] = bf16_to_f32(e[1] & 0xffffu) + h0.z;
    y[3] = bf16_to_f32(e[1] >> 16) + h0.w;
    y[4] = bf16_to_f32(e[2] & 0xffffu) + h1.x;
    y[5] = bf16_to_f32(e[2] >> 16) + h1.y;
    y[6] = bf16_to_f32(e[3] & 0xffffu) + h1.z;
    y[7] = bf16_to_f32(e[3] >> 16) + h1.w;
  }
  write_packed8(p.hi, p.lo, p.d, m, k, y);
}

hipError_t launch_prep_x(const PrepArgs& p, hipStream_t st) {
  const long n = (long)p.Mp * (p.d / 8);
  hipLaunchKernelGGL(k_prep_x, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace dt
