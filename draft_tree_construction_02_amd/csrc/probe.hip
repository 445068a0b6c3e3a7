// Measurement probes.  The streaming read probe of device memory gives the
// practical read-bandwidth ceiling that the head's weight stream is measured
// against, next to the chip's nominal 8 TB/s; the matrix-core rate probe (at
// the end of the file) gives the bf16 product rate for a given operand data,
// the bound of the 128-row head's hi/lo products.  Every byte of the buffer is read once with non-temporal
// 16-byte loads; the result is the sum of the buffer's 64-bit words modulo
// 2^64, so the loads cannot be removed and the read can be checked exactly
// (integer addition is order-free, so the sum does not depend on the grid).
//
// Read probe: every byte of the buffer is read once with non-temporal
// 16-byte loads (as described above).  Access pattern: one workgroup of four
// waves per compute unit, each wave
// streaming its own contiguous share of the buffer with 16 loads of 1 KB in
// flight.  Measured on MI355X over 2 GiB this reads at ~7.1 TB/s, where a
// grid-stride loop over all lanes reaches ~5.8 TB/s and many short per-
// workgroup chunks less still (more concurrent streams, lower throughput).
#include "../../include/dartree.h"
#include "common.hpp"

namespace dt {
namespace {

constexpr int PROBE_THREADS = 256;
constexpr int PROBE_WAVES = PROBE_THREADS / WAVE;
constexpr int PROBE_UNROLL = 16;    // 16-byte loads in flight per lane (1 KB per wave each)

constexpr int PROBE_MAX_DEVICES = 64;
int g_probe_cus[PROBE_MAX_DEVICES] = {};

int probe_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < PROBE_MAX_DEVICES && g_probe_cus[dev] > 0) return g_probe_cus[dev];
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  if (dev < PROBE_MAX_DEVICES) g_probe_cus[dev] = n;
  return n;
}

__global__ __launch_bounds__(64) void k_probe_clear(unsigned long long* sum) {
  if (threadIdx.x == 0) *sum = 0ull;
}

__device__ __forceinline__ unsigned long long words_of(u32x4 v) {
  return (((unsigned long long)v.y << 32) | v.x) + (((unsigned long long)v.w << 32) | v.z);
}

// n16 16-byte pieces; `tail` (when non-null) is one more 8-byte word.  Wave w
// of the grid reads pieces [w n16 / nw, (w + 1) n16 / nw).
__global__ __launch_bounds__(PROBE_THREADS) void k_probe_read(const u32x4* __restrict__ buf,
                                                              long n16,
                                                              const unsigned long long* tail,
                                                              unsigned long long* sum) {
  const int lane = threadIdx.x & (WAVE - 1);
  const long nw = (long)gridDim.x * PROBE_WAVES;
  const long w = (long)blockIdx.x * PROBE_WAVES + threadIdx.x / WAVE;
  const long hi = (w + 1) * n16 / nw;
  long i = w * n16 / nw + lane;
  unsigned long long acc = 0ull;
  // full rounds: the last load of a round is at i + (UNROLL - 1) WAVE < hi
  for (; i + (PROBE_UNROLL - 1) * WAVE < hi; i += PROBE_UNROLL * WAVE) {
    u32x4 v[PROBE_UNROLL];
#pragma unroll
    for (int u = 0; u < PROBE_UNROLL; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * WAVE);
#pragma unroll
    for (int u = 0; u < PROBE_UNROLL; ++u) acc += words_of(v[u]);
  }
  for (; i < hi; i += WAVE) acc += words_of(__builtin_nontemporal_load(buf + i));
  if (tail && blockIdx.x == 0 && threadIdx.x == 0) acc += *tail;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  __shared__ unsigned long long part[PROBE_WAVES];
  if ((threadIdx.x & (WAVE - 1)) == 0) part[threadIdx.x / WAVE] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long t = 0ull;
#pragma unroll
    for (int j = 0; j < PROBE_WAVES; ++j) t += part[j];
    atomicAdd(sum, t);                  // one device-scope vector atomic per workgroup
  }
}

// Matrix-core rate probe: one workgroup of 8 waves (two per SIMD) per
// compute unit; each wave holds 4 weight-like and 4 activation-like bf16
// fragments of the operand buffer in registers and runs `iters` rounds of 16
// `32x32x16` products into 4 accumulators (per round and K half, the 4 weight
// fragments times the hi-like, then times the lo-like activation fragment).
// The operands stay in registers, so the time is the matrix cores' alone,
// for whatever data the buffer holds.
constexpr int MFMA_PROBE_WAVES = 8;
constexpr int MFMA_PROBE_THREADS = 64 * MFMA_PROBE_WAVES;
constexpr int MFMA_PROBE_FRAGS = 8;                        // 1 KB fragments per wave
constexpr long MFMA_PROBE_WG_BYTES = (long)MFMA_PROBE_WAVES * MFMA_PROBE_FRAGS * 1024;

typedef __attribute__((ext_vector_type(16))) float f32x16_p;

__global__ __launch_bounds__(MFMA_PROBE_THREADS) void k_mfma_probe(const u32x4* __restrict__ ops,
                                                                   int iters, float* out) {
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const u32x4* src = ops + ((long)blockIdx.x * MFMA_PROBE_WAVES + wave) * MFMA_PROBE_FRAGS * WAVE;
  bf16x8 w[4], a[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    w[q] = __builtin_bit_cast(bf16x8, src[q * WAVE + lane]);
    a[q] = __builtin_bit_cast(bf16x8, src[(4 + q) * WAVE + lane]);
  }
  f32x16_p acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[q], a[2 * st], acc[q], 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[q], a[2 * st + 1], acc[q], 0, 0, 0);
    }
    // keeps the loop counter's update between the round's last product and
    // the loop branch: a branch issued right after a product measured ~30%
    // slower per round on gfx950 (the compiler otherwise moves the update to
    // the top of the round)
    __builtin_amdgcn_sched_barrier(0);
  }
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) sum += acc[c][e];
  out[(long)blockIdx.x * MFMA_PROBE_THREADS + threadIdx.x] = sum;
}

}  // namespace
}  // namespace dt

using namespace dt;

extern "C" int hbm_read_probe(const void* buf, size_t bytes, uint64_t* sum, void* stream) {
  if (!sum || (bytes > 0 && !buf)) return DT_EINVAL;
  if (bytes % 8 != 0 || (bytes > 0 && (uintptr_t)buf % 16 != 0)) return DT_EINVAL;
  if (bytes / 16 > (size_t)(1L << 40)) return DT_EUNSUPPORTED;
  const hipStream_t st = (hipStream_t)stream;
  unsigned long long* out = (unsigned long long*)sum;
  hipLaunchKernelGGL(k_probe_clear, dim3(1), dim3(64), 0, st, out);
  if (hipGetLastError() != hipSuccess) return DT_EHIP;
  if (bytes == 0) return DT_OK;
  const long n16 = (long)(bytes / 16);
  const unsigned long long* tail =
      bytes % 16 ? (const unsigned long long*)((const char*)buf + bytes - 8) : nullptr;
  // one workgroup per compute unit, fewer when there are not 16 KB per wave
  const long want = (n16 + PROBE_WAVES * PROBE_UNROLL * WAVE - 1) / (PROBE_WAVES * PROBE_UNROLL * WAVE);
  const int grid = (int)std::max(1L, std::min(want, (long)probe_cus()));
  hipLaunchKernelGGL(k_probe_read, dim3(grid), dim3(PROBE_THREADS), 0, st, (const u32x4*)buf, n16,
                     tail, out);
  return hipGetLastError() == hipSuccess ? DT_OK : DT_EHIP;
}

extern "C" int mfma_rate_probe(const void* operands, size_t bytes, int iters, float* out,
                               size_t out_count, void* stream) {
  if (!operands || !out || iters < 0) return DT_EINVAL;
  if ((uintptr_t)operands % 16 != 0) return DT_EINVAL;
  const int cus = probe_cus();
  if (bytes < (size_t)cus * MFMA_PROBE_WG_BYTES || out_count < (size_t)cus * MFMA_PROBE_THREADS)
    return DT_EINVAL;
  hipLaunchKernelGGL(k_mfma_probe, dim3(cus), dim3(MFMA_PROBE_THREADS), 0, (hipStream_t)stream,
                     (const u32x4*)operands, iters, out);
  return hipGetLastError() == hipSuccess ? DT_OK : DT_EHIP;
}
