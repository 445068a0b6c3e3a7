// Device helpers shared by the library's HIP kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dt {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;   // MFMA bf16 operand
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// float -> bfloat16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// x ~= hi + lo with hi = bf16(x), lo = bf16(x - hi): 16 significant bits,
// so a bf16 x bf16 product with fp32 accumulation sees x to ~2^-17 relative.
__device__ __forceinline__ void split_hi_lo(float x, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_bf16(x);
  lo = f32_to_bf16(x - bf16_to_f32(hi));
}

// Monotone map of a float onto uint32 (larger float -> larger integer).
__device__ __forceinline__ uint32_t float_order(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float float_unorder(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(u);
}

// Selection key: larger value first, then lower index.  0 = empty.
__device__ __forceinline__ uint64_t make_key(float v, uint32_t idx) {
  return ((uint64_t)float_order(v) << 32) | (uint64_t)(0xffffffffu - idx);
}
__device__ __forceinline__ float key_value(uint64_t k) { return float_unorder((uint32_t)(k >> 32)); }
__device__ __forceinline__ uint32_t key_index(uint64_t k) { return 0xffffffffu - (uint32_t)k; }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl_xor(lo, mask, WAVE);
  hi = __shfl_xor(hi, mask, WAVE);
  return ((uint64_t)hi << 32) | lo;
}

// Sorted (descending) top-K list held in registers; all indexing is static.
template <int K>
struct TopK {
  uint64_t v[K];
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] = 0;
  }
  __device__ __forceinline__ void insert(uint64_t key) {
    if (key > v[K - 1]) {
#pragma unroll
      for (int i = 0; i < K; ++i) {
        uint64_t a = v[i];
        bool sw = key > a;
        v[i] = sw ? key : a;
        key = sw ? a : key;
      }
    }
  }
  // Merge with another descending list: keep the K largest of the union.
  __device__ __forceinline__ void merge(const uint64_t (&o)[K]) {
    uint64_t c[K];
#pragma unroll
    for (int i = 0; i < K; ++i) c[i] = v[i] > o[K - 1 - i] ? v[i] : o[K - 1 - i];
    // c is bitonic; sort descending
#pragma unroll
    for (int s = K / 2; s >= 1; s >>= 1) {
#pragma unroll
      for (int i = 0; i < K; ++i) {
        if ((i & s) == 0) {
          uint64_t a = c[i], b = c[i + s];
          c[i] = a > b ? a : b;
          c[i + s] = a > b ? b : a;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] = c[i];
  }
  // Butterfly all-reduce over `group` consecutive lanes (power of two <= 64).
  __device__ __forceinline__ void reduce_lanes(int group) {
    for (int m = 1; m < group; m <<= 1) {
      uint64_t o[K];
#pragma unroll
      for (int i = 0; i < K; ++i) o[i] = shfl_xor_u64(v[i], m);
      merge(o);
    }
  }
};

// (max, sum exp(x - max)) pair, combined in a fixed order.
// Compare-exchange keeping the larger key in a.
__device__ __forceinline__ void ce_desc(uint64_t& a, uint64_t& b) {
  const bool sw = b > a;
  const uint64_t hi = sw ? b : a, lo = sw ? a : b;
  a = hi;
  b = lo;
}

// Bitonic sorting network over N keys (N a power of two), descending.
template <int N>
__device__ __forceinline__ void bitonic_sort_desc(uint64_t (&a)[N]) {
#pragma unroll
  for (int size = 2; size <= N; size <<= 1)
#pragma unroll
    for (int stride = size / 2; stride > 0; stride >>= 1)
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          if ((i & size) == 0) ce_desc(a[i], a[j]);
          else ce_desc(a[j], a[i]);
        }
      }
}

// The K largest of NV keys (NV a power of two; key 0 marks an empty entry):
// K = 1 is a maximum; otherwise runs of min(K, NV) keys are sorted by a
// network and folded in with the bitonic merge.  Keys are distinct (the
// column is part of them), so the list equals K one-at-a-time insertions.
template <int K, int NV>
__device__ __forceinline__ void topk_of(TopK<K>& tk, uint64_t (&keys)[NV]) {
  if constexpr (K == 1) {
    uint64_t m = keys[0];
#pragma unroll
    for (int j = 1; j < NV; ++j) m = keys[j] > m ? keys[j] : m;
    tk.v[0] = m;
  } else {
    constexpr int R = NV < K ? NV : K;
#pragma unroll
    for (int c = 0; c < NV / R; ++c) {
      uint64_t run[R];
#pragma unroll
      for (int i = 0; i < R; ++i) run[i] = keys[c * R + i];
      bitonic_sort_desc<R>(run);
      if (c == 0) {
#pragma unroll
        for (int i = 0; i < K; ++i) tk.v[i] = i < R ? run[i] : 0ull;
      } else {
        if constexpr (R == K) tk.merge(run);    // more than one run only when NV > K
      }
    }
  }
}

struct MaxSum {
  float m, s;
  // e^(m - M) as the hardware 2^x of (m - M) log2(e); the exponent is <= 0,
  // and -inf (an empty part) gives 0
  __device__ __forceinline__ void combine(float m2, float s2) {
    float M = fmaxf(m, m2);
    if (M == -INFINITY) { m = M; s = 0.f; return; }
    s = s * __builtin_amdgcn_exp2f((m - M) * 1.44269504088896341f) +
        s2 * __builtin_amdgcn_exp2f((m2 - M) * 1.44269504088896341f);
    m = M;
  }
};

// Packed hi/lo activation planes of an [Mp][K] matrix (K % 32 == 0): block
// (m / 16, k / 32) of 16 rows x 32 K is 512 contiguous bf16 in MFMA operand
// order; lane l of the block holds row l % 16, K 8 (l / 16) .. + 8.
// Writes 8 consecutive columns k .. k + 7 (k % 8 == 0) of row m.
__device__ __forceinline__ void write_packed8(uint16_t* hi, uint16_t* lo, int K, int m, int k,
                                              const float (&y)[8]) {
  const int lane = (m & 15) + 16 * ((k & 31) >> 3);
  const long off = ((long)(m >> 4) * (K >> 5) + (k >> 5)) * 512 + lane * 8;
  uint32_t h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) split_hi_lo(y[i], h[i], l[i]);
  *(u32x4*)(hi + off) = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                              h[6] | (h[7] << 16)};
  *(u32x4*)(lo + off) = u32x4{l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16),
                              l[6] | (l[7] << 16)};
}

}  // namespace dt
