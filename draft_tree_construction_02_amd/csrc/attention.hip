// One tree-attention layer of the verification forward (gfx950).
//
// Rows are (tree query i, query head hh within a key/value group), so the
// Hq / Hkv query heads that share a key/value head share every K/V tile.  A
// workgroup (4 waves x 16 rows) owns one key/value head, 64 rows and one
// contiguous range of keys, where keys [0, P) are the prefix (always visible)
// and keys [P, P + n) are the tree nodes (visible where the query's ancestor
// bitmask has the bit).  Keys are processed in blocks of 64 in one pass: the
// next block's K and V are loaded into registers while the current block,
// staged in LDS (K row-major, V transposed), feeds S^T = K Q^T and
// O^T += V^T P^T on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  In
// that orientation a lane's O values all belong to its own query row, so the
// softmax needs no exchange between lanes except when a row's reference
// maximum moves (see the block body).  Scores are in log2 units and
// exponentiated with exp2; P is rounded to bf16 for the PV product.  A
// combine kernel merges the key ranges:
//   out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
#include <cmath>
#include <type_traits>

#include "../../include/dartree.h"
#include "common.hpp"
#include "launch.hpp"

namespace dt {

constexpr int AT_THREADS = 256;
constexpr int AT_ROWS = 64;        // rows per workgroup (16 per wave)
constexpr int AT_KB = 64;          // keys per block
constexpr int HD = 128;
constexpr int KLD = HD + 8;        // K tile row stride (bf16)
constexpr int VLD = AT_KB + 8;     // transposed V tile row stride (bf16)
constexpr int AT_CH = AT_KB * (HD / 8) / AT_THREADS;   // 16-byte chunks per thread per tile
static_assert(AT_CH == 4 && AT_KB == 64 && AT_THREADS == 256, "staging map: 32 key pairs x 8 dim groups");

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* kp;
  const uint16_t* vp;
  const uint16_t* kt;
  const uint16_t* vt;
  const uint32_t* mask;
  int n, P, Hq, Hkv, group, words;
  float scale;
  int nsplit, keys_per_split;
  float* opart;      // [nsplit][Hkv][n*group][HD]
  float2* mlpart;    // [nsplit][Hkv][n*group]
};

__device__ __forceinline__ const uint16_t* key_row(const AttnArgs& a, const uint16_t* pre,
                                                   const uint16_t* tree, int key, int g) {
  return key < a.P ? pre + ((long)key * a.Hkv + g) * HD
                   : tree + ((long)(key - a.P) * a.Hkv + g) * HD;
}

// This thread's share of keys [kb, kb + 64): the key pair kk = 2 (tid % 32),
// kk + 1 and dims 16 (tid / 32) .. + 16 of K and V (keys >= kend are 0).
// kv[2 e + h] / vv[2 e + h] hold key kk + e, dims 16 (tid / 32) + 8 h .. + 8.
__device__ __forceinline__ void load_kv(const AttnArgs& a, int g, int kb, int kend,
                                        u32x4 (&kv)[AT_CH], u32x4 (&vv)[AT_CH]) {
  const int kk = 2 * (threadIdx.x % 32), d16 = 16 * (threadIdx.x / 32);
  // every load is issued (rows past the range re-read the last key and are
  // zeroed afterwards), so the vector-memory counter is the same on every path
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int key = kb + kk + e;
    const int kc = min(key, kend - 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      kv[2 * e + h] = *(const u32x4*)(key_row(a, a.kp, a.kt, kc, g) + d16 + 8 * h);
      vv[2 * e + h] = *(const u32x4*)(key_row(a, a.vp, a.vt, kc, g) + d16 + 8 * h);
    }
  }
}

__device__ __forceinline__ void zero_past_end(int kb, int kend, u32x4 (&kv)[AT_CH],
                                              u32x4 (&vv)[AT_CH]) {
  const int kk = 2 * (threadIdx.x % 32);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const uint32_t keep = kb + kk + e < kend ? 0xffffffffu : 0u;   // select, no branch
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        kv[2 * e + h][w] &= keep;
        vv[2 * e + h][w] &= keep;
      }
  }
}

// K rows as they are; V transposed, each 32-bit write holding the pair of
// keys (kk, kk + 1) of one dim, so a wave's writes of one dim are 32
// consecutive words.
__device__ __forceinline__ void store_kv(const u32x4 (&kv)[AT_CH], const u32x4 (&vv)[AT_CH],
                                         uint16_t* Ks, uint16_t* Vts) {
  const int kk = 2 * (threadIdx.x % 32), d16 = 16 * (threadIdx.x / 32);
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int h = 0; h < 2; ++h) *(u32x4*)(Ks + (kk + e) * KLD + d16 + 8 * h) = kv[2 * e + h];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t a0 = vv[h][w], a1 = vv[2 + h][w];    // keys kk, kk + 1: dims 2 w, 2 w + 1
      const int d = d16 + 8 * h + 2 * w;
      *(uint32_t*)(Vts + d * VLD + kk) = (a0 & 0xffffu) | (a1 << 16);
      *(uint32_t*)(Vts + (d + 1) * VLD + kk) = (a0 >> 16) | (a1 & 0xffff0000u);
    }
}

__global__ __launch_bounds__(AT_THREADS) void k_tree_attn(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[AT_KB * KLD];
  __shared__ __attribute__((aligned(16))) uint16_t Vts[HD * VLD];
  __shared__ uint32_t Ms[AT_ROWS * (DT_MAX_B / 32)];      // ancestor masks of the 64 rows
  const int g = blockIdx.x, rb = blockIdx.y, split = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int nrows = a.n * a.group;
  const int kbeg = split * a.keys_per_split;
  const int kend = min(a.P + a.n, kbeg + a.keys_per_split);

  // this lane's row (the MFMA B operand of S^T and the A operand of P V)
  const int row = rb * AT_ROWS + wave * 16 + r16;
  const bool row_ok = row < nrows;
  const int qi = row_ok ? row / a.group : 0;
  const int qh = g * a.group + (row_ok ? row % a.group : 0);
  u32x4 qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    qf[kk] = row_ok ? *(const u32x4*)(a.q + ((long)qi * a.Hq + qh) * HD + kk * 32 + g4 * 8)
                    : u32x4{0u, 0u, 0u, 0u};

  for (int idx = tid; idx < AT_ROWS * a.words; idx += AT_THREADS) {
    const int lr = idx / a.words, w = idx % a.words, rr = rb * AT_ROWS + lr;
    Ms[lr * (DT_MAX_B / 32) + w] = rr < nrows ? a.mask[(long)(rr / a.group) * a.words + w] : 0u;
  }
  const uint32_t* mrow = Ms + (wave * 16 + r16) * (DT_MAX_B / 32);

  // Scores are kept in log2 units (s * scale * log2 e), so the softmax is
  // exp2 of the shifted score; m, the running maximum, is in the same units.
  const float sl2 = a.scale * 1.4426950408889634f;
  float m = -INFINITY, l = 0.f;
  // O^T = V^T P^T: o[t][i] = O(row r16, dim 16 t + 4 g4 + i), so a lane holds
  // only its own row and the per-row rescale needs no exchange between lanes
  f32x4 o[HD / 16];
#pragma unroll
  for (int t = 0; t < HD / 16; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // two register sets: block b + 2 is requested while block b is computed
  u32x4 kv[2][AT_CH], vv[2][AT_CH];
  load_kv(a, g, kbeg, kend, kv[0], vv[0]);
  load_kv(a, g, kbeg + AT_KB, kend, kv[1], vv[1]);
  const int plain_end = min(a.P, kend);     // keys below this need no mask
  auto block = [&](int kb, auto set_tag) {
    constexpr int SET = decltype(set_tag)::value;
    __syncthreads();                       // every wave is done with the previous tiles
    zero_past_end(kb, kend, kv[SET], vv[SET]);
    store_kv(kv[SET], vv[SET], Ks, Vts);
    __syncthreads();
    load_kv(a, g, kb + 2 * AT_KB, kend, kv[SET], vv[SET]);

    // S^T: st[h][r] = s(key = kb + 16 h + 4 g4 + r, row = lane % 16), in
    // log2 units; masked or missing keys are -inf
    float st[4][4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u32x4 kf = *(const u32x4*)(Ks + (16 * h + r16) * KLD + kk * 32 + g4 * 8);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf),
                                                      __builtin_bit_cast(bf16x8, qf[kk]), acc,
                                                      0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) st[h][r] = acc[r] * sl2;
    }
    if (!(kb + AT_KB <= plain_end)) {      // wave-uniform: prefix blocks skip the mask
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kb + 16 * h + 4 * g4 + r;
          bool vis = key < kend;
          if (vis && key >= a.P) {
            const int j = key - a.P;
            vis = (mrow[j >> 5] >> (j & 31)) & 1u;
          }
          if (!vis) st[h][r] = -INFINITY;
        }
    }
    if (!row_ok) {
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) st[h][r] = -INFINITY;
    }
    // online softmax against a per-row reference m (not the running maximum):
    // p = exp2(s - m) is exact for any reference (O and l share it, and the
    // combine rescales by 2^(m - M)), so O is rescaled only when a score
    // exceeds m by more than RESCALE, which keeps p <= 2^RESCALE; the decision
    // is wave-uniform, and in the common case the block needs no exchange
    // between lanes.  l is summed per lane and reduced across the row's four
    // lane groups once, at the end.
    constexpr float RESCALE = 16.f;
    float lm = -INFINITY;
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) lm = fmaxf(lm, st[h][r]);
    if (__ballot(lm > m + RESCALE) != 0) {
      float bm = fmaxf(lm, __shfl_xor(lm, 16, 64));
      bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
      if (bm > m + RESCALE) {                 // this row takes a new reference
        const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - bm);
        l *= alpha;
#pragma unroll
        for (int t = 0; t < HD / 16; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[t][i] *= alpha;
        m = bm;
      }
    }
    const float msub = m == -INFINITY ? 0.f : m;     // no visible key yet: p = 0
    float p[4][4];
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[h][r] = __builtin_amdgcn_exp2f(st[h][r] - msub);     // exp2(-inf) = 0
        l += p[h][r];
      }
    // O^T += V^T P^T, 32 keys per MFMA.  k index 8 g4 + e of lane group g4
    // <-> key 32 q + 4 g4 + e (e < 4) and 32 q + 16 + 4 g4 + e - 4 (e >= 4):
    // the B operand (P^T) is then this lane's own p[2 q][.], p[2 q + 1][.],
    // rounded to bf16, and the A operand (V^T) two 8-byte pieces of a V^T row
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      typedef __attribute__((ext_vector_type(2))) float f2;
      typedef __attribute__((ext_vector_type(2))) __bf16 b2;
      uint32_t pk[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int h = 2 * qq + e / 2, r = 2 * (e % 2);
        pk[e] = __builtin_bit_cast(uint32_t,
                                   __builtin_convertvector(f2{p[h][r], p[h][r + 1]}, b2));
      }
      const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
      for (int t = 0; t < HD / 16; ++t) {
        const int dim = 16 * t + r16;
        const uint2 v0 = *(const uint2*)(Vts + dim * VLD + 32 * qq + 4 * g4);
        const uint2 v1 = *(const uint2*)(Vts + dim * VLD + 32 * qq + 16 + 4 * g4);
        const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{v0.x, v0.y, v1.x, v1.y});
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[t], 0, 0, 0);
      }
    }
  };
  // blocks in pairs; a block past the range (odd count) sees only masked
  // keys and leaves m, l and O unchanged
  for (int kb = kbeg; kb < kend; kb += 2 * AT_KB) {
    block(kb, std::integral_constant<int, 0>{});
    block(kb + AT_KB, std::integral_constant<int, 1>{});
  }

  // the row's sum over its four lane groups (all hold the same reference m)
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  // this lane's row, dims 16 t + 4 g4 .. + 3
  const long base = ((long)split * a.Hkv + g) * nrows;
  if (row_ok) {
#pragma unroll
    for (int t = 0; t < HD / 16; ++t)
      *(f32x4*)(a.opart + (base + row) * HD + 16 * t + 4 * g4) = o[t];
    if (g4 == 0) a.mlpart[base + row] = make_float2(m, l);
  }
}

// out[i][h][4 j .. 4 j + 3] for row (i, hh) of key/value head g = h / group:
// out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s (m in log2 units).
__global__ void k_tree_attn_combine(AttnArgs a, float* __restrict__ out) {
  const int nrows = a.n * a.group;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long)a.Hkv * nrows * (HD / 4)) return;
  const int d4 = gid % (HD / 4);
  const int row = (gid / (HD / 4)) % nrows;
  const int g = gid / ((long)(HD / 4) * nrows);
  float M = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s)
    M = fmaxf(M, a.mlpart[((long)s * a.Hkv + g) * nrows + row].x);
  f32x4 num = f32x4{0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (M != -INFINITY)
    for (int s = 0; s < a.nsplit; ++s) {
      const long b = ((long)s * a.Hkv + g) * nrows + row;
      const float2 ml = a.mlpart[b];
      const float w = ml.x == -INFINITY ? 0.f : exp2f(ml.x - M);
      const f32x4 v = *(const f32x4*)(a.opart + b * HD + 4 * d4);
      num += w * v;
      den += w * ml.y;
    }
  const int i = row / a.group, h = g * a.group + row % a.group;
  *(f32x4*)(out + ((long)i * a.Hq + h) * HD + 4 * d4) =
      den > 0.f ? num / den : f32x4{0.f, 0.f, 0.f, 0.f};
}

// Key ranges: about DT_ATTN_WGS workgroups (several per CU, so waves hide each
// other's latencies) with whole 64-key blocks per range.
#ifndef DT_ATTN_WGS
#define DT_ATTN_WGS 512
#endif
static void attn_plan(int n, int P, int Hkv, int group, int* nsplit, int* kps) {
  const int keys = P + n;
  const int rblocks = (n * group + AT_ROWS - 1) / AT_ROWS;
  int s = (DT_ATTN_WGS + Hkv * rblocks - 1) / (Hkv * rblocks);
  const int maxs = (keys + AT_KB - 1) / AT_KB;
  if (s > maxs) s = maxs;
  if (s < 1) s = 1;
  int per = (keys + s - 1) / s;
  per = (per + AT_KB - 1) / AT_KB * AT_KB;
  *kps = per;
  *nsplit = (keys + per - 1) / per;
}

}  // namespace dt

using namespace dt;

extern "C" size_t tree_attention_workspace_size(int n_tree, int P, int Hq, int Hkv, int hd) {
  if (n_tree < 1 || n_tree > DT_MAX_B || P < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv || hd != HD)
    return 0;
  int ns, kps;
  attn_plan(n_tree, P, Hkv, Hq / Hkv, &ns, &kps);
  const size_t rows = (size_t)Hkv * n_tree * (Hq / Hkv);
  const size_t o = ((size_t)ns * rows * HD * 4 + 255) / 256 * 256;
  return o + (size_t)ns * rows * sizeof(float2);
}

extern "C" int tree_attention_verify(const void* q, const void* k_prefix, const void* v_prefix,
                                     const void* k_tree, const void* v_tree, const uint32_t* mask,
                                     int n_tree, int P, int Hq, int Hkv, int hd, float scale,
                                     float* out, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  if (!q || !k_tree || !v_tree || !mask || !out) return DT_EINVAL;
  if (P > 0 && (!k_prefix || !v_prefix)) return DT_EINVAL;
  if (n_tree < 1 || P < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv || !std::isfinite(scale)) return DT_EINVAL;
  if (hd != HD || n_tree > DT_MAX_B) return DT_EUNSUPPORTED;
  const size_t need = tree_attention_workspace_size(n_tree, P, Hq, Hkv, hd);
  if (!workspace || workspace_bytes < need) return DT_EWORKSPACE;
  AttnArgs a;
  a.q = (const uint16_t*)q;
  a.kp = (const uint16_t*)k_prefix;
  a.vp = (const uint16_t*)v_prefix;
  a.kt = (const uint16_t*)k_tree;
  a.vt = (const uint16_t*)v_tree;
  a.mask = mask;
  a.n = n_tree;
  a.P = P;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.group = Hq / Hkv;
  a.words = (n_tree + 31) / 32;
  a.scale = scale;
  attn_plan(n_tree, P, Hkv, a.group, &a.nsplit, &a.keys_per_split);
  const size_t rows = (size_t)Hkv * n_tree * a.group;
  a.opart = (float*)workspace;
  a.mlpart = (float2*)((char*)workspace +
                       ((size_t)a.nsplit * rows * HD * 4 + 255) / 256 * 256);
  struct Ctx {
    AttnArgs a;
    float* out;
    hipStream_t st;
  } ctx{a, out, (hipStream_t)stream};
  auto run = [](void* p) -> hipError_t {
    Ctx& c = *(Ctx*)p;
    const int rblocks = (c.a.n * c.a.group + AT_ROWS - 1) / AT_ROWS;
    hipLaunchKernelGGL(k_tree_attn, dim3(c.a.Hkv, rblocks, c.a.nsplit), dim3(AT_THREADS), 0,
                       c.st, c.a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long tot = (long)c.a.Hkv * c.a.n * c.a.group * (HD / 4);
    hipLaunchKernelGGL(k_tree_attn_combine, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0,
                       c.st, c.a, c.out);
    return hipGetLastError();
  };
  return dt::timed_launch(DT_K_ATTN, ctx.st, run, &ctx) == hipSuccess ? DT_OK : DT_EHIP;
}
