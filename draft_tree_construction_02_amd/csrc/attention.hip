// One tree-attention layer of the verification forward (gfx950).
//
// Rows are (tree query i, query head hh within a key/value group), so the
// Hq / Hkv query heads that share a key/value head share every K/V tile.  A
// workgroup (4 waves x 16 rows) owns one key/value head, 64 rows and one
// contiguous range of keys, where keys [0, P) are the prefix (always visible)
// and keys [P, P + n) are the tree nodes (visible where the query's ancestor
// bitmask has the bit).  For each 32-key block the K and V tiles are staged in
// LDS; S^T = K Q^T runs on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
// Pass 1 finds each row's maximum over the range, pass 2 accumulates
// l = sum exp(s - max) in fp32 and O = P V with P rounded to bf16.  A combine
// kernel merges the key ranges: out = sum_s e^{m_s - M} O_s / sum_s e^{m_s - M} l_s.
#include <cmath>

#include "../../include/dartree.h"
#include "common.hpp"

namespace dt {

constexpr int AT_THREADS = 256;
constexpr int AT_ROWS = 64;        // rows per workgroup (16 per wave)
constexpr int AT_KB = 32;          // keys per block
constexpr int HD = 128;
constexpr int KLD = HD + 8;        // K tile row stride (bf16)
constexpr int VLD = AT_KB + 8;     // transposed V tile row stride (bf16)

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

// Stage K [32][128] and V^T [128][32] of keys [kb, kb + 32) into LDS.
__device__ __forceinline__ void stage_kv(const AttnArgs& a, int g, int kb, int kend,
                                         uint16_t* Ks, uint16_t* Vts) {
  const int tid = threadIdx.x;
  // 32 keys x 16 chunks of 8 bf16 = 512 chunks, 2 per thread
  for (int c = tid; c < AT_KB * (HD / 8); c += AT_THREADS) {
    const int kk = c / (HD / 8), d8 = (c % (HD / 8)) * 8;
    const int key = kb + kk;
    u32x4 kv = u32x4{0u, 0u, 0u, 0u}, vv = u32x4{0u, 0u, 0u, 0u};
    if (key < kend) {
      kv = *(const u32x4*)(key_row(a, a.kp, a.kt, key, g) + d8);
      vv = *(const u32x4*)(key_row(a, a.vp, a.vt, key, g) + d8);
    }
    *(u32x4*)(Ks + kk * KLD + d8) = kv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      Vts[(d8 + 2 * e) * VLD + kk] = (uint16_t)(vv[e] & 0xffffu);
      Vts[(d8 + 2 * e + 1) * VLD + kk] = (uint16_t)(vv[e] >> 16);
    }
  }
}

// S^T for 32 keys x 16 rows of this wave: st[h][r] = s(key = kb + 16 h + 4 g + r,
// row = lane % 16), scaled; masked or missing keys are -inf.
__device__ __forceinline__ void scores(const AttnArgs& a, const uint16_t* Ks, const u32x4 (&qf)[4],
                                       int kb, int kend, int qi, bool row_ok, float (&st)[2][4]) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u32x4 kf = *(const u32x4*)(Ks + (16 * h + r16) * KLD + kk * 32 + g4 * 8);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf),
                                                    __builtin_bit_cast(bf16x8, qf[kk]), acc, 0,
                                                    0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = kb + 16 * h + 4 * g4 + r;
      bool vis = row_ok && key < kend;
      if (vis && key >= a.P) {
        const int j = key - a.P;
        vis = (a.mask[(long)qi * a.words + (j >> 5)] >> (j & 31)) & 1u;
      }
      st[h][r] = vis ? acc[r] * a.scale : -INFINITY;
    }
  }
}

__global__ __launch_bounds__(AT_THREADS) void k_tree_attn(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[AT_KB * KLD];
  __shared__ __attribute__((aligned(16))) uint16_t Vts[HD * VLD];
  const int g = blockIdx.x, rb = blockIdx.y, split = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int nrows = a.n * a.group;
  const int kbeg = split * a.keys_per_split;
  const int kend = min(a.P + a.n, kbeg + a.keys_per_split);

  // this lane's row (as the MFMA B operand / S^T column)
  const int row = rb * AT_ROWS + wave * 16 + r16;
  const bool row_ok = row < nrows;
  const int qi = row_ok ? row / a.group : 0;
  const int qh = g * a.group + (row_ok ? row % a.group : 0);
  u32x4 qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    qf[kk] = row_ok ? *(const u32x4*)(a.q + ((long)qi * a.Hq + qh) * HD + kk * 32 + g4 * 8)
                    : u32x4{0u, 0u, 0u, 0u};

  // pass 1: row maximum over the key range
  float mx = -INFINITY;
  for (int kb = kbeg; kb < kend; kb += AT_KB) {
    __syncthreads();
    stage_kv(a, g, kb, kend, Ks, Vts);
    __syncthreads();
    float st[2][4];
    scores(a, Ks, qf, kb, kend, qi, row_ok, st);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, st[h][r]);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));

  // pass 2: l and O relative to mx
  float l = 0.f;
  f32x4 o[HD / 16];
#pragma unroll
  for (int t = 0; t < HD / 16; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kb = kbeg; kb < kend; kb += AT_KB) {
    __syncthreads();
    stage_kv(a, g, kb, kend, Ks, Vts);
    __syncthreads();
    float st[2][4];
    scores(a, Ks, qf, kb, kend, qi, row_ok, st);
    uint32_t pk[4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const float p0 = mx == -INFINITY ? 0.f : expf(st[h][r] - mx);
        const float p1 = mx == -INFINITY ? 0.f : expf(st[h][r + 1] - mx);
        l += p0 + p1;
        pk[h * 2 + r / 2] = f32_to_bf16(p0) | (f32_to_bf16(p1) << 16);
      }
    // P as the A operand: row = lane % 16, MFMA k index 8 g4 + e <-> key
    // 4 g4 + e (e < 4) and 16 + 4 g4 + e - 4 (e >= 4)
    const bf16x8 pa = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
    for (int t = 0; t < HD / 16; ++t) {
      const int dim = 16 * t + r16;
      const uint2 v0 = *(const uint2*)(Vts + dim * VLD + 4 * g4);
      const uint2 v1 = *(const uint2*)(Vts + dim * VLD + 16 + 4 * g4);
      const bf16x8 vb = __builtin_bit_cast(bf16x8, u32x4{v0.x, v0.y, v1.x, v1.y});
      o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, o[t], 0, 0, 0);
    }
  }
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);

  // O lane layout: row 4 g4 + r of the wave, dim 16 t + r16
  const long base = ((long)split * a.Hkv + g) * nrows;
#pragma unroll
  for (int t = 0; t < HD / 16; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int orow = rb * AT_ROWS + wave * 16 + 4 * g4 + r;
      if (orow < nrows) a.opart[(base + orow) * HD + 16 * t + r16] = o[t][r];
    }
  if (row_ok && g4 == 0) a.mlpart[base + row] = make_float2(mx, l);
}

// out[i][h][:] for row (i, hh) of key/value head g = h / group.
__global__ void k_tree_attn_combine(AttnArgs a, float* __restrict__ out) {
  const int nrows = a.n * a.group;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long)a.Hkv * nrows * HD) return;
  const int dim = gid % HD;
  const int row = (gid / HD) % nrows;
  const int g = gid / ((long)HD * nrows);
  float M = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s)
    M = fmaxf(M, a.mlpart[((long)s * a.Hkv + g) * nrows + row].x);
  float num = 0.f, den = 0.f;
  if (M != -INFINITY)
    for (int s = 0; s < a.nsplit; ++s) {
      const long b = ((long)s * a.Hkv + g) * nrows + row;
      const float2 ml = a.mlpart[b];
      const float w = ml.x == -INFINITY ? 0.f : expf(ml.x - M);
      num += w * a.opart[b * HD + dim];
      den += w * ml.y;
    }
  const int i = row / a.group, h = g * a.group + row % a.group;
  out[((long)i * a.Hq + h) * HD + dim] = den > 0.f ? num / den : 0.f;
}

static void attn_plan(int n, int P, int Hkv, int group, int* nsplit, int* kps) {
  const int keys = P + n;
  const int rblocks = (n * group + AT_ROWS - 1) / AT_ROWS;
  int s = (512 + Hkv * rblocks - 1) / (Hkv * rblocks);
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
  hipStream_t st = (hipStream_t)stream;
  const int rblocks = (n_tree * a.group + AT_ROWS - 1) / AT_ROWS;
  hipLaunchKernelGGL(k_tree_attn, dim3(Hkv, rblocks, a.nsplit), dim3(AT_THREADS), 0, st, a);
  if (hipGetLastError() != hipSuccess) return DT_EHIP;
  const long tot = (long)Hkv * n_tree * a.group * HD;
  hipLaunchKernelGGL(k_tree_attn_combine, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st,
                     a, out);
  return hipGetLastError() == hipSuccess ? DT_OK : DT_EHIP;
}
