// Selection kernels: per-row log-sum-exp and top-k merge, the per-request
// global top-W beam step, the global top-B prune and the ancestor bitmask.
//
// Every selection orders by a total key (value desc, index asc) packed into a
// u64, so ties are broken identically on every run; no floating-point atomics.
#include "../../include/dartree.h"
#include "common.hpp"
#include "launch.hpp"

namespace dt {

// ----------------------------------------------------------------------------
// merge: per row, the head's tile partials -> log-sum-exp and top-k
// ----------------------------------------------------------------------------
// Two passes.  Pass 1: workgroup (row, s) folds the s-th of S contiguous
// ranges of tiles: the (max, sum) pair of tile t goes to thread t % 256, the
// range's keys (one contiguous array) are read in consecutive 16-byte pieces
// (a wave's load covers 1 KB) and folded into per-thread register top-k
// lists; a butterfly in each wave and one over the 4 wave results leave the
// range's (max, sum) and top-KMAX keys.  Pass 2: one wave per row folds the
// S range results by a butterfly and writes the row's children.  Every
// combination follows a fixed tree, so the result does not depend on timing.
constexpr int MERGE_THREADS = 256;
constexpr int MERGE_TILES = 128;           // slices per merge range at least

template <int KMAX>
__global__ __launch_bounds__(MERGE_THREADS) void k_merge_part(const float2* __restrict__ ms_part,
                                                              const uint64_t* __restrict__ key_part,
                                                              int ntiles, int kt,
                                                              float2* __restrict__ ms2,
                                                              uint64_t* __restrict__ key2,
                                                              const int32_t* skip) {
  if (skip && *skip) return;
  constexpr int BATCH = 4;
  const int row = blockIdx.x, s = blockIdx.y, S = gridDim.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t_lo = (int)((long)s * ntiles / S), t_hi = (int)((long)(s + 1) * ntiles / S);
  MaxSum ms{-INFINITY, 0.f};
  TopK<KMAX> tk;
  tk.clear();
  const float2* mrow = ms_part + (long)row * ntiles;
  // keys of the range: words [w_lo, w_hi) of the row's array, read as
  // aligned pairs where possible; the first chunk is requested before the
  // statistics are combined, so both arrive in one round trip
  const uint64_t* krow = key_part + (long)row * ntiles * kt;
  long w_lo = (long)t_lo * kt;
  const long w_hi = (long)t_hi * kt;
  const bool head_word = ((uintptr_t)(krow + w_lo) & 15) != 0 && w_lo < w_hi;
  if (head_word) ++w_lo;
  const long np = (w_hi - w_lo) / 2;
  const ulonglong2* kp = (const ulonglong2*)(krow + w_lo);
  ulonglong2 v[BATCH];
#pragma unroll
  for (int b = 0; b < BATCH; ++b) {
    const long f = b * MERGE_THREADS + tid;
    v[b] = f < np ? kp[f] : make_ulonglong2(0ull, 0ull);
  }
  for (int t0 = t_lo; t0 < t_hi; t0 += MERGE_THREADS * BATCH) {
    float2 p[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int t = t0 + b * MERGE_THREADS + tid;
      p[b] = t < t_hi ? mrow[t] : make_float2(-INFINITY, 0.f);
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) ms.combine(p[b].x, p[b].y);
  }
  if (head_word && tid == 0) tk.insert(krow[w_lo - 1]);
  for (long f0 = 0; f0 < np; f0 += MERGE_THREADS * BATCH) {
    if (f0 > 0) {
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        const long f = f0 + b * MERGE_THREADS + tid;
        v[b] = f < np ? kp[f] : make_ulonglong2(0ull, 0ull);
      }
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      tk.insert(v[b].x);
      tk.insert(v[b].y);
    }
  }
  if (((w_hi - w_lo) & 1) && tid == MERGE_THREADS - 1) tk.insert(krow[w_hi - 1]);

  for (int off = 1; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(ms.m, off, 64);
    const float s2 = __shfl_xor(ms.s, off, 64);
    ms.combine(m2, s2);
  }
  tk.reduce_lanes(64);
  constexpr int NWV = MERGE_THREADS / 64;
  __shared__ float2 wms[NWV];
  __shared__ uint64_t wkeys[NWV][KMAX];
  if (lane == 0) {
    wms[wave] = make_float2(ms.m, ms.s);
#pragma unroll
    for (int i = 0; i < KMAX; ++i) wkeys[wave][i] = tk.v[i];
  }
  __syncthreads();
  if (wave != 0) return;
  const int src = lane < NWV ? lane : 0;
  MaxSum tot{lane < NWV ? wms[src].x : -INFINITY, lane < NWV ? wms[src].y : 0.f};
  TopK<KMAX> all;
#pragma unroll
  for (int i = 0; i < KMAX; ++i) all.v[i] = lane < NWV ? wkeys[src][i] : 0ull;
  for (int off = 1; off < NWV; off <<= 1) {
    const float m2 = __shfl_xor(tot.m, off, 64);
    const float s2 = __shfl_xor(tot.s, off, 64);
    tot.combine(m2, s2);
  }
  all.reduce_lanes(NWV);
  if (lane != 0) return;
  const long o = (long)row * S + s;
  ms2[o] = make_float2(tot.m, tot.s);
#pragma unroll
  for (int i = 0; i < KMAX; ++i) key2[o * KMAX + i] = all.v[i];
}

// One wave per row: lane s < S holds range s; butterfly over S2 lanes (S
// rounded up to a power of two).
template <int KMAX>
__global__ __launch_bounds__(64) void k_merge_final(const float2* __restrict__ ms2,
                                                    const uint64_t* __restrict__ key2, int S,
                                                    int k, int greedy,
                                                    int32_t* __restrict__ cand_tok,
                                                    float* __restrict__ cand_lp,
                                                    float* __restrict__ lse) {
  const int row = blockIdx.x, lane = threadIdx.x;
  const bool have = lane < S;
  const long o = (long)row * S + lane;
  MaxSum tot{-INFINITY, 0.f};
  TopK<KMAX> all;
  all.clear();
  if (have) {
    const float2 e = ms2[o];
    tot = MaxSum{e.x, e.y};
#pragma unroll
    for (int i = 0; i < KMAX; ++i) all.v[i] = key2[o * KMAX + i];
  }
  int S2 = 1;
  while (S2 < S) S2 <<= 1;
  for (int off = 1; off < S2; off <<= 1) {
    const float m2 = __shfl_xor(tot.m, off, 64);
    const float s2 = __shfl_xor(tot.s, off, 64);
    tot.combine(m2, s2);
  }
  all.reduce_lanes(S2);
  if (lane != 0) return;
  const float L = greedy ? tot.m : tot.m + logf(tot.s);
  lse[row] = L;
  for (int j = 0; j < k; ++j) {
    uint64_t key = 0;
#pragma unroll
    for (int q = 0; q < KMAX; ++q)
      if (q == j) key = all.v[q];
    const bool ok = (!greedy || j == 0) && key != 0;
    cand_tok[(long)row * k + j] = ok ? (int32_t)key_index(key) : -1;
    cand_lp[(long)row * k + j] = ok ? (greedy ? 0.f : key_value(key) - L) : -INFINITY;
  }
}

hipError_t launch_merge_part(const float2* ms_part, const uint64_t* key_part, int rows,
                             int ntiles, int kt, int kmax, float2* ms2, uint64_t* key2,
                             hipStream_t st, const int32_t* skip) {
  const int S = merge_splits(ntiles);
#define DT_MERGE1(KM)                                                                        \
  hipLaunchKernelGGL(k_merge_part<KM>, dim3(rows, S), dim3(MERGE_THREADS), 0, st, ms_part,     \
                     key_part, ntiles, kt, ms2, key2, skip)
  switch (kmax) {
    case 1: DT_MERGE1(1); break;
    case 4: DT_MERGE1(4); break;
    case 8: DT_MERGE1(8); break;
    case 16: DT_MERGE1(16); break;
    default: return hipErrorInvalidValue;
  }
#undef DT_MERGE1
  return hipGetLastError();
}

int merge_splits(int ntiles) {
  const int s = ntiles / MERGE_TILES;
  return s < 1 ? 1 : (s > MERGE_SPLITS_MAX ? MERGE_SPLITS_MAX : s);
}

hipError_t launch_merge(const float2* ms_part, const uint64_t* key_part, int rows, int ntiles,
                        int kt, int k, int kmax, int greedy, float2* ms2, uint64_t* key2,
                        int32_t* cand_tok, float* cand_lp, float* lse, hipStream_t st) {
  const int S = merge_splits(ntiles);
#define DT_MERGE(KM)                                                                          \
  hipLaunchKernelGGL(k_merge_part<KM>, dim3(rows, S), dim3(MERGE_THREADS), 0, st, ms_part,      \
                     key_part, ntiles, kt, ms2, key2, nullptr);                                 \
  hipLaunchKernelGGL(k_merge_final<KM>, dim3(rows), dim3(64), 0, st, ms2, key2, S, k, greedy,   \
                     cand_tok, cand_lp, lse)
  switch (kmax) {
    case 1: DT_MERGE(1); break;
    case 4: DT_MERGE(4); break;
    case 8: DT_MERGE(8); break;
    case 16: DT_MERGE(16); break;
    default: return hipErrorInvalidValue;
  }
#undef DT_MERGE
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// beam bookkeeping
// ----------------------------------------------------------------------------
// Depth-0 frontier: row r*W of request r holds the root (token root_tok[r],
// score 0, state row r of s0); every other row is empty.
__global__ void k_beam_init(int R, int W, int Mp, const int32_t* __restrict__ root_tok,
                            int32_t* tok, float* score, int32_t* src) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < Mp) {
    const bool root = i < R * W && i % W == 0;
    tok[i] = root ? root_tok[i / W] : -1;
    score[i] = root ? 0.f : -INFINITY;
    src[i] = root ? i / W : -1;
  }
}

hipError_t launch_beam_init(int R, int W, int Mp, const int32_t* root_tok, int32_t* tok,
                            float* score, int32_t* src, hipStream_t st) {
  hipLaunchKernelGGL(k_beam_init, dim3((Mp + 255) / 256), dim3(256), 0, st, R, W, Mp, root_tok,
                     tok, score, src);
  return hipGetLastError();
}

// Rows for a stand-alone state update: tokens copied from the caller, state
// row i of the caller's input for row i, padded rows empty.
__global__ void k_fill_rows(int rows, int Mp, const int32_t* __restrict__ tok_in, int32_t* tok,
                            int32_t* src) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < Mp) {
    tok[i] = i < rows ? tok_in[i] : -1;
    src[i] = i < rows ? i : -1;
  }
}

hipError_t launch_fill_rows(int rows, int Mp, const int32_t* tok_in, int32_t* tok, int32_t* src,
                            hipStream_t st) {
  hipLaunchKernelGGL(k_fill_rows, dim3((Mp + 255) / 256), dim3(256), 0, st, rows, Mp, tok_in, tok,
                     src);
  return hipGetLastError();
}

// One workgroup per request, two phases.
// 1. Children of each frontier row i (16 lanes per row, four rows per wave):
//    the row's S <= 16 merge range results are folded by a butterfly into
//    (max, sum exp) and the top-keff keys; child rank j gets logp = value -
//    log-sum-exp (0 at T=0).
// 2. Candidate c = i * keff + j scores score_in[i] + logp; the
//    n_t = min(W, n_{t-1} keff) best by (score desc, c asc) take slots
//    0..n_t-1 in that order.  A candidate's slot is the number of candidates
//    with a larger key (keys are distinct), counted by several lanes each.
constexpr int BEAM_THREADS = 1024;

template <int KMAX>
__global__ __launch_bounds__(BEAM_THREADS) void k_beam_step(BeamArgs b) {
  extern __shared__ uint64_t keys[];                       // [ncand]
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rin = b.rpr_in > 0 ? b.rpr_in : b.W, rout = b.rpr_out > 0 ? b.rpr_out : b.W;
  const int base = r * rin, obase = r * rout;
  const int n_prev = b.t == 0 ? 1 : b.n_valid[r * b.D + b.t - 1];
  const int keff = b.greedy ? 1 : b.k;
  const int ncand = n_prev * keff;
  const int nkeep = min(b.W, ncand);
  const int ncand_max = b.W * keff;
  int32_t* c_tok = (int32_t*)(keys + ncand_max);           // [ncand]

  if (!b.ms2) {
    // children already chosen per row (cand_tok / cand_lp, stride k)
    for (int c = tid; c < ncand; c += BEAM_THREADS) {
      const int i = c / keff, j = c % keff;
      const long o = (long)(base + i) * b.k + j;
      c_tok[c] = b.cand_tok[o];
      keys[c] = make_key(b.score_in[base + i] + b.cand_lp[o], (uint32_t)c);
    }
  }
  int S2 = 1;
  while (S2 < b.S) S2 <<= 1;
  // four rows per wave, one per group of 16 lanes (S <= 16 range results per
  // row, so every butterfly stays inside its group).  Every row of the request
  // is read (rows past n_prev are ignored below), so these loads need not
  // wait for n_valid.
  constexpr int RPW = WAVE / 16;
  for (int i0 = wave * RPW; b.ms2 && i0 < rin; i0 += (BEAM_THREADS / WAVE) * RPW) {
    const int sl = lane & 15, i = i0 + (lane >> 4);
    const bool row_ok = i < rin;
    const long o = (long)(base + (row_ok ? i : 0)) * b.S + sl;
    MaxSum tot{-INFINITY, 0.f};
    TopK<KMAX> all;
    all.clear();
    if (row_ok && sl < b.S) {
      const float2 e = b.ms2[o];
      tot = MaxSum{e.x, e.y};
#pragma unroll
      for (int q = 0; q < KMAX; ++q) all.v[q] = b.key2[o * KMAX + q];
    }
    const float sp = row_ok ? b.score_in[base + i] : 0.f;
    for (int off = 1; off < S2; off <<= 1) {
      const float m2 = __shfl_xor(tot.m, off, 64);
      const float s2 = __shfl_xor(tot.s, off, 64);
      tot.combine(m2, s2);
    }
    all.reduce_lanes(S2);
    if (sl == 0 && i < n_prev) {
      const float L = b.greedy ? tot.m : tot.m + logf(tot.s);
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (j < keff) {
          const uint64_t key = all.v[j];
          const bool ok = key != 0;
          const float lp = ok ? (b.greedy ? 0.f : key_value(key) - L) : -INFINITY;
          c_tok[i * keff + j] = ok ? (int32_t)key_index(key) : -1;
          keys[i * keff + j] = make_key(sp + lp, (uint32_t)(i * keff + j));
        }
      }
    }
  }
  __syncthreads();
  const long pool = ((long)r * b.D + b.t) * b.W;
  // rank of each candidate = number of larger keys, counted by P lanes each
  // (strided subsets of the keys, summed by a butterfly)
  int P = 1;
  while (P < WAVE && ncand * (2 * P) <= BEAM_THREADS) P *= 2;
  for (int c0 = 0; c0 < ncand; c0 += BEAM_THREADS / P) {
    const int c = c0 + tid / P, p = tid % P;
    const bool live = c < ncand;
    const uint64_t kc = live ? keys[c] : 0ull;
    int rank = 0;
    if (live) {
#pragma unroll 8
      for (int j = p; j < ncand; j += P) rank += keys[j] > kc;
    }
    for (int off = 1; off < P; off <<= 1) rank += __shfl_xor(rank, off, 64);
    if (live && p == 0 && rank < nkeep) {
      const int i = c / keff;
      const int32_t tk = c_tok[c];
      const float sc = key_value(kc);
      b.pool_tok[pool + rank] = tk;
      b.pool_parent[pool + rank] = b.t == 0 ? -1 : i;
      b.pool_score[pool + rank] = sc;
      b.tok_out[obase + rank] = tk;
      b.score_out[obase + rank] = sc;
      b.src_out[obase + rank] = base + i;
    }
  }
  for (int j = nkeep + tid; j < b.W; j += BEAM_THREADS) {
    b.pool_tok[pool + j] = -1;
    b.pool_parent[pool + j] = -1;
    b.pool_score[pool + j] = -INFINITY;
  }
  for (int j = nkeep + tid; j < rout; j += BEAM_THREADS) {
    b.tok_out[obase + j] = -1;
    b.score_out[obase + j] = -INFINITY;
    b.src_out[obase + j] = -1;
  }
  if (tid == 0) b.n_valid[r * b.D + b.t] = nkeep;
  // padded rows beyond R * rpr_out stay empty
  if (r == 0)
    for (int j = b.R * rout + tid; j < b.Mp; j += BEAM_THREADS) {
      b.tok_out[j] = -1;
      b.score_out[j] = -INFINITY;
      b.src_out[j] = -1;
    }
}

// Markov variant: every row's residual source is its request's s0 row.
__global__ void k_markov_src(int rows, int W, int Mp, int32_t* src) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < Mp) src[i] = i < rows ? i / W : -1;
}

hipError_t launch_markov_src(int rows, int W, int Mp, int32_t* src, hipStream_t st) {
  hipLaunchKernelGGL(k_markov_src, dim3((Mp + 255) / 256), dim3(256), 0, st, rows, W, Mp, src);
  return hipGetLastError();
}

// Output-head row c, columns kk .. kk + 7, as floats (kk % 8 == 0).
__device__ __forceinline__ void u_row8(const CandArgs& a, int c, int kk, float (&u)[8]) {
  if (!a.u_bf16) {
    const float* p = (const float*)a.Ut + (long)c * a.d + kk;
#pragma unroll
    for (int e = 0; e < 8; ++e) u[e] = p[e];
    return;
  }
  const uint16_t* p;
  if (a.u_packed) {
    // grouped packed layout: block (g, kb, t), lane (c % 16) + 16 ((kk % 32) / 8)
    constexpr int TPG = PACK_ROWS / 16;
    const int tile = c / 16;
    const int lane = (c & 15) + 16 * ((kk & 31) >> 3);
    p = (const uint16_t*)a.Ut +
        ((((long)(tile / TPG) * (a.d / 32) + kk / 32) * TPG + tile % TPG) * 512 + lane * 8);
  } else {
    p = (const uint16_t*)a.Ut + (long)c * a.d + kk;
  }
  const u32x4 v = *(const u32x4*)p;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    u[2 * e] = bf16_to_f32(v[e] & 0xffffu);
    u[2 * e + 1] = bf16_to_f32(v[e] >> 16);
  }
}

// Base-candidate variant: one workgroup per row i.  z_c = s'_i . U[c] for
// the depth's n_cand candidates (fp32), logp_c = z_c / T - lse_i, and the
// row's k best candidates by (logp desc, token asc); T == 0: the
// lowest-index argmax of z over the candidates, logp 0.
__global__ __launch_bounds__(256) void k_cand_score(CandArgs a) {
  __shared__ float zc[DT_MAX_K];
  const int i = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = i / a.W;
  const int32_t* cand = a.cand_base + ((long)r * a.D + a.t) * a.n_cand;
  const float* s = a.s + (long)i * a.d;
  for (int q = wave; q < a.n_cand; q += 4) {
    const int c = cand[q];
    float acc = 0.f;
    for (int kk = lane * 8; kk < a.d; kk += 64 * 8) {
      float u[8];
      u_row8(a, c, kk, u);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf(s[kk + e], u[e], acc);
    }
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (lane == 0) zc[q] = acc;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  int32_t* ot = a.cand_tok + (long)i * a.k;
  float* ol = a.cand_lp + (long)i * a.k;
  for (int j = 0; j < a.k; ++j) {
    ot[j] = -1;
    ol[j] = -INFINITY;
  }
  if (a.greedy) {
    int best = -1;
    float bz = -INFINITY;
    for (int q = 0; q < a.n_cand; ++q) {
      const int c = cand[q];
      if (best < 0 || zc[q] > bz || (zc[q] == bz && c < best)) {
        best = c;
        bz = zc[q];
      }
    }
    ot[0] = best;
    ol[0] = 0.f;
    return;
  }
  // insertion of the candidates into a (logp desc, token asc) list of k
  int nt = 0;
  for (int q = 0; q < a.n_cand; ++q) {
    const int c = cand[q];
    const float lp = zc[q] * a.inv_T - a.lse[i];
    int pos = nt;
    while (pos > 0 && (lp > ol[pos - 1] || (lp == ol[pos - 1] && c < ot[pos - 1]))) --pos;
    if (pos >= a.k) continue;
    for (int m = (nt < a.k ? nt : a.k - 1); m > pos; --m) {
      ot[m] = ot[m - 1];
      ol[m] = ol[m - 1];
    }
    ot[pos] = c;
    ol[pos] = lp;
    if (nt < a.k) ++nt;
  }
}

hipError_t launch_cand_score(const CandArgs& a, int rows, hipStream_t st) {
  hipLaunchKernelGGL(k_cand_score, dim3(rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_beam_step(const BeamArgs& b, hipStream_t st) {
  const int keff = b.greedy ? 1 : b.k;
  const size_t lds = (size_t)b.W * keff * (sizeof(uint64_t) + sizeof(int32_t));
  switch (b.kmax) {
    case 1: hipLaunchKernelGGL(k_beam_step<1>, dim3(b.R), dim3(BEAM_THREADS), lds, st, b); break;
    case 4: hipLaunchKernelGGL(k_beam_step<4>, dim3(b.R), dim3(BEAM_THREADS), lds, st, b); break;
    case 8: hipLaunchKernelGGL(k_beam_step<8>, dim3(b.R), dim3(BEAM_THREADS), lds, st, b); break;
    case 16: hipLaunchKernelGGL(k_beam_step<16>, dim3(b.R), dim3(BEAM_THREADS), lds, st, b); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// deferred pruning: global top-B per request
// ----------------------------------------------------------------------------
// Node f = t * W + j (t 0-based).  Key: prio = score + beta * (t + 1) desc,
// then f asc (= depth asc, slot asc).  Selected nodes are emitted in f order;
// the emitted index of a node is the number of selected nodes before it.
constexpr int PRUNE_THREADS = 1024;

__global__ __launch_bounds__(PRUNE_THREADS) void k_prune(
    const float* __restrict__ pool_score, const int32_t* __restrict__ pool_parent,
    const int32_t* __restrict__ n_valid, int D, int W, int B, float beta,
    int32_t* sel_node, int32_t* sel_parent, int32_t* sel_depth, int32_t* n_sel) {
  extern __shared__ unsigned char sm[];
  const int r = blockIdx.x, tid = threadIdx.x;
  const int P = D * W;
  uint64_t* keys = (uint64_t*)sm;                    // [P]; 0 = invalid node
  int32_t* emit = (int32_t*)(keys + P);              // [P]; emitted index or -1
  __shared__ int nv[DT_MAX_DEPTH];
  if (tid < D) nv[tid] = n_valid[r * D + tid];
  __syncthreads();
  int total = 0;
  for (int t = 0; t < D; ++t) total += nv[t];
  for (int f = tid; f < P; f += PRUNE_THREADS) {
    const int t = f / W, j = f % W;
    const bool valid = j < nv[t];
    // two roundings (no contraction into an fma), as documented
    const float pr = __fadd_rn(pool_score[(long)r * P + f], __fmul_rn(beta, (float)(t + 1)));
    keys[f] = valid ? make_key(pr, (uint32_t)f) : 0ull;
  }
  __syncthreads();
  const int m = min(B, total);
  for (int f = tid; f < P; f += PRUNE_THREADS) {
    const uint64_t kf = keys[f];
    int rank = 0;
    if (kf != 0)
      for (int g = 0; g < P; ++g) rank += keys[g] > kf;
    emit[f] = (kf != 0 && rank < m) ? 1 : 0;
  }
  __syncthreads();
  // emitted index = number of selected nodes with a smaller flat index
  __shared__ int wsum[PRUNE_THREADS / 64];
  // serial prefix over chunks of PRUNE_THREADS nodes
  int carry = 0;
  for (int c0 = 0; c0 < P; c0 += PRUNE_THREADS) {
    const int f = c0 + tid;
    const int v = f < P ? emit[f] : 0;
    // inclusive scan within the wave
    int x = v;
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, 64);
      if ((tid & 63) >= off) x += y;
    }
    if ((tid & 63) == 63) wsum[tid >> 6] = x;
    __syncthreads();
    int before = carry;
    for (int w = 0; w < (tid >> 6); ++w) before += wsum[w];
    int chunk_total = 0;
    for (int w = 0; w < PRUNE_THREADS / 64; ++w) chunk_total += wsum[w];
    __syncthreads();
    if (f < P) emit[f] = v ? before + x - 1 : -1;
    carry += chunk_total;
    __syncthreads();
  }
  const long o = (long)r * B;
  for (int f = tid; f < P; f += PRUNE_THREADS) {
    const int e = emit[f];
    if (e >= 0) {
      const int t = f / W;
      sel_node[o + e] = f;
      sel_depth[o + e] = t + 1;
      const int pj = t == 0 ? -1 : pool_parent[(long)r * P + f];
      sel_parent[o + e] = (pj >= 0 && pj < W) ? emit[(t - 1) * W + pj] : -1;
    }
  }
  for (int i = m + tid; i < B; i += PRUNE_THREADS) {
    sel_node[o + i] = -1;
    sel_parent[o + i] = -1;
    sel_depth[o + i] = -1;
  }
  if (tid == 0) n_sel[r] = m;
}

hipError_t launch_prune(const float* pool_score, const int32_t* pool_parent,
                        const int32_t* n_valid, int R, int D, int W, int B, float beta,
                        int32_t* sel_node, int32_t* sel_parent, int32_t* sel_depth,
                        int32_t* n_sel, hipStream_t st) {
  const size_t lds = (size_t)D * W * (sizeof(uint64_t) + sizeof(int32_t));
  hipLaunchKernelGGL(k_prune, dim3(R), dim3(PRUNE_THREADS), lds, st, pool_score, pool_parent,
                     n_valid, D, W, B, beta, sel_node, sel_parent, sel_depth, n_sel);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// ancestor bitmask: one thread per (request, row, word)
// ----------------------------------------------------------------------------
__global__ void k_mask(const int32_t* __restrict__ sel_parent, const int32_t* __restrict__ n_sel,
                       int R, int B, int words, uint32_t* mask) {
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long)R * B * words) return;
  const int w = gid % words;
  const int i = (gid / words) % B;
  const int r = gid / ((long)words * B);
  uint32_t bits = 0u;
  if (i < n_sel[r]) {
    const int32_t* par = sel_parent + (long)r * B;
    // walk from the node to its depth-1 ancestor; parents precede children,
    // and a parent index that does not (corrupt input) ends the walk
    for (int a = i; a >= 0;) {
      if ((a >> 5) == w) bits |= 1u << (a & 31);
      const int p = par[a];
      if (p >= a) break;
      a = p;
    }
  }
  mask[gid] = bits;
}

hipError_t launch_mask(const int32_t* sel_parent, const int32_t* n_sel, int R, int B,
                       uint32_t* mask, hipStream_t st) {
  const int words = (B + 31) / 32;
  const long n = (long)R * B * words;
  hipLaunchKernelGGL(k_mask, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, sel_parent,
                     n_sel, R, B, words, mask);
  return hipGetLastError();
}

}  // namespace dt
