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
// merge: one workgroup (8 waves) per row
// ----------------------------------------------------------------------------
// Each thread folds up to MERGE_BATCH tiles per pass (loads issued together),
// each wave reduces by a butterfly, then lanes 0..7 of wave 0 reduce the 8
// wave results by another butterfly.  The (max, sum) pairs combine in the same
// fixed tree, so the result does not depend on timing.
constexpr int MERGE_THREADS = 512;

template <int KMAX>
__global__ __launch_bounds__(MERGE_THREADS) void k_merge(const float2* __restrict__ ms_part,
                                                         const uint64_t* __restrict__ key_part,
                                                         int ntiles, int kt, int k, int greedy,
                                                         int32_t* __restrict__ cand_tok,
                                                         float* __restrict__ cand_lp,
                                                         float* __restrict__ lse) {
  constexpr int MERGE_BATCH = KMAX >= 16 ? 2 : 4;
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  MaxSum ms{-INFINITY, 0.f};
  TopK<KMAX> tk;
  tk.clear();
  const float2* mrow = ms_part + (long)row * ntiles;
  const uint64_t* krow = key_part + (long)row * ntiles * kt;
  for (int t0 = 0; t0 < ntiles; t0 += MERGE_THREADS * MERGE_BATCH) {
    float2 p[MERGE_BATCH];
    uint64_t kv[MERGE_BATCH][KMAX];
#pragma unroll
    for (int b = 0; b < MERGE_BATCH; ++b) {
      const int t = t0 + b * MERGE_THREADS + tid;
      p[b] = t < ntiles ? mrow[t] : make_float2(-INFINITY, 0.f);
#pragma unroll
      for (int i = 0; i < KMAX; ++i) kv[b][i] = (t < ntiles && i < kt) ? krow[(long)t * kt + i] : 0ull;
    }
#pragma unroll
    for (int b = 0; b < MERGE_BATCH; ++b) {
      ms.combine(p[b].x, p[b].y);
#pragma unroll
      for (int i = 0; i < KMAX; ++i) tk.insert(kv[b][i]);
    }
  }
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

hipError_t launch_merge(const float2* ms_part, const uint64_t* key_part, int rows, int ntiles,
                        int kt, int k, int kmax, int greedy, int32_t* cand_tok, float* cand_lp,
                        float* lse, hipStream_t st) {
#define DT_MERGE(KM)                                                                        \
  hipLaunchKernelGGL(k_merge<KM>, dim3(rows), dim3(MERGE_THREADS), 0, st, ms_part, key_part,   \
                     ntiles, kt, k, greedy, cand_tok, cand_lp, lse)
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

// One workgroup per request.  Candidate c = i * keff + rank of frontier row i
// scores score_in[i] + cand_lp[i][rank]; the n_t = min(W, n_{t-1} keff) best
// by (score desc, c asc) take slots 0..n_t-1 in that order.  A candidate's
// rank is the number of candidates with a larger key (keys are distinct).
constexpr int BEAM_THREADS = 1024;

__global__ __launch_bounds__(BEAM_THREADS) void k_beam_select(BeamArgs b) {
  extern __shared__ uint64_t keys[];              // [ncand]
  const int r = blockIdx.x, tid = threadIdx.x;
  const int base = r * b.W;
  const int n_prev = b.t == 0 ? 1 : b.n_valid[r * b.D + b.t - 1];
  const int keff = b.greedy ? 1 : b.k;
  const int ncand = n_prev * keff;
  const int nkeep = min(b.W, ncand);
  for (int c = tid; c < ncand; c += BEAM_THREADS) {
    const int i = c / keff, rk = c % keff;
    const float sc = b.score_in[base + i] + b.cand_lp[(long)(base + i) * b.k + rk];
    keys[c] = make_key(sc, (uint32_t)c);
  }
  __syncthreads();
  const long pool = ((long)r * b.D + b.t) * b.W;
  for (int c = tid; c < ncand; c += BEAM_THREADS) {
    const uint64_t kc = keys[c];
    int rank = 0;
    for (int j = 0; j < ncand; ++j) rank += keys[j] > kc;
    if (rank < nkeep) {
      const int i = c / keff, rk = c % keff;
      const int32_t tk = b.cand_tok[(long)(base + i) * b.k + rk];
      const float sc = key_value(kc);
      b.pool_tok[pool + rank] = tk;
      b.pool_parent[pool + rank] = b.t == 0 ? -1 : i;
      b.pool_score[pool + rank] = sc;
      b.tok_out[base + rank] = tk;
      b.score_out[base + rank] = sc;
      b.src_out[base + rank] = base + i;
    }
  }
  for (int j = nkeep + tid; j < b.W; j += BEAM_THREADS) {
    b.pool_tok[pool + j] = -1;
    b.pool_parent[pool + j] = -1;
    b.pool_score[pool + j] = -INFINITY;
    b.tok_out[base + j] = -1;
    b.score_out[base + j] = -INFINITY;
    b.src_out[base + j] = -1;
  }
  if (tid == 0) b.n_valid[r * b.D + b.t] = nkeep;
  // padded rows beyond R*W stay empty
  if (r == 0)
    for (int j = b.R * b.W + tid; j < b.Mp; j += BEAM_THREADS) {
      b.tok_out[j] = -1;
      b.score_out[j] = -INFINITY;
      b.src_out[j] = -1;
    }
}

hipError_t launch_beam_select(const BeamArgs& b, hipStream_t st) {
  const int ncand_max = b.W * (b.greedy ? 1 : b.k);
  const size_t lds = (size_t)ncand_max * sizeof(uint64_t);
  hipLaunchKernelGGL(k_beam_select, dim3(b.R), dim3(BEAM_THREADS), lds, st, b);
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
