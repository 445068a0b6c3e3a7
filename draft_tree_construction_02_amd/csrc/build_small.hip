// Whole supertree build for a small fp32 head in one launch (gfx950).
//
// The depth-wise batched construction ("DARTree: Teaching a Chain-Trained
// Corrector to Think in Trees", Core Mechanism; "Technische Samenvatting:
// DARTree", Methodologie part 1) run by one workgroup per request: for each
// depth, the state update s' = s_parent + GELU((E[tok] + h_t) W1) W2 of every
// frontier row, the scaled logits y = s' U / T, each row's log-sum-exp and
// top-k children, candidate scores by accumulated path log-probability, and
// the request's global top-W, which becomes the next frontier.  The frontier's
// states, x, H and the logits live in LDS, so the depths follow each other
// with workgroup barriers only: where the head is a few hundred KB, the
// multi-kernel path spends its time on launches, not on bytes.
//
// Results follow the same rules as the multi-kernel path: top-k by (value
// desc, token asc), candidates by (score desc, parent slot asc, rank asc),
// greedy (T = 0) keeps the lowest-index argmax with log-probability 0; pool
// rows past the kept count are (-1, -1, -inf).  Dot products run in fp32 (strided
// partial sums combined by a fixed butterfly); log-sum-exp is max-shifted.
#include "common.hpp"
#include "launch.hpp"

namespace dt {

namespace {

constexpr int SB_THREADS = 1024;
constexpr int SB_WAVES = SB_THREADS / WAVE;
constexpr int SB_MAX_W = 64;
constexpr int SB_RB = 4;                   // rows per pass over a weight row

__device__ __forceinline__ float sb_gelu(float y) {
  return 0.5f * y * (1.0f + erff(y * 0.70710678118654752f));
}

// out[i][j] = sum_c A[i][c] * Wt[j][c] for rows i < n, columns j < N (A in
// LDS, row stride K; Wt in global memory, row-major [N][K]).  A group of G
// consecutive lanes shares a column (G = the largest power of two <= 64 with
// N G <= the workgroup's threads and 4 G <= K, so narrow products still use
// every lane): lane g of the group adds the 4-wide K chunks g, g + G, ... in
// order, then the group sums its G partials by a fixed butterfly.  Each pass
// covers up to SB_RB rows, so a weight row is read once per SB_RB rows.
// epi(i, j, acc) stores the result.
template <class Epi>
__device__ __forceinline__ void sb_rows_times_wt(const float* A, int n, int K,
                                                 const float* __restrict__ Wt, int N, Epi epi) {
  int G = 1;
  while (G < WAVE && N * (2 * G) <= SB_THREADS && 4 * (2 * G) <= K) G *= 2;
  const int g = threadIdx.x % G, cols = SB_THREADS / G;
  for (int j0 = 0; j0 < N; j0 += cols) {
    const int j = j0 + threadIdx.x / G;
    const bool live = j < N;                 // every lane takes part in the butterflies
    const float* w = Wt + (long)(live ? j : 0) * K;
    for (int i0 = 0; i0 < n; i0 += SB_RB) {
      float acc[SB_RB] = {0.f, 0.f, 0.f, 0.f};
      if (live) {
        for (int c = 4 * g; c < K; c += 4 * G) {
          const float4 wv = *(const float4*)(w + c);
#pragma unroll
          for (int q = 0; q < SB_RB; ++q) {
            if (i0 + q < n) {
              const float4 av = *(const float4*)(A + (i0 + q) * K + c);
              acc[q] = fmaf(av.x, wv.x, acc[q]);
              acc[q] = fmaf(av.y, wv.y, acc[q]);
              acc[q] = fmaf(av.z, wv.z, acc[q]);
              acc[q] = fmaf(av.w, wv.w, acc[q]);
            }
          }
        }
      }
      for (int off = 1; off < G; off <<= 1)
#pragma unroll
        for (int q = 0; q < SB_RB; ++q) acc[q] += __shfl_xor(acc[q], off, WAVE);
      if (live && g == 0)
#pragma unroll
        for (int q = 0; q < SB_RB; ++q)
          if (i0 + q < n) epi(i0 + q, j, acc[q]);
    }
  }
}

template <int KMAX>
__global__ __launch_bounds__(SB_THREADS) void k_build_small(SmallBuildArgs a) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int d = a.d, d4 = 4 * d, V = a.V, W = a.W, D = a.D;
  const int keff = a.greedy ? 1 : a.k;
  const float scale = a.greedy ? 1.f : a.inv_T;
  // LDS: parent states, updated states, x, H, logits, candidate keys and tokens
  float* Sa = sm;                                   // [W][d]
  float* Sb = Sa + W * d;                           // [W][d]
  float* X = Sb + W * d;                            // [W][d]
  float* H = X + W * d;                             // [W][4d]
  float* Z = H + W * d4;                            // [W][V]
  uint64_t* keys = (uint64_t*)(Z + ((W * V + 1) & ~1));   // [W * KMAX]
  int32_t* ctok = (int32_t*)(keys + W * KMAX);            // [W * KMAX]
  __shared__ int32_t ftok[SB_MAX_W], fsrc[SB_MAX_W], ntok[SB_MAX_W], nsrc[SB_MAX_W];
  __shared__ float fscore[SB_MAX_W], nscore[SB_MAX_W];

  const float* E = (const float*)a.E;
  const float* W1t = (const float*)a.W1t;
  const float* W2t = (const float*)a.W2t;
  const float* Ut = (const float*)a.Ut;
  for (int c = tid; c < d; c += SB_THREADS) Sa[c] = a.s0[(long)r * d + c];
  if (tid == 0) {
    ftok[0] = a.root_tok[r];
    fscore[0] = 0.f;
    fsrc[0] = 0;
  }
  int n = 1;
  __syncthreads();

  for (int t = 0; t < D; ++t) {
    const float* ht = a.h + ((long)r * D + t) * d;
    for (int idx = tid; idx < n * d; idx += SB_THREADS) {
      const int i = idx / d, c = idx % d;
      const int tk = ftok[i];                         // a token outside [0, V) reads as zero
      X[idx] = (tk >= 0 && tk < V ? E[(long)tk * d + c] : 0.f) + ht[c];
    }
    __syncthreads();
    sb_rows_times_wt(X, n, d, W1t, d4, [&](int i, int j, float v) { H[i * d4 + j] = sb_gelu(v); });
    __syncthreads();
    sb_rows_times_wt(H, n, d4, W2t, d,
                     [&](int i, int j, float v) { Sb[i * d + j] = Sa[fsrc[i] * d + j] + v; });
    __syncthreads();
    sb_rows_times_wt(Sb, n, d, Ut, V, [&](int i, int j, float v) { Z[i * V + j] = v * scale; });
    __syncthreads();

    // one wave per frontier row: log-sum-exp and the row's top-keff children
    for (int i = wave; i < n; i += SB_WAVES) {
      const float* z = Z + i * V;
      float m = -INFINITY;
      TopK<KMAX> tk;
      tk.clear();
      for (int v = lane; v < V; v += WAVE) {
        m = fmaxf(m, z[v]);
        tk.insert(make_key(z[v], (uint32_t)v));
      }
      for (int off = 1; off < WAVE; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, WAVE));
      tk.reduce_lanes(WAVE);
      float L = m;
      if (!a.greedy) {
        float sum = 0.f;
        for (int v = lane; v < V; v += WAVE) sum += expf(z[v] - m);
        for (int off = 1; off < WAVE; off <<= 1) sum += __shfl_xor(sum, off, WAVE);
        L = m + logf(sum);
      }
      if (lane == 0) {
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
          if (j < keff) {
            const uint64_t key = tk.v[j];
            const bool ok = key != 0;
            const float lp = ok ? (a.greedy ? 0.f : key_value(key) - L) : -INFINITY;
            ctok[i * keff + j] = ok ? (int32_t)key_index(key) : -1;
            keys[i * keff + j] = make_key(fscore[i] + lp, (uint32_t)(i * keff + j));
          }
        }
      }
    }
    __syncthreads();

    // global top-W of the request's candidates: rank by counting (keys distinct)
    const int ncand = n * keff, nkeep = min(W, ncand);
    const long pool = ((long)r * D + t) * W;
    for (int c = tid; c < ncand; c += SB_THREADS) {
      const uint64_t kc = keys[c];
      int rank = 0;
      for (int j = 0; j < ncand; ++j) rank += keys[j] > kc;
      if (rank < nkeep) {
        const int i = c / keff;
        const float sc = key_value(kc);
        a.pool_tok[pool + rank] = ctok[c];
        a.pool_parent[pool + rank] = t == 0 ? -1 : i;
        a.pool_score[pool + rank] = sc;
        ntok[rank] = ctok[c];
        nscore[rank] = sc;
        nsrc[rank] = i;
      }
    }
    for (int j = nkeep + tid; j < W; j += SB_THREADS) {
      a.pool_tok[pool + j] = -1;
      a.pool_parent[pool + j] = -1;
      a.pool_score[pool + j] = -INFINITY;
    }
    if (tid == 0) a.n_valid[r * D + t] = nkeep;
    __syncthreads();
    // the kept children form the next frontier; their state rows are their
    // parents' updated states
    if (tid < nkeep) {
      ftok[tid] = ntok[tid];
      fscore[tid] = nscore[tid];
      fsrc[tid] = nsrc[tid];
    }
    float* tmp = Sa;
    Sa = Sb;
    Sb = tmp;
    n = nkeep;
    __syncthreads();
  }
}

size_t sb_lds_bytes(int W, int d, int V, int kmax) {
  const size_t floats = (size_t)W * d * 3 + (size_t)W * d * 4 + (((size_t)W * V + 1) & ~(size_t)1);
  return floats * 4 + (size_t)W * kmax * (8 + 4);
}

}  // namespace

bool small_build_ok(const SmallBuildArgs& a) {
  return a.W >= 1 && a.W <= SB_MAX_W && a.d % 4 == 0 && a.k >= 1 && a.k <= 16 &&
         sb_lds_bytes(a.W, a.d, a.V, a.kmax) <= SMALL_BUILD_LDS_MAX;
}

hipError_t launch_build_small(const SmallBuildArgs& a, hipStream_t st) {
  const size_t lds = sb_lds_bytes(a.W, a.d, a.V, a.kmax);
  switch (a.kmax) {
    case 1: hipLaunchKernelGGL(k_build_small<1>, dim3(a.R), dim3(SB_THREADS), lds, st, a); break;
    case 4: hipLaunchKernelGGL(k_build_small<4>, dim3(a.R), dim3(SB_THREADS), lds, st, a); break;
    case 8: hipLaunchKernelGGL(k_build_small<8>, dim3(a.R), dim3(SB_THREADS), lds, st, a); break;
    case 16: hipLaunchKernelGGL(k_build_small<16>, dim3(a.R), dim3(SB_THREADS), lds, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dt
