// Sequential heap-interleaved best-first construction: the per-node baseline
// that depth-wise batching replaces ("DARTree: Teaching a Chain-Trained
// Corrector to Think in Trees", Core Mechanism; "Technische Samenvatting:
// DARTree", Experimentele Resultaten, ablation of sequential heap-interleaved
// correction).
//
// Every expansion is one head call on one row (the same state-update and
// head kernels as the batched build, with Mp = 16).  Between two calls one
// workgroup pushes the expanded node's children, pops the best candidates
// until one can be expanded (depth < D) or the tree holds B nodes, appends
// every popped node to the output, and writes the next call's input x.  The
// host enqueues B call slots up front; a device flag turns the slots that
// are not needed into no-ops, so nothing synchronises with the host.
#include "../../include/dartree.h"
#include "common.hpp"
#include "launch.hpp"

namespace dt {

constexpr int SEQ_THREADS = 1024;

// Fold the merge range results of row 0 into its top-keff children (one
// wave); lane 0 returns them in tok / lp.
template <int KMAX>
__device__ __forceinline__ void fold_row0(const SeqArgs& a, int32_t (&tok)[KMAX],
                                          float (&lp)[KMAX]) {
  const int lane = threadIdx.x & 63;
  MaxSum tot{-INFINITY, 0.f};
  TopK<KMAX> all;
  all.clear();
  if (lane < a.S) {
    const float2 e = a.ms2[lane];
    tot = MaxSum{e.x, e.y};
#pragma unroll
    for (int q = 0; q < KMAX; ++q) all.v[q] = a.key2[(long)lane * KMAX + q];
  }
  int S2 = 1;
  while (S2 < a.S) S2 <<= 1;
  for (int off = 1; off < S2; off <<= 1) {
    const float m2 = __shfl_xor(tot.m, off, 64);
    const float s2 = __shfl_xor(tot.s, off, 64);
    tot.combine(m2, s2);
  }
  all.reduce_lanes(S2);
  const float L = a.greedy ? tot.m : tot.m + logf(tot.s);
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const uint64_t key = all.v[j];
    const bool ok = key != 0 && (!a.greedy || j == 0);
    tok[j] = ok ? (int32_t)key_index(key) : -1;
    lp[j] = ok ? (a.greedy ? 0.f : key_value(key) - L) : -INFINITY;
  }
}

// x of the next call: E[tok] + h[depth] for row 0 (packed planes for bf16
// heads, a dense fp32 row otherwise).  Rows 1.. stay zero.
__device__ __forceinline__ void write_x(const SeqArgs& a, int tok, int depth) {
  const float* hr = a.h + (long)depth * a.d;
  if (a.x_hi) {
    const uint16_t* er = (const uint16_t*)a.E + (long)tok * a.d;
    for (int kk = threadIdx.x * 8; kk < a.d; kk += SEQ_THREADS * 8) {
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = bf16_to_f32(er[kk + i]) + hr[kk + i];
      write_packed8(a.x_hi, a.x_lo, a.d, 0, kk, y);
    }
  } else {
    const float* er = (const float*)a.E + (long)tok * a.d;
    for (int kk = threadIdx.x; kk < a.d; kk += SEQ_THREADS) a.x_f32[kk] = er[kk] + hr[kk];
  }
}

__global__ __launch_bounds__(SEQ_THREADS) void k_seq_init(SeqArgs a, const float* s0,
                                                          const int32_t* root_tok) {
  const int tid = threadIdx.x;
  // s0 is the residual source of the root's call (state row B)
  for (int i = tid; i < a.d; i += SEQ_THREADS) a.state[(long)a.B * a.d + i] = s0[i];
  for (int i = tid; i < a.B; i += SEQ_THREADS) {
    a.out_tok[i] = -1;
    a.out_par[i] = -1;
    a.out_depth[i] = -1;
    a.out_score[i] = -INFINITY;
  }
  if (a.x_hi) {
    const long n8 = (long)a.Mp * (a.d / 8);
    for (long g = tid; g < n8; g += SEQ_THREADS) {
      float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      write_packed8(a.x_hi, a.x_lo, a.d, (int)(g / (a.d / 8)), (int)(g % (a.d / 8)) * 8, y);
    }
  } else {
    for (long i = tid; i < (long)a.Mp * a.d; i += SEQ_THREADS) a.x_f32[i] = 0.f;
  }
  __syncthreads();
  const int rt = root_tok[0];
  write_x(a, rt, 0);
  if (tid == 0) {
    a.ctl[SEQ_N_OUT] = 0;
    a.ctl[SEQ_N_CAND] = 0;
    a.ctl[SEQ_SKIP] = 0;
    a.ctl[SEQ_CUR_OUT] = -1;
    a.ctl[SEQ_CUR_DEPTH] = 0;
    a.ctl[SEQ_CUR_ROW] = a.B;
    a.ctl[SEQ_CALLS] = 0;
    a.cur_score[0] = 0.f;
    *a.n_out = 0;
  }
}

// After call `slot`: push the expanded node's children, then pop.  Which
// candidates are still in the heap is kept in an LDS bitmap for the whole
// kernel (loaded from and stored back to c_alive), so no thread ever reads a
// flag that another thread of this launch has changed in global memory.
template <int KMAX>
__global__ __launch_bounds__(SEQ_THREADS) void k_seq_step(SeqArgs a, int slot) {
  __shared__ uint64_t wbest[SEQ_THREADS / 64];
  __shared__ uint32_t alive[SEQ_MAX_CAND / 32];
  __shared__ int s_done, s_nout, s_ncand, s_expand, s_xtok, s_xdep;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int keff = a.greedy ? 1 : a.k;
  if (a.ctl[SEQ_SKIP]) return;                       // uniform: read before any write

  // push
  if (wave == 0) {
    int32_t ct[KMAX];
    float cl[KMAX];
    fold_row0<KMAX>(a, ct, cl);
    if (lane == 0) {
      const int base = a.ctl[SEQ_N_CAND];
      const int par = a.ctl[SEQ_CUR_OUT], dep = a.ctl[SEQ_CUR_DEPTH] + 1;
      const float sc0 = a.cur_score[0];
      int n = 0;
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (j < keff && ct[j] >= 0) {
          a.c_tok[base + n] = ct[j];
          a.c_par[base + n] = par;
          a.c_depth[base + n] = dep;
          a.c_row[base + n] = slot;
          a.c_score[base + n] = sc0 + cl[j];
          ++n;
        }
      s_ncand = base + n;
      s_nout = a.ctl[SEQ_N_OUT];
      a.ctl[SEQ_CALLS] += 1;
    }
  }
  __syncthreads();
  const int ncand = s_ncand, nold = a.ctl[SEQ_N_CAND];
  for (int w = tid; w < (ncand + 31) / 32; w += SEQ_THREADS) {
    // words of the previous launches (bits below nold), plus the new
    // candidates [nold, ncand), which are alive
    uint32_t v = 32 * w < nold ? a.c_alive[w] : 0u;
    for (int b = 0; b < 32; ++b) {
      const int c = 32 * w + b;
      if (c < nold) continue;
      if (c < ncand) v |= 1u << b;
      else v &= ~(1u << b);
    }
    alive[w] = v;
  }
  if (tid == 0) s_expand = 0;
  __syncthreads();

  // pop until a node can be expanded, the tree is full or nothing is left
  for (;;) {
    const int n_out = s_nout;
    uint64_t best = 0;
    if (n_out < a.B) {
      for (int c = tid; c < ncand; c += SEQ_THREADS) {
        if (!((alive[c >> 5] >> (c & 31)) & 1u)) continue;
        const int dep = a.c_depth[c];
        const float prio = __fadd_rn(a.c_score[c], __fmul_rn(a.beta, (float)dep));
        // order: prio desc, depth asc, push order asc
        const uint64_t key = make_key(prio, (uint32_t)dep * 65536u + (uint32_t)c);
        best = key > best ? key : best;
      }
    }
    for (int off = 32; off >= 1; off >>= 1) {
      const uint64_t o = shfl_xor_u64(best, off);
      best = o > best ? o : best;
    }
    if (lane == 0) wbest[wave] = best;
    __syncthreads();
    if (tid == 0) {
      uint64_t b = 0;
      for (int w = 0; w < SEQ_THREADS / 64; ++w) b = wbest[w] > b ? wbest[w] : b;
      int done = 1;
      if (b != 0) {
        const int c = (int)(key_index(b) & 65535u);
        alive[c >> 5] &= ~(1u << (c & 31));
        const int i = n_out;
        const int dep = a.c_depth[c];
        a.out_tok[i] = a.c_tok[c];
        a.out_par[i] = a.c_par[c];
        a.out_depth[i] = dep;
        a.out_score[i] = a.c_score[c];
        s_nout = i + 1;
        if (i + 1 < a.B && dep < a.D) {
          a.ctl[SEQ_CUR_OUT] = i;
          a.ctl[SEQ_CUR_DEPTH] = dep;
          a.ctl[SEQ_CUR_ROW] = a.c_row[c];
          a.ctl[SEQ_CUR_TOK] = a.c_tok[c];
          a.cur_score[0] = a.c_score[c];
          s_expand = 1;
          s_xtok = a.c_tok[c];
          s_xdep = dep;
        } else if (i + 1 < a.B) {
          done = 0;                                    // a leaf at depth D: keep popping
        } else {
          a.ctl[SEQ_SKIP] = 1;                         // the tree is full
        }
      } else {
        a.ctl[SEQ_SKIP] = 1;                           // nothing left to pop
      }
      s_done = done;
    }
    __syncthreads();
    if (s_done) break;
  }
  for (int w = tid; w < (ncand + 31) / 32; w += SEQ_THREADS) a.c_alive[w] = alive[w];
  if (tid == 0) {
    a.ctl[SEQ_N_CAND] = ncand;
    a.ctl[SEQ_N_OUT] = s_nout;
    *a.n_out = s_nout;
  }
  // the next call's input
  if (s_expand) write_x(a, s_xtok, s_xdep);
}

hipError_t launch_seq_init(const SeqArgs& a, const float* s0, const int32_t* root_tok,
                           hipStream_t st) {
  hipLaunchKernelGGL(k_seq_init, dim3(1), dim3(SEQ_THREADS), 0, st, a, s0, root_tok);
  return hipGetLastError();
}

hipError_t launch_seq_step(const SeqArgs& a, int slot, hipStream_t st) {
  switch (a.kmax) {
    case 1: hipLaunchKernelGGL(k_seq_step<1>, dim3(1), dim3(SEQ_THREADS), 0, st, a, slot); break;
    case 4: hipLaunchKernelGGL(k_seq_step<4>, dim3(1), dim3(SEQ_THREADS), 0, st, a, slot); break;
    case 8: hipLaunchKernelGGL(k_seq_step<8>, dim3(1), dim3(SEQ_THREADS), 0, st, a, slot); break;
    case 16: hipLaunchKernelGGL(k_seq_step<16>, dim3(1), dim3(SEQ_THREADS), 0, st, a, slot); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dt
