// Acceptance walk of draft trees against a synthetic greedy target: the
// verification step that closes a drafting round ("DARTree: Teaching a
// Chain-Trained Corrector to Think in Trees", Core Mechanism, last step; Key
// Concepts, accepted tokens per verification round).
//
// The target is a chain model of the correction head's form.  A node's state
// needs its parent's, so the states are computed depth by depth: k_walk_rows
// lists the nodes of one depth that have children (compacted over all
// requests), their x = E[tok] + h rows are written as the state update's
// input, the usual state-update kernels run on chunks of those rows, and
// k_walk_keep files the new states under the nodes' places in one inner-node
// list.  The target's output head then runs once over that whole list (greedy
// keys only), so its V x d matrix is streamed once per 128 inner nodes rather
// than once per depth; k_walk reads each node's argmax and follows, per
// request, the children that match the target.
#include "../../include/dartree.h"
#include "common.hpp"
#include "launch.hpp"

namespace dt {

constexpr int WALK_THREADS = 1024;
constexpr int WALK_X_THREADS = 256;

// Token of node i of request r, -1 if its index or token is out of range.
__device__ __forceinline__ int node_token(const WalkArgs& a, int r, int i) {
  int j = i;
  if (a.tok_index) {
    j = a.tok_index[(long)r * a.B + i];
    if (j < 0 || j >= a.tok_stride) return -1;
  }
  const int t = a.tok[(long)r * a.tok_stride + j];
  return t >= 0 && t < a.V ? t : -1;
}

__device__ __forceinline__ int node_count(const WalkArgs& a, int r) {
  const int n = a.n[r];
  return n < 0 ? 0 : (n > a.B ? a.B : n);
}

// One workgroup per request: clear its outputs and bookkeeping, then mark
// every node that is some valid node's parent.
__global__ __launch_bounds__(256) void k_walk_init(WalkArgs a) {
  const int r = blockIdx.x, B1 = a.B + 1;
  const long base = (long)r * B1;
  for (int j = threadIdx.x; j < B1; j += 256) {
    a.has_child[base + j] = 0;
    a.pos[base + j] = -1;
    a.target_tok[base + j] = -1;
  }
  for (int j = threadIdx.x; j < a.D; j += 256) a.path[(long)r * a.D + j] = -1;
  if (threadIdx.x == 0) a.accept_len[r] = 0;
  if (r == 0 && threadIdx.x == 0) a.ctl[1] = 0;
  __syncthreads();
  const int n = node_count(a, r);
  for (int i = threadIdx.x; i < n; i += 256) {
    const int p = a.parent[(long)r * a.B + i];
    if (p >= -1 && p < i) a.has_child[base + p + 1] = 1;   // same value from every writer
  }
}

// One workgroup.  t < D: list the rows of depth t - the root (t == 0) or the
// nodes at depth t whose parent has a row at depth t - 1, that have children
// and a valid token - and append them to the inner-node list.  t == D: chunk
// flags of the inner-node list, padding rows of its last chunk zeroed.
__global__ __launch_bounds__(WALK_THREADS) void k_walk_rows(WalkArgs a, int t) {
  __shared__ int s_wcount[WALK_THREADS / 64];
  __shared__ int s_base;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B1 = a.B + 1;
  const int gbase = a.ctl[1];                        // inner nodes listed before depth t
  if (t >= a.D) {
    for (int c = tid; c < a.nch; c += WALK_THREADS) a.skip[c] = c * a.CH >= gbase ? 1 : 0;
    const long lo = (long)gbase * a.d, hi = (long)(gbase + a.CH - 1) / a.CH * a.CH * a.d;
    for (long i = lo + tid; i < hi; i += WALK_THREADS) a.S_inner[i] = 0.f;
    return;
  }
  if (tid == 0) s_base = 0;
  __syncthreads();
  const long total = (long)a.R * B1;
  for (long g0 = 0; g0 < total; g0 += WALK_THREADS) {
    const long g = g0 + tid;
    int r = 0, j = 0, tokv = -1, src = -1;
    bool ok = false;
    if (g < total && a.has_child[g]) {
      r = (int)(g / B1);
      j = (int)(g % B1);
      if (j == 0) {
        if (t == 0) {
          tokv = a.root_tok[r];
          src = r;                                   // s0 row
          ok = tokv >= 0 && tokv < a.V;
        }
      } else if (t > 0 && j - 1 < node_count(a, r)) {
        const int i = j - 1;
        const long ri = (long)r * a.B;
        const int p = a.parent[ri + i];
        if (a.depth[ri + i] == t && p >= -1 && p < i) {
          tokv = node_token(a, r, i);
          const bool pok = p < 0 ? t == 1 : a.depth[ri + p] == t - 1;
          if (tokv >= 0 && pok) {
            src = a.pos[(long)r * B1 + p + 1];
            ok = src >= 0;
          }
        }
      }
    }
    const uint64_t bal = __ballot(ok);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) s_wcount[wave] = __popcll(bal);
    __syncthreads();
    int woff = 0;
    for (int w = 0; w < wave; ++w) woff += s_wcount[w];
    const int base = s_base;
    if (ok) {
      const int m = base + woff + before;
      a.row_req[m] = r;
      a.row_tok[m] = tokv;
      a.row_src[m] = src;
      a.row_gidx[m] = gbase + m;
      a.inner_req[gbase + m] = r;
      a.inner_node[gbase + m] = j - 1;
      a.pos[g] = m;
    }
    __syncthreads();
    if (tid == 0) {
      int tot = 0;
      for (int w = 0; w < WALK_THREADS / 64; ++w) tot += s_wcount[w];
      s_base = base + tot;
    }
    __syncthreads();
  }
  const int nt = s_base;
  if (tid == 0) {
    a.ctl[0] = nt;
    a.ctl[1] = gbase + nt;
  }
  for (int c = tid; c < a.nch; c += WALK_THREADS) a.skip[c] = c * a.CH >= nt ? 1 : 0;
  // padding rows of the last non-empty chunk have no residual source
  const int lim = (nt + a.CH - 1) / a.CH * a.CH;
  for (int m = nt + tid; m < lim; m += WALK_THREADS) a.row_src[m] = -1;
}

// x = E[tok] + h[req][t] of every listed row; the other rows of the last
// non-empty chunk are zero, empty chunks are left alone (their launches skip).
__global__ __launch_bounds__(WALK_X_THREADS) void k_walk_x(WalkArgs a, int t) {
  const int m = blockIdx.x;
  const int nt = a.ctl[0];
  if (m >= (nt + a.CH - 1) / a.CH * a.CH) return;
  const int kk = (blockIdx.y * WALK_X_THREADS + threadIdx.x) * 8;
  if (kk >= a.d) return;
  float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (m < nt) {
    const int r = a.row_req[m], tk = a.row_tok[m];
    const float* hr = a.h + ((long)r * a.D + t) * a.d + kk;
    if (a.bf16) {
      const uint16_t* er = (const uint16_t*)a.E + (long)tk * a.d + kk;
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = bf16_to_f32(er[i]) + hr[i];
    } else {
      const float* er = (const float*)a.E + (long)tk * a.d + kk;
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = er[i] + hr[i];
    }
  }
  if (a.x_hi) {
    const long cb = (long)(m / a.CH) * a.CH * a.d;
    write_packed8(a.x_hi + cb, a.x_lo + cb, a.d, m % a.CH, kk, y);
  } else {
    float* xr = a.x_f32 + (long)m * a.d + kk;
#pragma unroll
    for (int i = 0; i < 8; ++i) xr[i] = y[i];
  }
}

// States of the current depth's rows to their inner-node rows.
__global__ __launch_bounds__(WALK_X_THREADS) void k_walk_keep(WalkArgs a, const float* s_cur) {
  const int m = blockIdx.x;
  if (m >= a.ctl[0]) return;
  const int k = (blockIdx.y * WALK_X_THREADS + threadIdx.x) * 4;
  if (k >= a.d) return;
  *(float4*)(a.S_inner + (long)a.row_gidx[m] * a.d + k) = *(const float4*)(s_cur + (long)m * a.d + k);
}

// One workgroup per request: the target token of each of the request's inner
// nodes (the argmax over the head's greedy keys of its row), then one wave
// moves from the root to the lowest-index child whose token is the target's
// token after the current node.
__global__ __launch_bounds__(256) void k_walk(WalkArgs a) {
  const int r = blockIdx.x, B1 = a.B + 1;
  int32_t* tt = a.target_tok + (long)r * B1;
  const int ninner = a.ctl[1];
  for (int g = threadIdx.x; g < ninner; g += 256) {
    if (a.inner_req[g] != r) continue;
    const uint64_t* kr = a.key2 + (long)g * a.S;
    uint64_t best = 0;
    for (int s = 0; s < a.S; ++s) best = kr[s] > best ? kr[s] : best;
    tt[a.inner_node[g] + 1] = best != 0 ? (int32_t)key_index(best) : -1;
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  const int n = node_count(a, r);
  const long ri = (long)r * a.B;
  int cur = -1, len = 0;
  while (len < a.D) {
    const int want = tt[cur + 1];
    if (want < 0) break;
    int found = -1;
    for (int i0 = 0; i0 < n && found < 0; i0 += 64) {
      const int i = i0 + lane;
      bool match = false;
      if (i < n)
        match = a.parent[ri + i] == cur && a.depth[ri + i] == len + 1 &&
                node_token(a, r, i) == want;
      const uint64_t bal = __ballot(match);
      if (bal) found = i0 + __builtin_ctzll(bal);
    }
    if (found < 0) break;
    if (lane == 0) a.path[(long)r * a.D + len] = found;
    cur = found;
    ++len;
  }
  if (lane == 0) a.accept_len[r] = len;
}

hipError_t launch_walk_init(const WalkArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_walk_init, dim3(a.R), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_walk_rows(const WalkArgs& a, int t, hipStream_t st) {
  hipLaunchKernelGGL(k_walk_rows, dim3(1), dim3(WALK_THREADS), 0, st, a, t);
  if (t >= a.D) return hipGetLastError();
  const int ny = (a.d + WALK_X_THREADS * 8 - 1) / (WALK_X_THREADS * 8);
  hipLaunchKernelGGL(k_walk_x, dim3(a.nch * a.CH, ny), dim3(WALK_X_THREADS), 0, st, a, t);
  return hipGetLastError();
}

hipError_t launch_walk_keep(const WalkArgs& a, const float* s_cur, hipStream_t st) {
  const int ny = (a.d + WALK_X_THREADS * 4 - 1) / (WALK_X_THREADS * 4);
  hipLaunchKernelGGL(k_walk_keep, dim3(a.nch * a.CH, ny), dim3(WALK_X_THREADS), 0, st, a, s_cur);
  return hipGetLastError();
}

hipError_t launch_walk(const WalkArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_walk, dim3(a.R), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace dt
