// Skinny weight-streaming GEMMs of the correction-head step (gfx950).
//
// Every product here has the shape Y[M][N] = A[M][K] * Wt[N][K]^T with a few
// dozen rows M (the surviving branches), and N, K in the thousands: the time
// is the weight stream from HBM, read exactly once per call.  A workgroup
// (4 waves) owns a 128-column tile of Wt (one contiguous block of rows of the
// output-feature-major weight) and a K range; each wave streams its own 32
// weight rows with non-temporal 16-byte loads, one K iteration ahead of the
// MFMAs that consume them.
//
// bf16 weights: the fp32 activations are split into hi = bf16(a) and
// lo = bf16(a - hi) while being staged into LDS, and both halves go through
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation, which carries ~16
// significant bits of A (bf16 weights are exact).  fp32 weights use plain FMA.
//
// The head GEMM (z = s' U) never writes logits to HBM: each workgroup leaves
// its logit tile in LDS and reduces it per row to (max, sum exp) and the
// tile's top-k keys.  The state-update GEMMs use split-K; the last split to
// finish a column tile sums all splits in order and applies the epilogue
// (GELU, or residual add of the parent's state), so results are deterministic.
#include "common.hpp"
#include "launch.hpp"

namespace dt {

constexpr int NT = 256;               // threads per workgroup
constexpr int NWAVES = NT / WAVE;     // 4
constexpr int NW = 2;                 // 16-column MFMA tiles per wave
constexpr int TN_B = NWAVES * NW * 16;   // 128 columns per bf16 workgroup
constexpr int TN_F = 64;              // columns per fp32 workgroup
constexpr int KC_B = 128;             // K staged per LDS chunk (bf16 path)
constexpr int KC_F = 32;              // K staged per LDS chunk (fp32 path)
constexpr int CPAD = 4;               // C tile row padding (floats)

int gemm_tile_n(int w_bf16) { return w_bf16 ? TN_B : TN_F; }
int head_tile_n(int w_bf16) { return w_bf16 ? TN_B : TN_F; }
int gemm_k_chunk(int w_bf16, int) { return w_bf16 ? KC_B : KC_F; }

__device__ __forceinline__ float gelu_f(float y) {
  return 0.5f * y * (1.0f + erff(y * 0.70710678118654752f));
}

// ----------------------------------------------------------------------------
// A staging: fp32 activations (dense rows, or gathered embedding + hidden)
// ----------------------------------------------------------------------------
template <int Mp, int KC, bool GATHER, bool EBF16>
struct AStage {
  static constexpr int KQ = KC / 4;                       // float4 groups per row
  static constexpr int NG = Mp * KQ;                      // groups per chunk
  static constexpr int NA = (NG + NT - 1) / NT;           // groups per thread
  float4 a[NA];
  float4 hv[NA];
  uint2 eb[NA];

  __device__ __forceinline__ void issue(const ASrc& s, int k) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int g = tid + i * NT;
      const int m = g / KQ, kk = k + (g % KQ) * 4;
      a[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      hv[i] = a[i];
      eb[i] = make_uint2(0u, 0u);
      if (g < NG && m < s.rows) {
        if (GATHER) {
          const int t = s.tok[m];
          if (t >= 0) {
            hv[i] = *(const float4*)(s.h + (long)(m / s.rpr) * s.h_req_stride + kk);
            if (EBF16)
              eb[i] = *(const uint2*)((const uint16_t*)s.E + (long)t * s.ldE + kk);
            else
              a[i] = *(const float4*)((const float*)s.E + (long)t * s.ldE + kk);
          }
        } else {
          a[i] = *(const float4*)(s.a + (long)m * s.lda + kk);
        }
      }
    }
  }

  __device__ __forceinline__ float4 value(int i) const {
    if (!GATHER) return a[i];
    float4 e = a[i];
    if (EBF16) {
      e.x = bf16_to_f32(eb[i].x & 0xffffu);
      e.y = bf16_to_f32(eb[i].x >> 16);
      e.z = bf16_to_f32(eb[i].y & 0xffffu);
      e.w = bf16_to_f32(eb[i].y >> 16);
    }
    return make_float4(e.x + hv[i].x, e.y + hv[i].y, e.z + hv[i].z, e.w + hv[i].w);
  }

  // bf16 path: hi plane at As, lo plane at As + Mp * LDA.
  __device__ __forceinline__ void commit_split(uint16_t* As) const {
    constexpr int LDA = KC + 8;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int g = tid + i * NT;
      if (g < NG) {
        const int m = g / KQ, kk = (g % KQ) * 4;
        const float4 x = value(i);
        uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
        split_hi_lo(x.x, h0, l0);
        split_hi_lo(x.y, h1, l1);
        split_hi_lo(x.z, h2, l2);
        split_hi_lo(x.w, h3, l3);
        *(uint2*)(As + m * LDA + kk) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
        *(uint2*)(As + Mp * LDA + m * LDA + kk) = make_uint2(l0 | (l1 << 16), l2 | (l3 << 16));
      }
    }
  }

  // fp32 path
  __device__ __forceinline__ void commit_f32(float* As) const {
    constexpr int LDA = KC + 4;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int g = tid + i * NT;
      if (g < NG) {
        const int m = g / KQ, kk = (g % KQ) * 4;
        *(float4*)(As + m * LDA + kk) = value(i);
      }
    }
  }
};

// ----------------------------------------------------------------------------
// bf16 MFMA mainloop
// ----------------------------------------------------------------------------
// Lane (r = lane % 16, g = lane / 16) of a wave loads 32 consecutive K values
// (64 bytes) of weight row n = col0 + 16 c + r per 128-K iteration; MFMA j of
// the iteration uses elements [8 j, 8 j + 8) of that run, and the activation
// fragment uses the same K positions, so the product sums every K once.
template <int MT>
__device__ __forceinline__ void load_b(u32x4 (&b)[NW][4], const uint16_t* __restrict__ Wt,
                                       int ldw, int col0, int N, int kb, int lane) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int c = 0; c < NW; ++c) {
    const int n = col0 + 16 * c + r;
    if (n < N) {
      const u32x4* p = (const u32x4*)(Wt + (long)n * ldw + kb + g * 32);
#pragma unroll
      for (int q = 0; q < 4; ++q) b[c][q] = __builtin_nontemporal_load(p + q);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) b[c][q] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

template <int MT, int KC>
__device__ __forceinline__ void mma_iter(const uint16_t* As, int it, const u32x4 (&b)[NW][4],
                                         f32x4 (&acc)[NW][MT], int lane) {
  constexpr int Mp = 16 * MT;
  constexpr int LDA = KC + 8;
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint16_t* p = As + (16 * mt + r) * LDA + it * 128 + g * 32 + j * 8;
      const bf16x8 ahi = __builtin_bit_cast(bf16x8, *(const u32x4*)p);
      const bf16x8 alo = __builtin_bit_cast(bf16x8, *(const u32x4*)(p + Mp * LDA));
#pragma unroll
      for (int c = 0; c < NW; ++c)
        acc[c][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, b[c][j]), ahi, acc[c][mt], 0, 0, 0);
#pragma unroll
      for (int c = 0; c < NW; ++c)
        acc[c][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, b[c][j]), alo, acc[c][mt], 0, 0, 0);
    }
  }
}

template <int MT, int NBUF>
struct BfCfg {
  static constexpr int Mp = 16 * MT;
  static constexpr int KC = KC_B;
  static constexpr int LDA = KC + 8;
  static constexpr int ABUF = 2 * Mp * LDA;                 // uint16 per buffer
  static constexpr int A_BYTES = NBUF * ABUF * 2;
  static constexpr int C_BYTES = Mp * (TN_B + CPAD) * 4;
  static constexpr int LDS = A_BYTES > C_BYTES ? A_BYTES : C_BYTES;
};

// Accumulates Y[0..Mp)[n0..n0+128) over K range [k0, k0 + klen) and leaves it
// in the LDS C tile (row stride TN_B + CPAD floats), scaled by `scale`.
template <int MT, int NBUF, bool GATHER>
__device__ __forceinline__ void tile_bf16(const ASrc& src, const uint16_t* __restrict__ Wt,
                                          int K, int N, int n0, int k0, int klen, float scale,
                                          unsigned char* smem) {
  using C = BfCfg<MT, NBUF>;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  uint16_t* As = (uint16_t*)smem;
  f32x4 acc[NW][MT];
#pragma unroll
  for (int c = 0; c < NW; ++c)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[c][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  AStage<C::Mp, C::KC, GATHER, true> st;
  st.issue(src, k0);
  st.commit_split(As);
  __syncthreads();

  const int col0 = n0 + wave * NW * 16;
  const int nst = klen / C::KC;
  u32x4 bc[NW][4], bn[NW][4];
  load_b<MT>(bc, Wt, K, col0, N, k0, lane);
  for (int s = 0; s < nst; ++s) {
    const uint16_t* Ab = As + (NBUF == 2 ? (s & 1) * C::ABUF : 0);
    const bool more = s + 1 < nst;
    if (more) st.issue(src, k0 + (s + 1) * C::KC);
    if (more) load_b<MT>(bn, Wt, K, col0, N, k0 + (s + 1) * C::KC, lane);
    mma_iter<MT, C::KC>(Ab, 0, bc, acc, lane);
    if (more) {
      if (NBUF == 1) __syncthreads();
      st.commit_split(As + (NBUF == 2 ? ((s + 1) & 1) * C::ABUF : 0));
#pragma unroll
      for (int c = 0; c < NW; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) bc[c][q] = bn[c][q];
    }
    __syncthreads();
  }

  // accumulators -> LDS C tile; lane holds rows 16 mt + r, columns 4 g .. 4 g + 3
  float* Cs = (float*)smem;
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int c = 0; c < NW; ++c)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = 16 * mt + r;
      const int n = wave * NW * 16 + c * 16 + 4 * g;
      f32x4 v = acc[c][mt];
      *(float4*)(Cs + m * (TN_B + CPAD) + n) =
          make_float4(v[0] * scale, v[1] * scale, v[2] * scale, v[3] * scale);
    }
  __syncthreads();
}

// ----------------------------------------------------------------------------
// fp32 FMA mainloop (fp32 heads)
// ----------------------------------------------------------------------------
template <int MT>
struct F32Cfg {
  static constexpr int Mp = 16 * MT;
  static constexpr int KC = KC_F;
  static constexpr int LDA = KC + 4;
  static constexpr int A_BYTES = Mp * LDA * 4;
  static constexpr int C_BYTES = Mp * (TN_F + CPAD) * 4;
  static constexpr int LDS = A_BYTES + C_BYTES;
};

template <int MT, bool GATHER>
__device__ __forceinline__ void tile_f32(const ASrc& src, const float* __restrict__ Wt, int K,
                                         int N, int n0, int k0, int klen, float scale,
                                         unsigned char* smem, float*& Cs_out) {
  using C = F32Cfg<MT>;
  constexpr int RPT = C::Mp / 4;        // rows per thread
  const int tid = threadIdx.x, nl = tid % TN_F, mg = tid / TN_F;
  float* As = (float*)smem;
  float* Cs = (float*)(smem + C::A_BYTES);
  float acc[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) acc[i] = 0.f;
  const int n = n0 + nl;
  AStage<C::Mp, C::KC, GATHER, false> st;
  for (int s = 0; s < klen / C::KC; ++s) {
    const int kb = k0 + s * C::KC;
    st.issue(src, kb);
    st.commit_f32(As);
    __syncthreads();
    if (n < N) {
#pragma unroll
      for (int kk = 0; kk < C::KC; kk += 4) {
        const float4 w = *(const float4*)(Wt + (long)n * K + kb + kk);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          const float4 a = *(const float4*)(As + (mg + 4 * i) * C::LDA + kk);
          acc[i] = fmaf(a.x, w.x, acc[i]);
          acc[i] = fmaf(a.y, w.y, acc[i]);
          acc[i] = fmaf(a.z, w.z, acc[i]);
          acc[i] = fmaf(a.w, w.w, acc[i]);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) Cs[(mg + 4 * i) * (TN_F + CPAD) + nl] = acc[i] * scale;
  __syncthreads();
  Cs_out = Cs;
}

// ----------------------------------------------------------------------------
// split-K state-update GEMM with fused last-split epilogue
// ----------------------------------------------------------------------------
template <int MT, int TN>
__device__ __forceinline__ void splitk_epilogue(const GemmArgs& g, const float* Cs, int tile) {
  constexpr int Mp = 16 * MT;
  const int tid = threadIdx.x;
  const int n0 = tile * TN, split = blockIdx.y;
  const int nvalid = min(TN, g.N - n0);
  for (int idx = tid; idx < Mp * TN; idx += NT) {
    const int m = idx / TN, n = idx % TN;
    if (n < nvalid) g.part[((long)split * Mp + m) * g.N + n0 + n] = Cs[m * (TN + CPAD) + n];
  }
  __threadfence();
  __syncthreads();
  __shared__ int last;
  if (tid == 0) last = atomicAdd(&g.counters[tile], 1u) == (uint32_t)(g.splits - 1);
  __syncthreads();
  if (!last) return;
  __threadfence();
  const int rows = g.a.rows;
  for (int idx = tid; idx < Mp * TN; idx += NT) {
    const int m = idx / TN, n = idx % TN;
    if (n >= nvalid || m >= rows) continue;
    float y = 0.f;
    for (int s = 0; s < g.splits; ++s) y += g.part[((long)s * Mp + m) * g.N + n0 + n];
    float o;
    if (g.epi == EPI_GELU) {
      o = gelu_f(y);
    } else {
      const int sr = g.src_row[m];
      o = (sr >= 0 ? g.s_prev[(long)sr * g.N + n0 + n] : 0.f) + y;
    }
    g.out[(long)m * g.N + n0 + n] = o;
  }
  if (tid == 0) g.counters[tile] = 0u;
}

template <int MT, int NBUF, bool GATHER>
__global__ __launch_bounds__(NT) void k_gemm_bf16(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[BfCfg<MT, NBUF>::LDS];
  const int tile = blockIdx.x;
  const int klen = g.K / g.splits, k0 = blockIdx.y * klen;
  tile_bf16<MT, NBUF, GATHER>(g.a, (const uint16_t*)g.Wt, g.K, g.N, tile * TN_B, k0, klen, 1.f,
                              smem);
  splitk_epilogue<MT, TN_B>(g, (const float*)smem, tile);
}

template <int MT, bool GATHER>
__global__ __launch_bounds__(NT) void k_gemm_f32(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[F32Cfg<MT>::LDS];
  const int tile = blockIdx.x;
  const int klen = g.K / g.splits, k0 = blockIdx.y * klen;
  float* Cs;
  tile_f32<MT, GATHER>(g.a, (const float*)g.Wt, g.K, g.N, tile * TN_F, k0, klen, 1.f, smem, Cs);
  splitk_epilogue<MT, TN_F>(g, Cs, tile);
}

// ----------------------------------------------------------------------------
// corrected-logit head with fused per-tile log-softmax statistics and top-k
// ----------------------------------------------------------------------------
template <int MT, int KMAX, int TN>
__device__ __forceinline__ void head_epilogue(const HeadArgs& p, const float* Cs, int tile) {
  constexpr int Mp = 16 * MT;
  constexpr int G = NT / Mp;              // threads per row
  const int tid = threadIdx.x, m = tid / G, q = tid % G;
  const int n0 = tile * TN, ntiles = gridDim.x;
  const int nvalid = min(TN, p.V - n0);
  const float* row = Cs + m * (TN + CPAD);
  float mx = -INFINITY;
  TopK<KMAX> tk;
  tk.clear();
  for (int n = q; n < nvalid; n += G) {
    const float v = row[n];
    mx = fmaxf(mx, v);
    tk.insert(make_key(v, (uint32_t)(n0 + n)));
  }
  float s = 0.f;
  if (!p.greedy)
    for (int n = q; n < nvalid; n += G) s += expf(row[n] - mx);
  MaxSum ms{mx, s};
  for (int off = 1; off < G; off <<= 1) {
    const float m2 = __shfl_xor(ms.m, off, WAVE);
    const float s2 = __shfl_xor(ms.s, off, WAVE);
    ms.combine(m2, s2);
  }
  tk.reduce_lanes(G);
  if (q == 0) {
    const long o = (long)m * ntiles + tile;
    p.ms_part[o] = make_float2(ms.m, ms.s);
#pragma unroll
    for (int i = 0; i < KMAX; ++i)
      if (i < p.k) p.key_part[o * p.k + i] = tk.v[i];
  }
}

template <int MT, int NBUF, int KMAX>
__global__ __launch_bounds__(NT) void k_head_bf16(HeadArgs p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[BfCfg<MT, NBUF>::LDS];
  const int tile = blockIdx.x;
  tile_bf16<MT, NBUF, false>(p.a, (const uint16_t*)p.Ut, p.d, p.V, tile * TN_B, 0, p.d,
                             p.greedy ? 1.f : p.inv_T, smem);
  head_epilogue<MT, KMAX, TN_B>(p, (const float*)smem, tile);
}

template <int MT, int KMAX>
__global__ __launch_bounds__(NT) void k_head_f32(HeadArgs p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[F32Cfg<MT>::LDS];
  const int tile = blockIdx.x;
  float* Cs;
  tile_f32<MT, false>(p.a, (const float*)p.Ut, p.d, p.V, tile * TN_F, 0, p.d,
                      p.greedy ? 1.f : p.inv_T, smem, Cs);
  head_epilogue<MT, KMAX, TN_F>(p, Cs, tile);
}

// ----------------------------------------------------------------------------
// host launchers
// ----------------------------------------------------------------------------
template <int MT>
static hipError_t gemm_mt(const GemmArgs& g, hipStream_t st) {
  const int TN = g.w_bf16 ? TN_B : TN_F;
  dim3 grid((g.N + TN - 1) / TN, g.splits);
  if (g.w_bf16) {
    constexpr int NB = MT >= 8 ? 1 : 2;
    if (g.a.gather)
      hipLaunchKernelGGL((k_gemm_bf16<MT, NB, true>), grid, dim3(NT), 0, st, g);
    else
      hipLaunchKernelGGL((k_gemm_bf16<MT, NB, false>), grid, dim3(NT), 0, st, g);
  } else {
    if (g.a.gather)
      hipLaunchKernelGGL((k_gemm_f32<MT, true>), grid, dim3(NT), 0, st, g);
    else
      hipLaunchKernelGGL((k_gemm_f32<MT, false>), grid, dim3(NT), 0, st, g);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
  switch (g.Mp) {
    case 16: return gemm_mt<1>(g, st);
    case 32: return gemm_mt<2>(g, st);
    case 64: return gemm_mt<4>(g, st);
    case 128: return gemm_mt<8>(g, st);
    default: return hipErrorInvalidValue;
  }
}

template <int MT, int KMAX>
static hipError_t head_mk(const HeadArgs& p, hipStream_t st) {
  const int TN = p.w_bf16 ? TN_B : TN_F;
  dim3 grid((p.V + TN - 1) / TN);
  if (p.w_bf16) {
    constexpr int NB = MT >= 8 ? 1 : 2;
    hipLaunchKernelGGL((k_head_bf16<MT, NB, KMAX>), grid, dim3(NT), 0, st, p);
  } else {
    hipLaunchKernelGGL((k_head_f32<MT, KMAX>), grid, dim3(NT), 0, st, p);
  }
  return hipGetLastError();
}

template <int MT>
static hipError_t head_mt(const HeadArgs& p, hipStream_t st) {
  switch (p.kmax) {
    case 1: return head_mk<MT, 1>(p, st);
    case 4: return head_mk<MT, 4>(p, st);
    case 8: return head_mk<MT, 8>(p, st);
    case 16: return head_mk<MT, 16>(p, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_head(const HeadArgs& p, hipStream_t st) {
  switch (p.Mp) {
    case 16: return head_mt<1>(p, st);
    case 32: return head_mt<2>(p, st);
    case 64: return head_mt<4>(p, st);
    case 128: return head_mt<8>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dt
