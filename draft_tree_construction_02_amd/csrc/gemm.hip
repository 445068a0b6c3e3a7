// Skinny weight-streaming GEMMs of the correction-head step (gfx950).
//
// Every product here has the shape Y[M][N] = A[M][K] * Wt[N][K]^T with a few
// dozen rows M (the surviving branches), and N, K in the thousands: the time
// is the weight stream from HBM, read exactly once per call.
//
// bf16 path.  Weights are streamed in the packed block layout (1 KB blocks of
// 16 rows x 32 K in MFMA operand order, the 8 tiles of a 128-row group
// interleaved per 32-K step, see pack.hip) with non-temporal 16-byte loads, so
// every wave load instruction reads one contiguous 1 KB block and a
// workgroup's loads of one K step form one 8 KB run; row-major weights are
// also accepted (16 rows x 64 B per instruction).  Activations arrive as packed hi/lo bf16 planes (hi = bf16(a),
// lo = bf16(a - hi)), written by the producing kernel; both halves go through
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation, carrying ~16 significant
// bits of A (bf16 weights are exact).  A workgroup (4 waves) owns 128 output
// columns; each wave streams its own 2 x 16 weight rows one 128-K iteration
// ahead of the MFMAs, while the activation chunk is staged in LDS and shared
// by the 4 waves.
//
// fp32 path (fp32 heads): plain FMA with fp32 activations staged in LDS.
//
// The head GEMM (z = s' U) never writes logits to HBM: each workgroup leaves
// its logit tile in LDS and reduces it per row to (max, sum exp) and the
// tile's top-k keys.  The state-update GEMMs are split-K; each split writes
// its fp32 partial and a separate reduce kernel sums the splits in order and
// applies the epilogue (the kernel boundary makes the partials visible
// without a device-wide cache flush per workgroup).
#include "common.hpp"
#include "launch.hpp"

namespace dt {

// Tile shape of the bf16 path: NW_* 16-column MFMA tiles per wave (so
// 64 NW_* columns per workgroup) and register prefetch PF_* (1: the next
// K iteration's weights are loaded before the current MFMAs; 0: occupancy
// alone hides the load latency).
#ifndef DT_NW_HEAD
#define DT_NW_HEAD 2
#endif
#ifndef DT_PF_HEAD
#define DT_PF_HEAD 0
#endif
#ifndef DT_NW_GEMM
#define DT_NW_GEMM 2
#endif
#ifndef DT_PF_GEMM
#define DT_PF_GEMM 0
#endif
#ifndef DT_WV_HEAD
#define DT_WV_HEAD 4
#endif
#ifndef DT_WV_GEMM
#define DT_WV_GEMM 4
#endif
#ifndef DT_KC_B
#define DT_KC_B 128
#endif
// Wave priority schedule of the bf16 mainloop: 0 = none; 1 = priority falls
// from 3 to 0 as the wave progresses through its K range; 2 = priority 3 until
// the first iteration's data arrived, then 1.  Waves of one CU are otherwise
// served oldest first, which starves the last-dispatched workgroups.
#ifndef DT_PRIO
#define DT_PRIO 1
#endif
// 1: a K iteration requests its activation chunk before its weight
// fragments, so the wait before the LDS store of the activation does not also
// wait for the weights (vector memory counters complete in order); 0: after.
#ifndef DT_AFIRST
#define DT_AFIRST 1
#endif

constexpr int NT = 256;               // threads per workgroup (fp32 path, helpers)
constexpr int TN_HEAD = DT_WV_HEAD * DT_NW_HEAD * 16;
constexpr int TN_GEMM = DT_WV_GEMM * DT_NW_GEMM * 16;
constexpr int TN_F = 64;              // columns per fp32 workgroup
constexpr int KC_B = DT_KC_B;         // K staged per LDS chunk (bf16 path)
constexpr int KC_F = 32;              // K staged per LDS chunk (fp32 path)
constexpr int CPAD = 4;               // C tile row padding (floats)
constexpr int BLK = 512;              // bf16 elements per packed block (1 KB)


// bf16: largest row-tile count whose first product forms x while staging
// (beyond it a separate kernel writes the x planes first)
#ifndef DT_GATHER_MAX_MT
#define DT_GATHER_MAX_MT 2
#endif
int gemm_gather_max_rows() { return 16 * DT_GATHER_MAX_MT; }

int gemm_tile_n(int w_bf16) { return w_bf16 ? TN_GEMM : TN_F; }
int head_tile_n(int w_bf16) { return w_bf16 ? TN_HEAD : TN_F; }
// Balanced <=32-row bf16 head: G workgroups, the smallest multiple of the
// compute-unit count with at most 8 tiles of 16 columns each, workgroup j
// taking tiles [j nt / G, (j + 1) nt / G) of the nt = ceil(V / 16); so every
// unit streams the same number of workgroups and the slices differ by at most
// one 16-column tile (1280 workgroups at V = 151936 instead of 1187 tiles of
// 128 columns, which leave some units a fifth tile).  At 32 rows the
// activation chunk is single-buffered on this grid, the form that measured
// faster there (double-buffered, the balanced grid was slower than the fixed
// tiles).
static bool head_bal_ok(const HeadArgs& p) {
  return p.w_bf16 && (p.Mp == 16 || p.Mp == 32) && !head_rows128_ok(p) && !head_wide_ok(p);
}
static int head_bal_groups(int V) {
  const int nt = (V + 15) / 16, need = (nt + 7) / 8, cus = device_cu_count();
  const int g = (need + cus - 1) / cus * cus;
  return g <= nt ? g : need;
}
int head_tiles(const HeadArgs& p) {
  if (head_rows128_ok(p)) return head_rows128_slices(p);
  if (head_bal_ok(p)) return head_bal_groups(p.V);
  if (head_wide_ok(p)) return head_wide_slices(p);
  const int tn = head_tile_n(p.w_bf16);
  return (p.V + tn - 1) / tn;
}
int gemm_k_chunk(int w_bf16) { return w_bf16 ? KC_B : KC_F; }

__device__ __forceinline__ float gelu_f(float y) {
  return 0.5f * y * (1.0f + erff(y * 0.70710678118654752f));
}

// ----------------------------------------------------------------------------
// bf16 path: packed hi/lo activation chunk -> LDS
// ----------------------------------------------------------------------------
// LDS chunk layout: [hl][mt][kb][512] with kb the 32-wide K block inside the
// chunk; every block is copied whole (64 lanes x 16 B).
template <int MT, int KC, int WV>
struct AStagePacked {
  static constexpr int KB = KC / 32;                  // blocks per row tile
  static constexpr int NBLK = 2 * MT * KB;            // blocks per chunk
  static constexpr int PER_WAVE = (NBLK + WV - 1) / WV;   // blocks per wave
  u32x4 v[PER_WAVE];

  __device__ __forceinline__ void issue(const PackedA& a, int k) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kblocks = a.K / 32;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int bi = wave + i * WV;
      if (NBLK % WV == 0 || bi < NBLK) {
        const int hl = bi / (MT * KB), rem = bi % (MT * KB), mt = rem / KB, kb = rem % KB;
        const uint16_t* src = (hl ? a.lo : a.hi) + ((long)mt * kblocks + k / 32 + kb) * BLK;
        v[i] = *(const u32x4*)(src + lane * 8);
      }
    }
  }
  __device__ __forceinline__ void commit(uint16_t* As) const {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int bi = wave + i * WV;
      if (NBLK % WV == 0 || bi < NBLK) *(u32x4*)(As + bi * BLK + lane * 8) = v[i];
    }
  }
};

// The first state-update product's activation x = E[tok] + h_t formed while
// staging (no separate kernel writes x): block pair (mt, kb) of the chunk -
// the hi and lo blocks of rows 16 mt .. + 15, K 32 kb .. + 31 - is computed
// by one wave, lane l from E[tok[16 mt + l % 16]] and the row's h at K
// 32 kb + 8 (l / 16) .. + 8.  Rows >= rows and rows with tok < 0 are zero.
struct GatherA {
  ASrc s;
  int K;
};

template <int MT, int KC, int WV>
struct AStageGather {
  static constexpr int KB = KC / 32;
  static constexpr int NPAIR = MT * KB;
  static constexpr int PER_WAVE = (NPAIR + WV - 1) / WV;
  u32x4 e[PER_WAVE];
  float4 h0[PER_WAVE], h1[PER_WAVE];
  int tok[PER_WAVE];
  bool init = false;

  __device__ __forceinline__ void issue(const GatherA& a, int k) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int bi = wave + i * WV;
      if (NPAIR % WV == 0 || bi < NPAIR) {
        const int mt = bi / KB, kb = bi % KB;
        const int m = 16 * mt + (lane & 15);
        if (!init) tok[i] = m < a.s.rows ? a.s.tok[m] : -1;
        const int kk = k + 32 * kb + 8 * (lane >> 4);
        e[i] = u32x4{0u, 0u, 0u, 0u};
        h0[i] = h1[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (tok[i] >= 0) {
          e[i] = *(const u32x4*)((const uint16_t*)a.s.E + (long)tok[i] * a.K + kk);
          const float* hp = a.s.h + (long)(m / a.s.rpr) * a.s.h_req_stride + kk;
          h0[i] = *(const float4*)hp;
          h1[i] = *(const float4*)(hp + 4);
        }
      }
    }
    init = true;
  }
  __device__ __forceinline__ void commit(uint16_t* As) const {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int bi = wave + i * WV;
      if (NPAIR % WV == 0 || bi < NPAIR) {
        const int mt = bi / KB, kb = bi % KB;
        const float y[8] = {bf16_to_f32(e[i][0] & 0xffffu) + h0[i].x, bf16_to_f32(e[i][0] >> 16) + h0[i].y,
                            bf16_to_f32(e[i][1] & 0xffffu) + h0[i].z, bf16_to_f32(e[i][1] >> 16) + h0[i].w,
                            bf16_to_f32(e[i][2] & 0xffffu) + h1[i].x, bf16_to_f32(e[i][2] >> 16) + h1[i].y,
                            bf16_to_f32(e[i][3] & 0xffffu) + h1[i].z, bf16_to_f32(e[i][3] >> 16) + h1[i].w};
        uint32_t hi[8], lo[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) split_hi_lo(y[j], hi[j], lo[j]);
        const int blk = mt * KB + kb;
        *(u32x4*)(As + blk * BLK + lane * 8) =
            u32x4{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16),
                  hi[6] | (hi[7] << 16)};
        *(u32x4*)(As + (MT * KB + blk) * BLK + lane * 8) =
            u32x4{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16),
                  lo[6] | (lo[7] << 16)};
      }
    }
  }
};

// Weight fragments of one 128-K iteration: b[c][j] is the 16 x 32 block of
// column tile c and K step j, in MFMA operand order (lane l: row l % 16,
// K 8 (l / 16) .. + 8 of the step).  NTW makes the packed loads non-temporal.
// The head sets it: its weights are read once per depth, are far larger than
// the memory-side cache, and non-temporal loads do not evict what that cache
// holds.  The state-update products clear it, so their weights stay in that
// cache from one depth to the next (a probe on MI355X: 105 MB read ~15%
// faster from there, and still resident after a non-temporal 778 MB stream).
template <int NW, bool PACKED, bool NTW>
__device__ __forceinline__ void load_b(u32x4 (&b)[NW][4], const uint16_t* __restrict__ Wt,
                                       int K, int col0, int N, int kb, int lane) {
#pragma unroll
  for (int c = 0; c < NW; ++c) {
    const int nt = col0 + 16 * c;            // first row of this column tile
    if (PACKED) {
      if (nt < N) {
        // grouped block order: block (g, kb, t) of tile t of row group g
        constexpr int TPG = PACK_ROWS / 16;
        const int tile = nt / 16;
        const u32x4* p = (const u32x4*)(Wt + (((long)(tile / TPG) * (K / 32) + kb / 32) * TPG +
                                              tile % TPG) * BLK + lane * 8);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          b[c][j] = NTW ? __builtin_nontemporal_load(p + j * (TPG * BLK / 8)) : p[j * (TPG * BLK / 8)];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) b[c][j] = u32x4{0u, 0u, 0u, 0u};
      }
    } else {
      const int n = nt + (lane & 15);
      if (n < N) {
        const uint16_t* p = Wt + (long)n * K + kb + (lane >> 4) * 8;
#pragma unroll
        for (int j = 0; j < 4; ++j) b[c][j] = *(const u32x4*)(p + 32 * j);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) b[c][j] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
}

template <int MT, int KC, int NW>
__device__ __forceinline__ void mma_iter(const uint16_t* As, int it, const u32x4 (&b)[NW][4],
                                         f32x4 (&acc)[NW][MT], int lane) {
  constexpr int KB = KC / 32;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int blk = mt * KB + it * 4 + j;
      const bf16x8 ahi = __builtin_bit_cast(bf16x8, *(const u32x4*)(As + blk * BLK + lane * 8));
      const bf16x8 alo = __builtin_bit_cast(
          bf16x8, *(const u32x4*)(As + (MT * KB + blk) * BLK + lane * 8));
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

template <int MT, int NBUF, int NW, int WV>
struct BfCfg {
  static constexpr int Mp = 16 * MT;
  static constexpr int KC = KC_B;
  static constexpr int TN = WV * NW * 16;
  static constexpr int ABUF = 2 * MT * (KC / 32) * BLK;     // bf16 per buffer
  static constexpr int A_BYTES = NBUF * ABUF * 2;
  static constexpr int C_BYTES = Mp * (TN + CPAD) * 4;
  static constexpr int LDS = A_BYTES > C_BYTES ? A_BYTES : C_BYTES;
};

// Accumulates Y[0..Mp)[n0..n0+TN) over K range [k0, k0 + klen).  On return
// acc[c][mt] holds rows 16 mt + lane % 16, columns n0 + 16 NW wave + 16 c +
// 4 (lane / 16) + i (i = 0..3) in element i.
template <int MT, int NBUF, bool PW, int NW, int PF, int WV, bool NTW, class Stage, class ASource>
__device__ __forceinline__ void tile_bf16(const ASource& a, const uint16_t* __restrict__ Wt,
                                          int N, int n0, int k0, int klen, unsigned char* smem,
                                          f32x4 (&acc)[NW][MT]) {
  using C = BfCfg<MT, NBUF, NW, WV>;
  constexpr int IPS = C::KC / 128;          // 128-K iterations per staged chunk
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  uint16_t* As = (uint16_t*)smem;
#pragma unroll
  for (int c = 0; c < NW; ++c)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[c][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  Stage st;
  const int col0 = n0 + wave * NW * 16;
  const int nst = klen / C::KC;
  if constexpr (PF != 0) {
    u32x4 bc[NW][4], bn[NW][4];
    load_b<NW, PW, NTW>(bc, Wt, a.K, col0, N, k0, lane);
    st.issue(a, k0);
    st.commit(As);
    __syncthreads();
    for (int s = 0; s < nst; ++s) {
      const uint16_t* Ab = As + (NBUF == 2 ? (s & 1) * C::ABUF : 0);
      const bool more = s + 1 < nst;
      static_assert(IPS == 1, "register prefetch path stages one iteration per chunk");
      if (more) load_b<NW, PW, NTW>(bn, Wt, a.K, col0, N, k0 + (s + 1) * C::KC, lane);
      if (more) st.issue(a, k0 + (s + 1) * C::KC);
      mma_iter<MT, C::KC, NW>(Ab, 0, bc, acc, lane);
      if (more) {
        if (NBUF == 1) __syncthreads();
        st.commit(As + (NBUF == 2 ? ((s + 1) & 1) * C::ABUF : 0));
#pragma unroll
        for (int c = 0; c < NW; ++c)
#pragma unroll
          for (int q = 0; q < 4; ++q) bc[c][q] = bn[c][q];
      }
      __syncthreads();
    }
  } else {
    // no register prefetch: weights and the activation chunk of iteration s
    // are requested together; other resident waves cover the latency
    if (DT_PRIO != 0) __builtin_amdgcn_s_setprio(3);
    for (int s = 0; s < nst; ++s) {
      const int k = k0 + s * C::KC;
      if (DT_PRIO == 1) {
        const int pr = 3 - (4 * s) / nst;
        if (pr == 2) __builtin_amdgcn_s_setprio(2);
        else if (pr == 1) __builtin_amdgcn_s_setprio(1);
        else if (pr == 0) __builtin_amdgcn_s_setprio(0);
      } else if (DT_PRIO == 2 && s == 1) {
        __builtin_amdgcn_s_setprio(1);
      }
      uint16_t* Ab = As + (NBUF == 2 ? (s & 1) * C::ABUF : 0);
      u32x4 b[IPS][NW][4];
      if (DT_AFIRST) st.issue(a, k);
#pragma unroll
      for (int it = 0; it < IPS; ++it) load_b<NW, PW, NTW>(b[it], Wt, a.K, col0, N, k + 128 * it, lane);
      if (!DT_AFIRST) st.issue(a, k);
      if (NBUF == 1 && s > 0) __syncthreads();
      st.commit(Ab);
      __syncthreads();
#pragma unroll
      for (int it = 0; it < IPS; ++it) mma_iter<MT, C::KC, NW>(Ab, it, b[it], acc, lane);
    }
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------
// fp32 path
// ----------------------------------------------------------------------------
// A row m, columns k..k+3: dense rows or gathered embedding + hidden.
template <int Mp, int KC, bool GATHER>
struct AStageF32 {
  static constexpr int KQ = KC / 4;
  static constexpr int NG = Mp * KQ;
  static constexpr int NA = (NG + NT - 1) / NT;
  float4 a[NA];

  __device__ __forceinline__ void load(const ASrc& s, int k) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int g = tid + i * NT;
      const int m = g / KQ, kk = k + (g % KQ) * 4;
      a[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (g < NG && m < s.rows) {
        if (GATHER) {
          const int t = s.tok[m];
          if (t >= 0) {
            const float4 h = *(const float4*)(s.h + (long)(m / s.rpr) * s.h_req_stride + kk);
            const float4 e = *(const float4*)((const float*)s.E + (long)t * s.ldE + kk);
            a[i] = make_float4(e.x + h.x, e.y + h.y, e.z + h.z, e.w + h.w);
          }
        } else {
          a[i] = *(const float4*)(s.a + (long)m * s.lda + kk);
        }
      }
    }
  }
  __device__ __forceinline__ void commit(float* As) const {
    constexpr int LDA = KC + 4;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int g = tid + i * NT;
      if (g < NG) *(float4*)(As + (g / KQ) * LDA + (g % KQ) * 4) = a[i];
    }
  }
};

template <int MT>
struct F32Cfg {
  static constexpr int Mp = 16 * MT;
  static constexpr int KC = KC_F;
  static constexpr int LDA = KC + 4;
  static constexpr int A_BYTES = Mp * LDA * 4;
  static constexpr int C_BYTES = Mp * (TN_F + CPAD) * 4;
  static constexpr int LDS = A_BYTES + C_BYTES;
};

// Leaves Y (times `scale`) in the LDS C tile [Mp][TN_F + CPAD].
template <int MT, bool GATHER>
__device__ __forceinline__ float* tile_f32(const ASrc& src, const float* __restrict__ Wt, int K,
                                           int N, int n0, int k0, int klen, float scale,
                                           unsigned char* smem) {
  using C = F32Cfg<MT>;
  constexpr int RPT = C::Mp / 4;        // rows per thread
  const int tid = threadIdx.x, nl = tid % TN_F, mg = tid / TN_F;
  float* As = (float*)smem;
  float* Cs = (float*)(smem + C::A_BYTES);
  float acc[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) acc[i] = 0.f;
  const int n = n0 + nl;
  AStageF32<C::Mp, C::KC, GATHER> st;
  for (int s = 0; s < klen / C::KC; ++s) {
    const int kb = k0 + s * C::KC;
    st.load(src, kb);
    st.commit(As);
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
  return Cs;
}

// ----------------------------------------------------------------------------
// split-K partial products
// ----------------------------------------------------------------------------
template <int MT, int NBUF, bool PW, bool GATHER>
__global__ __launch_bounds__(64 * DT_WV_GEMM) void k_gemm_bf16(GemmArgs g) {
  if (g.skip && *g.skip) return;
  constexpr int NW = DT_NW_GEMM, WV = DT_WV_GEMM;
  using Cfg = BfCfg<MT, NBUF, NW, WV>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[Cfg::LDS];
  constexpr int Mp = 16 * MT;
  const int tile = blockIdx.x, split = blockIdx.y;
  const int klen = g.K / g.splits, k0 = split * klen;
  int n0 = tile * TN_GEMM, col_end = g.N;
  if (g.runs > 0) {
    // a balanced run of 16-column tiles; columns past col_end are zero-filled
    const int nt = g.N / 16;
    n0 = 16 * (int)((long)tile * nt / g.runs);
    col_end = 16 * (int)((long)(tile + 1) * nt / g.runs);
  }
  f32x4 acc[NW][MT];
  if constexpr (GATHER)
    tile_bf16<MT, NBUF, PW, NW, DT_PF_GEMM, WV, false, AStageGather<MT, Cfg::KC, WV>>(
        GatherA{g.a, g.K}, (const uint16_t*)g.Wt, col_end, n0, k0, klen, smem, acc);
  else
    tile_bf16<MT, NBUF, PW, NW, DT_PF_GEMM, WV, false, AStagePacked<MT, Cfg::KC, WV>>(
        g.pa, (const uint16_t*)g.Wt, col_end, n0, k0, klen, smem, acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
#pragma unroll
  for (int c = 0; c < NW; ++c) {
    const int n = n0 + wave * NW * 16 + c * 16 + 4 * q;
    if (n >= col_end) continue;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = 16 * mt + r;
      const f32x4 v = acc[c][mt];
      *(float4*)(g.part + ((long)split * Mp + m) * g.N + n) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

template <int MT, bool GATHER>
__global__ __launch_bounds__(NT) void k_gemm_f32(GemmArgs g) {
  if (g.skip && *g.skip) return;
  __shared__ __attribute__((aligned(16))) unsigned char smem[F32Cfg<MT>::LDS];
  constexpr int Mp = 16 * MT;
  const int tile = blockIdx.x, split = blockIdx.y;
  const int klen = g.K / g.splits, k0 = split * klen;
  const int n0 = tile * TN_F;
  const float* Cs = tile_f32<MT, GATHER>(g.a, (const float*)g.Wt, g.K, g.N, n0, k0, klen, 1.f,
                                         smem);
  const int nvalid = min(TN_F, g.N - n0);
  for (int idx = threadIdx.x; idx < Mp * TN_F; idx += NT) {
    const int m = idx / TN_F, n = idx % TN_F;
    if (n < nvalid) g.part[((long)split * Mp + m) * g.N + n0 + n] = Cs[m * (TN_F + CPAD) + n];
  }
}

// ----------------------------------------------------------------------------
// split-K reduction + epilogue; writes fp32 rows and (bf16 path) packed hi/lo
// ----------------------------------------------------------------------------
// G consecutive threads per (row m < Mp, 8 consecutive columns): thread q
// sums splits q, q + G, ... in order, the G partial sums are added by a
// butterfly (a fixed order), and thread 0 of the group applies the epilogue.
// Rows >= rows are zero.
template <int G>
__global__ __launch_bounds__(128) void k_reduce(ReduceArgs r) {
  if (r.skip && *r.skip) return;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int n8 = r.N / 8;
  const long grp = gid / G;
  const int q = (int)(gid % G);
  const bool live = grp < (long)r.Mp * n8;   // no early exit: the butterfly needs every lane
  // 64 consecutive groups make one packed block (16 rows x 32 columns): group
  // L of block b takes row 16 (b / (N / 32)) + L % 16, columns
  // 32 (b % (N / 32)) + 8 (L / 16) .. + 7, so a wave's packed stores are
  // contiguous and each row segment it reads is 128 bytes
  const long blk = grp >> 6;
  const int L = (int)(grp & 63), nb32 = r.N >> 5;
  const int m = live ? 16 * (int)(blk / nb32) + (L & 15) : 0;
  const int n = live ? 32 * (int)(blk % nb32) + 8 * (L >> 4) : 0;
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = 0.f;
  if (live && m < r.rows) {
#pragma unroll 4
    for (int s = q; s < r.splits; s += G) {
      const float* p = r.part + ((long)s * r.Mp + m) * r.N + n;
      const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
      y[0] += a.x; y[1] += a.y; y[2] += a.z; y[3] += a.w;
      y[4] += b.x; y[5] += b.y; y[6] += b.z; y[7] += b.w;
    }
  }
#pragma unroll
  for (int off = 1; off < G; off <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] += __shfl_xor(y[i], off, WAVE);
  if (!live || q != 0) return;
  if (m < r.rows) {
    if (r.epi == EPI_GELU) {
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = gelu_f(y[i]);
    } else {
      const int sr = r.src_row ? r.src_row[m] : -1;
      if (sr >= 0) {
        const float* sp = r.s_prev + (long)sr * r.N + n;
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = sp[i] + y[i];
      }
    }
  }
  if (r.out && m < r.rows_out) {
    float* o = r.out + (long)m * r.N + n;
    *(float4*)o = make_float4(y[0], y[1], y[2], y[3]);
    *(float4*)(o + 4) = make_float4(y[4], y[5], y[6], y[7]);
  }
  if (r.out_hi) write_packed8(r.out_hi, r.out_lo, r.N, m, n, y);
}

hipError_t launch_reduce(const ReduceArgs& r, hipStream_t st) {
  // whole packed blocks: rows in 16s, columns in 32s
  if (r.Mp % 16 != 0 || r.N % 32 != 0) return hipErrorInvalidValue;
  const long groups = (long)r.Mp * (r.N / 8);
  const int G = r.splits >= 12 ? 4 : (r.splits >= 3 ? 2 : 1);
  const unsigned blocks = (unsigned)((groups * G + 127) / 128);
  if (G == 4) hipLaunchKernelGGL(k_reduce<4>, dim3(blocks), dim3(128), 0, st, r);
  else if (G == 2) hipLaunchKernelGGL(k_reduce<2>, dim3(blocks), dim3(128), 0, st, r);
  else hipLaunchKernelGGL(k_reduce<1>, dim3(blocks), dim3(128), 0, st, r);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// corrected-logit head with fused per-tile log-softmax statistics and top-k
// ----------------------------------------------------------------------------
// Per-row (max, sum exp) and top-k keys of the logit tile in LDS: G threads
// per row, thread q holding columns q, q + G, ... of the tile.  FASTEXP takes
// e^x as the hardware 2^x of x log2(e) (bf16 heads); otherwise expf.
template <int MT, int KMAX, int TN, int THREADS, bool FASTEXP>
__device__ __forceinline__ void head_epilogue(const HeadArgs& p, const float* Cs, int tile, int n0,
                                              int nvalid) {
  constexpr int Mp = 16 * MT;
  constexpr int G = THREADS / Mp;         // threads per row (power of two <= 64)
  static_assert(G >= 1 && G <= 64, "row group must fit in a wave");
  constexpr int NV = TN / G;              // columns per thread
  static_assert(NV >= 1 && (NV & (NV - 1)) == 0 && NV * G == TN, "columns per thread");
  const int tid = threadIdx.x, m = tid / G, q = tid % G;
  const int ntiles = gridDim.x;
  const float* row = Cs + m * (TN + CPAD);
  auto ex = [](float x) {
    return FASTEXP ? __builtin_amdgcn_exp2f(x * 1.44269504088896341f) : expf(x);
  };
  float mx = -INFINITY, s = 0.f;
  TopK<KMAX> tk;
  if constexpr (NV <= 16) {
    // the thread's columns in registers, top-k by a sorting network
    float v[NV];
    uint64_t keys[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int n = q + G * j;
      const bool ok = n < nvalid;
      v[j] = ok ? row[n] : -INFINITY;
      keys[j] = ok ? make_key(v[j], (uint32_t)(n0 + n)) : 0ull;
      mx = fmaxf(mx, v[j]);
    }
    topk_of<KMAX, NV>(tk, keys);
    if (!p.greedy) {
      // empty entries are -inf and add +0
      const float m0 = mx > -INFINITY ? mx : 0.f;
#pragma unroll
      for (int j = 0; j < NV; ++j) s += ex(v[j] - m0);
    }
  } else {
    // many columns per thread (64 and 128 rows): one key at a time
    tk.clear();
    for (int n = q; n < nvalid; n += G) {
      const float v = row[n];
      mx = fmaxf(mx, v);
      tk.insert(make_key(v, (uint32_t)(n0 + n)));
    }
    if (!p.greedy)
      for (int n = q; n < nvalid; n += G) s += ex(row[n] - mx);
  }
  MaxSum ms{mx, s};
  if (p.greedy) {
    // T = 0 uses the maximum alone (the sums stay 0)
    for (int off = 1; off < G; off <<= 1) ms.m = fmaxf(ms.m, __shfl_xor(ms.m, off, WAVE));
  } else {
    for (int off = 1; off < G; off <<= 1) {
      const float m2 = __shfl_xor(ms.m, off, WAVE);
      const float s2 = __shfl_xor(ms.s, off, WAVE);
      ms.combine(m2, s2);
    }
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

#ifndef DT_HEAD_WPE
#define DT_HEAD_WPE 1
#endif
template <int MT, int NBUF, int KMAX, bool PW>
__global__ __launch_bounds__(64 * DT_WV_HEAD)
__attribute__((amdgpu_waves_per_eu(DT_HEAD_WPE, 8))) void k_head_bf16(HeadArgs p) {
  if (p.skip && *p.skip) return;
  constexpr int NW = DT_NW_HEAD;
  constexpr int TN = TN_HEAD;
  __shared__ __attribute__((aligned(16))) unsigned char smem[BfCfg<MT, NBUF, NW, DT_WV_HEAD>::LDS];
  const int tile = blockIdx.x;
  // this workgroup's columns [n0, col_end): a fixed 128-column tile, or with
  // the balanced grid a run of at most 8 tiles of 16 (columns past col_end are
  // zero-filled by the loads, not read)
  int n0 = tile * TN, col_end = p.V;
  if (p.bal) {
    const int nt = (p.V + 15) / 16, G = gridDim.x;
    const int tb = (int)((long)tile * nt / G), te = (int)((long)(tile + 1) * nt / G);
    n0 = 16 * tb;
    col_end = min(16 * te, p.V);
  }
  f32x4 acc[NW][MT];
  tile_bf16<MT, NBUF, PW, NW, DT_PF_HEAD, DT_WV_HEAD, true,
            AStagePacked<MT, BfCfg<MT, NBUF, NW, DT_WV_HEAD>::KC, DT_WV_HEAD>>(
      p.pa, (const uint16_t*)p.Ut, col_end, n0, 0, p.d, smem, acc);
  // accumulators -> LDS C tile (the A buffers are free after the last barrier)
  float* Cs = (float*)smem;
  const float scale = p.greedy ? 1.f : p.inv_T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
#pragma unroll
  for (int c = 0; c < NW; ++c)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const f32x4 v = acc[c][mt];
      *(float4*)(Cs + (16 * mt + r) * (TN + CPAD) + wave * NW * 16 + c * 16 + 4 * q) =
          make_float4(v[0] * scale, v[1] * scale, v[2] * scale, v[3] * scale);
    }
  __syncthreads();
  head_epilogue<MT, KMAX, TN, 64 * DT_WV_HEAD, true>(p, Cs, tile, n0, min(TN, col_end - n0));
}

template <int MT, int KMAX>
__global__ __launch_bounds__(NT) void k_head_f32(HeadArgs p) {
  if (p.skip && *p.skip) return;
  __shared__ __attribute__((aligned(16))) unsigned char smem[F32Cfg<MT>::LDS];
  const int tile = blockIdx.x;
  const float* Cs = tile_f32<MT, false>(p.a, (const float*)p.Ut, p.d, p.V, tile * TN_F, 0, p.d,
                                        p.greedy ? 1.f : p.inv_T, smem);
  head_epilogue<MT, KMAX, TN_F, NT, false>(p, Cs, tile, tile * TN_F, min(TN_F, p.V - tile * TN_F));
}

// ----------------------------------------------------------------------------
// host launchers
// ----------------------------------------------------------------------------
// LDS buffers of the activation chunk: double-buffered below DT_NBUF1_MT row
// tiles, single-buffered from there (keeps enough workgroups resident).
#ifndef DT_NBUF1_MT
#define DT_NBUF1_MT 8
#endif

template <int MT>
static hipError_t gemm_mt(const GemmArgs& g, hipStream_t st) {
  const int TN = g.w_bf16 ? TN_GEMM : TN_F;
  dim3 grid(g.w_bf16 && g.runs > 0 ? g.runs : (g.N + TN - 1) / TN, g.splits);
  if (g.w_bf16) {
    constexpr int NB = MT >= DT_NBUF1_MT ? 1 : 2;
    const dim3 blk(64 * DT_WV_GEMM);
    if (g.a.gather) {
      if constexpr (MT <= DT_GATHER_MAX_MT) {
        if (g.w_packed)
          hipLaunchKernelGGL((k_gemm_bf16<MT, NB, true, true>), grid, blk, 0, st, g);
        else
          hipLaunchKernelGGL((k_gemm_bf16<MT, NB, false, true>), grid, blk, 0, st, g);
      } else {
        return hipErrorInvalidValue;
      }
    } else if (g.w_packed) {
      hipLaunchKernelGGL((k_gemm_bf16<MT, NB, true, false>), grid, blk, 0, st, g);
    } else {
      hipLaunchKernelGGL((k_gemm_bf16<MT, NB, false, false>), grid, blk, 0, st, g);
    }
  } else {
    if (g.a.gather)
      hipLaunchKernelGGL((k_gemm_f32<MT, true>), grid, dim3(NT), 0, st, g);
    else
      hipLaunchKernelGGL((k_gemm_f32<MT, false>), grid, dim3(NT), 0, st, g);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
  if (gemm_rows128_ok(g)) return launch_gemm_rows128(g, st);
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
  const int TN = p.w_bf16 ? TN_HEAD : TN_F;
  dim3 grid((p.V + TN - 1) / TN);
  if (p.bal) grid = dim3(head_bal_groups(p.V));
  if (p.w_bf16) {
    constexpr int NB = MT >= DT_NBUF1_MT ? 1 : 2;
    if (MT == 2 && p.bal) {
      // balanced 32-row grid: one activation buffer (measured faster here)
      if (p.w_packed)
        hipLaunchKernelGGL((k_head_bf16<MT, 1, KMAX, true>), grid, dim3(64 * DT_WV_HEAD), 0, st, p);
      else
        hipLaunchKernelGGL((k_head_bf16<MT, 1, KMAX, false>), grid, dim3(64 * DT_WV_HEAD), 0, st, p);
    } else if (p.w_packed)
      hipLaunchKernelGGL((k_head_bf16<MT, NB, KMAX, true>), grid, dim3(64 * DT_WV_HEAD), 0, st, p);
    else
      hipLaunchKernelGGL((k_head_bf16<MT, NB, KMAX, false>), grid, dim3(64 * DT_WV_HEAD), 0, st, p);
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

hipError_t launch_head(const HeadArgs& p0, hipStream_t st) {
  if (head_rows128_ok(p0)) return launch_head_rows128(p0, st);
  if (head_wide_ok(p0)) return launch_head_wide(p0, st);
  HeadArgs p = p0;
  p.bal = head_bal_ok(p0) ? 1 : 0;
  switch (p.Mp) {
    case 16: return head_mt<1>(p, st);
    case 32: return head_mt<2>(p, st);
    case 64: return head_mt<4>(p, st);
    case 128: return head_mt<8>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dt
