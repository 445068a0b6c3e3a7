// Corrected-logit head for many surviving branches (64 or 128 rows), gfx950.
//
// Same contract as the head in gemm.hip (y = s' U / T over one slice of the
// vocabulary per workgroup, per-row (max, sum exp) and top-k keys of the
// slice written as partials), shaped for the case where the activation is
// large: every wave owns NW tiles of 16 columns for all rows, so each
// activation fragment read from LDS feeds NW weight tiles.  The slices are
// balanced runs of 16-column tiles: at 64 rows two workgroups per compute
// unit with 5 tiles per wave (18-19 tiles per slice at V = 151936, all
// workgroups resident at once), at 128 rows runs of at most 16 tiles with 4
// per wave.  A run may cross the packed layout's row groups, so every tile
// has its own block offset; a wave's tiles past its slice re-read the
// slice's last tile (in bounds, never reported).  The weight fragments of the
// next 64-K chunk are requested right after the MFMAs of the current one
// consume theirs, and the activation chunk is double-buffered in LDS with a
// single barrier per chunk, so two waves per SIMD keep both the HBM stream and
// the matrix cores busy.  Weights must be in the packed layout (pack.hip).
#include "common.hpp"
#include "launch.hpp"

#include <type_traits>

namespace dt {

namespace {

#ifndef DT_HW_RING
#define DT_HW_RING 1
#endif
#ifndef DT_HW_APF
#define DT_HW_APF 0
#endif

constexpr int HW_WAVES = 4;                       // waves per workgroup
// 16-column tiles per wave: 5 at 64 rows, 4 at 128 rows (register budget of
// two waves per SIMD)
constexpr int hw_nw(int MT) { return MT <= 4 ? 5 : 4; }
constexpr int HW_BLK = 512;                       // bf16 per packed 1 KB block
constexpr int HW_STEPS = 2;                       // 32-K steps per staged chunk

template <int MT, int KMAX>
struct HwCfg {
  static constexpr int Mp = 16 * MT;
  static constexpr int ABUF = 2 * MT * HW_STEPS * HW_BLK;        // bf16 per chunk buffer
  static constexpr int A_BYTES = 2 * ABUF * 2;                    // two buffers
  static constexpr int EPI_BYTES = HW_WAVES * Mp * (8 + 8 * KMAX);
  static constexpr int LDS = A_BYTES > EPI_BYTES ? A_BYTES : EPI_BYTES;
  static constexpr int ABLK = 2 * MT * HW_STEPS / HW_WAVES;      // blocks staged per wave
  static_assert((2 * MT * HW_STEPS) % HW_WAVES == 0, "activation blocks split evenly");
};

// Activation blocks of one chunk held by this wave: block bi = wave + 4 i is
// (hl, mt, j) with bi = (hl * MT + mt) * 2 + j, which is also its slot in the
// LDS chunk buffer.  ap[i] points at the block of chunk 0 (plus the lane's 16
// bytes); chunk ch is 2 ch blocks further.
template <int MT, int N>
__device__ __forceinline__ void hw_a_ptrs(const uint16_t* (&ap)[N], const PackedA& a, int wave,
                                          int lane) {
  const int kblocks = a.K / 32;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int bi = wave + HW_WAVES * i;
    const int hl = bi / (2 * MT), mt = (bi / 2) % MT, j = bi % 2;
    ap[i] = (hl ? a.lo : a.hi) + ((long)mt * kblocks + j) * HW_BLK + lane * 8;
  }
}

template <int N>
__device__ __forceinline__ void hw_load_a(u32x4 (&v)[N], const uint16_t* const (&ap)[N], int ch) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = *(const u32x4*)(ap[i] + ch * (HW_STEPS * HW_BLK));
}

template <int N>
__device__ __forceinline__ void hw_store_a(const u32x4 (&v)[N], uint16_t* buf, int wave,
                                           int lane) {
#pragma unroll
  for (int i = 0; i < N; ++i)
    *(u32x4*)(buf + (wave + HW_WAVES * i) * HW_BLK + lane * 8) = v[i];
}

// Weight fragments of one K step for the wave's NW tiles: tile c's block of
// the step starts toff[c] + kofs bytes into the grouped packed layout (both
// wave-uniform, so they stay in scalar registers), the lane's 16 bytes at
// vlane.  Non-temporal: the head's weights are streamed once per depth.
template <int NW>
__device__ __forceinline__ void hw_load_b(u32x4 (&b)[NW], __amdgpu_buffer_rsrc_t wrs, int vlane,
                                          const uint32_t (&toff)[NW], uint32_t kofs) {
#pragma unroll
  for (int c = 0; c < NW; ++c)
    b[c] = __builtin_amdgcn_raw_buffer_load_b128(wrs, vlane, toff[c] + kofs, 2 /* nt */);
}

template <int MT, int KMAX>
__global__ __launch_bounds__(64 * HW_WAVES)
__attribute__((amdgpu_waves_per_eu(2))) void k_head_wide(HeadArgs p) {
  if (p.skip && *p.skip) return;
  using C = HwCfg<MT, KMAX>;
  constexpr int Mp = C::Mp;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS];
  uint16_t* As = (uint16_t*)smem;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int NW = hw_nw(MT);
  const int tile = blockIdx.x;

  // this slice: 16-column tiles [tb, te) of the nt16 = ceil(V / 16), the
  // host's grid leaving 1 .. HW_WAVES NW tiles per slice.  Wave w owns tiles
  // tw .. tw + NW - 1; those at or past te load tile te - 1 again (its
  // columns are masked in the epilogue), so every weight load is
  // unconditional and in bounds (tiles below te lie in the stored groups).
  const int nt16 = (p.V + 15) / 16;
  const int tb = (int)((long)tile * nt16 / gridDim.x);
  const int te = (int)((long)(tile + 1) * nt16 / gridDim.x);
  const int tw = tb + wave * NW;
  // byte offsets fit 32 unsigned bits: the host admits heads of < 4 GiB
  const int tpg = PACK_ROWS / 16, kblocks = p.d / 32;
  const uint32_t wbytes = (uint32_t)((size_t)(nt16 + tpg - 1) / tpg * tpg * 16 * p.d * 2);
  const __amdgpu_buffer_rsrc_t wrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.Ut, (short)0, (int)wbytes, 0x00020000);
  uint32_t toff[NW];
#pragma unroll
  for (int c = 0; c < NW; ++c) {
    const int t = min(tw + c, te - 1);
    toff[c] = __builtin_amdgcn_readfirstlane(
        (uint32_t)(((t / tpg) * kblocks * tpg + t % tpg) * (uint32_t)(HW_BLK * 2)));
  }
  const int vlane = lane * 16;
  uint32_t kofs = 0;
  constexpr uint32_t WSTEP = (PACK_ROWS / 16) * HW_BLK * 2;     // bytes of one K step of a row group

  f32x4 acc[NW][MT];
#pragma unroll
  for (int c = 0; c < NW; ++c)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[c][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nch = p.d / (32 * HW_STEPS);
  const uint16_t* ap[C::ABLK];
  hw_a_ptrs<MT>(ap, p.pa, wave, lane);
  // weight fragments of RING chunks in flight: slot (ch % RING, j)
  constexpr int RING = DT_HW_RING;
  u32x4 b[RING][HW_STEPS][NW];
  u32x4 av[C::ABLK];
#pragma unroll
  for (int r = 0; r < RING; ++r)
#pragma unroll
    for (int j = 0; j < HW_STEPS; ++j, kofs += WSTEP) hw_load_b(b[r][j], wrs, vlane, toff, kofs);
  hw_load_a(av, ap, 0);
  hw_store_a(av, As, wave, lane);
  __syncthreads();

  // one chunk: MFMAs on the buffered activation and the weight fragments of
  // ring slot R; with LOADA the next chunk's activation is requested first
  // (so the wait before its LDS store does not cover the weight loads issued
  // after it), with LOADB each weight slot is refilled with the chunk RING
  // ahead as soon as its MFMAs have issued.  Tags keep the loop body free of
  // conditional loads.
  auto chunk = [&](int ch, auto slot_tag, auto loada_tag, auto loadb_tag) {
    constexpr int R = decltype(slot_tag)::value;
    constexpr bool LOADA = decltype(loada_tag)::value;
    constexpr bool LOADB = decltype(loadb_tag)::value;
    const uint16_t* cur = As + (ch & 1) * C::ABUF;
    if (LOADA) hw_load_a(av, ap, ch + 1);
    // keep the requests where they are written: the scheduler would
    // otherwise sink them below the MFMAs and expose their latency
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < HW_STEPS; ++j) {
#if DT_HW_APF
      u32x4 ah = *(const u32x4*)(cur + (0 * 2 + j) * HW_BLK + lane * 8);
      u32x4 al = *(const u32x4*)(cur + ((MT + 0) * 2 + j) * HW_BLK + lane * 8);
#endif
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#if DT_HW_APF
        const bf16x8 ahi = __builtin_bit_cast(bf16x8, ah);
        const bf16x8 alo = __builtin_bit_cast(bf16x8, al);
        if (mt + 1 < MT) {
          ah = *(const u32x4*)(cur + ((mt + 1) * 2 + j) * HW_BLK + lane * 8);
          al = *(const u32x4*)(cur + ((MT + mt + 1) * 2 + j) * HW_BLK + lane * 8);
        }
#else
        const bf16x8 ahi =
            __builtin_bit_cast(bf16x8, *(const u32x4*)(cur + (mt * 2 + j) * HW_BLK + lane * 8));
        const bf16x8 alo = __builtin_bit_cast(
            bf16x8, *(const u32x4*)(cur + ((MT + mt) * 2 + j) * HW_BLK + lane * 8));
#endif
#pragma unroll
        for (int c = 0; c < NW; ++c)
          acc[c][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, b[R][j][c]), ahi, acc[c][mt], 0, 0, 0);
#pragma unroll
        for (int c = 0; c < NW; ++c)
          acc[c][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, b[R][j][c]), alo, acc[c][mt], 0, 0, 0);
      }
      if (LOADB) {
        hw_load_b(b[R][j], wrs, vlane, toff, kofs);
        kofs += WSTEP;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (LOADA) hw_store_a(av, As + ((ch + 1) & 1) * C::ABUF, wave, lane);
    __syncthreads();
  };
  using T = std::true_type;
  using F = std::false_type;
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, RING - 1>;
  if constexpr (RING == 1) {
    for (int ch = 0; ch + 1 < nch; ++ch) chunk(ch, S0{}, T{}, T{});
    chunk(nch - 1, S0{}, F{}, F{});
  } else {
    // nch is even (d % 128 == 0)
    int ch = 0;
    for (; ch + 2 < nch; ch += 2) {
      chunk(ch, S0{}, T{}, T{});
      chunk(ch + 1, S1{}, T{}, T{});
    }
    chunk(ch, S0{}, T{}, F{});
    chunk(ch + 1, S1{}, F{}, F{});
  }

  // per-row statistics of the wave's tiles: lane l holds row 16 mt + l % 16,
  // columns 16 (tw + c) + 4 (l / 16) + i, those below min(16 te, V) valid;
  // the 4 lanes of a row combine by butterfly
  float2* ms_l = (float2*)smem;                                   // [wave][Mp]
  uint64_t* key_l = (uint64_t*)(smem + HW_WAVES * Mp * 8);        // [wave][Mp][KMAX]
  const float scale = p.greedy ? 1.f : p.inv_T;
  const int r = lane & 15, q = lane >> 4;
  const int colw = 16 * tw + 4 * q, colend = min(16 * te, p.V);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    float v[NW][4];
    float mx = -INFINITY;
    TopK<KMAX> tk;
    tk.clear();
#pragma unroll
    for (int c = 0; c < NW; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = colw + 16 * c + i;
        v[c][i] = acc[c][mt][i] * scale;
        if (col < colend) {
          mx = fmaxf(mx, v[c][i]);
          tk.insert(make_key(v[c][i], (uint32_t)col));
        }
      }
    float s = 0.f;
    if (!p.greedy) {
#pragma unroll
      for (int c = 0; c < NW; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (colw + 16 * c + i < colend) s += expf(v[c][i] - mx);
    }
    MaxSum ms{mx, s};
#pragma unroll
    for (int off = 16; off < 64; off <<= 1) {
      const float m2 = __shfl_xor(ms.m, off, WAVE);
      const float s2 = __shfl_xor(ms.s, off, WAVE);
      ms.combine(m2, s2);
      uint64_t o[KMAX];
#pragma unroll
      for (int i = 0; i < KMAX; ++i) o[i] = shfl_xor_u64(tk.v[i], off);
      tk.merge(o);
    }
    if (q == 0) {
      const int row = wave * Mp + 16 * mt + r;
      ms_l[row] = make_float2(ms.m, ms.s);
#pragma unroll
      for (int i = 0; i < KMAX; ++i) key_l[row * KMAX + i] = tk.v[i];
    }
  }
  __syncthreads();

  // combine the 4 waves of each row: G threads per row, each folding
  // HW_WAVES / G waves in wave order, then a butterfly over the G threads
  constexpr int G = 64 * HW_WAVES / Mp;
  constexpr int WPT = HW_WAVES / G;
  static_assert(G >= 1 && WPT >= 1 && G * WPT == HW_WAVES, "row groups");
  const int m = threadIdx.x / G, gq = threadIdx.x % G;
  MaxSum ms{-INFINITY, 0.f};
  TopK<KMAX> tk;
  tk.clear();
#pragma unroll
  for (int w = 0; w < WPT; ++w) {
    const int row = (gq * WPT + w) * Mp + m;
    const float2 e = ms_l[row];
    ms.combine(e.x, e.y);
    uint64_t o[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) o[i] = key_l[row * KMAX + i];
    tk.merge(o);
  }
#pragma unroll
  for (int off = 1; off < G; off <<= 1) {
    const float m2 = __shfl_xor(ms.m, off, WAVE);
    const float s2 = __shfl_xor(ms.s, off, WAVE);
    ms.combine(m2, s2);
    uint64_t o[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) o[i] = shfl_xor_u64(tk.v[i], off);
    tk.merge(o);
  }
  if (gq == 0) {
    const long o = (long)m * gridDim.x + tile;
    p.ms_part[o] = make_float2(ms.m, ms.s);
#pragma unroll
    for (int i = 0; i < KMAX; ++i)
      if (i < p.k) p.key_part[o * p.k + i] = tk.v[i];
  }
}

// Slices of the head: at 64 rows two workgroups per compute unit (more when
// V needs runs longer than 4 NW tiles, fewer for a small vocabulary, at
// least ~10 tiles each); at 128 rows runs of at most 16 tiles.  Every slice
// holds 1 .. 4 NW tiles.
int hw_slices(int Mp, int V) {
  const int nt16 = (V + 15) / 16;
  const int per = HW_WAVES * hw_nw(Mp / 16);
  const int need = (nt16 + per - 1) / per;
  if (Mp > 64) return need;
  return std::max(need, std::min(2 * device_cu_count(), std::max(1, nt16 / 10)));
}

template <int MT, int KMAX>
hipError_t head_wide_mk(const HeadArgs& p, hipStream_t st) {
  const dim3 grid(hw_slices(p.Mp, p.V));
  hipLaunchKernelGGL((k_head_wide<MT, KMAX>), grid, dim3(64 * HW_WAVES), 0, st, p);
  return hipGetLastError();
}

template <int MT>
hipError_t head_wide_mt(const HeadArgs& p, hipStream_t st) {
  switch (p.kmax) {
    case 1: return head_wide_mk<MT, 1>(p, st);
    case 4: return head_wide_mk<MT, 4>(p, st);
    case 8: return head_wide_mk<MT, 8>(p, st);
    case 16: return head_wide_mk<MT, 16>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

#ifndef DT_WIDE_MIN_MP
#define DT_WIDE_MIN_MP 64
#endif

bool head_wide_ok(const HeadArgs& p) {
  const size_t vpad = ((size_t)p.V + PACK_ROWS - 1) / PACK_ROWS * PACK_ROWS;
  return p.w_bf16 && p.w_packed && p.Mp >= DT_WIDE_MIN_MP && (p.Mp == 64 || p.Mp == 128) &&
         p.d % (32 * HW_STEPS) == 0 && vpad * (size_t)p.d * 2 < ((size_t)1 << 32);
}

int head_wide_slices(const HeadArgs& p) { return hw_slices(p.Mp, p.V); }

hipError_t launch_head_wide(const HeadArgs& p, hipStream_t st) {
  switch (p.Mp) {
    case 64: return head_wide_mt<4>(p, st);
    case 128: return head_wide_mt<8>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace dt
