// Corrected-logit head and state-update GEMM for 128 rows (many requests
// sharing one head), gfx950.
//
// The head (k_head_rows128) has the contract of the other heads (per-row
// (max, sum exp) and top-k keys of y = s' U / T over each vocabulary slice)
// and is shaped for a batch large enough that the matrix cores and the HBM
// stream have to run at full rate together:
//   * one workgroup of 8 waves (two per SIMD) per compute unit, each owning a
//     contiguous slice of 32-column tiles (slices differ by at most one tile);
//     wave w takes rows 32 (w % 4) .. + 31 for one half of the slice's tiles,
//     so its accumulators (up to 10 tiles of 32 x 32) and per-row statistics
//     are its own, and each half is reported as a slice of its own;
//   * both operands reach LDS by DMA (buffer loads with the LDS bit): the
//     weight fragments of one 32-K step (each wave a fifth of them) into one
//     of three slots two steps ahead, the hi/lo activation blocks of all 128
//     rows (each wave one row block of each plane) into one of two slots one
//     step ahead; no register holds data in flight, so the registers the
//     accumulators leave go to reading operands from LDS well ahead of use,
//     and the activation is read from L2 once per unit, not once per wave;
//   * one barrier per K step hands the slots over; it is split-phase: the
//     next step's activation and first weight fragments are read from LDS
//     right after it, while the MFMAs of the step's last tiles still run;
//   * v_mfma_f32_32x32x16_bf16 with the hi/lo activation split; a half of
//     nine tiles runs a loop without the tenth tile's MFMAs.
// The GEMM (k_gemm_rows128) keeps the four-wave organisation below
// (r8_mainloop): wave w owns rows 32 w .. + 31 for all the workgroup's tiles,
// weight fragments by DMA into four slots three steps ahead, activations
// straight from the packed planes into registers two steps ahead.
// Operand layout (both from 16-row x 32-K packed blocks): lane l takes row
// 16 ((l % 32) / 16) + l % 16 of a 32-row pair of blocks and, in K step st of
// the block, K values 16 st + 8 (l / 32) .. + 8, i.e. block lane
// l % 16 + 16 (2 st + l / 32); the K order inside a step is the same for both
// operands.  Accumulator element e of lane l is vocabulary column
// 8 (e / 4) + 4 (l / 32) + e % 4 of the tile and row l % 32 of the wave.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace dt {

namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int R8_WAVES = 4;                                     // one per 32-row tile
constexpr int R8_BLK = 512;                                     // bf16 per 1 KB fragment
constexpr int R8_ACT = 4;                                       // activation loads per step

constexpr int R8_MAX_DEVICES = 64;
std::atomic<int> g_cus[R8_MAX_DEVICES];     // 0 until queried

}  // namespace

// Compute units of the current device, queried once per device and cached in
// an atomic (two first callers may both query; they store the same value).
int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < R8_MAX_DEVICES) {
    const int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  if (dev < R8_MAX_DEVICES) g_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

namespace {

int cu_count() { return device_cu_count(); }

// Fragments per wave per K step and bf16 per LDS slot for NC tiles of 32
// columns per workgroup.
template <int NC>
struct R8Cfg {
  static constexpr int FPW = (2 * NC + R8_WAVES - 1) / R8_WAVES;
  static constexpr int SLOT = FPW * R8_WAVES * R8_BLK;
};

// The K loop shared by the 128-row head and the 128-row GEMM: wave w
// accumulates rows 32 w .. 32 w + 31 of Y = A W^T for the workgroup's tiles
// tb .. tb + T - 1 (T <= NC; 32 columns each) over K blocks kb0 .. kb0 + nkb
// - 1 (32 K each, nkb % 4 == 0).  W is a packed bf16 matrix (grouped layout)
// of nrows_pad rows and K columns; A the packed hi/lo planes of 128 rows.
// Ws holds the workgroup's NSLOT LDS slots, each its own array; weights run
// NSLOT - 1 steps ahead.  Only the first NCR tiles are computed (NCR < NC
// leaves the last tiles' accumulators at zero; their fragments are still
// loaded, so the load counts do not depend on NCR).  TAG makes the
// instantiation (and its lambdas) distinct per kernel: host stubs of kernels
// that share one instantiation are not all emitted.
template <int NC, int NCR, int TAG, int NSLOT>
__device__ __forceinline__ void r8_mainloop(const uint16_t* W, int nrows_pad, int K,
                                            const PackedA& pa, int tb, int T, int kb0, int nkb,
                                            f32x16 (&acc)[NC], uint16_t* const (&Ws)[NSLOT]) {
  static_assert(NCR <= NC, "tiles computed <= tiles loaded");
  constexpr int AHEAD = NSLOT - 1;
  using C = R8Cfg<NC>;
  constexpr int FPW = C::FPW;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kblocks = K / 32, kb_last = kb0 + nkb - 1;
  const int hh = lane >> 5, sub = (lane & 31) >> 4;
  const int lane_el = sub * R8_BLK + ((lane & 15) + 16 * hh) * 8;

  // weight fragments this wave loads each step: f = wave + 4 i is (tile f / 2,
  // K step f % 2); fragments past the workgroup's tiles repeat its last tile
  // (in bounds, loaded to LDS positions that are never read).  Buffer loads:
  // one lane offset in a VGPR, the fragment's offset in an SGPR; the buffer's
  // size bounds every access.
  const __amdgpu_buffer_rsrc_t wrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)W, (short)0, nrows_pad * K * 2, 0x00020000);
  const int w_lane = lane_el * 2;
  int wsoff[FPW];
#pragma unroll
  for (int i = 0; i < FPW; ++i) {
    const int f = wave + R8_WAVES * i;
    const int c = min(f / 2, T - 1), st = f % 2;
    const int j = tb + c;
    wsoff[i] = __builtin_amdgcn_readfirstlane(
        (((j / 4) * kblocks * 8 + 2 * (j % 4)) * R8_BLK + 256 * st) * 2);
  }
  // this wave's activation fragments: hi / lo planes, rows 32 wave + ..
  const __amdgpu_buffer_rsrc_t hrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)pa.hi, (short)0, 128 * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t lrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)pa.lo, (short)0, 128 * K * 2, 0x00020000);
  const int a_lane = (sub * kblocks * R8_BLK + ((lane & 15) + 16 * hh) * 8) * 2;
  const int a_wave = __builtin_amdgcn_readfirstlane(2 * wave * kblocks * R8_BLK * 2);

  // FPW loads of step kb's weight fragments into an LDS slot (always issued,
  // clamped to the last step, so that every step issues the same loads)
  auto load_w = [&](uint16_t* slot, int kb) {
    kb = min(kb, kb_last);
#pragma unroll
    for (int i = 0; i < FPW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wrs, (__attribute__((address_space(3))) void*)(slot + (wave + R8_WAVES * i) * R8_BLK),
          16, w_lane, wsoff[i] + kb * 8 * R8_BLK * 2, 0, 2 /* nt */);
  };
  // R8_ACT loads of step kb's activation fragments into registers
  u32x4 areg[2][R8_ACT];                                         // [kb % 2][st * 2 + hl]
  auto load_a = [&](u32x4 (&dst)[R8_ACT], int kb) {
    kb = min(kb, kb_last);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int so = a_wave + (kb * R8_BLK + 256 * st) * 2;
      dst[2 * st] =
          __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(hrs, a_lane, so, 0));
      dst[2 * st + 1] =
          __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(lrs, a_lane, so, 0));
    }
  };

#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;

  // Per step kb each wave issues R8_ACT activation loads for step kb + 2,
  // then FPW weight loads for step kb + AHEAD, and no other vector memory
  // operation.  The vector memory counter completes in issue order, so the
  // activation is requested before the weights: waiting for it never waits for
  // weights issued later.  Before the barrier that ends step kb a wave needs its
  // loads into step kb + 1's slot to be done.  The prologue issues W(kb0) ..
  // W(kb0 + AHEAD - 3), A(kb0), W(kb0 + AHEAD - 2), A(kb0 + 1),
  // W(kb0 + AHEAD - 1), so the loads issued after W(kb + 1) number
  // (AHEAD - 1) (FPW + R8_ACT) in the steady state and at least
  // (AHEAD - 1) FPW + min(3, AHEAD - 1) R8_ACT in the first steps; the wait
  // uses that smallest count, exact where it matters and never too lax.
  static_assert(AHEAD >= 3, "activation two steps ahead of at least three weight steps");
  constexpr int WAIT_AFTER = (AHEAD - 1) * FPW + (AHEAD - 1 < 3 ? AHEAD - 1 : 3) * R8_ACT;
  static_assert(WAIT_AFTER < 64, "vmcnt range");
  constexpr int WAITCNT = (WAIT_AFTER & 15) | ((WAIT_AFTER >> 4) << 14) | (7 << 4) | (15 << 8);

  // prologue, as if steps kb0 - AHEAD .. kb0 - 1 had run; then W(kb0)
  // complete (issued after it: AHEAD - 1 weight steps and two activation steps)
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) {
    if (i == AHEAD - 2) load_a(areg[0], kb0);
    if (i == AHEAD - 1) load_a(areg[1], kb0 + 1);
    __builtin_amdgcn_sched_barrier(0);
    load_w(Ws[i], kb0 + i);
    __builtin_amdgcn_sched_barrier(0);
  }
  constexpr int PRO = (AHEAD - 1) * FPW + 2 * R8_ACT;
  static_assert(PRO < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((PRO & 15) | ((PRO >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // one K step: request A(kb + 2) into the registers A(kb) leaves and
  // W(kb + AHEAD) into the slot freed by step kb - 1, then run the MFMAs of
  // step kb from its slot
  auto step = [&](int kb, uint16_t* cur, uint16_t* ahead, int par) {
    u32x4 acur[R8_ACT];
#pragma unroll
    for (int i = 0; i < R8_ACT; ++i) acur[i] = areg[par][i];
    __builtin_amdgcn_sched_barrier(0);
    load_a(areg[par], kb + 2);
    __builtin_amdgcn_sched_barrier(0);
    load_w(ahead, kb + AHEAD);
    __builtin_amdgcn_sched_barrier(0);
    const uint16_t* slot = cur + lane * 8;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const bf16x8 ahi = __builtin_bit_cast(bf16x8, acur[2 * st]);
      const bf16x8 alo = __builtin_bit_cast(bf16x8, acur[2 * st + 1]);
#pragma unroll
      for (int g = 0; g < NCR; g += 4) {
        bf16x8 w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (g + q < NCR)
            w[q] = __builtin_bit_cast(bf16x8,
                                      *(const u32x4*)(slot + (2 * (g + q) + st) * R8_BLK));
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (g + q < NCR)
            acc[g + q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[q], ahi, acc[g + q], 0, 0, 0);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (g + q < NCR)
            acc[g + q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[q], alo, acc[g + q], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(WAITCNT);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // nkb % NSLOT == 0 (NSLOT even): the slot of step kb0 + i is i % NSLOT and
  // its activation registers i % 2, static in the unrolled body
  for (int kb = kb0; kb <= kb_last; kb += NSLOT) {
#pragma unroll
    for (int i = 0; i < NSLOT; ++i)
      step(kb + i, Ws[i], Ws[(i + NSLOT - 1) % NSLOT], i & 1);
  }
  // loads past the last step may still be landing in LDS: let them finish
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
}

// ---------------------------------------------------------------------------
// 128-row head (see the file header).
constexpr int S8_WAVES = 8;
constexpr int S8_NC = 20;                          // 32-column tiles per slice at most
constexpr int S8_NCW = S8_NC / 2;                  // tiles per wave (half a slice)
constexpr int S8_FPW = 2 * S8_NC / S8_WAVES;       // weight fragments per wave per step
constexpr int S8_WSLOT = 2 * S8_NC * R8_BLK;       // bf16 per weight slot
constexpr int S8_ASLOT = 16 * R8_BLK;              // bf16 per activation slot
constexpr int S8_CAND = 19;                        // candidates per lane before the full insertion

// Workgroups of the head: one per compute unit (fewer for a small
// vocabulary, at least 128 columns each), each slice at most S8_NC tiles.
int s8_slices(int V) {
  const int nt = (V + 31) / 32;
  const int need = (nt + S8_NC - 1) / S8_NC;
  return std::max(std::min((V + 127) / 128, cu_count()), need);
}

template <int KMAX, int NCR>
__device__ __forceinline__ void s8_loop(const HeadArgs& p, int tb, int T, int c0, int nkb,
                                        f32x16 (&acc)[S8_NCW], uint16_t* const (&Wsl)[3],
                                        uint16_t* const (&Asl)[2]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r4 = wave & 3;
  const int kblocks = p.d / 32, kb_last = nkb - 1;
  const int hh = lane >> 5, sub = (lane & 31) >> 4;
  const int vpad = (p.V + PACK_ROWS - 1) / PACK_ROWS * PACK_ROWS;
  const __amdgpu_buffer_rsrc_t wrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.Ut, (short)0, vpad * p.d * 2, 0x00020000);
  const int w_lane = (sub * R8_BLK + ((lane & 15) + 16 * hh) * 8) * 2;
  int wsoff[S8_FPW];
#pragma unroll
  for (int i = 0; i < S8_FPW; ++i) {
    const int f = wave + S8_WAVES * i;
    const int c = min(f / 2, T - 1), st = f % 2;
    const int j = tb + c;
    wsoff[i] = __builtin_amdgcn_readfirstlane(
        (((j / 4) * kblocks * 8 + 2 * (j % 4)) * R8_BLK + 256 * st) * 2);
  }
  // activation blocks: wave w copies row block w of the hi and the lo plane
  const __amdgpu_buffer_rsrc_t hrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.pa.hi, (short)0, 128 * p.d * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t lrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.pa.lo, (short)0, 128 * p.d * 2, 0x00020000);
  const int a_lane = lane * 16;
  const int a_soff = __builtin_amdgcn_readfirstlane(wave * kblocks * R8_BLK * 2);

  auto load_w = [&](uint16_t* slot, int kb) {
    kb = min(kb, kb_last);
#pragma unroll
    for (int i = 0; i < S8_FPW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wrs, (__attribute__((address_space(3))) void*)(slot + (wave + S8_WAVES * i) * R8_BLK),
          16, w_lane, wsoff[i] + kb * 8 * R8_BLK * 2, 0, 2 /* nt */);
  };
  auto load_a = [&](uint16_t* slot, int kb) {
    kb = min(kb, kb_last);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        hrs, (__attribute__((address_space(3))) void*)(slot + wave * R8_BLK), 16, a_lane,
        a_soff + kb * R8_BLK * 2, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        lrs, (__attribute__((address_space(3))) void*)(slot + (8 + wave) * R8_BLK), 16, a_lane,
        a_soff + kb * R8_BLK * 2, 0, 0);
  };
  constexpr int WAITCNT = (S8_FPW & 15) | ((S8_FPW >> 4) << 14) | (7 << 4) | (15 << 8);
#pragma unroll
  for (int c = 0; c < S8_NCW; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  // prologue: W(0), A(0), W(1); W(0) and A(0) complete before the first barrier
  load_w(Wsl[0], 0);
  __builtin_amdgcn_sched_barrier(0);
  load_a(Asl[0], 0);
  __builtin_amdgcn_sched_barrier(0);
  load_w(Wsl[1], 1);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(WAITCNT);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  const int a_rd = ((2 * r4 + sub) * R8_BLK + ((lane & 15) + 16 * hh) * 8);   // + plane * 8 blocks + st * 256
  const int b_rd = 2 * c0 * R8_BLK + lane * 8;
  static_assert(NCR >= 5 && NCR <= 10, "two groups of tiles per half step");
  // Split-phase step: the barrier that hands over the next step's slots sits
  // before the MFMAs of tiles 4 .. NCR - 1 of the second K half, so the next
  // step's activation fragments and first weight fragments are read from LDS
  // while those MFMAs run (no LDS latency at the start of a step).
  struct Carry { bf16x8 a[4]; bf16x8 b[4]; };       // a: (st, hi/lo); b: st 0, tiles 0..3
  auto rd = [&](const uint16_t* p) { return __builtin_bit_cast(bf16x8, *(const u32x4*)p); };
  auto read_head = [&](const uint16_t* as, const uint16_t* ws, Carry& c) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      c.a[2 * st] = rd(as + 256 * st);
      c.a[2 * st + 1] = rd(as + 8 * R8_BLK + 256 * st);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) c.b[q] = rd(ws + (2 * q) * R8_BLK);
  };
  auto mfma2 = [&](int t, const bf16x8& w, const bf16x8& ahi, const bf16x8& alo) {
    acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w, ahi, acc[t], 0, 0, 0);
    acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w, alo, acc[t], 0, 0, 0);
  };
  Carry cur;
  read_head(Asl[0] + a_rd, Wsl[0] + b_rd, cur);
  // scheduling groups: DS reads (0x100) and MFMAs (0x008) in the order written
#define S8_GROUP(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)
  auto step = [&](auto sw, auto sa, int kb) {
    constexpr int SW = decltype(sw)::value, SA = decltype(sa)::value;
    load_a(Asl[(SA + 1) % 2], kb + 1);
    __builtin_amdgcn_sched_barrier(0);
    load_w(Wsl[(SW + 2) % 3], kb + 2);
    __builtin_amdgcn_sched_barrier(0);
    const uint16_t* ws = Wsl[SW] + b_rd;
    constexpr int N0 = NCR - 4;
    bf16x8 w0[N0], w1[NCR];
#pragma unroll
    for (int q = 0; q < N0; ++q) w0[q] = rd(ws + (2 * (4 + q)) * R8_BLK);
#pragma unroll
    for (int q = 0; q < 4; ++q) mfma2(q, cur.b[q], cur.a[0], cur.a[1]);
#pragma unroll
    for (int q = 0; q < 4; ++q) w1[q] = rd(ws + (2 * q + 1) * R8_BLK);
#pragma unroll
    for (int q = 0; q < N0; ++q) mfma2(4 + q, w0[q], cur.a[0], cur.a[1]);
#pragma unroll
    for (int q = 4; q < NCR; ++q) w1[q] = rd(ws + (2 * q + 1) * R8_BLK);
#pragma unroll
    for (int q = 0; q < 4; ++q) mfma2(q, w1[q], cur.a[2], cur.a[3]);
    S8_GROUP(0x100, N0);
    S8_GROUP(0x008, 8);
    S8_GROUP(0x100, 4);
    S8_GROUP(0x008, 2 * N0);
    S8_GROUP(0x100, N0);
    S8_GROUP(0x008, 8);
    // every read of this step's slots is done (its data is in registers);
    // own loads of A(kb + 1) and W(kb + 1) complete; then hand over
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(WAITCNT & ~(15 << 8));     // vmcnt(FPW), lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    const bf16x8 ahi = cur.a[2], alo = cur.a[3];
    read_head(Asl[(SA + 1) % 2] + a_rd, Wsl[(SW + 1) % 3] + b_rd, cur);
#pragma unroll
    for (int q = 4; q < NCR; ++q) mfma2(q, w1[q], ahi, alo);
    S8_GROUP(0x100, 8);
    S8_GROUP(0x008, 2 * N0);
    __builtin_amdgcn_sched_barrier(0);
  };
#undef S8_GROUP
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  int kb = 0;
  for (; kb + 6 <= nkb; kb += 6) {
    step(I0{}, I0{}, kb);
    step(I1{}, I1{}, kb + 1);
    step(I2{}, I0{}, kb + 2);
    step(I0{}, I1{}, kb + 3);
    step(I1{}, I0{}, kb + 4);
    step(I2{}, I1{}, kb + 5);
  }
  if (kb < nkb) {            // nkb % 6 is 2 or 4
    step(I0{}, I0{}, kb);
    step(I1{}, I1{}, kb + 1);
    if (kb + 2 < nkb) {
      step(I2{}, I0{}, kb + 2);
      step(I0{}, I1{}, kb + 3);
    }
  }
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
}

template <int KMAX>
__global__ __launch_bounds__(64 * S8_WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_head_rows128(HeadArgs p) {
  if (p.skip && *p.skip) return;
  __shared__ __attribute__((aligned(16))) uint16_t W0[S8_WSLOT];
  __shared__ __attribute__((aligned(16))) uint16_t W1[S8_WSLOT];
  __shared__ __attribute__((aligned(16))) uint16_t W2[S8_WSLOT];
  __shared__ __attribute__((aligned(16))) uint16_t A0[S8_ASLOT];
  __shared__ __attribute__((aligned(16))) uint16_t A1[S8_ASLOT];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r4 = wave & 3, hf = wave >> 2;
  const int G = gridDim.x, slice = blockIdx.x;
  const int nt = (p.V + 31) / 32;
  const int base = nt / G, extra = nt % G;
  const int tb = slice * base + min(slice, extra);
  const int T = base + (slice < extra ? 1 : 0);                   // 1 .. S8_NC
  const int T0 = (T + 1) / 2;
  const int c0 = hf ? T0 : 0, Tw = hf ? T - T0 : T0;            // this wave's tiles
  const int hh = lane >> 5;
  f32x16 acc[S8_NCW];
  uint16_t* const Wsl[3] = {W0, W1, W2};
  uint16_t* const Asl[2] = {A0, A1};
  if (Tw == S8_NCW)
    s8_loop<KMAX, S8_NCW>(p, tb, T, c0, p.d / 32, acc, Wsl, Asl);
  else
    s8_loop<KMAX, S8_NCW - 1>(p, tb, T, c0, p.d / 32, acc, Wsl, Asl);

  const float scale = p.greedy ? 1.f : p.inv_T;
  const int col0 = 32 * (tb + c0) + 4 * hh;
  const int lim = p.V - col0;
#pragma unroll
  for (int c = 0; c < S8_NCW; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int off = 32 * c + 8 * (e >> 2) + (e & 3);
      acc[c][e] = (c < Tw && off < lim) ? acc[c][e] * scale : -INFINITY;
    }
  float mx = -INFINITY;
  TopK<KMAX> tk;
  tk.clear();
  bool full = true;
  __syncthreads();
  if constexpr (KMAX == 4 || KMAX == 8) {
    float top[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) top[i] = -INFINITY;
#pragma unroll
    for (int g = 0; g < 2 * S8_NCW; ++g) {
      float x = acc[g >> 1][8 * (g & 1)];
#pragma unroll
      for (int i = 1; i < 8; ++i) x = fmaxf(x, acc[g >> 1][8 * (g & 1) + i]);
      mx = fmaxf(mx, x);
#pragma unroll
      for (int i = 0; i < KMAX; ++i) {
        const float hi = fmaxf(top[i], x);
        x = fminf(top[i], x);
        top[i] = hi;
      }
    }
    const float tau = top[KMAX - 1];
    // Candidate slots of the lane in W0 (waves 0..3) or W1 (waves 4..7):
    // values in the first half, columns in the second, slot j of thread t at
    // word 256 j + t % 256 of each half; slot S8_CAND takes the values that
    // are not kept.  Every value is written to the slot the count points at
    // and the count advances only for a value >= tau, so the scan has no
    // branch (a branch per value compiled to an exec-mask save and two taken
    // jumps each).
    static_assert(2 * (S8_CAND + 1) * 256 * 4 <= S8_WSLOT * 2, "candidate space");
    constexpr int SLOTB = 256 * 4, COLB = (S8_CAND + 1) * SLOTB;     // bytes
    float* cval = (float*)(hf ? W1 : W0) + (threadIdx.x & 255);
    uint32_t* ccol = (uint32_t*)(hf ? W1 : W0) + (S8_CAND + 1) * 256 + (threadIdx.x & 255);
    int cnt = 0;
    if (tau > -INFINITY) {
      char* const cb = (char*)cval;
      int off = 0;                                   // SLOTB * min(kept, S8_CAND)
#pragma unroll
      for (int c = 0; c < S8_NCW; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float v = acc[c][e];
          *(float*)(cb + off) = v;
          *(uint32_t*)(cb + off + COLB) = (uint32_t)(col0 + 32 * c + 8 * (e >> 2) + (e & 3));
          const bool keep = v >= tau;
          cnt += keep ? 1 : 0;
          off = min(off + (keep ? SLOTB : 0), S8_CAND * SLOTB);
        }
    } else {
      cnt = S8_CAND + 1;
    }
    full = __ballot(cnt > S8_CAND) != 0;
    if (!full) {
      int n = cnt;
#pragma unroll
      for (int m = 1; m < WAVE; m <<= 1) n = max(n, __shfl_xor(n, m, WAVE));
      n = __builtin_amdgcn_readfirstlane(n);
      // the candidates in runs of KMAX (empty keys past the lane's count),
      // each sorted by a network and folded in by a bitonic merge
      for (int r0 = 0; r0 < n; r0 += KMAX) {
        uint64_t run[KMAX];
#pragma unroll
        for (int i = 0; i < KMAX; ++i) {
          const int j = r0 + i;
          run[i] = j < cnt ? make_key(cval[256 * j], ccol[256 * j]) : 0ull;
        }
        TopK<KMAX> part;
        topk_of<KMAX, KMAX>(part, run);
        if (r0 == 0) {
#pragma unroll
          for (int i = 0; i < KMAX; ++i) tk.v[i] = part.v[i];
        } else {
          tk.merge(part.v);
        }
      }
    }
  }
  if (full) {
#pragma unroll
    for (int c = 0; c < S8_NCW; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float v = acc[c][e];
        if (v > -INFINITY) {
          mx = fmaxf(mx, v);
          tk.insert(make_key(v, (uint32_t)(col0 + 32 * c + 8 * (e >> 2) + (e & 3))));
        }
      }
  }
  float sum = 0.f;
  if (!p.greedy) {
    // e^(v - m0) as the hardware 2^x of (v - m0) log2(e): (v - m0) is within
    // the fp32 rounding of the value, the product adds one rounding
    const float m0 = mx > -INFINITY ? mx : 0.f;
#pragma unroll
    for (int c = 0; c < S8_NCW; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        sum += __builtin_amdgcn_exp2f((acc[c][e] - m0) * 1.44269504088896341f);
  }
  MaxSum ms{mx, sum};
  {
    const float m2 = __shfl_xor(ms.m, 32, WAVE);
    const float s2 = __shfl_xor(ms.s, 32, WAVE);
    ms.combine(m2, s2);
    uint64_t o[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) o[i] = shfl_xor_u64(tk.v[i], 32);
    tk.merge(o);
  }
  if (lane < 32) {
    // the two halves of a slice are reported as two consecutive slices
    const long o = (long)(32 * r4 + lane) * (2 * G) + 2 * slice + hf;
    p.ms_part[o] = make_float2(ms.m, ms.s);
#pragma unroll
    for (int i = 0; i < KMAX; ++i)
      if (i < p.k) p.key_part[o * p.k + i] = tk.v[i];
  }
}

// Split-K partial products of a 128-row GEMM on the same K loop: workgroup
// (slice, split) owns R8_GEMM_NC tiles of 32 output columns and K blocks
// [split * nkb, (split + 1) * nkb); wave w writes rows 32 w .. + 31 of
// part[split][128][N] (fp32), which the split-K reduction then sums in order.
constexpr int R8_GEMM_NC = 4;

__global__ __launch_bounds__(64 * R8_WAVES) __attribute__((amdgpu_waves_per_eu(2)))
void k_gemm_rows128(GemmArgs g) {
  if (g.skip && *g.skip) return;
  using C = R8Cfg<R8_GEMM_NC>;
  __shared__ __attribute__((aligned(16))) uint16_t Ws0[C::SLOT];
  __shared__ __attribute__((aligned(16))) uint16_t Ws1[C::SLOT];
  __shared__ __attribute__((aligned(16))) uint16_t Ws2[C::SLOT];
  __shared__ __attribute__((aligned(16))) uint16_t Ws3[C::SLOT];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slice = blockIdx.x, split = blockIdx.y;
  const int nt = g.N / 32;
  const int tb = slice * R8_GEMM_NC;
  const int T = min(R8_GEMM_NC, nt - tb);
  const int nkb = g.K / 32 / g.splits;
  const int npad = (g.N + PACK_ROWS - 1) / PACK_ROWS * PACK_ROWS;
  f32x16 acc[R8_GEMM_NC];
  uint16_t* const Ws[4] = {Ws0, Ws1, Ws2, Ws3};
  r8_mainloop<R8_GEMM_NC, R8_GEMM_NC, 0, 4>((const uint16_t*)g.Wt, npad, g.K, g.pa, tb, T,
                                            split * nkb, nkb, acc, Ws);
  // element e of lane l in tile c: row l % 32 of the wave, column
  // 32 (tb + c) + 8 (e / 4) + 4 (l / 32) + e % 4
  const int row = 32 * wave + (lane & 31);
  float* out = g.part + ((long)split * 128 + row) * g.N + 4 * (lane >> 5);
#pragma unroll
  for (int c = 0; c < R8_GEMM_NC; ++c)
    if (c < T)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(f32x4*)(out + 32 * (tb + c) + 8 * q) =
            f32x4{acc[c][4 * q], acc[c][4 * q + 1], acc[c][4 * q + 2], acc[c][4 * q + 3]};
}

}  // namespace

#ifndef DT_ROWS128
#define DT_ROWS128 1
#endif

bool head_rows128_ok(const HeadArgs& p) {
  const long vpad = (long)(p.V + PACK_ROWS - 1) / PACK_ROWS * PACK_ROWS;
  return DT_ROWS128 && p.w_bf16 && p.w_packed && p.Mp == 128 && p.d % 128 == 0 &&
         vpad * p.d * 2 < (1L << 31);
}

int head_rows128_slices(const HeadArgs& p) { return 2 * s8_slices(p.V); }

bool gemm_rows128_ok(const GemmArgs& g) {
  const long npad = (long)(g.N + PACK_ROWS - 1) / PACK_ROWS * PACK_ROWS;
  const int kblocks = g.K / 32;
  return DT_ROWS128 && g.w_bf16 && g.w_packed && g.Mp == 128 && g.N % 32 == 0 &&
         g.K % 32 == 0 && g.splits >= 1 && kblocks % g.splits == 0 &&
         (kblocks / g.splits) % 4 == 0 && npad * g.K * 2 < (1L << 31);
}

hipError_t launch_gemm_rows128(const GemmArgs& g, hipStream_t st) {
  const dim3 grid((g.N / 32 + R8_GEMM_NC - 1) / R8_GEMM_NC, g.splits);
  hipLaunchKernelGGL(k_gemm_rows128, grid, dim3(64 * R8_WAVES), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_head_rows128(const HeadArgs& p, hipStream_t st) {
  const dim3 grid(s8_slices(p.V));
  switch (p.kmax) {
    case 1: hipLaunchKernelGGL(k_head_rows128<1>, grid, dim3(64 * S8_WAVES), 0, st, p); break;
    case 4: hipLaunchKernelGGL(k_head_rows128<4>, grid, dim3(64 * S8_WAVES), 0, st, p); break;
    case 8: hipLaunchKernelGGL(k_head_rows128<8>, grid, dim3(64 * S8_WAVES), 0, st, p); break;
    case 16: hipLaunchKernelGGL(k_head_rows128<16>, grid, dim3(64 * S8_WAVES), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dt
