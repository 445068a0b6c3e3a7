// One tree-attention layer of the verification forward (gfx950).
//
// Rows are (tree query i, query head hh within a key/value group), so the
// Hq / Hkv query heads that share a key/value head share every K/V tile.
// Keys [0, P) are the prefix (always visible), keys [P, P + n) the tree nodes
// (visible where the query's ancestor bitmask has the bit); both are cut into
// blocks of 32 keys, the prefix blocks first, so no block mixes the two.
//
// Work split.  A workgroup of four waves owns one key/value head, 64 rows and
// a contiguous range of key blocks; each wave takes a quarter of that range
// for all 64 rows.  A wave therefore reads each K/V byte of its keys from LDS
// once (rows are not split across waves), needs no barrier inside its loop,
// and the four partial softmax states are merged through LDS at the end.
// When the rows alone do not fill the chip, the key blocks are also split
// across workgroups and a second kernel merges those partial states:
//   out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s   (m in log2 units).
// Workgroups that share a key range (same head and split, different rows) are
// numbered so that they land on the same XCD and share its L2.
//
// Per 32-key block a wave
//   * has had the block's K and V rows copied into one of its two LDS slots
//     by DMA (buffer loads with the LDS bit); a slot is refilled with the
//     block after next as soon as its data is in registers.  16-byte chunk c
//     of key row r sits at chunk c ^ sw(r), which makes both reads below free
//     of bank conflicts;
//   * forms S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (Q, the B operand,
//     stays in registers): lane l holds row 32 rt + l % 32 and keys
//     8 (e / 4) + 4 (l / 32) + e % 4 of the block;
//   * forms p = 2^(s log2(e) scale - m) against a per-row reference m that is
//     fixed for the whole pass (see the loop), so O is never rescaled inside
//     the loop and the accumulators stay in the matrix registers;
//   * forms O^T += V^T P^T: the B operand is the lane's own probabilities
//     rounded to bf16 (the contraction index runs over keys in the order the
//     lane holds them), the A operand V^T comes from the row-major V tile
//     through the LDS transpose read (ds_read_b64_tr_b16).
#include <cmath>
#include <cfloat>
#include <type_traits>

#include "../../include/dartree.h"
#include "common.hpp"
#include "launch.hpp"

namespace dt {

namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int AT_THREADS = 256;
constexpr int AT_WAVES = 4;
constexpr int AT_ROWS = 64;                          // rows per workgroup (each wave: all of them)
constexpr int AT_KB = 32;                            // keys per block
constexpr int HD = 128;
constexpr int AT_ROWB = HD * 2;                      // bytes of one key row of one head
constexpr int AT_TILE = AT_KB * AT_ROWB;             // bytes of one K (or V) block: 8 KB
constexpr int AT_SLOT = AT_WAVES * AT_TILE;          // one slot array: a tile per wave
constexpr int AT_MWORDS = DT_MAX_B / 32;
static_assert(AT_ROWS * HD * 4 == AT_SLOT, "a wave's merge rows fill one slot array");
static_assert(4 * AT_SLOT + AT_ROWS * AT_MWORDS * 4 <= 160 * 1024, "fits one compute unit's LDS");
constexpr float RESCALE = 16.f;                      // p <= 2^RESCALE under a pass's reference

// vmcnt / lgkmcnt encodings of s_waitcnt (expcnt left at its maximum)
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int WAIT_LGKM0 = 15 | (3 << 14) | (7 << 4);
constexpr int AT_DMA_PER_BLOCK = 16;                 // 8 K + 8 V loads of 1 KB

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* kp;
  const uint16_t* vp;
  const uint16_t* kt;
  const uint16_t* vt;
  const uint32_t* mask;
  int n, P, Hq, Hkv, group, words, nrows;
  float sl2;          // |scale| log2(e), at least FLT_MIN
  uint32_t qneg;      // sign bits flipped in q when the scale is negative
  int rblocks, nsplit, npair, pblk, nblk;
  float* out;
  float* opart;       // [nsplit][Hkv][nrows][HD]     (nsplit > 1)
  float2* mlpart;     // [nsplit][Hkv][nrows] (m, l)
};

// chunk swizzle of key row r (only r % 16 matters): a bijection of 0..15, so
// the 16 rows of a K operand read land on 16 distinct chunks, and the four
// rows of one transpose read on four distinct 64-byte groups
__device__ __forceinline__ int at_sw(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

typedef __attribute__((ext_vector_type(4))) int i32x4;

// Buffer resource of a byte range (raw buffer, no stride; loads past
// num_bytes return zero).
__device__ __forceinline__ i32x4 at_rsrc(const void* p, uint32_t num_bytes) {
  const uint64_t a = (uint64_t)p;
  return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)num_bytes, 0x00020000};
}

// One 16-byte-per-lane buffer load straight into LDS: lane l's 16 bytes from
// voff land at lds_addr + 16 l.  Written as inline assembly (M0 set inside,
// no output register) so that the compiler, which cannot follow which slot a
// copy fills across the loop, does not add waits of its own; the kernel
// waits for these copies itself with s_waitcnt vmcnt.
__device__ __forceinline__ void at_dma16(uint32_t lds_addr, int voff, int soff, i32x4 rsrc) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(const lds_void*)p);
}

__global__ __launch_bounds__(AT_THREADS) void k_tree_attn(AttnArgs a) {
  // two slots (K0/V0 and K1/V1), a tile per wave in each array
  __shared__ __attribute__((aligned(16))) unsigned char K0[AT_SLOT];
  __shared__ __attribute__((aligned(16))) unsigned char V0[AT_SLOT];
  __shared__ __attribute__((aligned(16))) unsigned char K1[AT_SLOT];
  __shared__ __attribute__((aligned(16))) unsigned char V1[AT_SLOT];
  __shared__ uint32_t Ms[AT_ROWS * AT_MWORDS];       // ancestor mask words of the 64 rows
  // workgroup -> (pair = head * nsplit + split, row block); the hardware
  // deals workgroups to the 8 XCDs round-robin, so every row block of a pair
  // gets a number with the same residue mod 8
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int pair = xcd + 8 * (j / a.rblocks), rb = j % a.rblocks;
  if (pair >= a.npair) return;
  const int g = pair / a.nsplit, split = pair % a.nsplit;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int row0 = rb * AT_ROWS;

  // this wave's key blocks
  const int wb = (int)((long)split * a.nblk / a.nsplit);
  const int we = (int)((long)(split + 1) * a.nblk / a.nsplit);
  const int b0 = wb + wave * (we - wb) / AT_WAVES;
  const int b1 = wb + (wave + 1) * (we - wb) / AT_WAVES;
  const int nb = b1 - b0;
  const int wo = wave * AT_TILE;                      // this wave's tile in each slot array

  const int rowstride = a.Hkv * AT_ROWB;
  const i32x4 kpr = at_rsrc(a.kp, (uint32_t)(a.P * rowstride));
  const i32x4 vpr = at_rsrc(a.vp, (uint32_t)(a.P * rowstride));
  const i32x4 ktr = at_rsrc(a.kt, (uint32_t)(a.n * rowstride));
  const i32x4 vtr = at_rsrc(a.vt, (uint32_t)(a.n * rowstride));

  // K and V rows of block b -> LDS at kd, vd: load j of 1 KB covers key rows
  // 4 j .. 4 j + 3, lane l writes chunk l % 16 of row 4 j + l / 16, i.e.
  // loads chunk (l % 16) ^ sw(row).  In a whole block the lane's offset is
  // one of four constants and the key offset is a scalar; in the last,
  // partial block keys past the end re-read the last key (masked).
  const int t4 = lane >> 4;
  int lpart[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) lpart[j] = t4 * rowstride + g * AT_ROWB + (((lane & 15) ^ (4 * t4 + j)) << 4);
  auto issue = [&](int b, unsigned char* kd, unsigned char* vd) {
    const bool pre = b < a.pblk;
    const int key0 = pre ? AT_KB * b : AT_KB * (b - a.pblk);
    const int kend = pre ? a.P : a.n;
    const i32x4 kr = pre ? kpr : ktr, vr = pre ? vpr : vtr;
    const uint32_t kl = lds_addr_of(kd), vl = lds_addr_of(vd);
    if (key0 + AT_KB <= kend) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int so = (key0 + 4 * jj) * rowstride;
        at_dma16(kl + 1024 * jj, lpart[jj & 3], so, kr);
        at_dma16(vl + 1024 * jj, lpart[jj & 3], so, vr);
      }
    } else {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int r = 4 * jj + t4;
        const int key = min(key0 + r, kend - 1);
        const int voff = (key * a.Hkv + g) * AT_ROWB + (((lane & 15) ^ at_sw(r)) << 4);
        at_dma16(kl + 1024 * jj, voff, 0, kr);
        at_dma16(vl + 1024 * jj, voff, 0, vr);
      }
    }
  };

  // the first two blocks are requested before anything else
  if (nb > 0) issue(b0, K0 + wo, V0 + wo);
  if (nb > 1) issue(b0 + 1, K1 + wo, V1 + wo);
  // ancestor mask words of the 64 rows, only where the range has tree blocks
  const bool any_tree = (int)((long)(split + 1) * a.nblk / a.nsplit) > a.pblk;
  if (any_tree) {
    for (int idx = tid; idx < AT_ROWS * a.words; idx += AT_THREADS) {
      const int r = idx / a.words, w = idx % a.words, rr = row0 + r;
      Ms[r * AT_MWORDS + w] = rr < a.nrows ? a.mask[(long)(rr / a.group) * a.words + w] : 0u;
    }
  }
  // Q, the B operand of S^T: row 32 rt + l32, dims 16 ks + 8 h .. + 7 (rows
  // past the end read the last row; their results are not written)
  u32x4 qf[2][8];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int rr = min(row0 + 32 * rt + l32, a.nrows - 1);
    const int qi = rr / a.group, hq = g * a.group + rr % a.group;
    const uint16_t* qp = a.q + ((long)qi * a.Hq + hq) * HD + 8 * h;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      qf[rt][ks] = *(const u32x4*)(qp + 16 * ks) ^ u32x4{a.qneg, a.qneg, a.qneg, a.qneg};
  }
  if (any_tree) __syncthreads();                      // mask words visible

  // LDS read offsets.  K (A operand of S^T): row l32, dims 16 ks + 8 h .. + 7.
  // V^T (A operand of O^T) by transpose read: this lane supplies key
  // 16 ks + 8 i + 4 (G / 2) + e4 and dims 32 dt + 16 (G % 2) + 4 q4 .. + 3,
  // G = lane / 16, e4 = lane % 16 / 4, q4 = lane % 4; it receives dims
  // 32 dt + lane % 32 of keys 16 ks + 8 i + 4 h + 0 .. 3.
  const int swk = at_sw(l32);
  int kofs[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) kofs[ks] = l32 * AT_ROWB + (((2 * ks + h) ^ swk) << 4);
  const int G = lane >> 4, e4 = (lane & 15) >> 2, q4 = lane & 3;
  int vofs[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int key = 8 * i + 4 * (G >> 1) + e4;
      const int chunk = 4 * dt + 2 * (G & 1) + (q4 >> 1);
      vofs[i][dt] = key * AT_ROWB + ((chunk ^ at_sw(key)) << 4) + 8 * (q4 & 1);
    }

  const float sl2 = a.sl2;
  f32x16 o[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[rt][dt][e] = 0.f;
  // m = -inf marks a row this wave saw no visible key of (weight 0 when merged)
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};

  // visibility of block b: whole prefix blocks see every key; otherwise keys
  // past the end and (tree blocks) keys off the row's ancestor path are masked
  struct Vis {
    bool masked;
    uint32_t w[2];
  };
  auto vis_of = [&](int b) {
    Vis v;
    const bool pre = b < a.pblk;
    const int key0 = pre ? AT_KB * b : AT_KB * (b - a.pblk);
    const int nvalid = (pre ? a.P : a.n) - key0;
    v.masked = !pre || nvalid < AT_KB;
    v.w[0] = v.w[1] = ~0u;
    if (v.masked) {
      const uint32_t lim = nvalid >= AT_KB ? ~0u : ((1u << nvalid) - 1u);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
        v.w[rt] = lim & (pre ? ~0u : Ms[(32 * rt + l32) * AT_MWORDS + (b - a.pblk)]);
    }
    return v;
  };
  auto kk_of = [&](int e) { return 8 * (e >> 2) + 4 * h + (e & 3); };
  // S^T of one block from slot Kt: s[rt] = K Q^T for rows 32 rt + l32
  auto scores = [&](const unsigned char* Kt, f32x16 (&s)[2]) {
    bf16x8 kf[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kf[ks] = *(const bf16x8*)(Kt + kofs[ks]);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[rt][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
        s[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            kf[ks], __builtin_bit_cast(bf16x8, qf[rt][ks]), s[rt], 0, 0, 0);
  };
  auto vread = [&](const unsigned char* Vt, bf16x8 (&vf)[4][2]) {
    typedef __attribute__((ext_vector_type(8))) short s16x8;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(Vt + vofs[0][dt] + ks * 16 * AT_ROWB));
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(Vt + vofs[1][dt] + ks * 16 * AT_ROWB));
        vf[dt][ks] = __builtin_bit_cast(bf16x8, s16x8{v0[0], v0[1], v0[2], v0[3],
                                                      v1[0], v1[1], v1[2], v1[3]});
      }
  };

  // The reference m of a row is fixed for a whole pass over the wave's
  // blocks.  It starts as the largest raw score of the first block (mask
  // ignored, so it is finite).  A pass is redone from its first block when a
  // visible score exceeds m by more than RESCALE (m becomes that block's
  // maximum, p stays <= 2^RESCALE) or when the row's largest visible score
  // ends up more than GAP below m (m becomes that maximum, so p does not
  // underflow).  Each redo raises m by more than RESCALE or sets it to the
  // true maximum, so passes end; with scores of ordinary size one pass is all
  // there is.
  constexpr float GAP = 64.f;
  if (nb > 0) {
    __builtin_amdgcn_s_waitcnt(wait_vm(0));           // q, the mask words, blocks 0 and 1
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s[2];
    scores(K0 + wo, s);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      float x = s[rt][0];
#pragma unroll
      for (int e = 1; e < 16; ++e) x = fmaxf(x, s[rt][e]);
      x *= sl2;
      m[rt] = fmaxf(x, __shfl_xor(x, 32, 64));
    }
  }
  for (int pass = 0; nb > 0; ++pass) {
    if (pass > 0) {
      __builtin_amdgcn_s_waitcnt(wait_vm(0));       // the last pass's copies have landed
      asm volatile("" ::: "memory");
      issue(b0, K0 + wo, V0 + wo);
      if (nb > 1) issue(b0 + 1, K1 + wo, V1 + wo);
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      l[rt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[rt][dt][e] = 0.f;
    }
    float mx[2] = {-INFINITY, -INFINITY};     // largest visible score (log2 units)
    bool redo = false;
    for (int i = 0; i < nb; ++i) {
      unsigned char* const Kt = ((i & 1) ? K1 : K0) + wo;
      unsigned char* const Vt = ((i & 1) ? V1 : V0) + wo;
      if (i + 1 < nb) __builtin_amdgcn_s_waitcnt(wait_vm(AT_DMA_PER_BLOCK));   // block i + 1 may be in flight
      else __builtin_amdgcn_s_waitcnt(wait_vm(0));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      f32x16 s[2];
      scores(Kt, s);
      bf16x8 vf[4][2];
      vread(Vt, vf);
      // the slot's data is in registers once these reads return: refill it
      // now, so the copy has this block's and the next block's work to land
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
      asm volatile("" ::: "memory");
      if (i + 2 < nb) issue(b0 + i + 2, Kt, Vt);
      __builtin_amdgcn_sched_barrier(0);
      const Vis v = vis_of(b0 + i);
      if (v.masked) {                      // masked scores become -inf (p = 0)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (!((v.w[rt] >> kk_of(e)) & 1u)) s[rt][e] = -INFINITY;
      }
      float lm[2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        float x = s[rt][0];
#pragma unroll
        for (int e = 1; e < 16; ++e) x = fmaxf(x, s[rt][e]);
        lm[rt] = x * sl2;
      }
      if (__ballot(lm[0] > m[0] + RESCALE || lm[1] > m[1] + RESCALE) != 0) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) m[rt] = fmaxf(m[rt], fmaxf(lm[rt], __shfl_xor(lm[rt], 32, 64)));
        redo = true;
        break;
      }
      bf16x8 pb[2][2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        mx[rt] = fmaxf(mx[rt], lm[rt]);
        const float nm = -m[rt];
        float p[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rt][e], sl2, nm));   // exp2(-inf) = 0
          l[rt] += p[e];
        }
        typedef __attribute__((ext_vector_type(2))) float f2;
        typedef __attribute__((ext_vector_type(2))) __bf16 b2;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          uint32_t pk[4];
#pragma unroll
          for (int c = 0; c < 4; ++c)
            pk[c] = __builtin_bit_cast(uint32_t, __builtin_convertvector(
                                                     f2{p[8 * ks + 2 * c], p[8 * ks + 2 * c + 1]}, b2));
          pb[rt][ks] = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
        }
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
            o[rt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[dt][ks], pb[rt][ks], o[rt][dt],
                                                                0, 0, 0);
    }
    if (!redo) {
      float bx[2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) bx[rt] = fmaxf(mx[rt], __shfl_xor(mx[rt], 32, 64));
      const bool low0 = bx[0] > -INFINITY && bx[0] < m[0] - GAP;
      const bool low1 = bx[1] > -INFINITY && bx[1] < m[1] - GAP;
      if (__ballot(low0 || low1) != 0) {
        if (low0) m[0] = bx[0];
        if (low1) m[1] = bx[1];
        redo = true;
      } else {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          if (bx[rt] == -INFINITY) m[rt] = -INFINITY;   // no visible key here (l = 0, O = 0)
      }
    }
    if (!redo) break;
  }

#pragma unroll
  for (int rt = 0; rt < 2; ++rt) l[rt] += __shfl_xor(l[rt], 32, 64);

  // merge the four waves' states through LDS (the slots are free now): wave w
  // writes its unnormalised O rows into slot array w, f32x4 chunk c of row r
  // at chunk c ^ (r % 32), and (m, l) into the mask array
  __syncthreads();
  unsigned char* const OW[AT_WAVES] = {K0, V0, K1, V1};
  float2* mlw = (float2*)Ms;
  {
    float* Ow = (float*)(wave == 0 ? K0 : wave == 1 ? V0 : wave == 2 ? K1 : V1);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int r = 32 * rt + l32;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int c4 = (8 * dt + 2 * c + h) ^ (r & 31);
          *(f32x4*)(Ow + r * HD + 4 * c4) = f32x4{o[rt][dt][4 * c], o[rt][dt][4 * c + 1],
                                                  o[rt][dt][4 * c + 2], o[rt][dt][4 * c + 3]};
        }
      if (h == 0) mlw[wave * AT_ROWS + r] = make_float2(m[rt], l[rt]);
    }
  }
  __syncthreads();
  {
    const int r = tid >> 2, qd = tid & 3, rr = row0 + r;
    if (rr < a.nrows) {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < AT_WAVES; ++w) M = fmaxf(M, mlw[w * AT_ROWS + r].x);
      float wt[AT_WAVES], L = 0.f;
#pragma unroll
      for (int w = 0; w < AT_WAVES; ++w) {
        const float2 ml = mlw[w * AT_ROWS + r];
        wt[w] = ml.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml.x - M);
        L += wt[w] * ml.y;
      }
      const int qi = rr / a.group, hq = g * a.group + rr % a.group;
      const float inv = L > 0.f ? 1.f / L : 0.f;
      float* dst = a.nsplit == 1 ? a.out + ((long)qi * a.Hq + hq) * HD
                                 : a.opart + (((long)split * a.Hkv + g) * a.nrows + rr) * HD;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int c4 = 8 * qd + c;
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < AT_WAVES; ++w)
          acc += wt[w] * *(const f32x4*)((const float*)OW[w] + r * HD + 4 * (c4 ^ (r & 31)));
        *(f32x4*)(dst + 4 * c4) = a.nsplit == 1 ? acc * inv : acc;
      }
      if (a.nsplit > 1 && qd == 0)
        a.mlpart[((long)split * a.Hkv + g) * a.nrows + rr] = make_float2(M, L);
    }
  }
}

// out[i][h][4 j .. 4 j + 3] for row (i, hh) of key/value head g = h / group:
// out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s (m in log2 units).
__global__ void k_tree_attn_combine(AttnArgs a) {
  const int nrows = a.nrows;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long)a.Hkv * nrows * (HD / 4)) return;
  const int d4 = gid % (HD / 4);
  const int row = (gid / (HD / 4)) % nrows;
  const int g = gid / ((long)(HD / 4) * nrows);
  // every split's (m, l) and partial output requested at once (one round
  // trip), in groups of CMB_SPLITS
  constexpr int CMB_SPLITS = 8;
  float M = -INFINITY;
  f32x4 num = f32x4{0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int s0 = 0; s0 < a.nsplit; s0 += CMB_SPLITS) {
    float2 ml[CMB_SPLITS];
    f32x4 v[CMB_SPLITS];
#pragma unroll
    for (int j = 0; j < CMB_SPLITS; ++j) {
      ml[j] = make_float2(-INFINITY, 0.f);
      v[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (s0 + j < a.nsplit) {
        const long b = ((long)(s0 + j) * a.Hkv + g) * nrows + row;
        ml[j] = a.mlpart[b];
        v[j] = *(const f32x4*)(a.opart + b * HD + 4 * d4);
      }
    }
    // the group's largest m; earlier groups' sums are rescaled to it (with
    // one group this is the plain sum against the global maximum)
    float Mg = M;
#pragma unroll
    for (int j = 0; j < CMB_SPLITS; ++j) Mg = fmaxf(Mg, ml[j].x);
    if (Mg == -INFINITY) continue;                   // no visible key so far
    if (Mg > M && M != -INFINITY) {
      const float c = __builtin_amdgcn_exp2f(M - Mg);
      num *= c;
      den *= c;
    }
    M = Mg;
#pragma unroll
    for (int j = 0; j < CMB_SPLITS; ++j) {
      const float w = ml[j].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[j].x - M);
      num += w * v[j];
      den += w * ml[j].y;
    }
  }
  const int i = row / a.group, h = g * a.group + row % a.group;
  *(f32x4*)(a.out + ((long)i * a.Hq + h) * HD + 4 * d4) =
      den > 0.f ? num / den : f32x4{0.f, 0.f, 0.f, 0.f};
}

// Key-block splits across workgroups: enough workgroups (about one per
// compute unit per round of 256) to fill the chip, at least four blocks per
// workgroup.
struct AttnPlan {
  int nrows, rblocks, pblk, nblk, nsplit, npair, grid;
};

AttnPlan attn_plan(int n, int P, int Hkv, int group) {
  AttnPlan p;
  p.nrows = n * group;
  p.rblocks = (p.nrows + AT_ROWS - 1) / AT_ROWS;
  p.pblk = (P + AT_KB - 1) / AT_KB;
  p.nblk = p.pblk + (n + AT_KB - 1) / AT_KB;
  const int base = Hkv * p.rblocks;
  const int rounds = (base + 255) / 256;
  int s = 256 * rounds / base;           // whole rounds of one workgroup per compute unit
  s = std::min(s, std::max(1, p.nblk / AT_WAVES));
  p.nsplit = std::max(1, s);
  p.npair = Hkv * p.nsplit;
  p.grid = (p.npair + 7) / 8 * 8 * p.rblocks;
  return p;
}

}  // namespace

}  // namespace dt

using namespace dt;

extern "C" size_t tree_attention_workspace_size(int n_tree, int P, int Hq, int Hkv, int hd) {
  if (n_tree < 1 || n_tree > DT_MAX_B || P < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv || hd != HD)
    return 0;
  const AttnPlan p = attn_plan(n_tree, P, Hkv, Hq / Hkv);
  if (p.nsplit == 1) return 256;
  const size_t rows = (size_t)Hkv * p.nrows;
  const size_t o = ((size_t)p.nsplit * rows * HD * 4 + 255) / 256 * 256;
  return o + (size_t)p.nsplit * rows * sizeof(float2);
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
  // key offsets of the buffer loads are 32-bit
  if ((long)P * Hkv * AT_ROWB >= (1L << 31)) return DT_EUNSUPPORTED;
  const size_t need = tree_attention_workspace_size(n_tree, P, Hq, Hkv, hd);
  if (!workspace || workspace_bytes < need) return DT_EWORKSPACE;
  const AttnPlan p = attn_plan(n_tree, P, Hkv, Hq / Hkv);
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
  a.nrows = p.nrows;
  // scores in log2 units; a negative scale negates q instead (exact in bf16)
  a.sl2 = std::max(std::fabs(scale) * 1.4426950408889634f, FLT_MIN);
  a.qneg = scale < 0.f ? 0x80008000u : 0u;
  a.rblocks = p.rblocks;
  a.nsplit = p.nsplit;
  a.npair = p.npair;
  a.pblk = p.pblk;
  a.nblk = p.nblk;
  a.out = out;
  const size_t rows = (size_t)Hkv * p.nrows;
  a.opart = (float*)workspace;
  a.mlpart = (float2*)((char*)workspace + ((size_t)p.nsplit * rows * HD * 4 + 255) / 256 * 256);
  struct Ctx {
    AttnArgs a;
    int grid;
    hipStream_t st;
  } ctx{a, p.grid, (hipStream_t)stream};
  auto run = [](void* c_) -> hipError_t {
    Ctx& c = *(Ctx*)c_;
    hipLaunchKernelGGL(k_tree_attn, dim3(c.grid), dim3(AT_THREADS), 0, c.st, c.a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || c.a.nsplit == 1) return e;
    const long tot = (long)c.a.Hkv * c.a.nrows * (HD / 4);
    hipLaunchKernelGGL(k_tree_attn_combine, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0,
                       c.st, c.a);
    return hipGetLastError();
  };
  return dt::timed_launch(DT_K_ATTN, ctx.st, run, &ctx) == hipSuccess ? DT_OK : DT_EHIP;
}
