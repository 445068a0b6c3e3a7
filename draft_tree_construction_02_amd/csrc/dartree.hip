// C ABI of the library: argument validation, workspace layout and the
// per-depth launch sequence of depth-wise batched supertree construction.
//
// One depth t (one batched head call over all R * W surviving branches):
//   gemm1  H  = GELU((E[tok] + h_t) W1)             split-K, last split reduces
//   gemm2  s' = s_parent + H W2                      split-K, last split reduces
//   head   per vocabulary tile: (max, sum exp) and top-k of s' U / T
//   merge  per row: log-sum-exp and top-k over all tiles -> children, logp
//   beam   per request: global top-W of parent score + logp, carry states
// Everything is enqueued on the caller's stream; nothing synchronises.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/dartree.h"
#include "launch.hpp"

using namespace dt;

namespace {

constexpr size_t ALIGN = 256;

size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

int padded_rows(int rows) {
  if (rows <= 16) return 16;
  if (rows <= 32) return 32;
  if (rows <= 64) return 64;
  return 128;
}

int kmax_for(int k, bool greedy) {
  if (greedy || k == 1) return 1;
  if (k <= 4) return 4;
  if (k <= 8) return 8;
  return 16;
}

// Split count for a split-K GEMM of K (nk chunks) over `tiles` column
// tiles: the largest divisor s of nk with at most 640 workgroups (1280 from
// 64 rows, where the MFMA work per byte is high, so more workgroups pay off)
// and fp32 partial traffic (written and read: 8 s Mp bytes per column) at
// most a quarter of the weight bytes (2 K per column).
int choose_splits(int nk, int tiles, int Mp, int K) {
  const long cap = Mp >= 64 ? 1280 : 640;
  int best = 1;
  for (int s = 1; s <= nk; ++s)
    if (nk % s == 0 && (long)tiles * s <= cap && 16L * s * Mp <= K) best = s;
  return best;
}

// Balanced split-K grid for 16-row bf16 products whose standard grid (tiles
// of 128 columns x choose_splits) is not a multiple of the compute units:
// runs x splits = 2 x CUs workgroups, splits a divisor of nk within the
// partial budget, each run at most 8 tiles of 16 columns.  Returns false when
// no such grid exists (the standard one stays).
bool choose_runs(int nk, int N, int Mp, int K, int std_wgs, int& splits, int& runs) {
  const int cus = device_cu_count();
  if (Mp != 16 || N % 16 != 0 || std_wgs % cus == 0) return false;
  const int nt = N / 16, G = 2 * cus;
  for (int s = nk; s >= 1; --s) {
    if (nk % s != 0 || G % s != 0 || 16L * s * Mp > K) continue;
    const int r = G / s;
    if (r <= nt && (nt + r - 1) / r <= 8) {
      splits = s;
      runs = r;
      return true;
    }
  }
  return false;
}

struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <class T>
  T* take(size_t n) {
    T* p = base ? (T*)(base + off) : nullptr;
    off += align_up(n * sizeof(T));
    return p;
  }
};

bool head_ok(const dt_head* h) {
  if (!h || !h->E || !h->W1t || !h->W2t || !h->Ut) return false;
  if (h->V < 1 || h->d < 1) return false;
  if (h->layout != DT_LAYOUT_ROWMAJOR && h->layout != DT_LAYOUT_PACKED) return false;
  if (h->wdtype == DT_BF16) return h->d % 128 == 0;
  if (h->wdtype == DT_F32) return h->d % 32 == 0 && h->layout == DT_LAYOUT_ROWMAJOR;
  return false;
}

int head_tiles_for(const dt_head* hd, int Mp);

// Workspace of the state update + head for Mp rows.
struct StepWs {
  float* part;                 // split-K partials (shared by both GEMMs)
  float* H;                    // [Mp][4d] fp32 (fp32 heads)
  uint16_t *H_hi, *H_lo;       // [Mp][4d] packed (bf16 heads)
  uint16_t *x_hi, *x_lo;       // [Mp][d] packed (bf16 heads)
  uint16_t *s_hi, *s_lo;       // [Mp][d] packed (bf16 heads)
  float2* ms_part;
  uint64_t* key_part;
  float2* ms2;                 // merge range results [Mp][MERGE_SPLITS_MAX]
  uint64_t* key2;
  int32_t* cand_tok;
  float* cand_lp;
  float* lse;
  int32_t* tok[2];
  float* score[2];
  int32_t* src[2];
  float* S[2];                 // [Mp][d] fp32 updated states (ping-pong)
  int Mp, tiles1, tiles2, tilesV, splits1, splits2;
  int runs1 = 0, runs2 = 0;    // balanced split-K grids (0: tiles of 128 columns)
};

// Launch shape of the state update and head for `rows` rows: padded rows,
// column tiles, split-K counts and balanced grids, vocabulary slices.
void shape_step(StepWs& w, const dt_head* h, int rows) {
  const int bf = h->wdtype == DT_BF16;
  const int d = h->d, V = h->V;
  const int TN = gemm_tile_n(bf), KC = gemm_k_chunk(bf);
  w.Mp = padded_rows(rows);
  w.tiles1 = (4 * d + TN - 1) / TN;
  w.tiles2 = (d + TN - 1) / TN;
  w.tilesV = (V + head_tile_n(bf) - 1) / head_tile_n(bf);
  w.tilesV = std::max(w.tilesV, head_tiles_for(h, w.Mp));   // slices of the launch, if more
  w.splits1 = choose_splits(d / KC, w.tiles1, w.Mp, d);
  w.splits2 = choose_splits(4 * d / KC, w.tiles2, w.Mp, 4 * d);
  w.runs1 = w.runs2 = 0;
  if (bf) {
    choose_runs(d / KC, 4 * d, w.Mp, d, w.tiles1 * w.splits1, w.splits1, w.runs1);
    choose_runs(4 * d / KC, d, w.Mp, 4 * d, w.tiles2 * w.splits2, w.splits2, w.runs2);
  }
}

// Workspace of the state update + head for up to `rows` rows: buffers that
// scale with the rows are sized for the largest padded count, the split-K
// partials and per-slice head results for the largest over every padded
// count up to it (a depth may run with fewer rows, so another launch shape).
StepWs carve_step(Carver& c, const dt_head* h, int rows, int k) {
  StepWs w{};
  const int bf = h->wdtype == DT_BF16;
  const int d = h->d;
  size_t part = 0, slices = 0;
  for (int m = 16;; m *= 2) {
    shape_step(w, h, m < rows ? m : rows);
    part = std::max(part, std::max((size_t)w.splits1 * w.Mp * 4 * d, (size_t)w.splits2 * w.Mp * d));
    slices = std::max(slices, (size_t)w.Mp * w.tilesV);
    if (m >= rows) break;
  }
  shape_step(w, h, rows);
  const size_t md = (size_t)w.Mp * d;
  w.part = c.take<float>(part);
  if (bf) {
    w.H_hi = c.take<uint16_t>(4 * md);
    w.H_lo = c.take<uint16_t>(4 * md);
    w.x_hi = c.take<uint16_t>(md);
    w.x_lo = c.take<uint16_t>(md);
    w.s_hi = c.take<uint16_t>(md);
    w.s_lo = c.take<uint16_t>(md);
  } else {
    w.H = c.take<float>(4 * md);
  }
  w.ms_part = c.take<float2>(slices);
  w.key_part = c.take<uint64_t>(slices * k);
  w.ms2 = c.take<float2>((size_t)w.Mp * MERGE_SPLITS_MAX);
  w.key2 = c.take<uint64_t>((size_t)w.Mp * MERGE_SPLITS_MAX * kmax_for(k, false));
  w.cand_tok = c.take<int32_t>((size_t)w.Mp * k);
  w.cand_lp = c.take<float>((size_t)w.Mp * k);
  w.lse = c.take<float>(w.Mp);
  for (int i = 0; i < 2; ++i) {
    w.tok[i] = c.take<int32_t>(w.Mp);
    w.score[i] = c.take<float>(w.Mp);
    w.src[i] = c.take<int32_t>(w.Mp);
    w.S[i] = c.take<float>(md);
  }
  return w;
}

// ---------------------------------------------------------------- timing
struct Timing {
  std::mutex mu;
  std::atomic<bool> on{false};     // read without the lock on every launch
  std::vector<hipEvent_t> free_ev;
  struct Rec { int cls; hipEvent_t a, b; };
  std::vector<Rec> pending;
  double total_ms[DT_K_COUNT] = {};
  int64_t count[DT_K_COUNT] = {};
} g_timing;

hipEvent_t take_event() {
  if (!g_timing.free_ev.empty()) {
    hipEvent_t e = g_timing.free_ev.back();
    g_timing.free_ev.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch` bracketed by events when timing is on.
template <class F>
hipError_t timed(int cls, hipStream_t st, F&& launch) {
  if (!g_timing.on.load(std::memory_order_relaxed)) return launch();
  std::lock_guard<std::mutex> lk(g_timing.mu);
  hipEvent_t a = take_event(), b = take_event();
  if (!a || !b) return launch();
  (void)hipEventRecord(a, st);
  hipError_t e = launch();
  (void)hipEventRecord(b, st);
  g_timing.pending.push_back({cls, a, b});
  return e;
}

}  // namespace

hipError_t dt::timed_launch(int cls, hipStream_t st, hipError_t (*fn)(void*), void* ctx) {
  return timed(cls, st, [&] { return fn(ctx); });
}

namespace {

void collect_pending() {
  for (auto& r : g_timing.pending) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      g_timing.total_ms[r.cls] += ms;
      g_timing.count[r.cls] += 1;
    }
    g_timing.free_ev.push_back(r.a);
    g_timing.free_ev.push_back(r.b);
  }
  g_timing.pending.clear();
}

// ---------------------------------------------------------------- one depth
struct DepthIo {
  const float* s_prev;      // residual source (rows indexed by src)
  const int32_t* tok;       // tokens entering the update (fp32 heads)
  const int32_t* src;       // residual row of each row (-1 none)
  const float* h;           // hidden base for this depth (fp32 heads)
  long h_req_stride;
  int rpr;
  int rows;
  float* s_out;             // updated states, rows_out rows of d
  int rows_out;
  const int32_t* skip = nullptr;   // device flag: launches do nothing when set
  bool prep = true;                // bf16: build the x planes here (else already built)
  const float* x_dense = nullptr;  // fp32: dense x rows instead of the gather
};

// s' = s_parent + GELU(x W1) W2 with x = E[tok] + h_t: (bf16 heads) x is
// formed as packed hi/lo planes, then two split-K GEMMs, each followed by its
// in-order reduction.
hipError_t run_update(const dt_head* hd, const StepWs& w, const DepthIo& io, hipStream_t st) {
  const int bf = hd->wdtype == DT_BF16, d = hd->d;
  const int packed = hd->layout == DT_LAYOUT_PACKED;
  hipError_t e = hipSuccess;
  // bf16 with few rows: the first product forms x while staging it
  const bool gather_bf16 = bf && io.prep && w.Mp <= gemm_gather_max_rows();
  if (bf && io.prep && !gather_bf16) {
    PrepArgs pr;
    pr.E = (const uint16_t*)hd->E;
    pr.d = d;
    pr.tok = io.tok;
    pr.h = io.h;
    pr.h_req_stride = io.h_req_stride;
    pr.rpr = io.rpr;
    pr.rows = io.rows;
    pr.Mp = w.Mp;
    pr.hi = w.x_hi;
    pr.lo = w.x_lo;
    e = timed(DT_K_REDUCE, st, [&] { return launch_prep_x(pr, st); });
    if (e != hipSuccess) return e;
  }
  GemmArgs g1;
  g1.skip = io.skip;
  g1.pa = PackedA{w.x_hi, w.x_lo, d};
  g1.a.gather = bf ? (gather_bf16 ? 1 : 0) : (io.x_dense ? 0 : 1);
  g1.a.a = io.x_dense;
  g1.a.lda = d;
  g1.a.E = hd->E;
  g1.a.ldE = d;
  g1.a.tok = io.tok;
  g1.a.h = io.h;
  g1.a.h_req_stride = io.h_req_stride;
  g1.a.rpr = io.rpr;
  g1.a.rows = io.rows;
  g1.Wt = hd->W1t;
  g1.w_bf16 = bf;
  g1.w_packed = packed;
  g1.N = 4 * d;
  g1.K = d;
  g1.Mp = w.Mp;
  g1.splits = w.splits1;
  g1.runs = w.runs1;
  g1.part = w.part;
  e = timed(DT_K_GEMM1, st, [&] { return launch_gemm(g1, st); });
  if (e != hipSuccess) return e;
  ReduceArgs r1;
  r1.skip = io.skip;
  r1.part = w.part;
  r1.splits = w.splits1;
  r1.Mp = w.Mp;
  r1.N = 4 * d;
  r1.rows = io.rows;
  r1.rows_out = io.rows;
  r1.epi = EPI_GELU;
  r1.out = bf ? nullptr : w.H;
  r1.out_hi = bf ? w.H_hi : nullptr;
  r1.out_lo = bf ? w.H_lo : nullptr;
  e = timed(DT_K_REDUCE, st, [&] { return launch_reduce(r1, st); });
  if (e != hipSuccess) return e;

  GemmArgs g2;
  g2.skip = io.skip;
  g2.pa = PackedA{w.H_hi, w.H_lo, 4 * d};
  g2.a.a = w.H;
  g2.a.lda = 4 * d;
  g2.a.rows = io.rows;
  g2.Wt = hd->W2t;
  g2.w_bf16 = bf;
  g2.w_packed = packed;
  g2.N = d;
  g2.K = 4 * d;
  g2.Mp = w.Mp;
  g2.splits = w.splits2;
  g2.runs = w.runs2;
  g2.part = w.part;
  e = timed(DT_K_GEMM2, st, [&] { return launch_gemm(g2, st); });
  if (e != hipSuccess) return e;
  ReduceArgs r2;
  r2.skip = io.skip;
  r2.part = w.part;
  r2.splits = w.splits2;
  r2.Mp = w.Mp;
  r2.N = d;
  r2.rows = io.rows;
  r2.rows_out = io.rows_out;
  r2.epi = EPI_RESID;
  r2.s_prev = io.s_prev;
  r2.src_row = io.src;
  r2.out = io.s_out;
  r2.out_hi = bf ? w.s_hi : nullptr;
  r2.out_lo = bf ? w.s_lo : nullptr;
  return timed(DT_K_REDUCE, st, [&] { return launch_reduce(r2, st); });
}

// Head + merge over `rows` states; bf16 heads read s' from w.s_* (packed),
// fp32 heads from the dense fp32 rows s.
// Vocabulary slices of the head launch for Mp rows.
int head_tiles_for(const dt_head* hd, int Mp) {
  HeadArgs p;
  p.w_bf16 = hd->wdtype == DT_BF16;
  p.w_packed = hd->layout == DT_LAYOUT_PACKED;
  p.V = hd->V;
  p.d = hd->d;
  p.Mp = Mp;
  return head_tiles(p);
}

hipError_t run_head(const dt_head* hd, const StepWs& w, const float* s, int rows, int k, float T,
                    int32_t* cand_tok, float* cand_lp, float* lse, hipStream_t st,
                    bool final_merge = true, const int32_t* skip = nullptr) {
  const bool greedy = T == 0.f;
  HeadArgs p;
  p.skip = skip;
  p.pa = PackedA{w.s_hi, w.s_lo, hd->d};
  p.a.a = s;
  p.a.lda = hd->d;
  p.a.rows = rows;
  p.Ut = hd->Ut;
  p.w_bf16 = hd->wdtype == DT_BF16;
  p.w_packed = hd->layout == DT_LAYOUT_PACKED;
  p.V = hd->V;
  p.d = hd->d;
  p.Mp = w.Mp;
  p.kmax = kmax_for(k, greedy);
  p.k = greedy ? 1 : k;
  p.inv_T = greedy ? 1.f : (float)(1.0 / (double)T);
  p.greedy = greedy;
  p.ms_part = w.ms_part;
  p.key_part = w.key_part;
  const int cls = head_rows128_ok(p) ? DT_K_HEAD128 : DT_K_HEAD;
  hipError_t e = timed(cls, st, [&] { return launch_head(p, st); });
  if (e != hipSuccess) return e;
  if (!final_merge)
    return timed(DT_K_MERGE, st, [&] {
      return launch_merge_part(w.ms_part, w.key_part, rows, head_tiles(p), p.k, p.kmax, w.ms2,
                               w.key2, st, skip);
    });
  return timed(DT_K_MERGE, st, [&] {
    return launch_merge(w.ms_part, w.key_part, rows, head_tiles(p), p.k, k, p.kmax, greedy,
                        w.ms2, w.key2, cand_tok, cand_lp, lse, st);
  });
}

}  // namespace

// ============================================================================
extern "C" {

const char* dartree_status_string(int s) {
  switch (s) {
    case DT_OK: return "ok";
    case DT_EINVAL: return "invalid argument";
    case DT_EWORKSPACE: return "workspace missing or too small";
    case DT_EUNSUPPORTED: return "outside this build's limits";
    case DT_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int dartree_version(void) { return (1 << 16) | 0; }

static int build_args_ok(const dt_head* head, int R, int D, int W, int k) {
  if (!head_ok(head)) return DT_EINVAL;
  if (R < 1 || D < 1 || W < 1 || k < 1 || k > head->V) return DT_EINVAL;
  if (D > DT_MAX_DEPTH || k > DT_MAX_K || (long)R * W > DT_MAX_ROWS ||
      (long)W * k > DT_MAX_CAND || (long)D * W > DT_MAX_POOL)
    return DT_EUNSUPPORTED;
  return DT_OK;
}

size_t build_supertree_workspace_size(const dt_head* head, int R, int D, int W, int k) {
  if (build_args_ok(head, R, D, W, k) != DT_OK) return 0;
  Carver c(nullptr);
  carve_step(c, head, R * W, k);
  return c.off;
}

namespace {

struct BuildWs {
  StepWs w;            // the depth loop (R * W rows)
  StepWs pre;          // base-candidate pass (chunks of rows of h)
  int32_t* cand_base;  // [R * D][n_cand]
  int32_t* msrc;       // Markov residual rows [Mp]
  int pre_rows;
};

int build_opts_ok(const dt_head* head, int k, const dt_build_opts* o) {
  if (!o) return DT_OK;
  if (o->flags & ~(DT_BUILD_MARKOV | DT_BUILD_BASE_CANDIDATES | DT_BUILD_MULTI_KERNEL))
    return DT_EINVAL;
  if (o->flags & DT_BUILD_BASE_CANDIDATES) {
    if (o->n_cand < k || o->n_cand > head->V) return DT_EINVAL;
    if (o->n_cand > DT_MAX_K) return DT_EUNSUPPORTED;
  }
  return DT_OK;
}

BuildWs carve_build(Carver& c, const dt_head* head, int R, int D, int W, int k,
                    const dt_build_opts* o) {
  BuildWs b{};
  b.w = carve_step(c, head, R * W, k);
  const bool base = o && (o->flags & DT_BUILD_BASE_CANDIDATES);
  if (base) {
    b.pre_rows = R * D < DT_MAX_ROWS ? R * D : DT_MAX_ROWS;
    b.pre = carve_step(c, head, b.pre_rows, o->n_cand);
    b.cand_base = c.take<int32_t>((size_t)R * D * o->n_cand);
  }
  if (o && (o->flags & DT_BUILD_MARKOV)) b.msrc = c.take<int32_t>(b.w.Mp);
  return b;
}

}  // namespace

size_t build_supertree_ex_workspace_size(const dt_head* head, int R, int D, int W, int k,
                                         const dt_build_opts* opts) {
  if (build_args_ok(head, R, D, W, k) != DT_OK || build_opts_ok(head, k, opts) != DT_OK)
    return 0;
  Carver c(nullptr);
  carve_build(c, head, R, D, W, k, opts);
  return c.off;
}

int build_supertree_ex(const dt_head* head, const float* h, const float* s0,
                       const int32_t* root_tok, int R, int D, int W, int k, float T,
                       const dt_build_opts* opts, int32_t* pool_tok, int32_t* pool_parent,
                       float* pool_score, int32_t* n_valid, void* workspace,
                       size_t workspace_bytes, void* stream) {
  int rc = build_args_ok(head, R, D, W, k);
  if (rc != DT_OK) return rc;
  rc = build_opts_ok(head, k, opts);
  if (rc != DT_OK) return rc;
  if (!h || !s0 || !root_tok || !pool_tok || !pool_parent || !pool_score || !n_valid)
    return DT_EINVAL;
  if (!(T >= 0.f) || !isfinite(T)) return DT_EINVAL;
  const size_t need = build_supertree_ex_workspace_size(head, R, D, W, k, opts);
  if (!workspace || workspace_bytes < need) return DT_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const bool greedy = T == 0.f, bf = head->wdtype == DT_BF16;
  const bool markov = opts && (opts->flags & DT_BUILD_MARKOV);
  const bool base = opts && (opts->flags & DT_BUILD_BASE_CANDIDATES);
  if (!bf && head->layout == DT_LAYOUT_ROWMAJOR && !markov && !base &&
      !(opts && (opts->flags & DT_BUILD_MULTI_KERNEL))) {
    // a head small enough for one workgroup's LDS: all depths in one launch
    SmallBuildArgs sa;
    sa.E = head->E; sa.W1t = head->W1t; sa.W2t = head->W2t; sa.Ut = head->Ut;
    sa.d = head->d; sa.V = head->V;
    sa.h = h; sa.s0 = s0; sa.root_tok = root_tok;
    sa.R = R; sa.D = D; sa.W = W; sa.k = k; sa.kmax = kmax_for(k, greedy);
    sa.greedy = greedy;
    sa.inv_T = greedy ? 1.f : (float)(1.0 / (double)T);
    sa.pool_tok = pool_tok; sa.pool_parent = pool_parent; sa.pool_score = pool_score;
    sa.n_valid = n_valid;
    if (small_build_ok(sa)) {
      const hipError_t e = timed(DT_K_BUILD_SMALL, st, [&] { return launch_build_small(sa, st); });
      return e == hipSuccess ? DT_OK : DT_EHIP;
    }
  }
  Carver c(workspace);
  BuildWs bw = carve_build(c, head, R, D, W, k, opts);
  const StepWs& w = bw.w;
  const int d = head->d, rows = R * W;
  const int n_cand = base ? opts->n_cand : 0;

  hipError_t e = hipSuccess;
  if (base) {
    // candidates of every (request, depth): the top n_cand of h_t U, in
    // chunks of rows of h
    for (int c0 = 0; c0 < R * D && e == hipSuccess; c0 += bw.pre_rows) {
      const int rc_rows = R * D - c0 < bw.pre_rows ? R * D - c0 : bw.pre_rows;
      const float* hs = h + (long)c0 * d;
      if (bf) {
        ReduceArgs r;
        r.part = hs;
        r.splits = 1;
        r.Mp = bw.pre.Mp;
        r.N = d;
        r.rows = rc_rows;
        r.rows_out = 0;
        r.epi = EPI_RESID;
        r.out_hi = bw.pre.s_hi;
        r.out_lo = bw.pre.s_lo;
        e = launch_reduce(r, st);
      }
      if (e == hipSuccess)
        e = run_head(head, bw.pre, hs, rc_rows, n_cand, 1.f, bw.cand_base + (long)c0 * n_cand,
                     bw.pre.cand_lp, bw.pre.lse, st);
    }
  }
  // Frontier rows per request: the frontier of depth t holds at most
  // min(W, keff^t) branches (the root alone at t = 0), so the plain build runs
  // depth t with that many rows per request, padded to the launch's rows;
  // the variants keep W rows throughout.
  const int keff = greedy ? 1 : k;
  const bool narrow = !markov && !base;
  auto width = [&](int t) {
    if (!narrow) return W;
    long r = 1;
    for (int i = 0; i < t && r < W; ++i) r *= keff;
    return (int)std::min<long>(r, W);
  };
  if (markov && e == hipSuccess) e = launch_markov_src(rows, W, w.Mp, bw.msrc, st);
  if (e == hipSuccess)
    e = launch_beam_init(R, width(0), padded_rows(R * width(0)), root_tok, w.tok[0], w.score[0],
                         w.src[0], st);
  for (int t = 0; t < D && e == hipSuccess; ++t) {
    const int cur = t & 1, nxt = cur ^ 1;
    const int rpr = width(t), rows_t = R * rpr;
    StepWs wt = w;                      // same buffers, this depth's launch shape
    shape_step(wt, head, rows_t);
    DepthIo io;
    io.s_prev = (t == 0 || markov) ? s0 : w.S[nxt];
    io.tok = w.tok[cur];
    io.src = markov ? bw.msrc : w.src[cur];
    io.h = h + (long)t * d;
    io.h_req_stride = (long)D * d;
    io.rpr = rpr;
    io.rows = rows_t;
    io.s_out = w.S[cur];
    io.rows_out = rows_t;
    e = run_update(head, wt, io, st);
    if (e != hipSuccess) break;
    // base candidates: the full merge gives each row's log-sum-exp, then the
    // children are chosen among the depth's candidates
    e = run_head(head, wt, w.S[cur], rows_t, k, T, w.cand_tok, w.cand_lp, w.lse, st, base);
    if (e != hipSuccess) break;
    if (base) {
      CandArgs ca;
      ca.s = w.S[cur];
      ca.lse = w.lse;
      ca.cand_base = bw.cand_base;
      ca.Ut = head->Ut;
      ca.u_bf16 = bf;
      ca.u_packed = head->layout == DT_LAYOUT_PACKED;
      ca.d = d; ca.W = W; ca.D = D; ca.t = t; ca.n_cand = n_cand; ca.k = k;
      ca.greedy = greedy;
      ca.inv_T = greedy ? 1.f : (float)(1.0 / (double)T);
      ca.cand_tok = w.cand_tok;
      ca.cand_lp = w.cand_lp;
      e = timed(DT_K_MERGE, st, [&] { return launch_cand_score(ca, rows_t, st); });
      if (e != hipSuccess) break;
    }
    BeamArgs b;
    b.R = R; b.W = W; b.k = k; b.D = D; b.t = t; b.greedy = greedy;
    if (base) {
      b.cand_tok = w.cand_tok;
      b.cand_lp = w.cand_lp;
    } else {
      b.ms2 = w.ms2;
      b.key2 = w.key2;
    }
    b.S = merge_splits(head_tiles_for(head, wt.Mp));
    b.kmax = kmax_for(k, greedy);
    b.score_in = w.score[cur];
    b.n_valid = n_valid;
    b.pool_tok = pool_tok;
    b.pool_parent = pool_parent;
    b.pool_score = pool_score;
    b.tok_out = w.tok[nxt];
    b.score_out = w.score[nxt];
    b.src_out = w.src[nxt];
    b.rpr_in = rpr;
    b.rpr_out = width(t + 1);
    b.Mp = padded_rows(R * b.rpr_out);
    e = timed(DT_K_MERGE, st, [&] { return launch_beam_step(b, st); });
  }
  return e == hipSuccess ? DT_OK : DT_EHIP;
}

int build_supertree(const dt_head* head, const float* h, const float* s0, const int32_t* root_tok,
                    int R, int D, int W, int k, float T, int32_t* pool_tok, int32_t* pool_parent,
                    float* pool_score, int32_t* n_valid, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return build_supertree_ex(head, h, s0, root_tok, R, D, W, k, T, nullptr, pool_tok, pool_parent,
                            pool_score, n_valid, workspace, workspace_bytes, stream);
}

size_t head_step_workspace_size(const dt_head* head, int rows, int k) {
  if (!head_ok(head) || rows < 1 || rows > DT_MAX_ROWS || k < 1 || k > DT_MAX_K ||
      k > head->V)
    return 0;
  Carver c(nullptr);
  carve_step(c, head, rows, k);
  return c.off;
}

int state_update(const dt_head* head, const float* s_in, const int32_t* tok, const float* h,
                 int rows, float* s_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!head_ok(head) || !s_in || !tok || !h || !s_out) return DT_EINVAL;
  if (rows < 1) return DT_EINVAL;
  if (rows > DT_MAX_ROWS) return DT_EUNSUPPORTED;
  if (s_in == s_out) return DT_EINVAL;
  const size_t need = head_step_workspace_size(head, rows, 1);
  if (!workspace || workspace_bytes < need) return DT_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  Carver c(workspace);
  StepWs w = carve_step(c, head, rows, 1);
  hipError_t e = launch_fill_rows(rows, w.Mp, tok, w.tok[0], w.src[0], st);
  if (e == hipSuccess) {
    DepthIo io;
    io.s_prev = s_in;
    io.tok = w.tok[0];
    io.src = w.src[0];
    io.h = h;
    io.h_req_stride = 0;
    io.rpr = 1;
    io.rows = rows;
    io.s_out = s_out;
    io.rows_out = rows;
    e = run_update(head, w, io, st);
  }
  return e == hipSuccess ? DT_OK : DT_EHIP;
}

int corrected_topk(const dt_head* head, const float* s, int rows, int k, float T,
                   int32_t* cand_tok, float* cand_lp, float* lse, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (!head_ok(head) || !s || !cand_tok || !cand_lp || !lse) return DT_EINVAL;
  if (rows < 1 || k < 1 || k > head->V) return DT_EINVAL;
  if (rows > DT_MAX_ROWS || k > DT_MAX_K) return DT_EUNSUPPORTED;
  if (!(T >= 0.f) || !isfinite(T)) return DT_EINVAL;
  const size_t need = head_step_workspace_size(head, rows, k);
  if (!workspace || workspace_bytes < need) return DT_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  Carver c(workspace);
  StepWs w = carve_step(c, head, rows, k);
  hipError_t e = hipSuccess;
  if (head->wdtype == DT_BF16) {
    // split the caller's fp32 states into the packed hi/lo planes
    ReduceArgs r;
    r.part = s;
    r.splits = 1;
    r.Mp = w.Mp;
    r.N = head->d;
    r.rows = rows;
    r.rows_out = 0;
    r.epi = EPI_RESID;
    r.out_hi = w.s_hi;
    r.out_lo = w.s_lo;
    e = launch_reduce(r, st);
  }
  if (e == hipSuccess) e = run_head(head, w, s, rows, k, T, cand_tok, cand_lp, lse, st);
  return e == hipSuccess ? DT_OK : DT_EHIP;
}

size_t pack_head_bytes(const dt_head* head) {
  if (!head_ok(head) || head->wdtype != DT_BF16) return 0;
  const size_t d = head->d, V = head->V;
  const size_t vpad = (V + PACK_ROWS - 1) / PACK_ROWS * PACK_ROWS;
  return align_up(4 * d * d * 2) * 2 + align_up(vpad * d * 2);
}

int pack_head(const dt_head* src, void* dst, size_t dst_bytes, dt_head* packed, void* stream) {
  if (!head_ok(src) || !packed) return DT_EINVAL;
  if (src->wdtype != DT_BF16 || src->layout != DT_LAYOUT_ROWMAJOR) return DT_EINVAL;
  const size_t need = pack_head_bytes(src);
  if (!dst || dst_bytes < need) return DT_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int d = src->d;
  char* base = (char*)dst;
  uint16_t* w1 = (uint16_t*)base;
  uint16_t* w2 = (uint16_t*)(base + align_up((size_t)4 * d * d * 2));
  uint16_t* u = (uint16_t*)(base + 2 * align_up((size_t)4 * d * d * 2));
  hipError_t e = launch_pack_weight((const uint16_t*)src->W1t, w1, 4 * d, d, st);
  if (e == hipSuccess) e = launch_pack_weight((const uint16_t*)src->W2t, w2, d, 4 * d, st);
  if (e == hipSuccess) e = launch_pack_weight((const uint16_t*)src->Ut, u, src->V, d, st);
  if (e != hipSuccess) return DT_EHIP;
  *packed = *src;
  packed->layout = DT_LAYOUT_PACKED;
  packed->W1t = w1;
  packed->W2t = w2;
  packed->Ut = u;
  return DT_OK;
}

// ---------------------------------------------------------------- sequential
struct SeqWs {
  StepWs step;
  SeqArgs a;
};

static SeqWs carve_seq(Carver& c, const dt_head* h, int D, int k, int B, bool greedy) {
  SeqWs s{};
  s.step = carve_step(c, h, 1, k);
  const int d = h->d, keff = greedy ? 1 : k, cap = B * keff;
  SeqArgs& a = s.a;
  a.state = c.take<float>((size_t)(B + 1) * d);
  if (h->wdtype != DT_BF16) a.x_f32 = c.take<float>((size_t)s.step.Mp * d);
  a.c_tok = c.take<int32_t>(cap);
  a.c_par = c.take<int32_t>(cap);
  a.c_depth = c.take<int32_t>(cap);
  a.c_row = c.take<int32_t>(cap);
  a.c_score = c.take<float>(cap);
  a.c_alive = c.take<uint32_t>((cap + 31) / 32);
  a.ctl = c.take<int32_t>(SEQ_CTL_WORDS);
  a.cur_score = c.take<float>(1);
  return s;
}

static int seq_args_ok(const dt_head* head, int D, int k, int B) {
  if (!head_ok(head)) return DT_EINVAL;
  if (D < 1 || k < 1 || k > head->V || B < 1) return DT_EINVAL;
  if (D > DT_MAX_DEPTH || k > DT_MAX_K || B > DT_MAX_B) return DT_EUNSUPPORTED;
  return DT_OK;
}

size_t build_tree_sequential_workspace_size(const dt_head* head, int D, int k, int B) {
  if (seq_args_ok(head, D, k, B) != DT_OK) return 0;
  Carver c(nullptr);
  carve_seq(c, head, D, k, B, false);
  return c.off;
}

int build_tree_sequential(const dt_head* head, const float* h, const float* s0,
                          const int32_t* root_tok, int D, int k, int B, float beta, float T,
                          int32_t* tok, int32_t* parent, int32_t* depth, float* score,
                          int32_t* n_out, void* workspace, size_t workspace_bytes,
                          void* stream) {
  int rc = seq_args_ok(head, D, k, B);
  if (rc != DT_OK) return rc;
  if (!h || !s0 || !root_tok || !tok || !parent || !depth || !score || !n_out) return DT_EINVAL;
  if (!(T >= 0.f) || !isfinite(T) || !(beta <= 0.f) || !isfinite(beta)) return DT_EINVAL;
  const size_t need = build_tree_sequential_workspace_size(head, D, k, B);
  if (!workspace || workspace_bytes < need) return DT_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const bool greedy = T == 0.f, bf = head->wdtype == DT_BF16;
  Carver c(workspace);
  SeqWs sw = carve_seq(c, head, D, k, B, greedy);
  const StepWs& w = sw.step;
  SeqArgs& a = sw.a;
  const int d = head->d;
  a.D = D; a.k = k; a.B = B; a.kmax = kmax_for(k, greedy);
  a.S = merge_splits(head_tiles_for(head, w.Mp));
  a.greedy = greedy; a.Mp = w.Mp; a.d = d; a.beta = beta;
  a.ms2 = w.ms2; a.key2 = w.key2;
  a.out_tok = tok; a.out_par = parent; a.out_depth = depth; a.out_score = score;
  a.n_out = n_out;
  a.E = head->E; a.h = h;
  if (bf) {
    a.x_hi = w.x_hi;
    a.x_lo = w.x_lo;
  }
  hipError_t e = launch_seq_init(a, s0, root_tok, st);
  // B call slots: the root's call and one per popped node that is expanded;
  // slots past the last expansion do nothing (device flag)
  for (int slot = 0; slot < B && e == hipSuccess; ++slot) {
    DepthIo io;
    io.s_prev = a.state;
    io.tok = nullptr;
    io.src = a.ctl + SEQ_CUR_ROW;
    io.h = h;
    io.h_req_stride = 0;
    io.rpr = 1;
    io.rows = 1;
    io.s_out = a.state + (long)slot * d;
    io.rows_out = 1;
    io.skip = a.ctl + SEQ_SKIP;
    io.prep = false;
    io.x_dense = bf ? nullptr : a.x_f32;
    e = run_update(head, w, io, st);
    if (e != hipSuccess) break;
    e = run_head(head, w, io.s_out, 1, k, T, w.cand_tok, w.cand_lp, w.lse, st, false,
                 io.skip);
    if (e != hipSuccess) break;
    e = timed(DT_K_MERGE, st, [&] { return launch_seq_step(a, slot, st); });
  }
  return e == hipSuccess ? DT_OK : DT_EHIP;
}

// ---------------------------------------------------------------- acceptance walk
struct WalkWs {
  StepWs step;                 // one chunk of CH rows, greedy keys
  WalkArgs a;
  float* S[2];                 // updated states of depth t (ping-pong) [nch * CH][d]
  uint64_t* key2_all;          // merge range results of every inner-node chunk
};

static WalkWs carve_walk(Carver& c, const dt_head* h, int R, int D, int B) {
  WalkWs w{};
  const int nodes = R * B;
  const int CH = padded_rows(nodes < DT_MAX_ROWS ? nodes : DT_MAX_ROWS);
  w.step = carve_step(c, h, CH, 1);
  WalkArgs& a = w.a;
  a.R = R; a.D = D; a.B = B; a.V = h->V; a.d = h->d;
  a.CH = CH;
  a.nch = (nodes + CH - 1) / CH;
  a.bf16 = h->wdtype == DT_BF16;
  a.S = merge_splits(head_tiles_for(h, CH));
  const size_t rows = (size_t)a.nch * CH, d = h->d, B1 = (size_t)B + 1;
  if (a.bf16) {
    a.x_hi = c.take<uint16_t>(rows * d);
    a.x_lo = c.take<uint16_t>(rows * d);
  } else {
    a.x_f32 = c.take<float>(rows * d);
  }
  w.S[0] = c.take<float>(rows * d);
  w.S[1] = c.take<float>(rows * d);
  w.key2_all = c.take<uint64_t>(rows * a.S);
  a.key2 = w.key2_all;
  a.has_child = c.take<uint8_t>((size_t)R * B1);
  a.pos = c.take<int32_t>((size_t)R * B1);
  a.row_req = c.take<int32_t>(rows);
  a.row_tok = c.take<int32_t>(rows);
  a.row_src = c.take<int32_t>(rows);
  a.row_gidx = c.take<int32_t>(rows);
  a.inner_req = c.take<int32_t>(rows);
  a.inner_node = c.take<int32_t>(rows);
  a.S_inner = c.take<float>(rows * d);
  a.ctl = c.take<int32_t>(2);
  a.skip = c.take<int32_t>(a.nch);
  return w;
}

static int walk_args_ok(const dt_head* target, int R, int D, int B) {
  if (!head_ok(target)) return DT_EINVAL;
  if (R < 1 || D < 1 || B < 1) return DT_EINVAL;
  if (D > DT_MAX_DEPTH || B > DT_MAX_B || (long)R * B > DT_MAX_WALK_NODES)
    return DT_EUNSUPPORTED;
  return DT_OK;
}

size_t accept_walk_workspace_size(const dt_head* target, int R, int D, int B) {
  if (walk_args_ok(target, R, D, B) != DT_OK) return 0;
  Carver c(nullptr);
  carve_walk(c, target, R, D, B);
  return c.off;
}

int accept_walk(const dt_head* target, const float* h, const float* s0, const int32_t* root_tok,
                int R, int D, int B, const int32_t* tok, int tok_stride,
                const int32_t* tok_index, const int32_t* parent, const int32_t* depth,
                const int32_t* n, int32_t* target_tok, int32_t* path, int32_t* accept_len,
                void* workspace, size_t workspace_bytes, void* stream) {
  int rc = walk_args_ok(target, R, D, B);
  if (rc != DT_OK) return rc;
  if (!h || !s0 || !root_tok || !tok || !parent || !depth || !n || !target_tok || !path ||
      !accept_len)
    return DT_EINVAL;
  if (tok_stride < (tok_index ? 1 : B)) return DT_EINVAL;
  const size_t need = accept_walk_workspace_size(target, R, D, B);
  if (!workspace || workspace_bytes < need) return DT_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  Carver c(workspace);
  WalkWs ww = carve_walk(c, target, R, D, B);
  WalkArgs& a = ww.a;
  a.root_tok = root_tok;
  a.tok = tok;
  a.tok_stride = tok_stride;
  a.tok_index = tok_index;
  a.parent = parent;
  a.depth = depth;
  a.n = n;
  a.E = target->E;
  a.h = h;
  a.target_tok = target_tok;
  a.path = path;
  a.accept_len = accept_len;
  const int d = target->d, CH = a.CH;
  hipError_t e = timed(DT_K_MERGE, st, [&] { return launch_walk_init(a, st); });
  // the target's states, depth by depth, filed under the inner-node list
  for (int t = 0; t < D && e == hipSuccess; ++t) {
    e = timed(DT_K_MERGE, st, [&] { return launch_walk_rows(a, t, st); });
    for (int ch = 0; ch < a.nch && e == hipSuccess; ++ch) {
      StepWs wc = ww.step;
      if (a.bf16) {
        wc.x_hi = a.x_hi + (size_t)ch * CH * d;
        wc.x_lo = a.x_lo + (size_t)ch * CH * d;
      }
      DepthIo io;
      io.s_prev = t == 0 ? s0 : ww.S[(t - 1) & 1];
      io.tok = nullptr;
      io.src = a.row_src + (size_t)ch * CH;
      io.h = nullptr;
      io.h_req_stride = 0;
      io.rpr = 1;
      io.rows = CH;
      io.s_out = ww.S[t & 1] + (size_t)ch * CH * d;
      io.rows_out = CH;
      io.skip = a.skip + ch;
      io.prep = false;
      io.x_dense = a.bf16 ? nullptr : a.x_f32 + (size_t)ch * CH * d;
      e = run_update(target, wc, io, st);
    }
    if (e == hipSuccess)
      e = timed(DT_K_MERGE, st, [&] { return launch_walk_keep(a, ww.S[t & 1], st); });
  }
  // one pass of the target's head over every inner node
  if (e == hipSuccess) e = timed(DT_K_MERGE, st, [&] { return launch_walk_rows(a, D, st); });
  for (int ch = 0; ch < a.nch && e == hipSuccess; ++ch) {
    StepWs wc = ww.step;
    wc.key2 = ww.key2_all + (size_t)ch * CH * a.S;
    const float* s_rows = a.S_inner + (size_t)ch * CH * d;
    if (a.bf16) {
      // split the fp32 states into the packed hi/lo planes
      ReduceArgs r;
      r.skip = a.skip + ch;
      r.part = s_rows;
      r.splits = 1;
      r.Mp = CH;
      r.N = d;
      r.rows = CH;
      r.rows_out = 0;
      r.epi = EPI_RESID;
      r.out_hi = wc.s_hi;
      r.out_lo = wc.s_lo;
      e = timed(DT_K_REDUCE, st, [&] { return launch_reduce(r, st); });
    }
    if (e == hipSuccess)
      e = run_head(target, wc, s_rows, CH, 1, 0.f, nullptr, nullptr, nullptr, st, false,
                   a.skip + ch);
  }
  if (e == hipSuccess) e = timed(DT_K_MERGE, st, [&] { return launch_walk(a, st); });
  return e == hipSuccess ? DT_OK : DT_EHIP;
}

int prune_topB(const float* pool_score, const int32_t* pool_parent, const int32_t* n_valid, int R,
               int D, int W, int B, float beta, int32_t* sel_node, int32_t* sel_parent,
               int32_t* sel_depth, int32_t* n_sel, void* stream) {
  if (!pool_score || !pool_parent || !n_valid || !sel_node || !sel_parent || !sel_depth || !n_sel)
    return DT_EINVAL;
  if (R < 1 || D < 1 || W < 1 || B < 1 || (long)B > (long)D * W) return DT_EINVAL;
  if (!(beta <= 0.f) || !isfinite(beta)) return DT_EINVAL;
  if ((long)D * W > DT_MAX_POOL || B > DT_MAX_B || D > DT_MAX_DEPTH) return DT_EUNSUPPORTED;
  hipError_t e = launch_prune(pool_score, pool_parent, n_valid, R, D, W, B, beta, sel_node,
                              sel_parent, sel_depth, n_sel, (hipStream_t)stream);
  return e == hipSuccess ? DT_OK : DT_EHIP;
}

int build_tree_mask(const int32_t* sel_parent, const int32_t* n_sel, int R, int B,
                    uint32_t* mask, void* stream) {
  if (!sel_parent || !n_sel || !mask) return DT_EINVAL;
  if (R < 1 || B < 1) return DT_EINVAL;
  if (B > DT_MAX_B) return DT_EUNSUPPORTED;
  hipError_t e = launch_mask(sel_parent, n_sel, R, B, mask, (hipStream_t)stream);
  return e == hipSuccess ? DT_OK : DT_EHIP;
}

}  // extern "C"

// ---------------------------------------------------------------- allocation-free build
// Device scratch of build_supertree_noalloc: one copy per GPU, held from the
// first call on that GPU until the process ends.  In host code `scratch`
// names a host-side stand-in, never the device address: kernels and copies
// take the per-device pointer resolved below.
static __device__ __align__(256) unsigned char scratch[DT_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[SCRATCH_MAX_DEVICES] = {};

// The current device's copy of `scratch`, resolved once per device with that
// device current.  Returns DT_OK or DT_EHIP / DT_EUNSUPPORTED.
int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return DT_EHIP;
  if (dev >= SCRATCH_MAX_DEVICES) return DT_EUNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DT_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DT_OK;
}

}  // namespace

extern "C" {

int build_supertree_noalloc(const dt_head* head, const float* h, const float* s0,
                            const int32_t* root_tok, int R, int D, int W, int k, float T,
                            int32_t* pool_tok, int32_t* pool_parent, float* pool_score,
                            int32_t* n_valid, void* stream) {
  int rc = build_args_ok(head, R, D, W, k);
  if (rc != DT_OK) return rc;
  if (!h || !s0 || !root_tok || !pool_tok || !pool_parent || !pool_score || !n_valid)
    return DT_EINVAL;
  if (!(T >= 0.f) || !isfinite(T)) return DT_EINVAL;
  // checked before the scratch is touched, so an oversized call launches nothing
  const size_t need = build_supertree_workspace_size(head, R, D, W, k);
  if (need > DT_NOALLOC_SCRATCH_BYTES) return DT_EUNSUPPORTED;
  void* ws = nullptr;
  rc = scratch_for_current_device(&ws);
  if (rc != DT_OK) return rc;
  // every kernel of the build writes what a later one reads (padding rows
  // included), so nothing in the scratch has to start at zero
  return build_supertree_ex(head, h, s0, root_tok, R, D, W, k, T, nullptr, pool_tok, pool_parent,
                            pool_score, n_valid, ws, DT_NOALLOC_SCRATCH_BYTES, stream);
}

int dartree_timing_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.on.store(enable != 0);
  return DT_OK;
}

int dartree_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  collect_pending();
  for (int i = 0; i < DT_K_COUNT; ++i) {
    g_timing.total_ms[i] = 0.0;
    g_timing.count[i] = 0;
  }
  return DT_OK;
}

int dartree_timing_read(int cls, double* total_ms, int64_t* launches) {
  if (cls < 0 || cls >= DT_K_COUNT || !total_ms || !launches) return DT_EINVAL;
  std::lock_guard<std::mutex> lk(g_timing.mu);
  collect_pending();
  *total_ms = g_timing.total_ms[cls];
  *launches = g_timing.count[cls];
  return DT_OK;
}

}  // extern "C"
