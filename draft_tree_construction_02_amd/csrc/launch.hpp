// Host-side launchers of the library's kernels (internal interface).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace dt {

// Packed bf16 weights (pack_head): rows are grouped by PACK_ROWS (8 tiles of
// 16); block (g, kb, t) of tile t, K block kb of group g sits at element
// offset ((g * K/32 + kb) * 8 + t) * 512, so the 8 tiles of a 128-column
// workgroup are read as one contiguous 8 KB run per 32-K step.
constexpr int PACK_ROWS = 128;

// fp32 activation source (fp32 heads): row m, column k of A.
//   dense:  A[m][k] = a[m * lda + k]
//   gather: A[m][k] = E[tok[m]][k] + h[(m / rpr) * h_req_stride + k]
// Rows with m >= rows, or with tok[m] < 0 in gather mode, read as zero.
struct ASrc {
  const float* a = nullptr;
  int lda = 0;
  const void* E = nullptr;
  int ldE = 0;
  const int32_t* tok = nullptr;
  const float* h = nullptr;
  long h_req_stride = 0;
  int rpr = 1;
  int gather = 0;
  int rows = 0;
};

// bf16 activation A [Mp][K] as packed hi/lo planes (see write_packed8):
// 1 KB block (mt, kb) of 16 rows x 32 K at element offset (mt * K/32 + kb) * 512,
// lane l of the block holding row 16 mt + l % 16, K 32 kb + 8 (l / 16) .. + 8.
struct PackedA {
  const uint16_t* hi = nullptr;
  const uint16_t* lo = nullptr;
  int K = 0;
};

enum Epi { EPI_GELU = 0, EPI_RESID = 1 };

// Split-K partial products part[split][Mp][N] of Y = A Wt^T, Wt [N][K].
// skip (optional, device): when *skip != 0 the launch does nothing; used by
// the sequential construction, whose number of head calls is data-dependent.
struct GemmArgs {
  const int32_t* skip = nullptr;
  PackedA pa;                 // bf16 path, packed activation planes
  ASrc a;                     // fp32 path
  const void* Wt = nullptr;
  int w_bf16 = 1;
  int w_packed = 0;           // bf16 weights in the packed block layout
  int N = 0, K = 0;
  int Mp = 0;                 // padded rows (16, 32, 64 or 128)
  int splits = 1;
  int runs = 0;               // bf16, > 0: workgroup x of a split takes the 16-column tiles
                              // [x nt / runs, (x + 1) nt / runs) (nt = N / 16, <= 8 each)
  float* part = nullptr;
};

// Sum of the splits in order plus the epilogue:
//   EPI_GELU : y = GELU(sum)
//   EPI_RESID: y = (src_row[m] >= 0 ? s_prev[src_row[m]][n] : 0) + sum
// Writes out [rows_out][N] fp32 (if out) and the packed hi/lo planes
// [Mp][N] (if out_hi); rows >= rows are zero.
struct ReduceArgs {
  const int32_t* skip = nullptr;
  const float* part = nullptr;
  int splits = 1, Mp = 0, N = 0, rows = 0, rows_out = 0;
  int epi = EPI_GELU;
  const float* s_prev = nullptr;
  const int32_t* src_row = nullptr;
  float* out = nullptr;
  uint16_t* out_hi = nullptr;
  uint16_t* out_lo = nullptr;
};

int gemm_tile_n(int w_bf16);
int gemm_gather_max_rows();   // bf16: rows up to which x = E[tok] + h is formed in staging
int gemm_k_chunk(int w_bf16);
hipError_t launch_gemm(const GemmArgs& g, hipStream_t st);
hipError_t launch_reduce(const ReduceArgs& r, hipStream_t st);

// Corrected-logit head: per (row, vocabulary tile) the tile's max, sum of
// exp(y - max) and top-kmax keys of y = z * inv_T (z raw when greedy).
struct HeadArgs {
  const int32_t* skip = nullptr;
  PackedA pa;                 // bf16 path: s' hi/lo
  ASrc a;                     // fp32 path: dense s'
  const void* Ut = nullptr;
  int w_bf16 = 1;
  int w_packed = 0;
  int V = 0, d = 0;
  int Mp = 0;
  int kmax = 1;               // 1, 4, 8 or 16
  int k = 1;                  // keys kept per tile (<= kmax)
  float inv_T = 1.f;
  int greedy = 0;
  float2* ms_part = nullptr;  // [Mp][ntiles]
  uint64_t* key_part = nullptr;  // [Mp][ntiles][k]
  int bal = 0;                // set by launch_head: balanced column runs (see head_tiles)
};
int device_cu_count();                       // compute units of the current device
int head_tile_n(int w_bf16);                 // smallest slice width (sizes workspaces)
int head_tiles(const HeadArgs& h);           // vocabulary slices of this launch
hipError_t launch_head(const HeadArgs& h, hipStream_t st);
// 64/128-row packed bf16 variant (head_wide.hip); launch_head dispatches to it
bool head_wide_ok(const HeadArgs& h);
int head_wide_slices(const HeadArgs& h);
hipError_t launch_head_wide(const HeadArgs& h, hipStream_t st);
// 128-row packed bf16 variant (head_rows128.hip): one vocabulary slice per
// compute unit; launch_head prefers it over the 64/128-row one
bool head_rows128_ok(const HeadArgs& h);
int head_rows128_slices(const HeadArgs& h);
hipError_t launch_head_rows128(const HeadArgs& h, hipStream_t st);
// 128-row packed bf16 GEMM on the same K loop (split-K partials as launch_gemm)
bool gemm_rows128_ok(const GemmArgs& g);
hipError_t launch_gemm_rows128(const GemmArgs& g, hipStream_t st);

// Per-row merge of the head's tile partials (kt keys per tile): log-sum-exp
// and global top-k, written to cand_tok / cand_lp rows of stride k.  ms2 and
// key2 hold the first pass's range results ([rows][merge_splits(ntiles)] and
// [..][kmax]).
int merge_splits(int ntiles);
constexpr int MERGE_SPLITS_MAX = 16;
hipError_t launch_merge(const float2* ms_part, const uint64_t* key_part, int rows,
                        int ntiles, int kt, int k, int kmax, int greedy, float2* ms2,
                        uint64_t* key2, int32_t* cand_tok, float* cand_lp, float* lse,
                        hipStream_t st);
// First pass only (the beam step folds the range results itself).
hipError_t launch_merge_part(const float2* ms_part, const uint64_t* key_part, int rows,
                             int ntiles, int kt, int kmax, float2* ms2, uint64_t* key2,
                             hipStream_t st, const int32_t* skip = nullptr);

// x = E[tok[m]] + h[(m / rpr) * h_req_stride] written as packed hi/lo planes
// [Mp][d] (bf16 heads); rows m >= rows or with tok[m] < 0 are zero.
struct PrepArgs {
  const uint16_t* E = nullptr;
  int d = 0;
  const int32_t* tok = nullptr;
  const float* h = nullptr;
  long h_req_stride = 0;
  int rpr = 1;
  int rows = 0, Mp = 0;
  uint16_t* hi = nullptr;
  uint16_t* lo = nullptr;
};
hipError_t launch_prep_x(const PrepArgs& p, hipStream_t st);

// Packed block layout of a bf16 matrix W [N][K] (K % 32 == 0): rows padded to
// a multiple of 16 with zeros; block (nb, kb) at element (nb * K/32 + kb) * 512.
hipError_t launch_pack_weight(const uint16_t* src, uint16_t* dst, int N, int K, hipStream_t st);

// Beam bookkeeping for one depth of R requests.
struct BeamArgs {
  int R = 0, W = 0, k = 0, D = 0, t = 0, greedy = 0;
  // children per row: either the merge range results (ms2 / key2) folded
  // here, or (ms2 == nullptr) already chosen in cand_tok / cand_lp [Mp][k]
  const int32_t* cand_tok = nullptr;
  const float* cand_lp = nullptr;
  const float2* ms2 = nullptr;         // merge range results [Mp][S]
  const uint64_t* key2 = nullptr;      // [Mp][S][kmax]
  int S = 1, kmax = 1;
  const float* score_in = nullptr;     // [R*W]
  int32_t* n_valid = nullptr;          // [R][D]
  int32_t* pool_tok = nullptr;         // [R][D][W]
  int32_t* pool_parent = nullptr;
  float* pool_score = nullptr;
  int32_t* tok_out = nullptr;          // [Mp]
  float* score_out = nullptr;          // [Mp]
  int32_t* src_out = nullptr;          // [Mp]
  int Mp = 0;                          // rows of the next depth's launches (padded)
  // frontier rows per request of this depth (input rows r * rpr_in + i) and
  // of the next one (output rows r * rpr_out + j); 0 means W
  int rpr_in = 0, rpr_out = 0;
};
hipError_t launch_beam_init(int R, int W, int Mp, const int32_t* root_tok, int32_t* tok,
                            float* score, int32_t* src, hipStream_t st);
// Base-candidate variant: children of each row among its depth's candidates.
struct CandArgs {
  const float* s = nullptr;            // updated states [rows][d] f32
  const float* lse = nullptr;          // [rows] logsumexp(z / T)
  const int32_t* cand_base = nullptr;  // [R * D][n_cand]
  const void* Ut = nullptr;
  int u_bf16 = 1, u_packed = 0;
  int d = 0, W = 1, D = 1, t = 0, n_cand = 1, k = 1, greedy = 0;
  float inv_T = 1.f;
  int32_t* cand_tok = nullptr;         // [rows][k]
  float* cand_lp = nullptr;
};
hipError_t launch_cand_score(const CandArgs& a, int rows, hipStream_t st);
hipError_t launch_markov_src(int rows, int W, int Mp, int32_t* src, hipStream_t st);

// Children of every frontier row from the merge range results, then the
// global top-W step.
hipError_t launch_beam_step(const BeamArgs& b, hipStream_t st);
hipError_t launch_fill_rows(int rows, int Mp, const int32_t* tok_in, int32_t* tok,
                            int32_t* src, hipStream_t st);

// Sequential best-first construction (sequential.hip).  ctl holds the
// control words below; candidates are pushed in order, each expansion adding
// its top-keff children.
enum SeqCtl {
  SEQ_N_OUT = 0,      // nodes in the output tree
  SEQ_N_CAND = 1,     // candidates pushed so far
  SEQ_SKIP = 2,       // 1: the remaining call slots do nothing
  SEQ_CUR_OUT = 3,    // output index of the node being expanded (-1: root)
  SEQ_CUR_DEPTH = 4,  // its depth (0: root)
  SEQ_CUR_ROW = 5,    // state row of its parent's update (the residual source)
  SEQ_CUR_TOK = 6,    // its token
  SEQ_CALLS = 7,      // head calls made
  SEQ_CTL_WORDS = 8
};
constexpr int SEQ_MAX_CAND = 16384;   // DT_MAX_B * DT_MAX_K
struct SeqArgs {
  int D = 0, k = 0, B = 0, kmax = 1, S = 1, greedy = 0, Mp = 0, d = 0;
  float beta = 0.f;
  const float2* ms2 = nullptr;         // merge range results of row 0 [S]
  const uint64_t* key2 = nullptr;      // [S][kmax]
  int32_t* ctl = nullptr;              // [SEQ_CTL_WORDS]
  float* cur_score = nullptr;          // [1] score of the node being expanded
  int32_t* c_tok = nullptr;            // candidates [B * keff]
  int32_t* c_par = nullptr;
  int32_t* c_depth = nullptr;
  int32_t* c_row = nullptr;
  float* c_score = nullptr;
  uint32_t* c_alive = nullptr;         // bitmap
  float* state = nullptr;              // [B + 1][d] updated states; row B = s0
  int32_t* out_tok = nullptr;          // [B]
  int32_t* out_par = nullptr;
  int32_t* out_depth = nullptr;
  float* out_score = nullptr;
  int32_t* n_out = nullptr;
  const void* E = nullptr;             // embedding (bf16 or fp32, as the head)
  const float* h = nullptr;            // [D][d]
  uint16_t* x_hi = nullptr;            // bf16 heads: packed x planes [Mp][d]
  uint16_t* x_lo = nullptr;
  float* x_f32 = nullptr;              // fp32 heads: dense x [Mp][d]
};
hipError_t launch_seq_init(const SeqArgs& a, const float* s0, const int32_t* root_tok,
                           hipStream_t st);
hipError_t launch_seq_step(const SeqArgs& a, int slot, hipStream_t st);

// Acceptance walk (verify.hip).  Rows of one depth are the tree nodes of that
// depth that have children, compacted over all requests in (request, node)
// order and evaluated in chunks of CH rows; ctl[0] holds the row count of the
// current depth, ctl[1] the number of inner nodes listed so far (all depths,
// in depth order: inner_req / inner_node, their states in S_inner).
struct WalkArgs {
  int R = 0, D = 0, B = 0, V = 0, d = 0, CH = 0, nch = 0, S = 1, bf16 = 1;
  const int32_t* root_tok = nullptr;   // [R]
  const int32_t* tok = nullptr;        // node tokens, see node_token
  int tok_stride = 0;
  const int32_t* tok_index = nullptr;  // [R][B] or null
  const int32_t* parent = nullptr;     // [R][B]
  const int32_t* depth = nullptr;      // [R][B]
  const int32_t* n = nullptr;          // [R]
  const void* E = nullptr;             // target embedding (bf16 or fp32)
  const float* h = nullptr;            // [R][D][d]
  int32_t* target_tok = nullptr;       // [R][B + 1]
  int32_t* path = nullptr;             // [R][D]
  int32_t* accept_len = nullptr;       // [R]
  uint8_t* has_child = nullptr;        // [R][B + 1], slot 0 = root
  int32_t* pos = nullptr;              // [R][B + 1] row of the node at its depth
  int32_t* row_req = nullptr;          // [nch * CH]
  int32_t* row_tok = nullptr;
  int32_t* row_src = nullptr;          // residual row (previous depth's rows; s0 row at depth 0)
  int32_t* ctl = nullptr;              // [2] rows of the current depth, inner nodes so far
  int32_t* skip = nullptr;             // [nch] chunk flags
  int32_t* row_gidx = nullptr;         // [nch * CH] inner-node index of each row
  int32_t* inner_req = nullptr;        // [nch * CH]
  int32_t* inner_node = nullptr;       // [nch * CH] node index, -1 = root
  float* S_inner = nullptr;            // [nch * CH][d] target states of the inner nodes
  const uint64_t* key2 = nullptr;      // merge range results [nch][CH][S] (greedy keys)
  uint16_t* x_hi = nullptr;            // bf16: packed x planes [nch][CH][d]
  uint16_t* x_lo = nullptr;
  float* x_f32 = nullptr;              // fp32: dense x [nch * CH][d]
};
hipError_t launch_walk_init(const WalkArgs& a, hipStream_t st);
// t < D: compact the rows of depth t, list them as inner nodes and write their
// x.  t == D: chunk flags of the inner-node list and zero padding rows.
hipError_t launch_walk_rows(const WalkArgs& a, int t, hipStream_t st);
// Copy the updated states of the current depth's rows (s_cur, [rows][d]) to
// their inner-node rows.
hipError_t launch_walk_keep(const WalkArgs& a, const float* s_cur, hipStream_t st);
// Target token of every inner node from the head's greedy keys, then the walk.
hipError_t launch_walk(const WalkArgs& a, hipStream_t st);

// One-launch build of a small fp32 head (build_small.hip): one workgroup of
// 1024 threads per request runs all D depths with the frontier in LDS.
constexpr size_t SMALL_BUILD_LDS_MAX = 61440;   // dynamic LDS; static arrays add 1.5 KB
struct SmallBuildArgs {
  const void* E = nullptr;             // fp32 row-major head
  const void* W1t = nullptr;
  const void* W2t = nullptr;
  const void* Ut = nullptr;
  int d = 0, V = 0;
  const float* h = nullptr;            // [R][D][d]
  const float* s0 = nullptr;           // [R][d]
  const int32_t* root_tok = nullptr;   // [R]
  int R = 0, D = 0, W = 0, k = 0, kmax = 1, greedy = 0;
  float inv_T = 1.f;
  int32_t* pool_tok = nullptr;         // [R][D][W]
  int32_t* pool_parent = nullptr;
  float* pool_score = nullptr;
  int32_t* n_valid = nullptr;          // [R][D]
};
bool small_build_ok(const SmallBuildArgs& a);
hipError_t launch_build_small(const SmallBuildArgs& a, hipStream_t st);

// Runs fn(ctx) bracketed by timing events of kernel class cls when kernel
// timing is on (dartree_timing_enable).
hipError_t timed_launch(int cls, hipStream_t st, hipError_t (*fn)(void*), void* ctx);

hipError_t launch_prune(const float* pool_score, const int32_t* pool_parent,
                        const int32_t* n_valid, int R, int D, int W, int B, float beta,
                        int32_t* sel_node, int32_t* sel_parent, int32_t* sel_depth,
                        int32_t* n_sel, hipStream_t st);
hipError_t launch_mask(const int32_t* sel_parent, const int32_t* n_sel, int R, int B,
                       uint32_t* mask, hipStream_t st);

}  // namespace dt
