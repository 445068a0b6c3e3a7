// Host-side launchers of the library's kernels (internal interface).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dt {

// Activation source of a skinny GEMM: row m, column k of the fp32 matrix A.
//   dense:  A[m][k] = a[m * lda + k]
//   gather: A[m][k] = E[tok[m]][k] + h[(m / rpr) * h_req_stride + k]
// Rows with m >= rows, or with tok[m] < 0 in gather mode, read as zero.
struct ASrc {
  const float* a = nullptr;
  int lda = 0;
  const void* E = nullptr;
  int ldE = 0;
  int e_bf16 = 0;
  const int32_t* tok = nullptr;
  const float* h = nullptr;
  long h_req_stride = 0;
  int rpr = 1;
  int gather = 0;
  int rows = 0;
};

enum Epi { EPI_GELU = 0, EPI_RESID = 1 };

// Split-K skinny GEMM Y = A Wt^T (Wt [N][K]) with a fused epilogue run by the
// last split to finish each column tile, summing the splits in order:
//   EPI_GELU : out[m][n] = GELU(Y[m][n])
//   EPI_RESID: out[m][n] = (src_row[m] >= 0 ? s_prev[src_row[m]][n] : 0) + Y[m][n]
struct GemmArgs {
  ASrc a;
  const void* Wt = nullptr;
  int w_bf16 = 1;
  int N = 0, K = 0;
  int Mp = 0;                 // padded rows (16, 32, 64, 128 or 256)
  int splits = 1;
  float* part = nullptr;      // [splits][Mp][N]
  uint32_t* counters = nullptr;  // [ceil(N / TN)] zero on entry, zero on exit
  int epi = EPI_GELU;
  float* out = nullptr;       // [Mp][N]
  const float* s_prev = nullptr;
  const int32_t* src_row = nullptr;
};

// Column-tile width and K-chunk of a GEMM configuration.
int gemm_tile_n(int w_bf16);
int gemm_k_chunk(int w_bf16, int Mp);
hipError_t launch_gemm(const GemmArgs& g, hipStream_t st);

// Corrected-logit head: per (row, vocabulary tile) the tile's max, sum of
// exp(y - max) and top-kmax keys of y = z * inv_T (z raw when greedy).
struct HeadArgs {
  ASrc a;                     // dense s'
  const void* Ut = nullptr;
  int w_bf16 = 1;
  int V = 0, d = 0;
  int Mp = 0;
  int kmax = 1;               // 1, 4, 8 or 16
  int k = 1;                  // keys kept per tile (<= kmax)
  float inv_T = 1.f;
  int greedy = 0;
  float2* ms_part = nullptr;  // [Mp][ntiles]
  uint64_t* key_part = nullptr;  // [Mp][ntiles][k]
};
int head_tile_n(int w_bf16);
hipError_t launch_head(const HeadArgs& h, hipStream_t st);

// Per-row merge of the head's tile partials (kt keys per tile): log-sum-exp
// and global top-k, written to cand_tok / cand_lp rows of stride k.
hipError_t launch_merge(const float2* ms_part, const uint64_t* key_part, int rows,
                        int ntiles, int kt, int k, int kmax, int greedy, int32_t* cand_tok,
                        float* cand_lp, float* lse, hipStream_t st);

// Beam bookkeeping for one depth of R requests.
struct BeamArgs {
  int R = 0, W = 0, k = 0, D = 0, t = 0, greedy = 0;
  const int32_t* cand_tok = nullptr;   // [R*W][k]
  const float* cand_lp = nullptr;      // [R*W][k]
  const float* score_in = nullptr;     // [R*W]
  int32_t* n_valid = nullptr;          // [R][D]
  int32_t* pool_tok = nullptr;         // [R][D][W]
  int32_t* pool_parent = nullptr;
  float* pool_score = nullptr;
  int32_t* tok_out = nullptr;          // [Mp]
  float* score_out = nullptr;          // [Mp]
  int32_t* src_out = nullptr;          // [Mp]
  int Mp = 0;
};
hipError_t launch_beam_init(int R, int W, int Mp, const int32_t* root_tok, int32_t* tok,
                            float* score, int32_t* src, uint32_t* counters, int n_counters,
                            hipStream_t st);
hipError_t launch_beam_select(const BeamArgs& b, hipStream_t st);
hipError_t launch_fill_rows(int rows, int Mp, const int32_t* tok_in, int32_t* tok,
                            int32_t* src, uint32_t* counters, int n_counters, hipStream_t st);

hipError_t launch_prune(const float* pool_score, const int32_t* pool_parent,
                        const int32_t* n_valid, int R, int D, int W, int B, float beta,
                        int32_t* sel_node, int32_t* sel_parent, int32_t* sel_depth,
                        int32_t* n_sel, hipStream_t st);
hipError_t launch_mask(const int32_t* sel_parent, const int32_t* n_sel, int R, int B,
                       uint32_t* mask, hipStream_t st);

}  // namespace dt
