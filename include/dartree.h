/*
 * dartree.h - C ABI of the MI355X (gfx950) library for DARTree's depth-wise
 * batched draft-supertree construction, deferred top-B pruning, the ancestor
 * attention mask and one tree-attention verification layer.
 *
 * Method sources (page title, section):
 *  [P1] "DARTree: Teaching a Chain-Trained Corrector to Think in Trees"
 *       (alanhou.org), Core Mechanism and its diagram.
 *  [P2] "Technische Samenvatting: DARTree" (gist.science), Methodologie,
 *       part 1 "Depth-Wise Parallel AR Expansie" and part 2 "Deferred
 *       Best-First Pruning" (Lemma 1).
 *  [P3] "Accelerating Language Models with Diffusion Draft Trees"
 *       (legiblepapers), Summary & Methodology Analysis.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or retains them.  Scratch space comes from a
 *    caller-provided device workspace sized by the matching *_workspace_size.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *    is enqueued on it and the call returns; outputs are valid once the
 *    caller has synchronised the stream.  Nothing synchronises the host.
 *  - Arguments are validated on the host before anything is launched.  On an
 *    error the call returns a negative dt_status, launches nothing and writes
 *    no output.  Launch failures reported by HIP return DT_EHIP.
 *  - Results are bitwise reproducible for identical inputs on a device with
 *    the same number of compute units: reductions run in a fixed order and no
 *    floating-point atomics are used, but the launch grids (vocabulary
 *    slices, split-K counts) are sized from the compute-unit count, so the
 *    fp32 summation order, and with it the last bits of a score, can differ
 *    between devices with different counts.
 *  - Calls that share one workspace must not overlap in time.
 *  - Global state: the library keeps only (a) a per-device cache of the
 *    compute-unit count (atomic, filled on first use), (b) the kernel timing
 *    registry of dartree_timing_* (mutex-protected; off by default) and (c)
 *    the per-device address of build_supertree_noalloc's static scratch
 *    (mutex-protected, resolved on first use).  Everything else lives in the
 *    caller's buffers.
 *  - Row-major layouts throughout; "[A][B]" means B is the fastest index.
 */
#ifndef DARTREE_H
#define DARTREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DT_OK = 0,
  DT_EINVAL = -1,       /* a null pointer, a size or a hyper-parameter out of range */
  DT_EWORKSPACE = -2,   /* workspace null or smaller than *_workspace_size        */
  DT_EUNSUPPORTED = -3, /* valid by the method but outside this build's limits    */
  DT_EHIP = -4          /* the HIP runtime reported an error                      */
} dt_status;

typedef enum { DT_F32 = 0, DT_BF16 = 1 } dt_dtype;

/* Storage layout of the streamed head weights W1t, W2t and Ut. */
typedef enum {
  DT_LAYOUT_ROWMAJOR = 0, /* [N][K] row-major as documented for dt_head          */
  DT_LAYOUT_PACKED = 1    /* bf16 only: written by pack_head (see there)          */
} dt_layout;

/* Limits of this build (checked on the host). */
#define DT_MAX_K 16         /* children per branch                              */
#define DT_MAX_ROWS 128     /* R * W: branch rows evaluated per head call        */
#define DT_MAX_CAND 4096    /* W * k candidates per request and depth           */
#define DT_MAX_POOL 4096    /* D * W pool nodes per request                      */
#define DT_MAX_B 1024       /* verification budget per request                   */
#define DT_MAX_DEPTH 64

/*
 * The correction head (read-only, device memory).  The pages fix no head
 * architecture; this is the synthetic head of the evaluated workloads:
 *     x  = E[tok] + h_t
 *     s' = s + GELU(x W1) W2          (exact erf GELU)
 *     z  = s' U                       (corrected logits)
 * Storage is output-feature-major so that each weight row is contiguous:
 *     E   [V][d]      token embedding
 *     W1t [4d][d]     W1 transposed
 *     W2t [d][4d]     W2 transposed
 *     Ut  [V][d]      U transposed (vocab-major: a vocabulary tile is one
 *                     contiguous block)
 * wdtype DT_BF16: all four are bfloat16; DT_F32: all four are float32.
 * d must be a multiple of 128 for DT_BF16 and of 32 for DT_F32.
 * layout DT_LAYOUT_PACKED (bf16 only) means W1t, W2t and Ut were produced by
 * pack_head; E is always row-major (rows are gathered by token).
 */
typedef struct {
  int32_t d;
  int32_t V;
  int32_t wdtype;      /* dt_dtype  */
  int32_t layout;      /* dt_layout */
  const void* E;
  const void* W1t;
  const void* W2t;
  const void* Ut;
} dt_head;

/* Human-readable text of a status code (static storage). */
const char* dartree_status_string(int status);

/* Library version, (major << 16) | minor. */
int dartree_version(void);

/* ------------------------------------------------------------------------ */
/* Weight packing (once per model load)                                      */
/* ------------------------------------------------------------------------ */

/* Device bytes pack_head writes for a row-major bf16 head (0 if invalid). */
size_t pack_head_bytes(const dt_head* head);

/*
 * pack_head - copy the streamed bf16 weights W1t [4d][d], W2t [d][4d] and
 * Ut [V][d] into `dst` (device, pack_head_bytes bytes, caller-owned) in the
 * packed block layout, and fill `*packed` (host struct) with a head that
 * points there (E still points to the caller's row-major E).
 * Packed layout of a matrix [N][K]: rows padded with zeros to a multiple of
 * 128 and split into groups g of 128 rows, each of 8 tiles t of 16 rows;
 * 1 KB blocks of 16 rows x 32 columns, block (g, kb, t) at element offset
 * ((g * K/32 + kb) * 8 + t) * 512; inside a block, the 8 bf16 at offset 8 l
 * hold row 128 g + 16 t + (l mod 16), columns 32 kb + 8 (l / 16) .. + 7
 * (l = 0..63).  This is the operand order of the gfx950 bf16 MFMA, so one
 * wave load instruction streams one contiguous block, and the 8 tiles of a
 * row group advance through K as one contiguous run.  Asynchronous on `stream`; `dst` must stay
 * alive while the packed head is used.
 */
int pack_head(const dt_head* src, void* dst, size_t dst_bytes, dt_head* packed, void* stream);

/* ------------------------------------------------------------------------ */
/* Supertree construction                                                    */
/* ------------------------------------------------------------------------ */

/* Bytes of device workspace build_supertree needs (0 on invalid arguments). */
size_t build_supertree_workspace_size(const dt_head* head, int R, int D, int W, int k);

/*
 * build_supertree - depth-wise batched construction of R independent
 * supertrees that share one correction head ([P1] Core Mechanism; [P2]
 * part 1; [P3]).
 *
 * For t = 1..D, one batched head call runs over every surviving branch of
 * every request: the state update, the corrected logits z = s'U, the
 * temperature log-softmax logp = z/T - logsumexp(z/T) and each branch's top-k
 * children by (logp desc, token asc).  A child's score is its parent's score
 * plus its logp (accumulated path log-probability).  Per request the best
 * n_t = min(W, n_{t-1} * k) candidates by (score desc, parent slot asc, child
 * rank asc) survive and carry their parent's updated state forward; the
 * child's token enters the next depth's update.  The root (depth 0) is one
 * branch with state s0, token root_tok and score 0; so n_0 = 1.
 * T == 0 is the greedy limit: only the lowest-index argmax of z survives as a
 * child, with logp 0, so each request's supertree is a chain.
 *
 * Inputs:
 *   h         [R][D][d] f32   drafter hidden state for each depth (h[r][t-1]
 *                             feeds the step producing depth-t tokens)
 *   s0        [R][d]    f32   root branch state
 *   root_tok  [R]       i32   last verified token, 0 <= root_tok < V
 *   1 <= R, 1 <= D <= DT_MAX_DEPTH, 1 <= W, 1 <= k <= min(V, DT_MAX_K),
 *   R*W <= DT_MAX_ROWS, W*k <= DT_MAX_CAND, D*W <= DT_MAX_POOL, T >= 0 finite.
 * Outputs (slot j of depth t at index [r][t-1][j]):
 *   pool_tok    [R][D][W] i32  token, -1 for unused slots
 *   pool_parent [R][D][W] i32  parent slot at depth t-1; -1 at depth 1 and
 *                              for unused slots
 *   pool_score  [R][D][W] f32  accumulated log-probability; -inf if unused
 *   n_valid     [R][D]    i32  used slots per depth
 * Slots are in (score desc, parent slot asc, rank asc) order.
 * Inputs must be finite.
 * A small fp32 head (row-major, W <= 64, and the states, x, H and logits of
 * W rows within 60 KB: 4 (7 W d + W V) + 12 W kmax bytes) is built by one
 * launch with one workgroup per request; the workspace is then unused.
 */
int build_supertree(const dt_head* head, const float* h, const float* s0,
                    const int32_t* root_tok, int R, int D, int W, int k, float T,
                    int32_t* pool_tok, int32_t* pool_parent, float* pool_score,
                    int32_t* n_valid, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * build_supertree_noalloc - build_supertree for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same kernels and the same results, bit for bit,
 * with the scratch memory taken from a static device array of
 * DT_NOALLOC_SCRATCH_BYTES inside the library instead of a caller workspace.
 * Each GPU the library runs on holds its own copy of that array from the
 * first call on it until the process ends; the call itself allocates and
 * frees nothing.  The caller still passes every input and output; arguments,
 * outputs and errors are those of build_supertree, plus DT_EUNSUPPORTED when
 * build_supertree_workspace_size for these arguments exceeds
 * DT_NOALLOC_SCRATCH_BYTES (checked on the host; nothing is launched).
 * The current device must be the one `stream` belongs to.  All calls on one
 * GPU share its array: calls that overlap in time on one GPU (two streams, two
 * threads) race and give undefined results.  The array keeps the last call's
 * contents; no part of it needs to start at zero.
 */
#define DT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

int build_supertree_noalloc(const dt_head* head, const float* h, const float* s0,
                            const int32_t* root_tok, int R, int D, int W, int k, float T,
                            int32_t* pool_tok, int32_t* pool_parent, float* pool_score,
                            int32_t* n_valid, void* stream);

/* Build variants (dt_build_opts.flags). */
#define DT_BUILD_MARKOV 1           /* no carried state: every update starts from s0    */
#define DT_BUILD_BASE_CANDIDATES 2  /* children only among the depth's base candidates   */
#define DT_BUILD_MULTI_KERNEL 4     /* same result; small fp32 heads run the per-depth   */
                                    /* kernels instead of the one-launch build           */

typedef struct {
  int32_t flags;    /* DT_BUILD_* bits                                                   */
  int32_t n_cand;   /* DT_BUILD_BASE_CANDIDATES: candidates per depth, k <= n_cand <= DT_MAX_K */
} dt_build_opts;

/* Device bytes of workspace build_supertree_ex needs (0 if invalid). */
size_t build_supertree_ex_workspace_size(const dt_head* head, int R, int D, int W, int k,
                                         const dt_build_opts* opts);

/*
 * build_supertree_ex - build_supertree with the variants the pages discuss
 * (opts == NULL or flags == 0: exactly build_supertree).
 *  - DT_BUILD_MARKOV: a Markov correction head that carries no state along
 *    the branch (the DSpark drafter of [P2] Experimentele Resultaten,
 *    Generaliseerbaarheid): every row's update
 *    is s' = s0[r] + GELU((E[tok] + h_t) W1) W2, so a node's children depend
 *    on its token and depth only.
 *  - DT_BUILD_BASE_CANDIDATES: at each depth the n_cand candidate tokens are
 *    the top of the drafter's base logits, read here as h_t U (by logit desc,
 *    token asc), shared by the request's branches ([P2] part 1, Kandidaat
 *    Selectie); each branch's children are its k best candidates by the
 *    corrected log-probability (full-vocabulary normaliser), token asc on
 *    ties.  T == 0: the single child is the lowest-index argmax of z over the
 *    candidates, logp 0.  The candidates of all D depths come from one extra
 *    head pass over the R*D hidden rows before the depth loop.
 * Arguments and outputs as build_supertree; opts is a host pointer.
 */
int build_supertree_ex(const dt_head* head, const float* h, const float* s0,
                       const int32_t* root_tok, int R, int D, int W, int k, float T,
                       const dt_build_opts* opts, int32_t* pool_tok, int32_t* pool_parent,
                       float* pool_score, int32_t* n_valid, void* workspace,
                       size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Stages of one depth (the same kernels build_supertree runs)               */
/* ------------------------------------------------------------------------ */

/* Bytes of workspace for the two stage calls below with `rows` rows. */
size_t head_step_workspace_size(const dt_head* head, int rows, int k);

/*
 * state_update - the head's state step for `rows` branches:
 *   s_out[i] = s_in[i] + GELU((E[tok[i]] + h) W1) W2.
 *   s_in, s_out [rows][d] f32 (may not alias); tok [rows] i32; h [d] f32.
 * 1 <= rows <= DT_MAX_ROWS.
 */
int state_update(const dt_head* head, const float* s_in, const int32_t* tok,
                 const float* h, int rows, float* s_out, void* workspace,
                 size_t workspace_bytes, void* stream);

/*
 * corrected_topk - corrected logits z = s U for `rows` states, the temperature
 * log-softmax over the whole vocabulary and each row's top-k children
 * ([P1] Core Mechanism: W corrected conditional distributions, top-k each).
 *   s        [rows][d] f32
 *   cand_tok [rows][k] i32   tokens by (logp desc, token asc)
 *   cand_lp  [rows][k] f32   their log-probabilities (T > 0)
 *   lse      [rows]    f32   logsumexp(z/T) (T > 0); max z when T == 0
 * With T == 0 only column 0 is meaningful (the lowest-index argmax, lp 0);
 * the other columns hold token -1 and lp -inf.
 */
int corrected_topk(const dt_head* head, const float* s, int rows, int k, float T,
                   int32_t* cand_tok, float* cand_lp, float* lse, void* workspace,
                   size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Sequential best-first construction (the per-node baseline)               */
/* ------------------------------------------------------------------------ */

/* Device bytes of workspace build_tree_sequential needs (0 if invalid). */
size_t build_tree_sequential_workspace_size(const dt_head* head, int D, int k, int B);

/*
 * build_tree_sequential - the costly alternative to depth-wise batching that
 * the pages measure against ([P1] Core Mechanism; [P2] Experimentele
 * Resultaten, ablation of sequential heap-interleaved correction): best-first
 * growth with a max-heap and ONE HEAD CALL PER EXPANDED NODE, for one
 * request.  The root is expanded first (h row 0); then the best candidate by
 * (score + beta * depth desc, depth asc, push order asc) is popped and
 * appended to the tree, and, unless the tree holds B nodes or the node is at
 * depth D, expanded at once: the head's state step on its parent's updated
 * state with its token and h row `depth`, its top-k children (temperature T,
 * T == 0 the argmax) pushed with score = node score + logp.  Repeats until B
 * nodes or no candidate is left.  Head calls = 1 + expanded popped nodes.
 *   h [D][d] f32, s0 [d] f32, root_tok [1] i32 (device)
 * Outputs, in pop order (entries >= *n_out are -1 / -inf):
 *   tok    [B] i32   node token
 *   parent [B] i32   index of the parent entry (earlier), -1 at depth 1
 *   depth  [B] i32   1..D
 *   score  [B] f32   accumulated log-probability (0 when T == 0)
 *   n_out  [1] i32   nodes in the tree
 * 1 <= k <= min(V, DT_MAX_K), 1 <= B <= DT_MAX_B, 1 <= D <= DT_MAX_DEPTH,
 * beta <= 0 finite, T >= 0 finite.  Everything runs on `stream`: B call
 * slots are enqueued and the ones after the last expansion do nothing.
 */
int build_tree_sequential(const dt_head* head, const float* h, const float* s0,
                          const int32_t* root_tok, int D, int k, int B, float beta, float T,
                          int32_t* tok, int32_t* parent, int32_t* depth, float* score,
                          int32_t* n_out, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ------------------------------------------------------------------------ */
/* Deferred best-first pruning and the verification mask                    */
/* ------------------------------------------------------------------------ */

/*
 * prune_topB - deferred best-first pruning as one global top-B per request
 * ([P2] part 2, Globale Selectie and Lemma 1; [P3]).
 *   prio = pool_score + beta * depth (depth 1..D).  The min(B, sum n_valid)
 *   best valid pool nodes by (prio desc, depth asc, slot asc) are selected and
 *   emitted in (depth asc, slot asc) order.  For beta <= 0 this set is the
 *   set a sequential best-first max-heap pops (Lemma 1) and it is
 *   ancestor-closed, so every emitted parent is emitted earlier.
 * Inputs: the build_supertree outputs for R requests of D x W slots.
 *   1 <= B <= min(D*W, DT_MAX_B); beta <= 0 finite (beta > 0 -> DT_EINVAL).
 * Outputs (row r, entry i < n_sel[r]; entries >= n_sel[r] are -1):
 *   sel_node   [R][B] i32  flat pool index (t-1)*W + slot
 *   sel_parent [R][B] i32  index of the parent entry, -1 for depth-1 nodes
 *   sel_depth  [R][B] i32  depth 1..D
 *   n_sel      [R]    i32  min(B, number of valid pool nodes)
 */
int prune_topB(const float* pool_score, const int32_t* pool_parent,
               const int32_t* n_valid, int R, int D, int W, int B, float beta,
               int32_t* sel_node, int32_t* sel_parent, int32_t* sel_depth,
               int32_t* n_sel, void* stream);

/*
 * build_tree_mask - ancestor bitmask of each verification tree ([P1] Core
 * Mechanism: the sparse attention mask lets the target check every branch in
 * one forward; [P3]: tree-attention mask of the prefix tree).
 *   mask [R][B][ceil(B/32)] u32: bit (i mod 32) of word (i / 32) of row j is
 *   set iff entry i is entry j or an ancestor of it.  Rows >= n_sel are zero.
 *   The verified prefix is visible to every node and is not in the mask.
 *   sel_parent as written by prune_topB (parents precede children).
 */
int build_tree_mask(const int32_t* sel_parent, const int32_t* n_sel, int R, int B,
                    uint32_t* mask, void* stream);

/* ------------------------------------------------------------------------ */
/* Verification: one tree-attention layer                                    */
/* ------------------------------------------------------------------------ */

size_t tree_attention_workspace_size(int n_tree, int P, int Hq, int Hkv, int hd);

/*
 * tree_attention_verify - one attention layer of the target's single
 * verification forward over the tree ([P1] Core Mechanism, last step; [P2]
 * part 2, Verificatie; [P3]).  Query i (a tree node) of head h attends to all
 * P prefix keys and to the tree keys its mask row marks; key/value head
 * h / (Hq / Hkv) (grouped-query attention).  Softmax in fp32.
 *   q        [n_tree][Hq][hd]  bf16
 *   k_prefix, v_prefix [P][Hkv][hd] bf16
 *   k_tree,   v_tree   [n_tree][Hkv][hd] bf16
 *   mask     [n_tree][ceil(n_tree/32)] u32 (build_tree_mask row layout)
 *   out      [n_tree][Hq][hd]  f32
 *   hd == 128, Hq % Hkv == 0, 1 <= n_tree <= 1024, P >= 0.
 */
int tree_attention_verify(const void* q, const void* k_prefix, const void* v_prefix,
                          const void* k_tree, const void* v_tree, const uint32_t* mask,
                          int n_tree, int P, int Hq, int Hkv, int hd, float scale,
                          float* out, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ------------------------------------------------------------------------ */
/* Acceptance walk against a synthetic greedy target                         */
/* ------------------------------------------------------------------------ */

#define DT_MAX_WALK_NODES 8192   /* R * B: draft nodes per accept_walk call */

/* Device bytes of workspace accept_walk needs (0 if the arguments are invalid). */
size_t accept_walk_workspace_size(const dt_head* target, int R, int D, int B);

/*
 * accept_walk - verification of R draft trees by a synthetic greedy target
 * ([P1] Core Mechanism: one target forward checks every branch and the
 * longest agreeing prefix is kept; [P1] Key Concepts: accepted tokens per
 * verification round; [P1] Expert Assessment: compare trees of matched size).
 * The pages' target is a language model; here it is a chain model of the
 * correction head's form with its own weights (`target`, any dt_head).  Its
 * state after node v follows v's path: s'(root) = s0 + step(root_tok, h row 0),
 * s'(v) = s'(parent v) + step(tok v, h row depth(v)), with
 * step(t, x) = GELU((E[t] + x) W1) W2, and its token after v is the
 * lowest-index argmax of s'(v) U.  It is evaluated depth by depth, once for
 * every node that has children, in batches of up to 128 rows (the same
 * state-update and head kernels as the builds, T == 0).
 * The walk starts at the root and moves to the child (lowest index first)
 * whose token is the target's token after the current node, until no child
 * matches; tokens per round = accept_len + 1.
 * Tree of request r (device arrays, row stride B): n[r] nodes (clamped to
 * [0, B]); node i has parent parent[r][i] (-1: child of the root) with
 * parent < i, depth depth[r][i] = depth of the parent + 1 (1..D), token
 *   tok[r * tok_stride + i]                       when tok_index == NULL,
 *   tok[r * tok_stride + tok_index[r * B + i]]    otherwise
 * (so prune_topB's sel_node indexes build_supertree's pool_tok directly,
 * tok_stride = D * W; the sequential tree is tok_stride = B, no index).
 * Nodes that break these rules, have a token outside [0, V) or an index
 * outside [0, tok_stride) get no target token and are never accepted.
 *   h [R][D][d] f32, s0 [R][d] f32, root_tok [R] i32.
 * Outputs:
 *   target_tok [R][B + 1] i32  target's token after the root (column 0) and
 *                              after node i (column 1 + i); -1 where the node
 *                              has no children
 *   path       [R][D] i32      accepted nodes in depth order, then -1
 *   accept_len [R] i32         accepted draft nodes
 * 1 <= R, 1 <= B <= DT_MAX_B, R * B <= DT_MAX_WALK_NODES,
 * 1 <= D <= DT_MAX_DEPTH; everything runs on `stream`.
 */
int accept_walk(const dt_head* target, const float* h, const float* s0,
                const int32_t* root_tok, int R, int D, int B, const int32_t* tok,
                int tok_stride, const int32_t* tok_index, const int32_t* parent,
                const int32_t* depth, const int32_t* n, int32_t* target_tok,
                int32_t* path, int32_t* accept_len, void* workspace,
                size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Read-bandwidth probe                                                      */
/* ------------------------------------------------------------------------ */

/*
 * hbm_read_probe - reads every byte of a device buffer once (a plain
 * streaming read by a grid of resident workgroups) and writes the sum of its
 * little-endian 64-bit words modulo 2^64 to *sum (device memory).  Timed over
 * a buffer of a few GB it gives the practical device-memory read bandwidth
 * against which the head's weight stream (2 d V bytes per depth, [P3]
 * Summary & Methodology Analysis: drafting is memory-bandwidth bound) is
 * reported; the sum makes the read checkable and keeps it from being elided.
 *   buf   device pointer, 16-byte aligned (may be NULL when bytes == 0)
 *   bytes multiple of 8; 0 gives *sum = 0
 *   sum   device uint64_t[1], written on `stream`
 * Two launches (clear, read); no workspace.
 */
int hbm_read_probe(const void* buf, size_t bytes, uint64_t* sum, void* stream);

/*
 * mfma_rate_probe - runs bf16 32x32x16 matrix-core products with operands held
 * in registers, the bound of the corrected-logit head when its rows are many
 * (its hi/lo products are 2 * 2 * rows * d * V flop per depth; at 128 rows
 * they, not the weight stream of [P3] Summary & Methodology Analysis, set its
 * time, and the product rate depends on the operand data).  One workgroup of
 * 8 waves per compute unit (cus = the device's compute units); wave w of
 * workgroup g holds 8 fragments of 1 KB from operands + (8 g + w) * 8 KB
 * (4 weight-like, 4 activation-like bf16 tiles) and runs `iters` rounds of
 * 16 products into 4 accumulators, then writes each thread's sum of its
 * accumulators to out[512 g + thread].  With every operand 1.0 each output is
 * exactly 4096 * iters.
 *   operands  device bf16 buffer, 16-byte aligned, >= cus * 64 KB
 *   bytes     its size in bytes
 *   iters     rounds, >= 0 (cus * 8 * iters * 16 * 32768 flop per call)
 *   out       device float[out_count], out_count >= cus * 512
 * One launch on `stream`; DT_EINVAL on a NULL, misaligned or short buffer.
 */
int mfma_rate_probe(const void* operands, size_t bytes, int iters, float* out, size_t out_count,
                    void* stream);

/* ------------------------------------------------------------------------ */
/* Kernel timing (off by default)                                            */
/* ------------------------------------------------------------------------ */

/* Kernel classes that can be timed. */
typedef enum {
  DT_K_GEMM1 = 0,   /* state update, first projection (split-K partials)  */
  DT_K_GEMM2 = 1,   /* state update, second projection (split-K partials) */
  DT_K_HEAD = 2,    /* corrected-logit head + per-tile softmax/top-k (the */
                    /* 16- to 64-row and fp32 kernels)                    */
  DT_K_MERGE = 3,   /* per-row merge and per-request beam select          */
  DT_K_REDUCE = 4,  /* split-K reductions (GELU / residual epilogues)     */
  DT_K_ATTN = 5,    /* tree-attention verification layer (both kernels)   */
  DT_K_BUILD_SMALL = 6, /* one-launch build of a small fp32 head (all depths) */
  DT_K_HEAD128 = 7, /* corrected-logit head launches of the 128-row kernel */
  DT_K_COUNT = 8
} dt_kernel_class;

/*
 * dartree_timing_enable - when enabled, every launch of a kernel class is
 * bracketed by HIP events recorded on the launch's stream; after the caller
 * synchronises, dartree_timing_read returns the summed milliseconds and the
 * launch count since the last reset.  Process-wide; not thread-safe; adds an
 * event pair per launch.
 */
int dartree_timing_enable(int enable);
int dartree_timing_reset(void);
int dartree_timing_read(int kernel_class, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* DARTREE_H */
