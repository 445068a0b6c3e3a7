"""fp64 CPU oracle for DARTree's depth-wise batched draft-supertree construction.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It
shares no code with the HIP library and never imports it.

Sources (page title, section):

* "DARTree: Teaching a Chain-Trained Corrector to Think in Trees" (alanhou.org),
  section "Core Mechanism" and its diagram: each depth makes one batched call
  of the AR correction head over the W live branches, each branch proposes
  its k best children, the W*k children are ranked by path log-probability
  and W of them survive, for D depths (so D head calls); best-first pruning
  over the stored scores then gives the verification tree and its sparse
  attention mask.
* "Technische Samenvatting: DARTree" (gist.science), section "Methodologie",
  part 1 "Depth-Wise Parallel AR Expansie": candidates scored by corrected
  cumulative probability, the top-W branches kept and their correction states
  carried forward; part 2 "Deferred Best-First Pruning": one global top-B over
  all materialised prefixes, equal (Lemma 1) to the sequential best-first
  max-heap selection when the depth bonus beta is <= 0.
* "Accelerating Language Models with Diffusion Draft Trees" (legiblepapers),
  "Summary & Methodology Analysis": global top-W child prefixes per depth (W the
  layer width), global top-B nodes (B the verification budget), prefix tree
  verified with a tree-attention mask in one forward.

The pages give no head architecture.  The synthetic correction head used here
is the workload recipe: ``s' = s + GELU((E[tok] + h_t) W1) W2`` with the exact
erf GELU, logits ``z = s' U``, temperature log-softmax ``z/T - logsumexp(z/T)``.

Readings where the pages are silent (each listed in the design notes):

* the root (last verified token) is a single frontier row at depth 0, expanded
  like any node, so the width at depth t is ``min(W, n_{t-1} * k)``;
* h_t feeds the step that produces the depth-t tokens; the carried state of a
  kept child is its parent's updated state, and the child's token is consumed
  by the next depth's update;
* T = 0 is the T -> 0+ limit: only the lowest-index argmax has finite
  log-probability (0), so each row has one child;
* tie-breaks: children by (logp desc, token asc); survivors by (score desc,
  parent slot asc, child rank asc); pruning by (prio desc, depth asc,
  slot asc) with ``prio = score + beta * depth``;
* the verification tree is emitted in (depth, slot) order; its mask row i holds
  node i and its ancestors among the draft nodes (the prefix is always visible
  and is not part of the bitmask).
"""
from __future__ import annotations

import heapq
import math
from dataclasses import dataclass, field

import numpy as np
from scipy.special import erf

NEG_INF = -math.inf


# ----------------------------------------------------------------------------
# weights
# ----------------------------------------------------------------------------
def _widen(a: np.ndarray, wdtype: str) -> np.ndarray:
    """Storage array -> exact float64 (bf16 bit patterns or float32)."""
    if wdtype == "bf16":
        return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, np.float32).astype(np.float64)


class OracleHead:
    """The synthetic correction head in math layout, fp64.

    Takes storage-layout arrays: E [V][d], W1t [4d][d], W2t [d][4d], Ut [V][d]
    (float32 or bf16 bit patterns).  W1 = W1t^T, W2 = W2t^T, U = Ut^T.
    The output head U is widened lazily in column chunks unless ``cache_u``.
    """

    def __init__(self, wdtype, E, W1t, W2t, Ut, cache_u=True, chunk=16384):
        self.wdtype = wdtype
        self.V, self.d = Ut.shape
        self._E = E
        self.W1 = _widen(W1t, wdtype).T          # [d][4d]
        self.W2 = _widen(W2t, wdtype).T          # [4d][d]
        self._Ut = Ut
        self.chunk = chunk
        self._U = _widen(Ut, wdtype).T if cache_u else None   # [d][V]

    def embed(self, tok) -> np.ndarray:
        return _widen(self._E[np.asarray(tok, np.int64)], self.wdtype)

    def logits(self, s: np.ndarray) -> np.ndarray:
        """z = s U for rows s [n][d] -> [n][V] fp64."""
        if self._U is not None:
            return s @ self._U
        z = np.empty((s.shape[0], self.V), np.float64)
        for lo in range(0, self.V, self.chunk):
            hi = min(self.V, lo + self.chunk)
            z[:, lo:hi] = s @ _widen(self._Ut[lo:hi], self.wdtype).T
        return z


# ----------------------------------------------------------------------------
# one correction-head step (workload recipe)
# ----------------------------------------------------------------------------
def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU, x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2))."""
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def state_update(head: OracleHead, s: np.ndarray, tok, h_t: np.ndarray) -> np.ndarray:
    """s' = s + GELU((E[tok] + h_t) W1) W2 for every frontier row (fp64)."""
    x = head.embed(tok) + np.asarray(h_t, np.float64)[None, :]
    return np.asarray(s, np.float64) + gelu(x @ head.W1) @ head.W2


def log_softmax_T(z: np.ndarray, T: float) -> np.ndarray:
    """Temperature log-softmax of one row, fp64, max-shifted.

    T > 0: z/T - log sum exp(z/T).  T == 0: the T -> 0+ limit, 0 at the
    lowest-index maximum of z and -inf elsewhere.
    """
    z = np.asarray(z, np.float64)
    if T == 0.0:
        out = np.full(z.shape, NEG_INF)
        out[int(np.argmax(z))] = 0.0        # argmax returns the first maximum
        return out
    y = z / T
    m = np.max(y)
    return y - (m + math.log(np.sum(np.exp(y - m))))


def topk_children(logp: np.ndarray, k: int):
    """The k best tokens of one row by (logp desc, token asc), finite only.

    Returns (tokens int64 [<=k], logps float64 [<=k]).
    """
    idx = np.arange(logp.size)
    order = np.lexsort((idx, -logp))          # primary -logp, then token
    order = order[np.isfinite(logp[order])][:k]
    return order.astype(np.int64), logp[order]


def entropy_T(z: np.ndarray, T: float) -> float:
    """Entropy (nats) of softmax(z / T); used only for input calibration."""
    lp = log_softmax_T(z, T)
    p = np.exp(lp)
    return float(-np.sum(p[p > 0] * lp[p > 0]))


# ----------------------------------------------------------------------------
# depth-wise batched supertree construction
# ----------------------------------------------------------------------------
@dataclass
class Supertree:
    """Scored pool of one request: slot j at depth t (0-based t = depth - 1)."""
    tok: np.ndarray          # [D][W] int64, -1 where invalid
    parent: np.ndarray       # [D][W] int64, parent slot at depth t-1 (-1 at t=0 / invalid)
    score: np.ndarray        # [D][W] float64, accumulated log-prob, -inf where invalid
    n_valid: np.ndarray      # [D] int64
    head_calls: int = 0
    entropies: list = field(default_factory=list)   # per depth: entropies of the rows (T>0)
    lse: list = field(default_factory=list)         # per depth: logsumexp(z/T) of each row


def base_candidates(head: OracleHead, h_t: np.ndarray, K: int) -> np.ndarray:
    """The K candidate tokens of one depth from the drafter's base logits
    ("Technische Samenvatting: DARTree", Methodologie part 1, Kandidaat
    Selectie).  Reading: the base logits are h_t U (the drafter hidden of the
    depth through the same output head); the K best by (logit desc, token
    asc)."""
    z = head.logits(np.asarray(h_t, np.float64)[None, :])[0]
    order = np.lexsort((np.arange(z.size), -z))
    return order[:K].astype(np.int64)


def restricted_children(z: np.ndarray, lp: np.ndarray, cand: np.ndarray, k: int, T: float):
    """Top-k children of one row among the candidate tokens: by corrected
    log-probability (full-vocabulary normaliser) desc, token asc.  At T = 0
    the single child is the lowest-index argmax of z over the candidates, with
    log-probability 0 (the T -> 0+ limit of the softmax restricted to them)."""
    cand = np.asarray(cand, np.int64)
    if T == 0.0:
        best = cand[np.lexsort((cand, -z[cand]))][0]
        return np.array([best], np.int64), np.array([0.0])
    order = np.lexsort((cand, -lp[cand]))[:k]
    return cand[order], lp[cand[order]]


def build_supertree(head: OracleHead, h: np.ndarray, s0: np.ndarray, root_tok: int,
                    D: int, W: int, k: int, T: float,
                    want_entropy: bool = False, markov: bool = False,
                    n_cand: int = 0) -> Supertree:
    """Depth-wise batched construction for one request (fp64).

    Variants (the pages' head and candidate variants; off by default):
    * markov: no carried state - every row's update starts from s0, so a
      node's children depend only on its token and depth (a Markov
      correction head, as in the DSpark drafter of "Technische Samenvatting:
      DARTree", Experimentele Resultaten, Generaliseerbaarheid);
    * n_cand > 0: each row's children are chosen among the depth's n_cand
      base-logit candidates (``base_candidates``), scored with the corrected
      log-probability (``restricted_children``).
    """
    pool_tok = np.full((D, W), -1, np.int64)
    pool_parent = np.full((D, W), -1, np.int64)
    pool_score = np.full((D, W), NEG_INF)
    n_valid = np.zeros(D, np.int64)
    out = Supertree(pool_tok, pool_parent, pool_score, n_valid)

    f_state = np.asarray(s0, np.float64)[None, :]     # frontier: root only
    f_tok = np.array([root_tok], np.int64)
    f_score = np.array([0.0])
    for t in range(D):
        # one batched head call over every frontier row
        out.head_calls += 1
        src = np.repeat(np.asarray(s0, np.float64)[None, :], f_tok.size, 0) if markov else f_state
        s_new = state_update(head, src, f_tok, h[t])
        z = head.logits(s_new)
        cand_t = base_candidates(head, h[t], n_cand) if n_cand > 0 else None
        cands = []                                    # (score, parent, rank, token)
        ents, lses = [], []
        for i in range(z.shape[0]):
            lp = log_softmax_T(z[i], T)
            if T > 0.0:
                y = z[i] / T
                lses.append(float(np.max(y) + math.log(np.sum(np.exp(y - np.max(y))))))
                if want_entropy:
                    ents.append(entropy_T(z[i], T))
            if cand_t is None:
                toks, lps = topk_children(lp, k)
            else:
                toks, lps = restricted_children(z[i], lp, cand_t, k, T)
            for r in range(toks.size):
                cands.append((f_score[i] + lps[r], i, r, int(toks[r])))
        out.entropies.append(ents)
        out.lse.append(lses)
        cands.sort(key=lambda c: (-c[0], c[1], c[2]))
        keep = cands[:W]
        n = len(keep)
        n_valid[t] = n
        for j, (sc, i, r, c) in enumerate(keep):
            pool_tok[t, j] = c
            pool_parent[t, j] = i if t > 0 else -1
            pool_score[t, j] = sc
        # carry the parent's updated state; the child's token is consumed next
        f_state = s_new[[c[1] for c in keep]]
        f_tok = np.array([c[3] for c in keep], np.int64)
        f_score = np.array([c[0] for c in keep])
    return out


# ----------------------------------------------------------------------------
# deferred best-first pruning
# ----------------------------------------------------------------------------
@dataclass
class VerifyTree:
    node: np.ndarray         # [n] flat pool index t*W + j
    parent: np.ndarray       # [n] index into this list, -1 for depth-1 nodes
    depth: np.ndarray        # [n] 1-based depth
    n: int


def _pool_nodes(score, n_valid):
    return [(t, j) for t in range(score.shape[0]) for j in range(int(n_valid[t]))]


def prune_topB(score, parent, n_valid, B: int, beta: float) -> VerifyTree:
    """Global top-B over the scored pool with prio = score + beta * depth.

    Order (prio desc, depth asc, slot asc); the chosen nodes are emitted in
    (depth, slot) order with parents remapped to emitted indices.
    """
    D, W = score.shape
    nodes = _pool_nodes(score, n_valid)
    prio = {n: float(score[n]) + beta * (n[0] + 1) for n in nodes}
    ranked = sorted(nodes, key=lambda n: (-prio[n], n[0], n[1]))
    chosen = sorted(ranked[:min(B, len(nodes))])
    index = {n: i for i, n in enumerate(chosen)}
    m = len(chosen)
    node = np.array([t * W + j for t, j in chosen], np.int64)
    depth = np.array([t + 1 for t, _ in chosen], np.int64)
    par = np.full(m, -1, np.int64)
    for i, (t, j) in enumerate(chosen):
        if t > 0:
            p = (t - 1, int(parent[t, j]))
            if p not in index:
                raise AssertionError(f"selection not ancestor-closed at {(t, j)}")
            par[i] = index[p]
    return VerifyTree(node, par, depth, m)


def heap_prune(score, parent, n_valid, B: int, beta: float) -> set:
    """Sequential best-first selection with a max-heap over the cached pool.

    Start from the depth-1 nodes; pop the best (prio desc, depth asc, slot
    asc), then push its children; stop after B pops.  Returns the popped set of
    (t, j).  (Lemma 1 states this equals the global top-B when beta <= 0.)
    """
    D, W = score.shape
    kids = {}
    for t in range(1, D):
        for j in range(int(n_valid[t])):
            kids.setdefault((t - 1, int(parent[t, j])), []).append((t, j))

    def key(n):
        return (-(float(score[n]) + beta * (n[0] + 1)), n[0], n[1])

    heap = [key((0, j)) for j in range(int(n_valid[0]))]
    heapq.heapify(heap)
    popped = set()
    while heap and len(popped) < B:
        _, t, j = heapq.heappop(heap)
        popped.add((t, j))
        for c in kids.get((t, j), []):
            heapq.heappush(heap, key(c))
    return popped


# ----------------------------------------------------------------------------
# sequential heap-interleaved best-first construction (the per-node baseline)
# ----------------------------------------------------------------------------
@dataclass
class SeqTree:
    """Tree built one head call per expanded node, in pop order."""
    tok: np.ndarray          # [n] int64
    parent: np.ndarray       # [n] index of the parent in this list, -1 at depth 1
    depth: np.ndarray        # [n] 1-based depth
    score: np.ndarray        # [n] float64 accumulated log-prob
    n: int
    head_calls: int


def sequential_best_first(head: OracleHead, h: np.ndarray, s0: np.ndarray, root_tok: int,
                          D: int, k: int, B: int, beta: float, T: float) -> SeqTree:
    """Best-first tree growth with a max-heap and one head call per expanded
    node: the costly alternative the pages set against depth-wise batching
    ("DARTree: Teaching a Chain-Trained Corrector to Think in Trees", Core
    Mechanism; "Technische Samenvatting: DARTree", Experimentele Resultaten,
    ablation of sequential heap-interleaved correction against depth-wise
    batching).

    Reading used here (the pages give the idea, not the steps): the root is
    expanded first (one head call, h_1); every popped node is appended to the
    tree and, unless the tree holds B nodes or the node sits at depth D, is
    expanded at once (one head call on its own row: its parent's updated
    state, its token and h_{depth+1}) and its top-k children are pushed.  The
    heap orders by (score + beta * depth desc, depth asc, push order asc).
    Children, scores and carried states are exactly those of the batched
    step for the same row.
    """
    out_tok, out_par, out_depth, out_score = [], [], [], []
    heap = []
    pushed = 0
    calls = 0

    def expand(state, tok, depth, score, node_index):
        # one head call on one row; returns the row's updated state
        nonlocal pushed, calls
        calls += 1
        s_new = state_update(head, np.asarray(state, np.float64)[None, :], [int(tok)], h[depth])[0]
        lp = log_softmax_T(head.logits(s_new[None, :])[0], T)
        toks, lps = topk_children(lp, k)
        for r in range(toks.size):
            sc = score + float(lps[r])
            d = depth + 1
            heapq.heappush(heap, (-(sc + beta * d), d, pushed, int(toks[r]), node_index, sc,
                                  s_new))
            pushed += 1
        return s_new

    expand(s0, root_tok, 0, 0.0, -1)
    while heap and len(out_tok) < B:
        _, d, _, tok, par, sc, parent_state = heapq.heappop(heap)
        i = len(out_tok)
        out_tok.append(tok)
        out_par.append(par)
        out_depth.append(d)
        out_score.append(sc)
        if len(out_tok) < B and d < D:
            expand(parent_state, tok, d, sc, i)
    n = len(out_tok)
    return SeqTree(np.array(out_tok, np.int64), np.array(out_par, np.int64),
                   np.array(out_depth, np.int64), np.array(out_score, np.float64), n, calls)


# ----------------------------------------------------------------------------
# acceptance walk against a synthetic target (verification stand-in)
# ----------------------------------------------------------------------------
@dataclass
class Walk:
    target_tok: np.ndarray   # [B + 1]: target's greedy token after the root (0) and node i (1 + i);
                             # -1 for nodes without children
    path: list               # accepted node indices, depth 1, 2, ...
    tau: int                 # tokens per verification round = len(path) + 1


def acceptance_walk(target: OracleHead, h: np.ndarray, s0: np.ndarray, root_tok: int,
                    tok, parent, depth, n: int, D: int, B: int) -> Walk:
    """Verify one draft tree against a synthetic greedy target.

    "DARTree: Teaching a Chain-Trained Corrector to Think in Trees": Core
    Mechanism (the target checks the whole tree in one forward and keeps the
    longest prefix it agrees with), Key Concepts (tokens accepted per
    verification round), Expert Assessment (compare trees of matched size).

    The pages' target is a language model; the stand-in is a chain model of
    the correction head's form with weights of its own (``target``).  Its
    state after a node follows the node's path from the root:
    s'_root = s0 + step(root_tok, h[0]), s'_v = s'_parent(v) + step(tok_v,
    h[depth(v)]), the draft head's recurrence, and its greedy token
    after v is the lowest-index argmax of s'_v U_target.  The target's token
    is needed only after nodes that have children.

    The walk starts at the root; while the current node has a child whose
    token is the target's token after it, it moves to that child (the
    lowest-index one if several match); it stops at a node with no such
    child.  tau counts the accepted draft tokens plus the target's own token
    after the last of them.  Tree: node i < n has token tok[i], parent
    parent[i] (-1: the root) earlier in the list and depth depth[i] =
    depth of the parent + 1, at most D.
    """
    tok = np.asarray(tok)[:n]; parent = np.asarray(parent)[:n]; depth = np.asarray(depth)[:n]
    has_child = np.zeros(n + 1, bool)                 # slot 0: the root
    for i in range(n):
        has_child[int(parent[i]) + 1] = True
    states = {-1: state_update(target, np.asarray(s0, np.float64)[None, :], [int(root_tok)],
                               h[0])[0]}
    target_tok = np.full(B + 1, -1, np.int64)
    if has_child[0]:
        target_tok[0] = int(np.argmax(target.logits(states[-1][None, :])[0]))
    for i in range(n):
        if not has_child[i + 1]:
            continue
        states[i] = state_update(target, states[int(parent[i])][None, :], [int(tok[i])],
                                 h[int(depth[i])])[0]
        target_tok[i + 1] = int(np.argmax(target.logits(states[i][None, :])[0]))
    path, cur, dcur = [], -1, 0
    while dcur < D and target_tok[cur + 1] >= 0:
        want = int(target_tok[cur + 1])
        match = [i for i in range(n) if int(parent[i]) == cur and int(tok[i]) == want]
        if not match:
            break
        cur = match[0]
        dcur = int(depth[cur])
        path.append(cur)
    return Walk(target_tok, path, len(path) + 1)


# ----------------------------------------------------------------------------
# ancestor mask
# ----------------------------------------------------------------------------
def tree_mask(parent: np.ndarray, n: int, B: int) -> np.ndarray:
    """Bitmask [B][ceil(B/32)] uint32: row i has bit i and the bits of all its
    ancestors among the tree nodes (bit b of word w is node 32 w + b)."""
    words = (B + 31) // 32
    mask = np.zeros((B, words), np.uint32)
    for i in range(n):
        a = i
        while a >= 0:
            mask[i, a // 32] |= np.uint32(1 << (a % 32))
            a = int(parent[a])
    return mask


def mask_to_bool(mask: np.ndarray, n: int) -> np.ndarray:
    """Visible[i][j] (j a tree node) from the bitmask."""
    vis = np.zeros((n, n), bool)
    for i in range(n):
        for j in range(n):
            vis[i, j] = bool((int(mask[i, j // 32]) >> (j % 32)) & 1)
    return vis


# ----------------------------------------------------------------------------
# verification: one tree-attention layer
# ----------------------------------------------------------------------------
def tree_attention(q, k_prefix, v_prefix, k_tree, v_tree, mask, n: int, scale: float):
    """Tree attention in fp64.

    q [n][Hq][hd]; k/v_prefix [P][Hkv][hd]; k/v_tree [n][Hkv][hd]; query head h
    reads key/value head h // (Hq / Hkv).  Each tree query sees every prefix key
    and the tree keys its mask row marks.  Returns out [n][Hq][hd] fp64.
    """
    q = np.asarray(q, np.float64)
    kp, vp = np.asarray(k_prefix, np.float64), np.asarray(v_prefix, np.float64)
    kt, vt = np.asarray(k_tree, np.float64), np.asarray(v_tree, np.float64)
    Hq, Hkv = q.shape[1], kp.shape[1]
    group = Hq // Hkv
    vis = mask_to_bool(mask, n)
    out = np.zeros((n, Hq, q.shape[2]))
    for h in range(Hq):
        g = h // group
        sp = (q[:n, h] @ kp[:, g].T) * scale                 # [n][P]
        st = (q[:n, h] @ kt[:n, g].T) * scale                # [n][n]
        st = np.where(vis, st, NEG_INF)
        s = np.concatenate([sp, st], axis=1)
        m = np.max(s, axis=1, keepdims=True)
        p = np.exp(s - m)
        p /= np.sum(p, axis=1, keepdims=True)
        out[:, h] = p @ np.concatenate([vp[:, g], vt[:n, g]], axis=0)
    return out


# ----------------------------------------------------------------------------
# measurement: checksum of the read-bandwidth probe
# ----------------------------------------------------------------------------
def word_sum64(buf) -> int:
    """Sum of the little-endian unsigned 64-bit words of a byte buffer, modulo
    2^64: what the streaming read probe returns for the buffer it reads (the
    probe sets the ceiling for the memory-bound weight stream of "Accelerating
    Language Models with Diffusion Draft Trees", Summary & Methodology
    Analysis).  ``buf`` is bytes or a numpy array; its size must be a
    multiple of 8."""
    raw = np.frombuffer(buf, np.uint8) if isinstance(buf, (bytes, bytearray)) else \
        np.ascontiguousarray(buf).reshape(-1).view(np.uint8)
    if raw.size % 8:
        raise ValueError("buffer size must be a multiple of 8 bytes")
    words = raw.view("<u8")
    # numpy's unsigned integer sums wrap modulo 2^64
    return int(np.sum(words, dtype=np.uint64)) if words.size else 0
