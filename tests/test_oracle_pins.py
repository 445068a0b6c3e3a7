"""Pins of the fp64 oracle to facts outside itself.

Each test checks the oracle against a closed form, a textbook special case, a
library routine it does not use, brute force on tiny inputs, or a hand-worked
example under tests/golden/.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
from hypothesis import given, settings, strategies as st

from oracle import dartree_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def gold():
    with open(GOLD) as f:
        return json.load(f)


def tiny_head(V=7, d=8, seed=0, wscale=0.5, uscale=1.5):
    """A float32 head small enough for brute force (storage layout)."""
    g = np.random.default_rng(seed)
    E = (g.standard_normal((V, d)) * wscale).astype(np.float32)
    W1t = (g.standard_normal((4 * d, d)) * wscale).astype(np.float32)
    W2t = (g.standard_normal((d, 4 * d)) * wscale).astype(np.float32)
    Ut = (g.standard_normal((V, d)) * uscale).astype(np.float32)
    return O.OracleHead("f32", E, W1t, W2t, Ut)


# ----------------------------------------------------------------------------
# GELU and the state update
# ----------------------------------------------------------------------------
def test_gelu_matches_math_erf_and_table_values():
    xs = np.linspace(-8, 8, 1601)
    ref = np.array([0.5 * x * (1 + math.erf(x / math.sqrt(2))) for x in xs])
    assert np.max(np.abs(O.gelu(xs) - ref)) < 1e-15
    # textbook Phi values: GELU(1) = Phi(1), GELU(2) = 2 Phi(2)
    assert abs(O.gelu(np.array(1.0)) - 0.8413447460685429) < 1e-15
    assert abs(O.gelu(np.array(2.0)) - 2 * 0.9772498680518208) < 1e-15
    # GELU(x) - GELU(-x) = x, GELU(0) = 0, GELU -> identity / 0 in the tails
    assert np.max(np.abs(O.gelu(xs) - O.gelu(-xs) - xs)) < 1e-14
    assert O.gelu(np.array(0.0)) == 0.0
    assert abs(O.gelu(np.array(40.0)) - 40.0) < 1e-12
    assert abs(O.gelu(np.array(-40.0))) < 1e-12


def test_state_update_hand_example():
    g = gold()["state_update_d1"]
    E = np.array(g["E"], np.float32)
    W1t = np.array(g["W1"], np.float32).T.copy()      # stored transposed
    W2t = np.array(g["W2"], np.float32).T.copy()
    head = O.OracleHead("f32", E, W1t, W2t, np.zeros((2, 1), np.float32))
    s = O.state_update(head, np.array([g["s"]]), [g["tok"]], np.array(g["h"]))
    assert abs(s[0, 0] - g["s_new"][0]) < 1e-14


def test_state_update_degenerate_weights_keep_state():
    head = tiny_head()
    s = np.random.default_rng(1).standard_normal((3, 8))
    h = np.random.default_rng(2).standard_normal(8)
    for zero in ("W1", "W2"):
        hz = tiny_head()
        setattr(hz, zero, np.zeros_like(getattr(hz, zero)))
        assert np.array_equal(O.state_update(hz, s, [0, 1, 2], h), s)
    # E[tok] + h = 0 -> GELU(0) = 0 -> state unchanged
    hz = tiny_head()
    tok = [4, 4, 4]
    s2 = O.state_update(hz, s, tok, -hz.embed([4])[0])
    assert np.array_equal(s2, s)
    assert head.d == 8


def test_state_update_linear_regime_orientation():
    # With a large positive pre-activation GELU is the identity, so the update
    # is the linear map s + x W1 W2, computed here by a different association.
    d = 5
    g = np.random.default_rng(3)
    E = np.zeros((3, d), np.float32)
    W1 = np.abs(g.standard_normal((d, 4 * d))).astype(np.float32) + 1.0
    W2 = g.standard_normal((4 * d, d)).astype(np.float32)
    head = O.OracleHead("f32", E, W1.T.copy(), W2.T.copy(), np.zeros((3, d), np.float32))
    x = np.full(d, 20.0)
    s = g.standard_normal((1, d))
    got = O.state_update(head, s, [1], x)
    want = s + x[None, :] @ (W1.astype(np.float64) @ W2.astype(np.float64))
    assert np.allclose(got, want, rtol=1e-12, atol=1e-9)


def test_head_storage_layout_is_transposed_u():
    V, d = 6, 4
    Ut = np.zeros((V, d), np.float32)
    Ut[3, 1] = 1.0
    head = O.OracleHead("f32", np.zeros((V, d), np.float32), np.zeros((4 * d, d), np.float32),
                        np.zeros((d, 4 * d), np.float32), Ut)
    s = np.array([[0.1, 0.7, -0.2, 0.3]])
    z = head.logits(s)
    assert z[0, 3] == pytest.approx(0.7) and np.count_nonzero(z) == 1


def test_bf16_widening_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F], np.uint16)
    want = [1.0, -1.0, 3.140625, 2.0 ** -133, 3.3895313892515355e38]
    head = O.OracleHead("bf16", bits.reshape(5, 1), np.zeros((4, 1), np.uint16),
                        np.zeros((1, 4), np.uint16), np.zeros((5, 1), np.uint16))
    got = head.embed(np.arange(5))[:, 0]
    assert list(got) == want


def test_chunked_and_cached_logits_agree():
    g = np.random.default_rng(5)
    V, d = 1000, 16
    Ut = g.standard_normal((V, d)).astype(np.float32)
    args = ("f32", np.zeros((V, d), np.float32), np.zeros((4 * d, d), np.float32),
            np.zeros((d, 4 * d), np.float32), Ut)
    a = O.OracleHead(*args, cache_u=True)
    b = O.OracleHead(*args, cache_u=False, chunk=96)
    s = g.standard_normal((3, d))
    assert np.allclose(a.logits(s), b.logits(s), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# temperature log-softmax and top-k
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("T", [0.25, 1.0, 3.0])
def test_log_softmax_matches_scipy(T):
    g = np.random.default_rng(7)
    for scale in (1.0, 30.0, 300.0):
        z = g.standard_normal(5000) * scale
        got = O.log_softmax_T(z, T)
        want = scipy.special.log_softmax(z / T)
        assert np.max(np.abs(got - want)) < 1e-9 * max(1.0, scale / T)
        assert abs(np.sum(np.exp(got)) - 1.0) < 1e-12


def test_log_softmax_T0_is_lowest_index_argmax():
    z = np.array([1.0, 3.0, -2.0, 3.0, 0.5])
    lp = O.log_softmax_T(z, 0.0)
    assert lp[1] == 0.0 and np.all(np.isneginf(np.delete(lp, 1)))
    # the T -> 0+ limit of the temperature log-softmax on a gap-ful row
    z2 = np.array([0.0, 1.0, 0.2])
    lim = scipy.special.log_softmax(z2 / 1e-4)
    assert np.argmax(lim) == 1 and abs(lim[1]) < 1e-12 and lim[0] < -1e3


@given(st.lists(st.integers(-3, 3), min_size=1, max_size=12), st.integers(1, 14))
@settings(max_examples=200, deadline=None)
def test_topk_children_brute_force(vals, k):
    lp = np.array(vals, np.float64)
    toks, lps = O.topk_children(lp, k)
    m = min(k, lp.size)
    assert toks.size == m
    chosen = set(toks.tolist())
    # every chosen >= every unchosen, equal values resolved to the lower token
    for a in chosen:
        for b in set(range(lp.size)) - chosen:
            assert lp[a] > lp[b] or (lp[a] == lp[b] and a < b)
    # sorted by (logp desc, token asc)
    keys = [(-lp[t], t) for t in toks]
    assert keys == sorted(keys)
    assert np.array_equal(lps, lp[toks])


def test_topk_children_skips_minus_inf():
    lp = np.array([-np.inf, -1.0, -np.inf, -0.5])
    toks, _ = O.topk_children(lp, 4)
    assert toks.tolist() == [3, 1]


# ----------------------------------------------------------------------------
# depth-wise batched construction
# ----------------------------------------------------------------------------
def _greedy_chain(head, h, s0, root, D):
    """Textbook greedy decoding: feed back the argmax token each step."""
    s, tok, score, toks, scores = np.asarray(s0, np.float64)[None], root, 0.0, [], []
    for t in range(D):
        s = O.state_update(head, s, [tok], h[t])
        lp = scipy.special.log_softmax(head.logits(s)[0])
        tok = int(np.argmax(lp))
        score += lp[tok]
        toks.append(tok); scores.append(score)
    return toks, scores


def _inputs(head, D, seed=11):
    g = np.random.default_rng(seed)
    return g.standard_normal((D, head.d)), g.standard_normal(head.d)


def test_width_one_is_the_greedy_chain():
    head = tiny_head(V=40, d=8)
    h, s0 = _inputs(head, 6)
    tree = O.build_supertree(head, h, s0, 3, D=6, W=1, k=4, T=1.0)
    toks, scores = _greedy_chain(head, h, s0, 3, 6)
    assert tree.tok[:, 0].tolist() == toks
    assert np.allclose(tree.score[:, 0], scores, atol=1e-12)
    assert tree.n_valid.tolist() == [1] * 6


def test_T0_is_the_same_chain_with_zero_scores():
    head = tiny_head(V=40, d=8)
    h, s0 = _inputs(head, 6)
    t0 = O.build_supertree(head, h, s0, 3, D=6, W=5, k=4, T=0.0)
    toks, _ = _greedy_chain(head, h, s0, 3, 6)
    assert t0.n_valid.tolist() == [1] * 6
    assert t0.tok[:, 0].tolist() == toks
    assert np.all(t0.score[:, 0] == 0.0)
    assert np.all(t0.tok[:, 1:] == -1)


def test_exhaustive_enumeration_when_beam_keeps_everything():
    V, D = 3, 3
    head = tiny_head(V=V, d=6, seed=4)
    h, s0 = _inputs(head, D, seed=12)
    tree = O.build_supertree(head, h, s0, 0, D=D, W=V ** D, k=V, T=1.0)
    # brute force: every token sequence, its state chain and summed log-prob
    for t in range(1, D + 1):
        want = {}
        for seq in itertools.product(range(V), repeat=t):
            s, tok, sc = np.asarray(s0)[None], 0, 0.0
            for i, c in enumerate(seq):
                s = O.state_update(head, s, [tok], h[i])
                sc += scipy.special.log_softmax(head.logits(s)[0])[c]
                tok = c
            want[seq] = sc
        assert int(tree.n_valid[t - 1]) == V ** t
        got = {}
        for j in range(V ** t):
            seq, tt, jj = [], t - 1, j
            while tt >= 0:
                seq.append(int(tree.tok[tt, jj]))
                jj = int(tree.parent[tt, jj]); tt -= 1
            got[tuple(reversed(seq))] = tree.score[t - 1, j]
        assert got.keys() == want.keys()
        assert max(abs(got[s] - want[s]) for s in want) < 1e-12
        # the depth-t path probabilities form a distribution
        assert abs(sum(math.exp(v) for v in got.values()) - 1.0) < 1e-12
        # slots in non-increasing score order
        assert np.all(np.diff(tree.score[t - 1, :V ** t]) <= 0)


def test_width_formula_head_calls_and_structure():
    head = tiny_head(V=50, d=8)
    h, s0 = _inputs(head, 7)
    for W, k in ((4, 4), (16, 3), (5, 8), (1, 1)):
        tree = O.build_supertree(head, h, s0, 2, D=7, W=W, k=k, T=1.0)
        assert tree.head_calls == 7
        n = 1
        for t in range(7):
            n = min(W, n * k)
            assert tree.n_valid[t] == n
            for j in range(n):
                p = tree.parent[t, j]
                if t == 0:
                    assert p == -1 and tree.score[t, j] <= 0
                else:
                    assert 0 <= p < tree.n_valid[t - 1]
                    assert tree.score[t, j] <= tree.score[t - 1, p]
            assert np.all(np.isneginf(tree.score[t, n:]))


def _paths_with_scores(tree, t):
    """{token path: score} of the depth-t pool (0-based t)."""
    out = {}
    W = tree.tok.shape[1]
    for j in range(int(tree.n_valid[t])):
        seq, tt, jj = [], t, j
        while tt >= 0:
            seq.append(int(tree.tok[tt, jj]))
            jj = int(tree.parent[tt, jj]); tt -= 1
        out[tuple(reversed(seq))] = float(tree.score[t, j])
    return out


def test_markov_width_one_is_the_markov_greedy_chain():
    # textbook greedy decoding with a head that restarts from s0 every step
    head = tiny_head(V=40, d=8)
    h, s0 = _inputs(head, 6)
    tree = O.build_supertree(head, h, s0, 3, D=6, W=1, k=4, T=1.0, markov=True)
    tok, score = 3, 0.0
    for t in range(6):
        s = O.state_update(head, np.asarray(s0)[None], [tok], h[t])
        lp = scipy.special.log_softmax(head.logits(s)[0])
        tok = int(np.argmax(lp))
        score += lp[tok]
        assert tree.tok[t, 0] == tok and abs(tree.score[t, 0] - score) < 1e-12


def test_markov_children_depend_only_on_token_and_depth():
    head = tiny_head(V=6, d=8, seed=3)
    h, s0 = _inputs(head, 3, seed=5)
    tree = O.build_supertree(head, h, s0, 1, D=3, W=6 ** 3, k=6, T=1.0, markov=True)
    for t in range(1, 3):
        seen = {}
        for j in range(int(tree.n_valid[t])):
            p = int(tree.parent[t, j])
            key = (int(tree.tok[t - 1, p]), int(tree.tok[t, j]))
            lp = float(tree.score[t, j] - tree.score[t - 1, p])
            if key in seen:
                assert abs(seen[key] - lp) < 1e-12
            seen[key] = lp
    # at depth 3 the same (token, child) pair occurs under many depth-1 tokens
    assert len(seen) < int(tree.n_valid[2])
    # a carried-state head does not have this property on the same inputs
    plain = O.build_supertree(head, h, s0, 1, D=3, W=6 ** 3, k=6, T=1.0)
    assert not np.allclose(plain.score, tree.score)


@pytest.mark.parametrize("T", [1.0, 0.7, 0.0])
def test_base_candidates_over_the_whole_vocabulary_is_the_plain_build(T):
    head = tiny_head(V=30, d=8, seed=6)
    h, s0 = _inputs(head, 4, seed=2)
    a = O.build_supertree(head, h, s0, 2, D=4, W=7, k=3, T=T)
    b = O.build_supertree(head, h, s0, 2, D=4, W=7, k=3, T=T, n_cand=30)
    for x, y in ((a.tok, b.tok), (a.parent, b.parent), (a.n_valid, b.n_valid)):
        assert np.array_equal(x, y)
    assert np.array_equal(a.score, b.score)


def test_base_candidates_brute_force():
    # every node's children: the k best of the depth's K base-logit candidates
    # (np.argsort of h_t U) by scipy's full-vocabulary log_softmax
    V, D, k, K = 9, 3, 2, 4
    head = tiny_head(V=V, d=6, seed=9)
    h, s0 = _inputs(head, D, seed=4)
    tree = O.build_supertree(head, h, s0, 0, D=D, W=k ** D, k=k, T=1.0, n_cand=K)
    cands = []
    for t in range(D):
        z = head.logits(np.asarray(h[t])[None])[0]
        cands.append(sorted(range(V), key=lambda c: (-z[c], c))[:K])
    want = {}

    def rec(state, tok, t, path, score):
        if t == D:
            return
        s = O.state_update(head, np.asarray(state)[None], [tok], h[t])
        lp = scipy.special.log_softmax(head.logits(s)[0])
        kids = sorted(cands[t], key=lambda c: (-lp[c], c))[:k]
        for c in kids:
            want[path + (c,)] = score + lp[c]
            rec(s[0], c, t + 1, path + (c,), score + lp[c])

    rec(np.asarray(s0, np.float64), 0, 0, (), 0.0)
    got = {}
    for t in range(D):
        got.update(_paths_with_scores(tree, t))
    assert got.keys() == want.keys()
    assert max(abs(got[p] - want[p]) for p in want) < 1e-12


@pytest.mark.parametrize("markov,n_cand", [(True, 0), (False, 8), (True, 6)])
@pytest.mark.parametrize("T", [1.0, 0.0])
def test_build_checker_follows_the_variants(markov, n_cand, T):
    # the teacher-forced checker accepts a variant's own build and rejects it
    # as a plain build (the variants are told apart)
    from oracle import parity as P
    head = tiny_head(V=50, d=8, seed=0)
    h, s0 = _inputs(head, 5, seed=1)
    t = O.build_supertree(head, h, s0, 3, D=5, W=6, k=3, T=T, markov=markov, n_cand=n_cand)
    dev = dict(tok=t.tok, parent=t.parent, score=t.score, n_valid=t.n_valid)
    assert P.check_build(head, h, s0, 3, 5, 6, 3, T, dev, 1e-9, 1e-9, markov=markov,
                         base_cand=n_cand).ok
    assert not P.check_build(head, h, s0, 3, 5, 6, 3, T, dev, 1e-9, 1e-9).ok


def test_survivor_tie_break_on_exact_ties():
    # With E = 0 and h = 0 the update leaves every state equal to s0, so every
    # row has the same children a, b, c with log-probs l0 > l1 > l2.  At depth
    # 2 the candidates (parent 0, b) and (parent 1, a) both score l0 + l1
    # exactly; the tie goes to the lower parent slot.
    V, d = 9, 4
    Ut = np.random.default_rng(0).standard_normal((V, d)).astype(np.float32)
    head = O.OracleHead("f32", np.zeros((V, d), np.float32), np.zeros((4 * d, d), np.float32),
                        np.zeros((d, 4 * d), np.float32), Ut)
    s0 = np.ones(d)
    tree = O.build_supertree(head, np.zeros((2, d)), s0, 0, D=2, W=6, k=3, T=1.0)
    assert tree.n_valid.tolist() == [3, 6]
    a, b, c = tree.tok[0, :3].tolist()
    got = [(int(tree.parent[1, j]), int(tree.tok[1, j])) for j in range(3)]
    assert got == [(0, a), (0, b), (1, a)]
    assert tree.score[1, 1] == tree.score[1, 2]



# ----------------------------------------------------------------------------
# sequential heap-interleaved best-first construction
# ----------------------------------------------------------------------------
def _full_topk_tree(head, h, s0, root, D, k, T):
    """Brute force: every node of the k-ary tree to depth D, where a node's
    children are the k best tokens of its row (logp desc, token asc) by
    scipy's log_softmax; returns {token path: score}."""
    out = {}

    def rec(state, tok, depth, path, score):
        if depth == D:
            return
        s = O.state_update(head, np.asarray(state)[None], [tok], h[depth])
        z = head.logits(s)[0]
        lp = scipy.special.log_softmax(z / T)
        order = np.lexsort((np.arange(lp.size), -lp))[:k]
        for c in order:
            p = path + (int(c),)
            out[p] = score + float(lp[c])
            rec(s[0], int(c), depth + 1, p, out[p])

    rec(np.asarray(s0, np.float64), root, 0, (), 0.0)
    return out


def _seq_paths(tree):
    paths = []
    for i in range(tree.n):
        p, j = [], i
        while j >= 0:
            p.append(int(tree.tok[j]))
            j = int(tree.parent[j])
        paths.append(tuple(reversed(p)))
    return paths


@settings(max_examples=12, deadline=None)
@given(B=st.integers(1, 30), beta=st.floats(-1.5, 0.0), seed=st.integers(0, 50),
       T=st.sampled_from([0.5, 1.0, 2.0]))
def test_sequential_best_first_is_top_b_of_the_full_tree(B, beta, seed, T):
    # Lemma 1 on the whole k-ary tree: with beta <= 0 the sequential pops are
    # the B best nodes of the full tree by score + beta * depth
    D, k = 3, 3
    head = tiny_head(V=9, d=6, seed=seed)
    h, s0 = _inputs(head, D, seed=seed + 100)
    full = _full_topk_tree(head, h, s0, 1, D, k, T)
    seq = O.sequential_best_first(head, h, s0, 1, D=D, k=k, B=B, beta=beta, T=T)
    ranked = sorted(full, key=lambda p: -(full[p] + beta * len(p)))
    want = set(ranked[:min(B, len(full))])
    paths = _seq_paths(seq)
    assert seq.n == min(B, len(full))
    assert set(paths) == want
    for i, p in enumerate(paths):
        assert abs(seq.score[i] - full[p]) < 1e-12
        assert seq.depth[i] == len(p)
        # ancestor-closed, parents popped first
        assert seq.parent[i] < i and (seq.parent[i] == -1) == (len(p) == 1)
    # pop order is best-first: priorities never increase
    prio = seq.score + beta * seq.depth
    assert np.all(np.diff(prio) <= 1e-12)


def test_sequential_matches_batched_prune_when_beam_keeps_everything():
    D, k, B = 3, 3, 11
    head = tiny_head(V=12, d=6, seed=7)
    h, s0 = _inputs(head, D, seed=3)
    for beta in (0.0, -0.3):
        tree = O.build_supertree(head, h, s0, 2, D=D, W=k ** D, k=k, T=1.0)
        vt = O.prune_topB(tree.score, tree.parent, tree.n_valid, B, beta)
        want = set()
        for node in vt.node:
            t, j = divmod(int(node), k ** D)
            p = []
            while t >= 0:
                p.append(int(tree.tok[t, j]))
                j = int(tree.parent[t, j]); t -= 1
            want.add(tuple(reversed(p)))
        seq = O.sequential_best_first(head, h, s0, 2, D=D, k=k, B=B, beta=beta, T=1.0)
        assert set(_seq_paths(seq)) == want
        # one head call per expanded node: the root plus every popped node that
        # is neither the last one nor at depth D
        expanded = sum(1 for i in range(seq.n - 1) if seq.depth[i] < D)
        assert seq.head_calls == 1 + expanded


def test_sequential_checker_accepts_the_oracle_and_rejects_planted_mistakes():
    from oracle import parity as P
    head = tiny_head(V=50, d=8, seed=2)
    h, s0 = _inputs(head, 5, seed=8)
    t = O.sequential_best_first(head, h, s0, 3, D=5, k=4, B=20, beta=-0.1, T=1.0)
    dev = dict(tok=t.tok, parent=t.parent, depth=t.depth, score=t.score, n=[t.n])
    assert P.check_sequential(head, h, s0, 3, 5, 4, 20, -0.1, 1.0, dev, 1e-9, 1e-9).ok
    for mut in ("tok", "score", "order"):
        bad = {k: np.array(v).copy() for k, v in dev.items()}
        if mut == "tok":
            bad["tok"][2] = (bad["tok"][2] + 1) % 50
        elif mut == "score":
            bad["score"][3] += 1e-6
        else:
            for key in ("tok", "parent", "depth", "score"):
                bad[key][[1, 2]] = bad[key][[2, 1]]
        assert not P.check_sequential(head, h, s0, 3, 5, 4, 20, -0.1, 1.0, bad, 1e-9,
                                      1e-9).ok, mut


def test_sequential_T0_is_the_greedy_chain():
    head = tiny_head(V=40, d=8)
    h, s0 = _inputs(head, 6)
    toks, _ = _greedy_chain(head, h, s0, 3, 6)
    for B in (3, 6, 10):
        seq = O.sequential_best_first(head, h, s0, 3, D=6, k=4, B=B, beta=0.0, T=0.0)
        n = min(B, 6)
        assert seq.n == n and seq.head_calls == n
        assert seq.tok.tolist() == toks[:n]
        assert seq.parent.tolist() == list(range(-1, n - 1))
        assert np.all(seq.score == 0.0)


# ----------------------------------------------------------------------------
# acceptance walk against a synthetic target
# ----------------------------------------------------------------------------
def _perturbed(head, sigma, seed):
    """A target sharing E, W1, W2 with `head`, U perturbed (float32 storage)."""
    g = np.random.default_rng(seed)
    Ut = (head._Ut + sigma * g.standard_normal(head._Ut.shape)).astype(np.float32)
    return O.OracleHead("f32", head._E, head.W1.T.astype(np.float32),
                        head.W2.T.astype(np.float32), Ut)


def _state_from_scratch(head, h, s0, root, path_toks):
    """State after a token sequence, recomputed position by position."""
    s = np.asarray(s0, np.float64)[None]
    for j, t in enumerate([root] + list(path_toks)):
        s = O.state_update(head, s, [t], h[j])
    return s[0]


def test_walk_with_the_draft_head_as_target_accepts_the_whole_greedy_chain():
    head = tiny_head(V=40, d=8)
    D = 6
    h, s0 = _inputs(head, D)
    toks, _ = _greedy_chain(head, h, s0, 3, D)
    seq = O.sequential_best_first(head, h, s0, 3, D=D, k=4, B=D, beta=0.0, T=0.0)
    w = O.acceptance_walk(head, h, s0, 3, seq.tok, seq.parent, seq.depth, seq.n, D, B=D)
    assert w.tau == D + 1 and w.path == list(range(D))
    # the target's token after each chain node is the next chain token; the
    # depth-D leaf has no children and no target token
    assert w.target_tok.tolist() == toks + [-1]


@settings(max_examples=15, deadline=None)
@given(seed=st.integers(0, 60), sigma=st.sampled_from([0.05, 0.3, 1.0]),
       kind=st.sampled_from(["sequential", "pruned"]))
def test_walk_is_the_longest_tree_prefix_of_the_target_greedy_continuation(seed, sigma, kind):
    D, k, B = 4, 3, 14
    head = tiny_head(V=9, d=6, seed=seed)
    target = _perturbed(head, sigma, seed + 1)
    h, s0 = _inputs(head, D, seed=seed + 200)
    if kind == "sequential":
        t = O.sequential_best_first(head, h, s0, 1, D=D, k=k, B=B, beta=-0.2, T=1.0)
        tok, par, dep, n = t.tok, t.parent, t.depth, t.n
    else:
        W = 5
        tr = O.build_supertree(head, h, s0, 1, D=D, W=W, k=k, T=1.0)
        vt = O.prune_topB(tr.score, tr.parent, tr.n_valid, B, -0.2)
        n = vt.n
        tok = np.array([tr.tok[int(x) // W, int(x) % W] for x in vt.node[:n]], np.int64)
        par, dep = vt.parent[:n], vt.depth[:n]
    w = O.acceptance_walk(target, h, s0, 1, tok, par, dep, n, D, B)
    # independent formulation: the target decodes greedily from the root; tau
    # is 1 + the longest prefix of that continuation that is a root path
    g, _ = _greedy_chain(target, h, s0, 1, D)
    paths = {}
    for i in range(n):
        p, j = [], i
        while j >= 0:
            p.append(int(tok[j])); j = int(par[j])
        paths[tuple(reversed(p))] = i
    L = 0
    while L < D and tuple(g[:L + 1]) in paths:
        L += 1
    assert w.tau == L + 1
    assert [int(tok[i]) for i in w.path] == g[:L]
    assert [paths[tuple(g[:j + 1])] for j in range(L)] == w.path
    # target token of every node with children, from the state recomputed along
    # its token sequence
    kids = {int(p) for p in par}
    for i in range(n):
        if i not in kids:
            assert w.target_tok[i + 1] == -1
            continue
        seqtoks = [int(tok[x]) for x in _seq_ancestry(par, i)]
        s = _state_from_scratch(target, h, s0, 1, seqtoks)
        assert w.target_tok[i + 1] == int(np.argmax(target.logits(s[None])[0]))
    assert w.target_tok[0] == (g[0] if n else -1)
    assert np.all(w.target_tok[n + 1:] == -1)


def _seq_ancestry(par, i):
    out = []
    while i >= 0:
        out.append(i); i = int(par[i])
    return list(reversed(out))


def test_walk_edge_cases():
    head = tiny_head(V=9, d=6, seed=4)
    D, B = 3, 5
    h, s0 = _inputs(head, D)
    empty = O.acceptance_walk(head, h, s0, 2, [], [], [], 0, D, B)
    assert empty.tau == 1 and empty.path == [] and np.all(empty.target_tok == -1)
    g, _ = _greedy_chain(head, h, s0, 2, D)
    wrong = (g[0] + 1) % 9
    # a root child that is not the target's token stops the walk at once
    w = O.acceptance_walk(head, h, s0, 2, [wrong], [-1], [1], 1, D, B)
    assert w.tau == 1 and w.target_tok[0] == g[0] and w.target_tok[1] == -1
    # the matching child is found among siblings, whatever its position
    w = O.acceptance_walk(head, h, s0, 2, [wrong, g[0], g[1]], [-1, -1, 1], [1, 1, 2], 3, D, B)
    assert w.path == [1, 2] and w.tau == 3
    assert w.target_tok.tolist()[:3] == [g[0], -1, g[1]]


def test_walk_checker_accepts_the_oracle_and_rejects_planted_mistakes():
    from oracle import parity as P
    head = tiny_head(V=30, d=8, seed=5)
    target = _perturbed(head, 0.1, 9)
    D, k, B = 4, 3, 12
    h, s0 = _inputs(head, D, seed=6)
    t = O.sequential_best_first(head, h, s0, 2, D=D, k=k, B=B, beta=0.0, T=1.0)
    tree = dict(tok=t.tok, parent=t.parent, depth=t.depth, n=t.n)
    w = O.acceptance_walk(target, h, s0, 2, t.tok, t.parent, t.depth, t.n, D, B)
    assert w.tau >= 2          # the seed is chosen so that the walk goes somewhere
    path = np.array(w.path + [-1] * (D - len(w.path)))
    dev = dict(target_tok=w.target_tok.copy(), path=path, accept_len=[len(w.path)])
    assert P.check_walk(target, h, s0, 2, D, B, tree, dev, 1e-9).ok
    inner = [j for j in range(B + 1) if w.target_tok[j] >= 0]
    for mut in ("target", "leaf", "path", "len"):
        bad = {kk: np.array(v).copy() for kk, v in dev.items()}
        if mut == "target":
            bad["target_tok"][inner[-1]] = (bad["target_tok"][inner[-1]] + 1) % 30
        elif mut == "leaf":
            leaf = [j for j in range(1, t.n + 1) if w.target_tok[j] < 0][0]
            bad["target_tok"][leaf] = 0
        elif mut == "path":
            bad["path"][0] = (bad["path"][0] + 1) % t.n
        else:
            bad["accept_len"][0] += 1
        assert not P.check_walk(target, h, s0, 2, D, B, tree, bad, 1e-9).ok, mut


# ----------------------------------------------------------------------------
# deferred pruning (Lemma 1), ancestor closure, mask
# ----------------------------------------------------------------------------
def test_prune_and_mask_hand_examples():
    g = gold()["pool_prune_mask"]
    score = np.array(g["score"]); parent = np.array(g["parent"]); nv = np.array(g["n_valid"])
    for case in g["cases"]:
        vt = O.prune_topB(score, parent, nv, case["B"], case["beta"])
        assert vt.node.tolist() == case["node"]
        assert vt.parent.tolist() == case["sel_parent"]
        assert vt.depth.tolist() == case["depth"]
        B = case["B"]
        m = O.tree_mask(vt.parent, vt.n, B)
        assert m[:vt.n, 0].tolist() == case["mask"]
        assert np.all(m[vt.n:] == 0)


@st.composite
def pools(draw):
    D = draw(st.integers(1, 4))
    W = draw(st.integers(1, 4))
    integer = draw(st.booleans())
    score = np.full((D, W), -np.inf)
    parent = np.full((D, W), -1, np.int64)
    nv = np.zeros(D, np.int64)
    prev = 1
    for t in range(D):
        n = draw(st.integers(1, W)) if prev > 0 else 0
        nv[t] = n
        for j in range(n):
            p = draw(st.integers(0, prev - 1)) if t > 0 else -1
            base = 0.0 if t == 0 else score[t - 1, p]
            step = draw(st.integers(0, 3)) if integer else draw(
                st.floats(0, 3, allow_nan=False, allow_infinity=False))
            score[t, j] = base - step
            parent[t, j] = p
        prev = n
    return score, parent, nv


@given(pools(), st.integers(1, 20), st.sampled_from([0.0, -0.5, -1.0, -2.0]))
@settings(max_examples=400, deadline=None)
def test_lemma1_top_b_equals_best_first_heap(pool, B, beta):
    score, parent, nv = pool
    vt = O.prune_topB(score, parent, nv, B, beta)
    W = score.shape[1]
    got = {divmod(int(x), W) for x in vt.node}
    assert got == O.heap_prune(score, parent, nv, B, beta)
    assert vt.n == min(B, int(nv.sum()))
    # ancestor closed, emitted in (depth, slot) order, parents index earlier rows
    for i in range(vt.n):
        assert vt.parent[i] < i
        assert (vt.parent[i] == -1) == (vt.depth[i] == 1)
    assert list(vt.node) == sorted(vt.node)


def test_lemma1_needs_nonpositive_beta():
    # a deep node with a higher priority than a shallow one once beta > 0:
    # global top-B then picks a node whose parent it does not pick
    score = np.array([[-1.0, -1.05], [-1.1, -np.inf]])
    parent = np.array([[-1, -1], [1, -1]])
    nv = np.array([2, 1])
    beta = 1.0     # prios: (0,0) 0.0, (0,1) -0.05, (1,0) 0.9
    with pytest.raises(AssertionError):
        O.prune_topB(score, parent, nv, 1, beta)
    assert O.heap_prune(score, parent, nv, 1, beta) == {(0, 0)}


def test_mask_closed_forms():
    B = 70
    chain = np.arange(-1, B - 1)
    m = O.tree_mask(chain, B, B)
    vis = O.mask_to_bool(m, B)
    assert np.array_equal(vis, np.tril(np.ones((B, B), bool)))
    star = np.full(B, -1)
    assert np.array_equal(O.mask_to_bool(O.tree_mask(star, B, B), B), np.eye(B, dtype=bool))
    # popcount of a row = depth of the node
    g = np.random.default_rng(0)
    par = np.array([-1] + [int(g.integers(-1, i)) for i in range(1, B)])
    m = O.tree_mask(par, B, B)
    for i in range(B):
        dep, a = 0, i
        while a >= 0:
            dep += 1; a = par[a]
        assert sum(bin(int(w)).count("1") for w in m[i]) == dep


# ----------------------------------------------------------------------------
# tree attention
# ----------------------------------------------------------------------------
def _attn_inputs(n, P, Hq, Hkv, hd, seed=0):
    g = np.random.default_rng(seed)
    return (g.standard_normal((n, Hq, hd)), g.standard_normal((P, Hkv, hd)),
            g.standard_normal((P, Hkv, hd)), g.standard_normal((n, Hkv, hd)),
            g.standard_normal((n, Hkv, hd)))


def test_attention_star_tree_without_prefix_returns_own_value():
    n, Hq, Hkv, hd = 9, 4, 2, 8
    q, kp, vp, kt, vt = _attn_inputs(n, 0, Hq, Hkv, hd)
    m = O.tree_mask(np.full(n, -1), n, n)
    out = O.tree_attention(q, kp, vp, kt, vt, m, n, 0.3)
    for h in range(Hq):
        assert np.array_equal(out[:, h], vt[:, h // 2])


def test_attention_chain_is_causal_sdpa():
    n, P, Hq, Hkv, hd = 12, 0, 4, 4, 16
    q, kp, vp, kt, vt = _attn_inputs(n, P, Hq, Hkv, hd, seed=1)
    m = O.tree_mask(np.arange(-1, n - 1), n, n)
    out = O.tree_attention(q, kp, vp, kt, vt, m, n, 1 / 4)
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(kt).permute(1, 0, 2)
    tv = torch.from_numpy(vt).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=1 / 4)
    assert np.max(np.abs(out - ref.permute(1, 0, 2).numpy())) < 1e-12


def test_attention_prefix_and_tree_mask_match_sdpa_with_gqa():
    n, P, Hq, Hkv, hd = 10, 37, 8, 2, 16
    q, kp, vp, kt, vt = _attn_inputs(n, P, Hq, Hkv, hd, seed=2)
    g = np.random.default_rng(3)
    par = np.array([-1] + [int(g.integers(-1, i)) for i in range(1, n)])
    m = O.tree_mask(par, n, n)
    out = O.tree_attention(q, kp, vp, kt, vt, m, n, 0.17)
    vis = torch.from_numpy(np.concatenate([np.ones((n, P), bool), O.mask_to_bool(m, n)], 1))
    K = torch.from_numpy(np.concatenate([kp, kt], 0)).permute(1, 0, 2)
    Vv = torch.from_numpy(np.concatenate([vp, vt], 0)).permute(1, 0, 2)
    K = K.repeat_interleave(Hq // Hkv, 0)
    Vv = Vv.repeat_interleave(Hq // Hkv, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2), K, Vv, attn_mask=vis, scale=0.17)
    assert np.max(np.abs(out - ref.permute(1, 0, 2).numpy())) < 1e-12


# ----------------------------------------------------------------------------
# read-probe checksum
# ----------------------------------------------------------------------------
def test_word_sum64_closed_forms():
    # words 0 .. n-1: n (n - 1) / 2, reduced modulo 2^64 only by the definition
    n = 1_000_003
    assert O.word_sum64(np.arange(n, dtype=np.uint64)) == n * (n - 1) // 2 % 2 ** 64
    # all-ones bytes: n words of 2^64 - 1 sum to -n modulo 2^64
    assert O.word_sum64(b"\xff" * (8 * n)) == (-n) % 2 ** 64
    # large words wrap: 2^63 + 2^63 = 0
    assert O.word_sum64(np.array([2 ** 63, 2 ** 63], np.uint64)) == 0
    assert O.word_sum64(b"") == 0
    with pytest.raises(ValueError):
        O.word_sum64(b"\x00" * 12)


def test_word_sum64_byte_order_and_brute_force():
    # little-endian: byte j of a word weighs 256^j
    assert O.word_sum64(bytes([1, 2, 0, 0, 0, 0, 0, 0])) == 1 + 2 * 256
    assert O.word_sum64(bytes([0] * 7 + [1])) == 2 ** 56
    rng = np.random.default_rng(7)
    raw = rng.integers(0, 256, 8 * 1001, dtype=np.uint8).tobytes()
    want = 0
    for i in range(0, len(raw), 8):
        w = 0
        for j in range(8):
            w += raw[i + j] << (8 * j)
        want = (want + w) % 2 ** 64
    assert O.word_sum64(raw) == want
    # any dtype is read as its bytes
    assert O.word_sum64(np.frombuffer(raw, np.uint16)) == want


# ----------------------------------------------------------------------------
# entropy of the temperature softmax (the input calibration of the Qwen3-8B
# workload rests on it)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
def test_entropy_closed_forms(T):
    # uniform logits: log V nats at any temperature
    for V in (1, 2, 7, 1000):
        assert abs(O.entropy_T(np.zeros(V), T) - math.log(V)) < 1e-12
    # one token far above the rest: a point mass, 0 nats
    z = np.zeros(50)
    z[17] = 1e4
    assert abs(O.entropy_T(z, T)) < 1e-12
    # two tokens with probabilities p, 1 - p (logits log p, log(1 - p) at T = 1;
    # scaled by T so that z / T gives them): the binary entropy in nats
    for p in (0.5, 0.11, 0.9, 1e-3):
        z2 = T * np.array([math.log(p), math.log(1 - p)])
        want = -p * math.log(p) - (1 - p) * math.log(1 - p)
        assert abs(O.entropy_T(z2, T) - want) < 1e-12
    assert abs(O.entropy_T(np.array([0.0, 0.0]), T) - math.log(2)) < 1e-15


@pytest.mark.parametrize("T", [0.3, 0.7, 1.0, 1.7])
def test_entropy_matches_scipy_entr(T):
    g = np.random.default_rng(int(T * 10))
    for V in (3, 64, 5000):
        z = g.standard_normal(V) * 4.0
        want = float(np.sum(scipy.special.entr(scipy.special.softmax(z / T))))
        got = O.entropy_T(z, T)
        assert abs(got - want) < 1e-10 * max(1.0, want)
        assert 0.0 <= got <= math.log(V) + 1e-12
    # masked (-inf) logits contribute nothing
    z = np.array([1.0, -np.inf, 2.0, -np.inf])
    want = float(np.sum(scipy.special.entr(scipy.special.softmax(np.array([1.0, 2.0]) / T))))
    assert abs(O.entropy_T(z, T) - want) < 1e-12


def test_calibrated_scale_is_the_recorded_one():
    # the workload generator uses the scale the calibration script recorded
    from draft_tree_construction_02_amd import synth
    rec = json.load(open(os.path.join(os.path.dirname(GOLD), "h_scale_qwen3_8b.json")))
    assert synth.H_SCALE_QWEN3_8B == rec["alpha"]
    assert abs(rec["mean_entropy_nats"] - 2.0) <= 0.05
    assert synth.workloads()["qwen3_8b"].h_scale == rec["alpha"]


# ----------------------------------------------------------------------------
# the parity checkers: each accepts the oracle's own output and rejects a
# planted mistake in every failure branch (the message names the branch)
# ----------------------------------------------------------------------------
def _plain_case(T=1.0, seed=3):
    head = tiny_head(V=50, d=8, seed=seed)
    h, s0 = _inputs(head, 5, seed=21)
    t = O.build_supertree(head, h, s0, 3, D=5, W=6, k=3, T=T)
    return head, h, s0, t


def _dev(t):
    return dict(tok=t.tok.copy(), parent=t.parent.copy(), score=t.score.copy(),
                n_valid=t.n_valid.copy())


def _parent_logp(head, h, s0, root, tree, t, j, T=1.0):
    """scipy log-softmax of the row that produced pool node (t, j): the path
    of tokens from the root to its parent replayed through the state update."""
    path, tt, jj = [], t - 1, int(tree.parent[t, j]) if t > 0 else -1
    while tt >= 0:
        path.append(int(tree.tok[tt, jj]))
        jj = int(tree.parent[tt, jj])
        tt -= 1
    toks = [root] + path[::-1]
    s = np.asarray(s0, np.float64)[None]
    for d, c in enumerate(toks):
        s = O.state_update(head, s, [c], h[d])
    return scipy.special.log_softmax(head.logits(s)[0] / T)


def _build_fails(head, h, s0, dev, T=1.0, tol=1e-9, tau=1e-9, D=5, W=6, k=3):
    from oracle import parity as P
    rep = P.check_build(head, h, s0, 3, D, W, k, T, dev, tol, tau)
    return rep


def _has(rep_or_list, text):
    msgs = rep_or_list.failures if hasattr(rep_or_list, "failures") else rep_or_list
    return any(text in m for m in msgs)


def test_check_build_accepts_the_oracle_and_counts_no_exemption():
    for T in (1.0, 0.0):
        head, h, s0, t = _plain_case(T)
        rep = _build_fails(head, h, s0, _dev(t), T)
        assert rep.ok and rep.exemptions == 0, rep.failures
        assert rep.max_score_err == 0.0
        fin = np.isfinite(t.score)
        assert np.array_equal(np.isfinite(rep.forced_score), fin)
        assert np.array_equal(rep.forced_score[fin], t.score[fin])


def test_check_build_rejects_planted_mistakes():
    head, h, s0, t = _plain_case()
    D, W = 5, 6
    last, n_last = D - 1, int(t.n_valid[D - 1])
    assert t.n_valid.tolist()[:2] == [3, 6] and n_last == W

    # a token that is not among its parent's top-3 children, with the score it
    # would have (parent score + its log-probability)
    dev = _dev(t)
    j = n_last - 1
    lp = _parent_logp(head, h, s0, 3, t, last, j)
    c = int(np.argsort(-lp, kind="stable")[9])
    dev["tok"][last, j] = c
    dev["score"][last, j] = t.score[last - 1, t.parent[last, j]] + lp[c]
    assert _has(_build_fails(head, h, s0, dev), "not a top-3 child")

    # a score off by more than the tolerance
    dev = _dev(t)
    dev["score"][2, 1] += 1e-6
    assert _has(_build_fails(head, h, s0, dev), "vs oracle")

    # two slots of the last depth in the wrong order
    dev = _dev(t)
    for key in ("tok", "parent", "score"):
        dev[key][last, [0, 1]] = dev[key][last, [1, 0]]
    assert _has(_build_fails(head, h, s0, dev), "out of order")
    # ... accepted, and counted, when the gap is within tau
    rep = _build_fails(head, h, s0, dev, tau=10.0)
    assert rep.ok and rep.exemptions >= 1

    # an unused slot that is not padded (depth 1 holds 3 of 6 slots)
    dev = _dev(t)
    dev["tok"][0, 4] = 5
    assert _has(_build_fails(head, h, s0, dev), "not padded")
    dev = _dev(t)
    dev["score"][0, 5] = -1.0
    assert _has(_build_fails(head, h, s0, dev), "not padded")

    # a wrong width
    dev = _dev(t)
    dev["n_valid"][2] = 5
    assert _has(_build_fails(head, h, s0, dev), "n_valid")

    # a depth-1 node with a parent slot
    dev = _dev(t)
    dev["parent"][0, 1] = 0
    assert _has(_build_fails(head, h, s0, dev), "parent 0 != -1")

    # a parent slot outside the previous depth
    dev = _dev(t)
    dev["parent"][2, 0] = 99
    assert _has(_build_fails(head, h, s0, dev), "bad parent/token")

    # the same child kept twice
    dev = _dev(t)
    for key in ("tok", "parent", "score"):
        dev[key][last, n_last - 1] = dev[key][last, n_last - 2]
    assert _has(_build_fails(head, h, s0, dev), "duplicate child")

    # the last kept node swapped for the best rejected top-3 candidate: every
    # slot is a valid child with its own score, but the kept set is not a top-6
    dev = _dev(t)
    kept = {(int(t.parent[last, q]), int(t.tok[last, q])) for q in range(n_last)}
    best = None
    for p in range(int(t.n_valid[last - 1])):
        # the row of frontier slot p at the last depth: replay its path + itself
        row = _row_logp(head, h, s0, 3, t, last - 1, p)
        for c in np.argsort(-row, kind="stable")[:3]:
            if (p, int(c)) not in kept:
                sc = t.score[last - 1, p] + row[c]
                if best is None or sc > best[0]:
                    best = (sc, p, int(c))
    assert best is not None and best[0] < t.score[last, n_last - 1] - 1e-6
    dev["tok"][last, n_last - 1] = best[2]
    dev["parent"][last, n_last - 1] = best[1]
    dev["score"][last, n_last - 1] = best[0]
    rep = _build_fails(head, h, s0, dev)
    assert _has(rep, "kept set not a top-6"), rep.failures


def _row_logp(head, h, s0, root, tree, t, j, T=1.0):
    """scipy log-softmax of the row of pool node (t, j) one depth later (the
    row whose children form depth t + 1)."""
    path, tt, jj = [], t, j
    while tt >= 0:
        path.append(int(tree.tok[tt, jj]))
        jj = int(tree.parent[tt, jj])
        tt -= 1
    toks = [root] + path[::-1]
    s = np.asarray(s0, np.float64)[None]
    for d, c in enumerate(toks):
        s = O.state_update(head, s, [c], h[d])
    return scipy.special.log_softmax(head.logits(s)[0] / T)


def test_check_build_rejects_a_wrong_exact_tie_break_and_a_wrong_argmax():
    from oracle import parity as P
    # exact ties (the survivor tie-break setting): (parent 0, b) and (parent 1,
    # a) score l0 + l1 exactly; slots 1 and 2 of depth 2 swapped
    V, d = 9, 4
    Ut = np.random.default_rng(0).standard_normal((V, d)).astype(np.float32)
    head = O.OracleHead("f32", np.zeros((V, d), np.float32), np.zeros((4 * d, d), np.float32),
                        np.zeros((d, 4 * d), np.float32), Ut)
    s0, h = np.ones(d), np.zeros((2, d))
    t = O.build_supertree(head, h, s0, 0, D=2, W=6, k=3, T=1.0)
    dev = _dev(t)
    assert P.check_build(head, h, s0, 0, 2, 6, 3, 1.0, dev, 1e-9, 1e-9).ok
    for key in ("tok", "parent", "score"):
        dev[key][1, [1, 2]] = dev[key][1, [2, 1]]
    rep = P.check_build(head, h, s0, 0, 2, 6, 3, 1.0, dev, 1e-9, 1e-9)
    assert _has(rep, "broken wrongly"), rep.failures
    # greedy limit: a child that is not the argmax of its row
    head, h, s0, t = _plain_case(T=0.0)
    dev = _dev(t)
    lp = _parent_logp(head, h, s0, 3, t, 4, 0)
    dev["tok"][4, 0] = int(np.argsort(-lp, kind="stable")[1])
    assert _has(_build_fails(head, h, s0, dev, T=0.0), "not argmax")


def _prune_case(B=10, beta=-0.3):
    from oracle import parity as P
    head, h, s0, t = _plain_case()
    forced = P.check_build(head, h, s0, 3, 5, 6, 3, 1.0, _dev(t), 1e-9, 1e-9).forced_score
    vt = O.prune_topB(t.score, t.parent, t.n_valid, B, beta)

    def pad(a):
        out = np.full(B, -1, np.int64)
        out[:len(a)] = a
        return out
    sel = dict(node=pad(vt.node), parent=pad(vt.parent), depth=pad(vt.depth), n=vt.n)
    return t, forced, vt, sel


def _sel_from_nodes(t, nodes, B):
    """A verification tree emitting the given (t, j) set in (depth, slot)
    order, parents remapped (-1 where the parent is not in the set)."""
    chosen = sorted(nodes)
    index = {c: i for i, c in enumerate(chosen)}
    W = t.tok.shape[1]
    node = np.full(B, -1, np.int64); par = np.full(B, -1, np.int64); dep = np.full(B, -1, np.int64)
    for i, (tt, j) in enumerate(chosen):
        node[i] = tt * W + j
        dep[i] = tt + 1
        par[i] = index.get((tt - 1, int(t.parent[tt, j])), -1) if tt > 0 else -1
    return dict(node=node, parent=par, depth=dep, n=len(chosen))


def test_check_prune_accepts_the_oracle_and_rejects_planted_mistakes():
    from oracle import parity as P
    B, beta = 10, -0.3
    t, forced, vt, sel = _prune_case(B, beta)

    def run(s):
        return P.check_prune(forced, t.parent, t.n_valid, B, beta, s, 1e-9)

    assert run(sel).ok and run(sel).exemptions == 0
    W = t.tok.shape[1]
    chosen = {divmod(int(x), W) for x in vt.node}

    bad = {kk: (np.array(v).copy() if kk != "n" else v) for kk, v in sel.items()}
    bad["n"] = vt.n - 1
    assert _has(run(bad), "n_sel")

    i = int(np.nonzero(vt.parent > 0)[0][0])
    bad = {kk: (np.array(v).copy() if kk != "n" else v) for kk, v in sel.items()}
    bad["parent"][i] -= 1
    assert _has(run(bad), "parent index")

    bad = {kk: (np.array(v).copy() if kk != "n" else v) for kk, v in sel.items()}
    bad["depth"][i] += 1
    assert _has(run(bad), "depth")

    bad = {kk: (np.array(v).copy() if kk != "n" else v) for kk, v in sel.items()}
    bad["node"][[0, 1]] = bad["node"][[1, 0]]
    assert _has(run(bad), "order")

    # a budget above the pool (27 nodes) leaves padding to plant in
    tp, fp, vp, sp = _prune_case(30, beta)
    assert vp.n == 27
    assert P.check_prune(fp, tp.parent, tp.n_valid, 30, beta, sp, 1e-9).ok
    for key in ("node", "parent", "depth"):
        bad = {kk: (np.array(v).copy() if kk != "n" else v) for kk, v in sp.items()}
        bad[key][vp.n] = 0
        assert _has(P.check_prune(fp, tp.parent, tp.n_valid, 30, beta, bad, 1e-9), "padded")

    # not ancestor-closed: a selected parent dropped, the best unselected node added
    nodes = [(tt, j) for tt in range(5) for j in range(int(t.n_valid[tt]))]
    prio = {c: t.score[c] + beta * (c[0] + 1) for c in nodes}
    deep = max(c for c in chosen if c[0] > 0)
    par = (deep[0] - 1, int(t.parent[deep]))
    out = [c for c in nodes if c not in chosen]
    add = max(out, key=lambda c: prio[c])
    rep = run(_sel_from_nodes(t, (chosen - {par}) | {add}, B))
    assert _has(rep, "not ancestor-closed"), rep.failures

    # closed but not a top-B: a selected leaf swapped for a worse node whose
    # parent is selected
    kids = {(c[0] - 1, int(t.parent[c])) for c in chosen if c[0] > 0}
    leaf = min((c for c in chosen if c not in kids), key=lambda c: prio[c])
    worse = [c for c in out if (c[0] == 0 or (c[0] - 1, int(t.parent[c])) in chosen)
             and prio[c] < prio[leaf] - 1e-6]
    swap = max(worse, key=lambda c: prio[c])
    rep = run(_sel_from_nodes(t, (chosen - {leaf}) | {swap}, B))
    assert rep.failures == [f for f in rep.failures if "not a top-" in f] and rep.failures

    # an exact priority tie at the boundary goes to the lower slot
    score = np.array([[-1.0, -1.0, -1.0]]); par0 = np.full((1, 3), -1); nv = np.array([3])
    good = dict(node=np.array([0, 1]), parent=np.array([-1, -1]), depth=np.array([1, 1]), n=2)
    wrong = dict(node=np.array([0, 2]), parent=np.array([-1, -1]), depth=np.array([1, 1]), n=2)
    assert P.check_prune(score, par0, nv, 2, 0.0, good, 1e-9).ok
    assert _has(P.check_prune(score, par0, nv, 2, 0.0, wrong, 1e-9), "broken wrongly")


def test_check_mask_and_compare_exact_reject_planted_mistakes():
    from oracle import parity as P
    B = 30
    t, _, vt, sel = _prune_case(B)
    mask = O.tree_mask(vt.parent, vt.n, B)
    assert P.check_mask(sel["parent"], vt.n, B, mask) == []
    bad = mask.copy(); bad[3, 0] ^= np.uint32(1 << 1)
    assert P.check_mask(sel["parent"], vt.n, B, bad)
    bad = mask.copy(); bad[B - 1, 0] = 1          # a row past n_sel must stay empty
    assert vt.n < B and P.check_mask(sel["parent"], vt.n, B, bad)

    assert P.compare_exact(t, _dev(t), 1e-9) == []
    checks = {"tok": "tokens differ", "parent": "parents differ", "n_valid": "n_valid differs",
              "score": "scores differ", "pattern": "valid-score pattern"}
    for what, msg in checks.items():
        dev = _dev(t)
        if what == "tok":
            dev["tok"][3, 2] += 1
        elif what == "parent":
            dev["parent"][3, 2] = (dev["parent"][3, 2] + 1) % 6
        elif what == "n_valid":
            dev["n_valid"][1] -= 1
        elif what == "score":
            dev["score"][2, 2] += 3e-9
        else:
            dev["score"][4, 5] = -np.inf
        got = P.compare_exact(t, dev, 1e-9)
        assert any(msg in m for m in got), (what, got)


def test_sampled_checkers_accept_the_oracle_and_reject_planted_mistakes():
    from oracle import sampled as S
    head, h, s0, t = _plain_case()
    D, W, k = 5, 6, 3
    paths = S.sample_paths(t.tok, t.parent, t.n_valid, 1, seed=0)
    fails, st = S.check_paths(head, h, s0, 3, k, 1.0, _dev(t), 1e-9, 1e-9, paths)
    assert fails == [] and st["exemptions"] == 0
    assert S.check_structure(t.tok, t.parent, t.score, t.n_valid, W, k, 50, 1.0) == []
    last = D - 1

    # a sampled end node (slot 0 of the last depth) given a non-top-3 token
    dev = _dev(t)
    lp = _parent_logp(head, h, s0, 3, t, last, 0)
    c = int(np.argsort(-lp, kind="stable")[9])
    dev["tok"][last, 0] = c
    dev["score"][last, 0] = t.score[last - 1, t.parent[last, 0]] + lp[c]
    f, _ = S.check_paths(head, h, s0, 3, k, 1.0, dev, 1e-9, 1e-9, paths)
    assert _has(f, "not a top-3 child")

    dev = _dev(t)
    dev["score"][last, 0] += 1e-6
    f, _ = S.check_paths(head, h, s0, 3, k, 1.0, dev, 1e-9, 1e-9, paths)
    assert _has(f, "vs oracle")

    # a sampled last-depth node replaced by a worse unkept sibling: its parent's
    # better child is then dropped although it beats the worst kept node
    kept = {(int(t.parent[last, q]), int(t.tok[last, q])) for q in range(int(t.n_valid[last]))}
    ends = [p[-1] for p in paths if p[-1][0] == last]
    planted = False
    for (_, j) in ends:
        p = int(t.parent[last, j])
        row = _row_logp(head, h, s0, 3, t, last - 1, p)
        for c in np.argsort(-row, kind="stable")[:k]:
            sc = t.score[last - 1, p] + row[c]
            if (p, int(c)) not in kept and sc < t.score[last, j] - 1e-6:
                dev = _dev(t)
                dev["tok"][last, j] = int(c)
                dev["score"][last, j] = sc
                f, _ = S.check_paths(head, h, s0, 3, k, 1.0, dev, 1e-9, 1e-9, paths)
                assert _has(f, "dropped child"), f
                planted = True
                break
        if planted:
            break
    assert planted

    # depth 1 (the root's children) kept in another order
    dev = _dev(t)
    for key in ("tok", "score"):
        dev[key][0, [0, 1]] = dev[key][0, [1, 0]]
    f, _ = S.check_paths(head, h, s0, 3, k, 1.0, dev, 1e-9, 1e-9, paths)
    assert _has(f, "depth 1 kept")


def test_check_structure_rejects_planted_mistakes():
    from oracle import sampled as S
    _, _, _, t = _plain_case()
    W, k, V = 6, 3, 50
    cases = {
        "n_valid": lambda d: d["n_valid"].__setitem__(2, 5),
        "not non-increasing": lambda d: d["score"].__setitem__((2, 1), d["score"][2, 0] + 1.0),
        "invalid score": lambda d: d["score"].__setitem__((0, 0), 0.5),
        "token out of range": lambda d: d["tok"].__setitem__((3, 1), V),
        "depth 1 parents": lambda d: d["parent"].__setitem__((0, 2), 0),
        "parent out of range": lambda d: d["parent"].__setitem__((3, 1), 6),
        "duplicate children": lambda d: (d["parent"].__setitem__((4, 5), d["parent"][4, 4]),
                                         d["tok"].__setitem__((4, 5), d["tok"][4, 4])),
        "padding": lambda d: d["tok"].__setitem__((0, 3), 0),
    }
    for msg, plant in cases.items():
        dev = _dev(t)
        plant(dev)
        got = S.check_structure(dev["tok"], dev["parent"], dev["score"], dev["n_valid"], W, k, V,
                                1.0)
        assert any(msg in m for m in got), (msg, got)
    # a child scored above its parent: the scores of depth 2 raised above
    # depth 1 (kept in order)
    dev = _dev(t)
    dev["score"][1, :] = 0.0
    got = S.check_structure(dev["tok"], dev["parent"], dev["score"], dev["n_valid"], W, k, V, 1.0)
    assert any("above parent" in m for m in got), got
    # greedy limit: every score is 0
    _, _, _, t0 = _plain_case(T=0.0)
    assert S.check_structure(t0.tok, t0.parent, t0.score, t0.n_valid, W, k, V, 0.0) == []
    dev = _dev(t0)
    dev["score"][2, 0] = -0.5
    got = S.check_structure(dev["tok"], dev["parent"], dev["score"], dev["n_valid"], W, k, V, 0.0)
    assert any("greedy scores not 0" in m for m in got), got


def test_full_check_accepts_the_oracle_and_rejects_a_planted_mistake():
    # the whole-request check the GPU tests run, fed the oracle's own build,
    # top-B and mask in the device's storage types ([R][D][W] int32 / float32)
    from draft_tree_construction_02_amd import synth
    from tests.gpu_util import full_check, oracle_head
    wl = synth.Workload("cpu_full_check", V=300, d=128, wdtype="bf16", D=4, W=6, k=3, B=10,
                        beta=-0.05, T=1.0, R=2, seeds=(5, 6))
    hw, req = synth.make_workload_inputs(wl)
    ohead = oracle_head(hw)
    pool = dict(pool_tok=[], pool_parent=[], pool_score=[], n_valid=[])
    sel = dict(sel_node=[], sel_parent=[], sel_depth=[], n_sel=[])
    masks = []
    for r in range(wl.R):
        t = O.build_supertree(ohead, req.h[r], req.s0[r], int(req.root_tok[r]), wl.D, wl.W,
                              wl.k, wl.T)
        vt = O.prune_topB(t.score, t.parent, t.n_valid, wl.B, wl.beta)
        pool["pool_tok"].append(t.tok); pool["pool_parent"].append(t.parent)
        pool["pool_score"].append(t.score); pool["n_valid"].append(t.n_valid)

        def pad(a):
            o = np.full(wl.B, -1, np.int32)
            o[:vt.n] = a
            return o
        sel["sel_node"].append(pad(vt.node)); sel["sel_parent"].append(pad(vt.parent))
        sel["sel_depth"].append(pad(vt.depth)); sel["n_sel"].append(vt.n)
        masks.append(O.tree_mask(vt.parent, vt.n, wl.B))
    pool = {kk: np.stack(v).astype(np.float32 if kk == "pool_score" else np.int32)
            for kk, v in pool.items()}
    sel = {kk: np.array(v, np.int32) for kk, v in sel.items()}
    mask = np.stack(masks)
    for r in range(wl.R):
        st = full_check(ohead, req, r, wl, pool, sel, mask)
        assert st["exact"] and st["exemptions"] == 0 and st["max_score_err"] < 1e-6
        assert st["n_sel"] == wl.B
    bad = mask.copy()
    bad[1, 4, 0] ^= np.uint32(1)
    with pytest.raises(AssertionError):
        full_check(ohead, req, 1, wl, pool, sel, bad)
    badsel = {kk: v.copy() for kk, v in sel.items()}
    badsel["sel_parent"][0, 5] = -1 if badsel["sel_parent"][0, 5] >= 0 else 0
    with pytest.raises(AssertionError):
        full_check(ohead, req, 0, wl, pool, badsel, mask)
