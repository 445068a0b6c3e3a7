"""Teacher-forced parity checks of a device-built supertree against the oracle.

TEST INFRASTRUCTURE ONLY (see ``dartree_oracle``).  The device's outputs are
treated as a claimed answer: the checker follows the device's tokens and parent
pointers, recomputes every state, log-probability and score along those paths
in fp64 with the oracle, and checks that every choice the device made is a
valid one.  A choice that differs from the oracle's own preference is accepted
("exempted") only when the fp64 score gap it depends on is at most ``tau``;
the number of exemptions is reported.  With zero exemptions the device's tree
must equal the oracle's independent build exactly.

No floating-point value computed by the device is ever fed to the oracle: only
its discrete choices (tokens, parent slots, selected nodes) are followed.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import dartree_oracle as O


@dataclass
class Report:
    exemptions: int = 0
    max_score_err: float = 0.0
    failures: list = field(default_factory=list)
    notes: list = field(default_factory=list)
    # oracle scores along the device paths, [D][W] (-inf where invalid)
    forced_score: np.ndarray | None = None

    def fail(self, msg):
        self.failures.append(msg)

    @property
    def ok(self):
        return not self.failures


def check_build(head, h, s0, root_tok, D, W, k, T, dev, tol, tau,
                report: Report | None = None, markov: bool = False,
                base_cand: int = 0) -> Report:
    """Check one request's scored pool.

    dev: dict with 'tok', 'parent', 'score' ([D][W]) and 'n_valid' ([D]).
    markov / base_cand select the build variants of ``build_supertree``
    (base_cand is its n_cand).
    """
    rep = report or Report()
    V = head.V
    tok = np.asarray(dev["tok"]); par = np.asarray(dev["parent"])
    sco = np.asarray(dev["score"], np.float64); nv = np.asarray(dev["n_valid"])
    forced = np.full((D, W), -math.inf)
    f_state = np.asarray(s0, np.float64)[None, :]
    f_tok = np.array([root_tok], np.int64)
    f_score = np.array([0.0])
    for t in range(D):
        src = np.repeat(np.asarray(s0, np.float64)[None, :], f_tok.size, 0) if markov else f_state
        s_new = O.state_update(head, src, f_tok, h[t])
        z = head.logits(s_new)
        n_prev = z.shape[0]
        cand_t = O.base_candidates(head, h[t], base_cand) if base_cand > 0 else None
        lps, kids = [], []
        for i in range(n_prev):
            lp = O.log_softmax_T(z[i], T)
            lps.append(lp)
            kids.append(O.topk_children(lp, k) if cand_t is None
                        else O.restricted_children(z[i], lp, cand_t, k, T))
        n_cand = sum(kt.size for kt, _ in kids)
        n_exp = min(W, n_cand)
        if int(nv[t]) != n_exp:
            rep.fail(f"depth {t + 1}: n_valid {int(nv[t])} != {n_exp}")
            return rep
        n = n_exp
        seen = set()
        ps, cs, os_ = [], [], []
        for j in range(n):
            p = 0 if t == 0 else int(par[t, j])
            c = int(tok[t, j])
            if t == 0 and int(par[t, j]) != -1:
                rep.fail(f"depth 1 slot {j}: parent {int(par[t, j])} != -1")
            if not (0 <= p < n_prev) or not (0 <= c < V):
                rep.fail(f"depth {t + 1} slot {j}: bad parent/token ({p}, {c})")
                return rep
            if (p, c) in seen:
                rep.fail(f"depth {t + 1} slot {j}: duplicate child ({p}, {c})")
            seen.add((p, c))
            if cand_t is not None and c not in set(cand_t.tolist()):
                rep.fail(f"depth {t + 1} slot {j}: token {c} is not a base-logit candidate")
                return rep
            ktoks, klps = kids[p]
            if T == 0.0:
                # greedy limit: the child must be the argmax up to tau in logit
                a = int(ktoks[0])
                if c != a:
                    gap = float(z[p, a] - z[p, c])
                    if gap <= tau:
                        rep.exemptions += 1
                    else:
                        rep.fail(f"depth {t + 1} slot {j}: token {c} not argmax {a} (gap {gap:.3g})")
                lpc = 0.0
            else:
                lpc = float(lps[p][c])
                if c not in set(ktoks.tolist()):
                    gap = float(klps[-1] - lpc)
                    if gap <= tau:
                        rep.exemptions += 1
                    else:
                        rep.fail(f"depth {t + 1} slot {j}: token {c} not a top-{k} child "
                                 f"of slot {p} (gap {gap:.3g})")
            o = float(f_score[p]) + lpc
            err = abs(float(sco[t, j]) - o)
            rep.max_score_err = max(rep.max_score_err, err)
            if not err <= tol:
                rep.fail(f"depth {t + 1} slot {j}: score {float(sco[t, j]):.7g} vs oracle {o:.7g}")
            ps.append(p); cs.append(c); os_.append(o)
            forced[t, j] = o
        for j in range(n, W):
            if int(tok[t, j]) != -1 or int(par[t, j]) != -1 or not (sco[t, j] == -math.inf):
                rep.fail(f"depth {t + 1} slot {j}: invalid slot not padded")
        # the kept set is a valid top-n of the oracle candidates
        if n < n_cand:
            rejected = [float(f_score[i]) + float(lp) for i in range(n_prev)
                        for c, lp in zip(*kids[i]) if (i, int(c)) not in seen]
            if rejected:
                gap = min(os_) - max(rejected)
                if gap < 0:
                    if gap >= -tau:
                        rep.exemptions += 1
                    else:
                        rep.fail(f"depth {t + 1}: kept set not a top-{n} (gap {gap:.3g})")
        # slots in non-increasing score order; exact ties follow (parent, rank)
        for j in range(1, n):
            dlt = os_[j] - os_[j - 1]
            if dlt > 0:
                if dlt <= tau:
                    rep.exemptions += 1
                else:
                    rep.fail(f"depth {t + 1}: slots {j - 1},{j} out of order ({dlt:.3g})")
            elif dlt == 0 and T > 0.0:
                r0 = list(kids[ps[j - 1]][0]).index(cs[j - 1]) if cs[j - 1] in kids[ps[j - 1]][0] else k
                r1 = list(kids[ps[j]][0]).index(cs[j]) if cs[j] in kids[ps[j]][0] else k
                if (ps[j - 1], r0) > (ps[j], r1):
                    rep.fail(f"depth {t + 1}: exact tie at slots {j - 1},{j} broken wrongly")
        f_state = s_new[ps]
        f_tok = np.array(cs, np.int64)
        f_score = np.array(os_)
    rep.forced_score = forced
    return rep


def check_prune(forced_score, pool_parent, n_valid, B, beta, sel, tau,
                report: Report | None = None) -> Report:
    """Check a device verification tree against oracle priorities.

    forced_score: oracle scores along the device pool ([D][W]).
    sel: dict with 'node', 'parent', 'depth' ([B], -1 padded) and 'n' (int).
    """
    rep = report or Report()
    D, W = forced_score.shape
    nodes = [(t, j) for t in range(D) for j in range(int(n_valid[t]))]
    m = min(B, len(nodes))
    n = int(sel["n"])
    if n != m:
        rep.fail(f"n_sel {n} != {m}")
        return rep
    node = np.asarray(sel["node"]); spar = np.asarray(sel["parent"]); sdep = np.asarray(sel["depth"])
    chosen = [divmod(int(x), W) for x in node[:n]]
    for i, (t, j) in enumerate(chosen):
        if not (0 <= t < D and 0 <= j < int(n_valid[t])):
            rep.fail(f"sel {i}: node {(t, j)} not a valid pool node")
            return rep
        if int(sdep[i]) != t + 1:
            rep.fail(f"sel {i}: depth {int(sdep[i])} != {t + 1}")
    if chosen != sorted(set(chosen)):
        rep.fail("selected nodes not emitted in (depth, slot) order / duplicated")
        return rep
    index = {c: i for i, c in enumerate(chosen)}
    for i, (t, j) in enumerate(chosen):
        want = -1 if t == 0 else index.get((t - 1, int(pool_parent[t, j])), None)
        if want is None:
            rep.fail(f"sel {i}: parent of {(t, j)} not selected (not ancestor-closed)")
        elif int(spar[i]) != want:
            rep.fail(f"sel {i}: parent index {int(spar[i])} != {want}")
    for arr, name in ((node, "node"), (spar, "parent"), (sdep, "depth")):
        if np.any(np.asarray(arr[n:]) != -1):
            rep.fail(f"sel {name} not -1 padded")
    prio = {c: float(forced_score[c]) + beta * (c[0] + 1) for c in nodes}
    cset = set(chosen)
    rest = [prio[c] for c in nodes if c not in cset]
    if rest and chosen:
        gap = min(prio[c] for c in chosen) - max(rest)
        if gap < 0:
            if gap >= -tau:
                rep.exemptions += 1
            else:
                rep.fail(f"selection not a top-{m} under oracle priorities (gap {gap:.3g})")
        elif gap == 0:
            lo = min(prio[c] for c in chosen)
            worst_in = max(c for c in chosen if prio[c] == lo)
            best_out = min(c for c in nodes if c not in cset and prio[c] == lo)
            if best_out < worst_in:
                rep.fail("exact prio tie at the top-B boundary broken wrongly")
    return rep


def check_mask(sel_parent, n, B, mask) -> list:
    """The device bitmask must equal the ancestor closure of its own tree."""
    want = O.tree_mask(np.asarray(sel_parent), int(n), B)
    got = np.asarray(mask, np.uint32).reshape(want.shape)
    bad = np.argwhere(got != want)
    return [f"mask row {int(r)} word {int(w)}: {int(got[r, w]):#x} != {int(want[r, w]):#x}"
            for r, w in bad[:10]]


def compare_exact(ora: O.Supertree, dev, tol) -> list:
    """With no exemptions the device pool must equal the oracle's own build."""
    out = []
    if not np.array_equal(np.asarray(dev["n_valid"]), ora.n_valid):
        out.append("n_valid differs from the oracle build")
    if not np.array_equal(np.asarray(dev["tok"]), ora.tok):
        out.append("tokens differ from the oracle build")
    if not np.array_equal(np.asarray(dev["parent"]), ora.parent):
        out.append("parents differ from the oracle build")
    fin = np.isfinite(ora.score)
    if not np.array_equal(np.isfinite(np.asarray(dev["score"], np.float64)), fin):
        out.append("valid-score pattern differs from the oracle build")
    elif fin.any():
        err = np.max(np.abs(np.asarray(dev["score"], np.float64)[fin] - ora.score[fin]))
        if not err <= tol:
            out.append(f"scores differ from the oracle build by {err:.3g}")
    return out


def check_sequential(head, h, s0, root_tok, D, k, B, beta, T, dev, tol, tau) -> Report:
    """Teacher-forced check of a device-built sequential best-first tree.

    dev: dict of tok, parent, depth, score ([B], pop order) and n.  The
    oracle replays the heap along the device's pops: each popped node must be
    a candidate (a top-k child of its parent in fp64, or within tau of the
    k-th child), its fp64 priority must be within tau of the best candidate
    left, its score within tol of the fp64 path score, and every expansion
    the device performs is repeated in fp64 from the device's token path.
    """
    rep = Report()
    n = int(np.asarray(dev["n"]).reshape(-1)[0])
    tok = np.asarray(dev["tok"]); par = np.asarray(dev["parent"])
    dep = np.asarray(dev["depth"]); sco = np.asarray(dev["score"], np.float64)
    cand = {}          # (parent index, token) -> (score, depth)
    row_lp = {}        # parent index -> (full logp row, top-k tokens, its state)
    states = {}

    def expand(idx, state, t, depth, score):
        s_new = O.state_update(head, np.asarray(state, np.float64)[None, :], [int(t)],
                               h[depth])[0]
        lp = O.log_softmax_T(head.logits(s_new[None, :])[0], T)
        toks, lps = O.topk_children(lp, k)
        row_lp[idx] = (lp, set(int(x) for x in toks), float(lps[-1]) if lps.size else -math.inf,
                       score)
        states[idx] = s_new
        for c, l in zip(toks.tolist(), lps.tolist()):
            cand[(idx, int(c))] = (score + l, depth + 1)

    expand(-1, s0, root_tok, 0, 0.0)
    for i in range(n):
        key = (int(par[i]), int(tok[i]))
        if key[0] not in row_lp:
            rep.fail(f"pop {i}: parent {key[0]} was never expanded")
            return rep
        if key not in cand:
            lp, top, kth, psc = row_lp[key[0]]
            c = key[1]
            gap = kth - float(lp[c]) if 0 <= c < lp.size else math.inf
            if T > 0.0 and gap <= tau:
                rep.exemptions += 1
                cand[key] = (psc + float(lp[c]), int(dep[i]))
            else:
                rep.fail(f"pop {i}: token {c} is not a child of entry {key[0]} (gap {gap:.3g})")
                return rep
        sc, d = cand[key]
        if d != int(dep[i]):
            rep.fail(f"pop {i}: depth {dep[i]} != {d}")
        err = abs(float(sco[i]) - sc)
        rep.max_score_err = max(rep.max_score_err, err)
        if not err <= tol:
            rep.fail(f"pop {i}: score {sco[i]:.7g} vs oracle {sc:.7g}")
        prio = sc + beta * d
        best = max(v[0] + beta * v[1] for v in cand.values())
        if best - prio > tau:
            rep.fail(f"pop {i}: priority {prio:.6g} below the best candidate {best:.6g}")
        elif best - prio > 0.0:
            rep.exemptions += 1
        del cand[key]
        if i + 1 < B and d < D:
            # the node carries its parent's updated state (the root's for depth 1)
            expand(i, states[key[0]], key[1], d, sc)
    if n < B and cand:
        rep.fail(f"device stopped after {n} pops with {len(cand)} candidates left")
    if n > B:
        rep.fail(f"n = {n} > B")
    rep.notes.append(dict(head_calls=len(row_lp)))
    return rep


def check_walk(target, h, s0, root_tok, D, B, tree, dev, tau) -> Report:
    """Check a device acceptance walk of one tree against the synthetic target.

    tree: dict of tok, parent, depth ([>= n]) and n.  dev: dict of target_tok
    ([B + 1]), path ([D]) and accept_len.  Every target token the device
    reports is compared with the fp64 argmax of the target's logits at that
    node (a different token passes only when its fp64 logit is within tau of
    the maximum, counted as an exemption); nodes without children must report
    -1.  The walk is then replayed on the device's target tokens and must
    equal the device's path exactly.
    """
    rep = Report()
    n = int(tree["n"])
    tok = np.asarray(tree["tok"])[:n]; par = np.asarray(tree["parent"])[:n]
    dep = np.asarray(tree["depth"])[:n]
    tt = np.asarray(dev["target_tok"]).reshape(-1)
    has_child = np.zeros(B + 1, bool)
    for i in range(n):
        has_child[int(par[i]) + 1] = True
    states = {-1: O.state_update(target, np.asarray(s0, np.float64)[None, :], [int(root_tok)],
                                 h[0])[0]}
    inner = []
    for j in range(B + 1):
        i = j - 1
        if not has_child[j]:
            if int(tt[j]) != -1:
                rep.fail(f"entry {i}: target token {tt[j]} for a node without children")
            continue
        if i >= 0:
            states[i] = O.state_update(target, states[int(par[i])][None, :], [int(tok[i])],
                                       h[int(dep[i])])[0]
        inner.append(j)
    # one pass over the target's output matrix for every node with children
    Z = target.logits(np.stack([states[j - 1] for j in inner])) if inner else None
    for q, j in enumerate(inner):
        i = j - 1
        z = Z[q]
        best = int(np.argmax(z))
        got = int(tt[j])
        if got == best:
            continue
        if not 0 <= got < z.size:
            rep.fail(f"entry {i}: target token {got} out of range")
            continue
        gap = float(z[best] - z[got])
        if gap <= tau:
            rep.exemptions += 1
        else:
            rep.fail(f"entry {i}: target token {got} vs argmax {best} (gap {gap:.3g})")
    # the walk over the device's target tokens
    path, cur = [], -1
    while len(path) < D and int(tt[cur + 1]) >= 0:
        want = int(tt[cur + 1])
        match = [i for i in range(n) if int(par[i]) == cur and int(tok[i]) == want]
        if not match:
            break
        cur = match[0]
        path.append(cur)
    got_path = [int(x) for x in np.asarray(dev["path"]).reshape(-1)]
    want_path = path + [-1] * (D - len(path))
    if got_path != want_path:
        rep.fail(f"path {got_path} vs {want_path}")
    if int(np.asarray(dev["accept_len"]).reshape(-1)[0]) != len(path):
        rep.fail(f"accept_len {dev['accept_len']} vs {len(path)}")
    rep.notes.append(dict(tau=len(path) + 1))
    return rep
