"""Sampled oracle checks for full-size builds (test infrastructure only).

At the full vocabulary and hidden sizes the oracle cannot re-run every
branch of every depth in seconds, so it checks sampled root-to-node paths of
the device's supertree: along each path it recomputes, in fp64, every state
(following the device's tokens, teacher-forced), the full temperature
log-softmax of every row on the path, and checks

* the device token at each step is one of the oracle's top-k children of its
  parent row, up to a score gap tau;
* the device's accumulated score matches the oracle's path score within tol;
* every oracle top-k child of a sampled row that the device dropped scores no
  better than the worst kept node of that depth, up to tau + tol;
* at depth 1 (a single root row) the device's kept set is exactly the
  oracle's top-n_1 unless a boundary gap is below tau.

Only discrete device choices (tokens, parent slots) are followed; no device
floating-point value is fed to the oracle.
"""
from __future__ import annotations

import numpy as np

from . import dartree_oracle as O


def sample_paths(pool_tok, pool_parent, n_valid, nodes_per_depth=1, seed=0):
    """Root-to-node paths ending at sampled slots: always slot 0 and the last
    valid slot of the deepest depth, plus `nodes_per_depth` random nodes of
    every depth.  Returns a list of [(t, j), ...] from depth 1 down."""
    g = np.random.default_rng(seed)
    D = pool_tok.shape[0]
    ends = {(D - 1, 0), (D - 1, int(n_valid[D - 1]) - 1)}
    for t in range(D):
        for _ in range(nodes_per_depth):
            ends.add((t, int(g.integers(0, int(n_valid[t])))))
    paths = []
    for t, j in sorted(ends):
        path = []
        while t >= 0:
            path.append((t, j))
            j = int(pool_parent[t, j])
            t -= 1
        paths.append(path[::-1])
    return paths


def check_paths(head: O.OracleHead, h, s0, root_tok, k, T, dev, tol, tau, paths):
    """Teacher-forced oracle check of sampled paths; returns (failures, stats)."""
    tok = np.asarray(dev["tok"]); par = np.asarray(dev["parent"])
    sco = np.asarray(dev["score"], np.float64); nv = np.asarray(dev["n_valid"])
    D = tok.shape[0]
    # rows to evaluate: every path prefix, keyed by the node whose state it is
    # (None = root); the row of node (t, j) yields the children at depth t + 1
    prefixes = {None: None}
    for p in paths:
        for i, node in enumerate(p):
            prefixes[node] = p[i - 1] if i else None
    # updated state of every row on the paths (the MLP is cheap); a node's
    # carried state is its parent's updated state, its own token enters the
    # update that produces its children; the root row updates s0 with root_tok
    order = sorted((n for n in prefixes if n is not None), key=lambda n: n[0])
    rows = [None] + order
    upd = {None: O.state_update(head, np.asarray(s0, np.float64)[None, :], [int(root_tok)],
                                h[0])[0]}
    for node in order:
        t, _ = node
        if t + 1 < D:
            upd[node] = O.state_update(head, upd[prefixes[node]][None, :], [int(tok[node])],
                                       h[t + 1])[0]
    logits_rows = {}
    keys = [n for n in rows if n in upd]
    z = head.logits(np.stack([upd[n] for n in keys]))
    for n, zr in zip(keys, z):
        logits_rows[n] = zr

    fails, exempt, max_err = [], 0, 0.0
    worst_kept = [float(np.min(sco[t, :int(nv[t])])) for t in range(D)]
    path_score = {None: 0.0}
    for node in order:
        t, j = node
        parent = prefixes[node]
        zr = logits_rows[parent]
        lp = O.log_softmax_T(zr, T)
        ktok, klp = O.topk_children(lp, k)
        c = int(tok[node])
        if T == 0.0:
            if c != int(ktok[0]):
                gap = float(zr[int(ktok[0])] - zr[c])
                if gap <= tau:
                    exempt += 1
                else:
                    fails.append(f"depth {t + 1} slot {j}: token {c} not argmax (gap {gap:.3g})")
            lpc = 0.0
        else:
            lpc = float(lp[c])
            if c not in set(ktok.tolist()):
                gap = float(klp[-1] - lpc)
                if gap <= tau:
                    exempt += 1
                else:
                    fails.append(f"depth {t + 1} slot {j}: token {c} not a top-{k} child (gap {gap:.3g})")
        ps = path_score[parent] + lpc
        path_score[node] = ps
        err = abs(float(sco[t, j]) - ps)
        max_err = max(max_err, err)
        if not err <= tol:
            fails.append(f"depth {t + 1} slot {j}: score {sco[t, j]:.7g} vs oracle {ps:.7g}")
        # dropped children of this parent row must not beat the worst kept node
        if T > 0.0:
            pslot = -1 if parent is None else parent[1]
            kept = {int(tok[t, q]) for q in range(int(nv[t]))
                    if (t == 0 or int(par[t, q]) == pslot)}
            for ct, cl in zip(ktok.tolist(), klp.tolist()):
                if ct not in kept:
                    cand = path_score[parent] + cl
                    if cand > worst_kept[t] + tau + tol:
                        fails.append(f"depth {t + 1}: dropped child {ct} of slot {pslot} scores "
                                     f"{cand:.6g} > worst kept {worst_kept[t]:.6g}")
    # depth 1 comes from the single root row: the kept set is the oracle's top-n_1
    if T > 0.0:
        lp = O.log_softmax_T(logits_rows[None], T)
        ktok, klp = O.topk_children(lp, k)
        n1 = int(nv[0])
        got = [int(x) for x in tok[0, :n1]]
        if got != ktok[:n1].tolist():
            gaps = np.abs(np.diff(klp))
            if np.min(gaps) <= tau:
                exempt += 1
            else:
                fails.append(f"depth 1 kept {got} != oracle {ktok[:n1].tolist()}")
    return fails, dict(exemptions=exempt, max_score_err=max_err, paths=len(paths),
                       rows=len(keys))


def check_structure(tok, par, score, n_valid, W, k, V, T):
    """Size-independent properties of a device pool."""
    out = []
    D = tok.shape[0]
    keff = 1 if T == 0.0 else k
    n_prev = 1
    for t in range(D):
        n = int(n_valid[t])
        want = min(W, n_prev * keff)
        if n != want:
            out.append(f"depth {t + 1}: n_valid {n} != {want}")
            return out
        s = score[t, :n].astype(np.float64)
        if n > 1 and np.any(np.diff(s) > 0):
            out.append(f"depth {t + 1}: scores not non-increasing")
        if not np.all(np.isfinite(s)) or np.any(s > 0):
            out.append(f"depth {t + 1}: invalid score")
        if np.any(tok[t, :n] < 0) or np.any(tok[t, :n] >= V):
            out.append(f"depth {t + 1}: token out of range")
        if t == 0:
            if np.any(par[t, :n] != -1):
                out.append("depth 1 parents not -1")
        else:
            p = par[t, :n]
            if np.any(p < 0) or np.any(p >= n_prev):
                out.append(f"depth {t + 1}: parent out of range")
            elif np.any(s > score[t - 1, p] + 1e-6):
                out.append(f"depth {t + 1}: child scores above parent")
            pairs = set(zip(p.tolist(), tok[t, :n].tolist()))
            if len(pairs) != n:
                out.append(f"depth {t + 1}: duplicate children")
        if np.any(tok[t, n:] != -1) or np.any(par[t, n:] != -1) or \
                not np.all(np.isneginf(score[t, n:])):
            out.append(f"depth {t + 1}: padding")
        if T == 0.0 and np.any(s != 0.0):
            out.append(f"depth {t + 1}: greedy scores not 0")
        n_prev = n
    return out
