"""Helpers shared by the GPU tests: upload seeded inputs, run the library,
bring results back to numpy."""
from __future__ import annotations

import numpy as np
import torch

from draft_tree_construction_02_amd import _abi as A
from draft_tree_construction_02_amd import synth
from oracle import dartree_oracle as O

DEV = "cuda:0"


def dev_weights(hw: synth.HeadWeights, packed: bool = False) -> A.Head:
    def up(a):
        if hw.wdtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    head = A.Head(up(hw.E), up(hw.W1t), up(hw.W2t), up(hw.Ut))
    return head.packed() if packed else head


def oracle_head(hw: synth.HeadWeights, cache_u=True) -> O.OracleHead:
    return O.OracleHead(hw.wdtype, hw.E, hw.W1t, hw.W2t, hw.Ut, cache_u=cache_u)


def dev_requests(req: synth.Requests):
    return (torch.from_numpy(req.h).to(DEV), torch.from_numpy(req.s0).to(DEV),
            torch.from_numpy(req.root_tok).to(DEV))


def to_np(d: dict) -> dict:
    return {k: v.cpu().numpy() for k, v in d.items()}


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def tolerances(wdtype: str, ymax: float = 8.0):
    """(score tolerance, near-tie gap tau) for a head dtype.

    bf16 heads: 2e-3 absolute on log-probabilities and path scores, tau = 2 tol.
    fp32 heads: fp32 rounding of a logit is relative to its size, so the
    tolerance is 1e-5 for logits up to 8 in magnitude and grows with them.
    """
    if wdtype == "bf16":
        return 2e-3, 4e-3
    tol = 1e-5 * max(1.0, ymax / 8.0)
    return tol, 2 * tol


def full_check(ohead: O.OracleHead, req: synth.Requests, r: int, wl: synth.Workload, pool: dict,
               sel: dict, mask: np.ndarray, want_entropy: bool = False) -> dict:
    """The whole oracle check of request r of a device build (numpy outputs of
    build_supertree, prune_topB and build_tree_mask):

    * teacher-forced check of every depth (every row, every child, the top-W
      survivors and their order), following the device's tokens and parents;
    * the device's top-B against the oracle priorities along the same paths;
    * the mask against the ancestor closure of the device's own tree, exactly;
    * with zero near-tie exemptions: equality with the oracle's independent
      build (tokens, parents, widths exact; scores within tol) and with its
      top-B (nodes, parents, depths exact).

    Returns a summary (exemptions, max score error, sizes; the oracle build's
    mean entropy when asked); raises AssertionError on any failure."""
    from oracle import parity as PAR
    tol, tau = tolerances(wl.wdtype)
    dev = dict(tok=pool["pool_tok"][r], parent=pool["pool_parent"][r],
               score=pool["pool_score"][r], n_valid=pool["n_valid"][r])
    rep = PAR.check_build(ohead, req.h[r], req.s0[r], int(req.root_tok[r]), wl.D, wl.W, wl.k,
                          wl.T, dev, tol, tau)
    assert rep.ok, rep.failures[:5]
    dsel = dict(node=sel["sel_node"][r], parent=sel["sel_parent"][r], depth=sel["sel_depth"][r],
                n=sel["n_sel"][r])
    PAR.check_prune(rep.forced_score, dev["parent"], dev["n_valid"], wl.B, wl.beta, dsel, tau, rep)
    assert rep.ok, rep.failures[:5]
    bad = PAR.check_mask(dsel["parent"], dsel["n"], wl.B, mask[r])
    assert not bad, bad
    out = dict(exemptions=rep.exemptions, max_score_err=float(rep.max_score_err),
               pool=int(np.sum(dev["n_valid"])), n_sel=int(dsel["n"]), exact=False)
    if rep.exemptions == 0 or want_entropy:
        ora = O.build_supertree(ohead, req.h[r], req.s0[r], int(req.root_tok[r]), wl.D, wl.W,
                                wl.k, wl.T, want_entropy=want_entropy)
        if want_entropy:
            out["mean_entropy"] = float(np.mean([e for row in ora.entropies for e in row]))
        if rep.exemptions == 0:
            diff = PAR.compare_exact(ora, dev, tol)
            assert not diff, diff
            vt = O.prune_topB(ora.score, ora.parent, ora.n_valid, wl.B, wl.beta)
            assert np.array_equal(dsel["node"][:vt.n], vt.node)
            assert np.array_equal(dsel["parent"][:vt.n], vt.parent)
            assert np.array_equal(dsel["depth"][:vt.n], vt.depth)
            out["exact"] = True
    return out
