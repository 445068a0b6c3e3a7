"""GPU parity of the build variants (Markov head, base-logit candidates)
against the fp64 oracle: teacher-forced replay of every depth, exact equality
with the oracle's own build when no near-tie was exempted, and the pruned tree
and mask of the variant's pool."""
import numpy as np
import pytest
import torch

from draft_tree_construction_02_amd import _abi as A
from draft_tree_construction_02_amd import synth
from oracle import dartree_oracle as O
from oracle import parity as PAR
from tests.gpu_util import dev_requests, dev_weights, oracle_head, to_np, tolerances
from tests.test_gpu_parity import case_inputs, layouts, small_cases

pytestmark = pytest.mark.gpu

VARIANTS = {"markov": dict(markov=True, n_cand=0), "base": dict(markov=False, n_cand=-1),
            "markov_base": dict(markov=True, n_cand=-1)}


def n_cand_for(wl):
    return min(wl.V, 16, wl.k + 4)


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name,packed", layouts(small_cases()))
def test_variant_build_matches_oracle(name, packed, variant):
    wl = small_cases()[name]
    v = dict(VARIANTS[variant])
    if v["n_cand"] < 0:
        v["n_cand"] = n_cand_for(wl)
    print(f"variant {variant} case {name} packed={packed} {v}", flush=True)
    hw, req, head, ohead = case_inputs(wl, packed)
    tol, tau = tolerances(wl.wdtype)
    h, s0, root = dev_requests(req)
    out = A.build_supertree(head, h, s0, root, wl.D, wl.W, wl.k, wl.T, **v)
    sel = A.prune_topB(out["pool_score"], out["pool_parent"], out["n_valid"], wl.B, wl.beta)
    mask = A.build_tree_mask(sel["sel_parent"], sel["n_sel"])
    torch.cuda.synchronize()
    pool, sel, mask = to_np(out), to_np(sel), mask.cpu().numpy().view(np.uint32)
    for r in range(wl.R):
        dev = dict(tok=pool["pool_tok"][r], parent=pool["pool_parent"][r],
                   score=pool["pool_score"][r], n_valid=pool["n_valid"][r])
        rep = PAR.check_build(ohead, req.h[r], req.s0[r], int(req.root_tok[r]), wl.D, wl.W,
                              wl.k, wl.T, dev, tol, tau, markov=v["markov"],
                              base_cand=v["n_cand"])
        assert rep.ok, rep.failures[:5]
        dsel = dict(node=sel["sel_node"][r], parent=sel["sel_parent"][r],
                    depth=sel["sel_depth"][r], n=sel["n_sel"][r])
        PAR.check_prune(rep.forced_score, dev["parent"], dev["n_valid"], wl.B, wl.beta, dsel,
                        tau, rep)
        assert rep.ok, rep.failures[:5]
        assert not PAR.check_mask(dsel["parent"], dsel["n"], wl.B, mask[r])
        if rep.exemptions == 0:
            ora = O.build_supertree(ohead, req.h[r], req.s0[r], int(req.root_tok[r]), wl.D,
                                    wl.W, wl.k, wl.T, markov=v["markov"], n_cand=v["n_cand"])
            assert not PAR.compare_exact(ora, dev, tol)


def test_fullsize_variants():
    # the Qwen3-4B shape with both variants on, checked at every depth
    wl = synth.workloads()["qwen3_4b"]
    print("full-size variants qwen3_4b", flush=True)
    hw, req = synth.make_workload_inputs(wl)
    head = dev_weights(hw, packed=True)
    h, s0, root = dev_requests(req)
    out = to_np(A.build_supertree(head, h, s0, root, wl.D, wl.W, wl.k, wl.T, markov=True,
                                  n_cand=16))
    del head
    torch.cuda.empty_cache()
    tol, tau = tolerances(wl.wdtype)
    dev = dict(tok=out["pool_tok"][0], parent=out["pool_parent"][0],
               score=out["pool_score"][0], n_valid=out["n_valid"][0])
    rep = PAR.check_build(oracle_head(hw), req.h[0], req.s0[0], int(req.root_tok[0]), wl.D,
                          wl.W, wl.k, wl.T, dev, tol, tau, markov=True, base_cand=16)
    assert rep.ok, rep.failures[:5]
    print(f"variants: exemptions {rep.exemptions} max score err {rep.max_score_err:.3g}",
          flush=True)
