"""GPU parity of the sequential best-first construction (one head call per
expanded node) against the fp64 oracle: teacher-forced replay of every pop,
and exact equality with the oracle's own run when no near-tie was exempted."""
import numpy as np
import pytest
import torch

from draft_tree_construction_02_amd import _abi as A
from oracle import dartree_oracle as O
from oracle import parity as PAR
from tests.gpu_util import DEV, to_np, tolerances
from tests.test_gpu_parity import case_inputs, layouts, small_cases

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,packed", layouts(small_cases()))
def test_sequential_matches_oracle(name, packed):
    wl = small_cases()[name]
    print(f"sequential case {name} packed={packed}", flush=True)
    hw, req, head, ohead = case_inputs(wl, packed)
    tol, tau = tolerances(wl.wdtype)
    for beta in sorted({wl.beta, 0.0}):
        h = torch.from_numpy(req.h[0]).to(DEV)
        s0 = torch.from_numpy(req.s0[0]).to(DEV)
        root = torch.from_numpy(req.root_tok[:1]).to(DEV)
        out = to_np(A.build_tree_sequential(head, h, s0, root, wl.D, wl.k, wl.B, beta, wl.T))
        rep = PAR.check_sequential(ohead, req.h[0], req.s0[0], int(req.root_tok[0]), wl.D, wl.k,
                                   wl.B, beta, wl.T, out, tol, tau)
        assert rep.ok, rep.failures[:5]
        n = int(out["n"][0])
        assert np.all(out["tok"][n:] == -1) and np.all(out["parent"][n:] == -1)
        if rep.exemptions == 0:
            ora = O.sequential_best_first(ohead, req.h[0], req.s0[0], int(req.root_tok[0]), wl.D,
                                          wl.k, wl.B, beta, wl.T)
            assert n == ora.n
            assert np.array_equal(out["tok"][:n], ora.tok)
            assert np.array_equal(out["parent"][:n], ora.parent)
            assert np.array_equal(out["depth"][:n], ora.depth)
            assert np.max(np.abs(out["score"][:n] - ora.score), initial=0.0) <= tol
        # the verification mask of the tree (parents precede children)
        mask = A.build_tree_mask(torch.from_numpy(out["parent"][None]).to(DEV),
                                 torch.from_numpy(out["n"]).to(DEV)).cpu().numpy()
        bad = PAR.check_mask(out["parent"], n, wl.B, mask[0].view(np.uint32))
        assert not bad, bad
        print(f"{name} beta={beta}: n={n} exemptions={rep.exemptions} "
              f"head_calls={rep.notes[-1]['head_calls']}", flush=True)


def test_sequential_small_budget_and_leaf_pops():
    # B larger than the whole reachable tree: the device must stop when the
    # heap is empty; D=1 pops only leaves after the root's single call
    wl = small_cases()["bf16_T1"].with_(D=1, B=30)
    hw, req, head, ohead = case_inputs(small_cases()["bf16_T1"], True)
    h = torch.from_numpy(req.h[0][:1].copy()).to(DEV)
    s0 = torch.from_numpy(req.s0[0]).to(DEV)
    root = torch.from_numpy(req.root_tok[:1]).to(DEV)
    out = to_np(A.build_tree_sequential(head, h, s0, root, 1, wl.k, 30, 0.0, 1.0))
    assert int(out["n"][0]) == wl.k
    assert np.all(out["depth"][:wl.k] == 1) and np.all(out["parent"][:wl.k] == -1)
    ora = O.sequential_best_first(ohead, req.h[0][:1], req.s0[0], int(req.root_tok[0]), 1, wl.k,
                                  30, 0.0, 1.0)
    assert np.array_equal(out["tok"][:wl.k], ora.tok)
