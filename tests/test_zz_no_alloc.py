"""The allocation-free build (static per-GPU scratch) against the workspace
build on the same inputs: two calls in a row, the second with fewer rows, a
smaller head and a different row organisation, so it runs over the first
call's leftover scratch contents.  Outputs must be identical bit for bit
(same kernels, fixed-order reductions)."""
import numpy as np
import pytest
import torch

from draft_tree_construction_02_amd import _abi as A
from draft_tree_construction_02_amd import synth
from tests.gpu_util import dev_requests, dev_weights, to_np

pytestmark = pytest.mark.gpu


def _pool_like(R, D, W, dev):
    return dict(pool_tok=torch.full((R, D, W), 7, dtype=torch.int32, device=dev),
                pool_parent=torch.full((R, D, W), 7, dtype=torch.int32, device=dev),
                pool_score=torch.full((R, D, W), 7.0, dtype=torch.float32, device=dev),
                n_valid=torch.full((R, D), 7, dtype=torch.int32, device=dev))


CALLS = [
    # 128 rows (8 requests x 16): the 128-row head and GEMM, packed weights
    synth.Workload("noalloc_rows128", V=5000, d=512, wdtype="bf16", D=5, W=16, k=8, B=40,
                   beta=0.0, T=1.0, R=8, seeds=tuple(range(20, 28))),
    # then 16 rows at a smaller head, row-major weights, greedy
    synth.Workload("noalloc_rows16", V=3001, d=256, wdtype="bf16", D=4, W=8, k=4, B=8,
                   beta=0.0, T=0.0, R=2, seeds=(40, 41)),
]


def test_noalloc_build_matches_workspace_build_twice():
    dev = "cuda:0"
    for i, wl in enumerate(CALLS):
        packed = i == 0
        print(f"noalloc call {i}: {wl.name} rows={wl.R * wl.W} packed={packed}", flush=True)
        hw, req = synth.make_workload_inputs(wl)
        head = dev_weights(hw, packed)
        h, s0, root = dev_requests(req)
        want = to_np(A.build_supertree(head, h, s0, root, wl.D, wl.W, wl.k, wl.T))
        out = _pool_like(wl.R, wl.D, wl.W, dev)
        got = to_np(A.build_supertree_noalloc(head, h, s0, root, wl.D, wl.W, wl.k, wl.T, out))
        for key in want:
            assert np.array_equal(want[key].view(np.uint8), got[key].view(np.uint8)), (i, key)
        assert int(got["n_valid"].sum()) > 0
        del head
    torch.cuda.synchronize()


def test_noalloc_refuses_a_call_beyond_its_scratch():
    # a 128-row build at d = 8192, V = 262144 needs more than the static array
    # holds: refused on the host with a clear error, nothing launched
    wl = CALLS[0]
    dev = "cuda:0"
    hw, req = synth.make_workload_inputs(wl)
    head = dev_weights(hw, True)
    h, s0, root = dev_requests(req)
    big = A.Head.__new__(A.Head)
    big.__dict__.update(head.__dict__)
    big.c = A.dt_head(8192, 262144, A.DT_BF16, A.DT_LAYOUT_PACKED, head.c.E, head.c.W1t,
                      head.c.W2t, head.c.Ut)
    big.d, big.V = 8192, 262144
    hb = torch.zeros((wl.R, wl.D, 8192), dtype=torch.float32, device=dev)
    sb = torch.zeros((wl.R, 8192), dtype=torch.float32, device=dev)
    out = _pool_like(wl.R, wl.D, wl.W, dev)
    with pytest.raises(A.DartreeError, match="static array holds"):
        A.build_supertree_noalloc(big, hb, sb, root, wl.D, wl.W, 16, wl.T, out)
    torch.cuda.synchronize()
    assert int(out["n_valid"][0, 0].item()) == 7      # outputs untouched
