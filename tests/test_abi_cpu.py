"""CPU checks of the C ABI: the library loads, exports every symbol the header
declares, and rejects bad arguments on the host before launching anything.
No call here reaches a kernel (all use invalid arguments or size queries)."""
import ctypes as C
import os
import re

import pytest

from draft_tree_construction_02_amd import _abi as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dartree.h")

DT_EINVAL, DT_EWORKSPACE, DT_EUNSUPPORTED = -1, -2, -3


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"^\s*#.*$", "", text, flags=re.M)
    # every prototype: an identifier, a parenthesised parameter list, then ';'
    names = re.findall(r"\b([A-Za-z_]\w*)\s*\([^;{}]*\)\s*;", text)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = header_functions()
    assert len(names) == 25, names
    L = A.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(A.EXPORTS) == names


def test_version_and_status_strings():
    L = A.lib()
    assert L.dartree_version() >> 16 == 1
    for code in (0, -1, -2, -3, -4):
        assert A.status_string(code)
    assert A.status_string(-99) == "unknown status"


def fake_head(d=2560, V=151936, wdtype=A.DT_BF16):
    # non-null but never dereferenced: every call below fails validation first
    return A.dt_head(d, V, wdtype, 0, 16, 32, 48, 64)


def build(hd, R=1, D=16, W=16, k=8, T=1.0, ws=1 << 40, wsp=1, **kw):
    p = dict(hid=1, s0=1, root=1, tok=1, par=1, score=1, nv=1)
    p.update(kw)
    return A.lib().build_supertree(C.byref(hd), p["hid"], p["s0"], p["root"], R, D, W, k, T,
                                   p["tok"], p["par"], p["score"], p["nv"], wsp, ws, None)


def test_build_supertree_validation():
    h = fake_head()
    assert build(h, k=0) == DT_EINVAL
    assert build(h, W=0) == DT_EINVAL
    assert build(h, D=0) == DT_EINVAL
    assert build(h, R=0) == DT_EINVAL
    assert build(h, T=-1.0) == DT_EINVAL
    assert build(h, T=float("nan")) == DT_EINVAL
    assert build(h, T=float("inf")) == DT_EINVAL
    assert build(h, k=17) == DT_EUNSUPPORTED
    assert build(h, W=129) == DT_EUNSUPPORTED          # R*W > 128 rows
    assert build(h, R=9, W=16) == DT_EUNSUPPORTED
    assert build(h, D=65) == DT_EUNSUPPORTED
    assert build(h, hid=None) == DT_EINVAL
    assert build(h, nv=None) == DT_EINVAL
    assert build(h, ws=10) == DT_EWORKSPACE
    assert build(h, wsp=None) == DT_EWORKSPACE
    assert build(fake_head(d=2500)) == DT_EINVAL        # bf16 needs d % 128 == 0
    assert build(fake_head(d=48, wdtype=A.DT_F32)) == DT_EINVAL
    assert build(fake_head(wdtype=7)) == DT_EINVAL
    bad = fake_head()
    bad.Ut = None
    assert build(bad) == DT_EINVAL
    assert build(fake_head(V=4), k=8) == DT_EINVAL        # k > V


def seq(hd, D=16, k=8, B=64, beta=0.0, T=1.0, ws=1 << 40, wsp=1, **kw):
    p = dict(hid=1, s0=1, root=1, tok=1, par=1, depth=1, score=1, n=1)
    p.update(kw)
    return A.lib().build_tree_sequential(C.byref(hd), p["hid"], p["s0"], p["root"], D, k, B,
                                         beta, T, p["tok"], p["par"], p["depth"], p["score"],
                                         p["n"], wsp, ws, None)


def noalloc(hd, R=1, D=16, W=16, k=8, T=1.0, **kw):
    p = dict(hid=1, s0=1, root=1, tok=1, par=1, score=1, nv=1)
    p.update(kw)
    return A.lib().build_supertree_noalloc(C.byref(hd), p["hid"], p["s0"], p["root"], R, D, W,
                                           k, T, p["tok"], p["par"], p["score"], p["nv"], None)


def test_build_supertree_noalloc_validation():
    # argument checks as build_supertree; a call whose scratch would exceed the
    # static array is refused on the host before the array is looked up
    h = fake_head()
    assert noalloc(h, k=0) == DT_EINVAL
    assert noalloc(h, T=-1.0) == DT_EINVAL
    assert noalloc(h, T=float("nan")) == DT_EINVAL
    assert noalloc(h, tok=None) == DT_EINVAL
    assert noalloc(h, R=9, W=16) == DT_EUNSUPPORTED          # 144 rows
    assert noalloc(fake_head(d=100)) == DT_EINVAL
    big = fake_head(d=8192, V=262144)
    need = A.lib().build_supertree_workspace_size(C.byref(big), 8, 16, 16, 16)
    assert need > A.NOALLOC_SCRATCH_BYTES
    assert noalloc(big, R=8, D=16, W=16, k=16) == DT_EUNSUPPORTED
    # every benchmarked workload fits the static array
    from draft_tree_construction_02_amd import synth
    for wl in synth.workloads().values():
        hd = fake_head(d=wl.d, V=wl.V, wdtype=A.DT_BF16 if wl.wdtype == "bf16" else A.DT_F32)
        assert 0 < A.lib().build_supertree_workspace_size(C.byref(hd), wl.R, wl.D, wl.W,
                                                          wl.k) <= A.NOALLOC_SCRATCH_BYTES
    # the limit the binding states is the header's
    text = open(HEADER).read()
    assert "#define DT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in text
    assert A.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_build_tree_sequential_validation():
    h = fake_head()
    L = A.lib()
    assert L.build_tree_sequential_workspace_size(C.byref(h), 16, 8, 64) > 0
    assert L.build_tree_sequential_workspace_size(C.byref(h), 16, 0, 64) == 0
    assert seq(h, k=0) == DT_EINVAL
    assert seq(h, B=0) == DT_EINVAL
    assert seq(h, D=0) == DT_EINVAL
    assert seq(h, beta=0.5) == DT_EINVAL
    assert seq(h, beta=float("nan")) == DT_EINVAL
    assert seq(h, T=-1.0) == DT_EINVAL
    assert seq(h, k=17) == DT_EUNSUPPORTED
    assert seq(h, B=1025) == DT_EUNSUPPORTED
    assert seq(h, D=65) == DT_EUNSUPPORTED
    assert seq(h, hid=None) == DT_EINVAL
    assert seq(h, n=None) == DT_EINVAL
    assert seq(h, ws=10) == DT_EWORKSPACE
    assert seq(h, wsp=None) == DT_EWORKSPACE
    assert seq(fake_head(V=4), k=8) == DT_EINVAL


def walk(hd, R=1, D=16, B=64, stride=64, index=None, ws=1 << 40, wsp=1, **kw):
    p = dict(hid=1, s0=1, root=1, tok=1, par=1, depth=1, n=1, tt=1, path=1, alen=1)
    p.update(kw)
    return A.lib().accept_walk(C.byref(hd), p["hid"], p["s0"], p["root"], R, D, B, p["tok"],
                               stride, index, p["par"], p["depth"], p["n"], p["tt"], p["path"],
                               p["alen"], wsp, ws, None)


def test_accept_walk_validation():
    h = fake_head()
    L = A.lib()
    assert L.accept_walk_workspace_size(C.byref(h), 1, 16, 64) > 0
    assert L.accept_walk_workspace_size(C.byref(h), 0, 16, 64) == 0
    assert L.accept_walk_workspace_size(C.byref(h), 8, 16, 1025) == 0
    # the workspace grows with the number of nodes
    assert L.accept_walk_workspace_size(C.byref(h), 8, 16, 128) > \
        L.accept_walk_workspace_size(C.byref(h), 1, 16, 128)
    assert walk(h, R=0) == DT_EINVAL
    assert walk(h, D=0) == DT_EINVAL
    assert walk(h, B=0) == DT_EINVAL
    assert walk(h, B=1025, stride=1025) == DT_EUNSUPPORTED
    assert walk(h, R=9, B=1024, stride=1024) == DT_EUNSUPPORTED     # R * B > 8192
    assert walk(h, D=65) == DT_EUNSUPPORTED
    assert walk(h, stride=63) == DT_EINVAL                           # row of B tokens
    assert walk(h, stride=0, index=1) == DT_EINVAL
    for name in ("hid", "s0", "root", "tok", "par", "depth", "n", "tt", "path", "alen"):
        assert walk(h, **{name: None}) == DT_EINVAL, name
    assert walk(h, ws=10) == DT_EWORKSPACE
    assert walk(h, wsp=None) == DT_EWORKSPACE
    assert walk(fake_head(d=2500)) == DT_EINVAL


def test_build_supertree_ex_validation():
    L = A.lib()
    h = fake_head()
    o = A.dt_build_opts(A.DT_BUILD_MARKOV, 0)
    assert L.build_supertree_ex_workspace_size(C.byref(h), 1, 16, 16, 8, C.byref(o)) > 0
    assert L.build_supertree_ex_workspace_size(C.byref(h), 1, 16, 16, 8, None) == \
        L.build_supertree_workspace_size(C.byref(h), 1, 16, 16, 8)

    def ex(opts, **kw):
        p = dict(k=8, T=1.0, ws=1 << 40)
        p.update(kw)
        return L.build_supertree_ex(C.byref(h), 1, 1, 1, 1, 16, 16, p["k"], p["T"],
                                    C.byref(opts) if opts is not None else None, 1, 1, 1, 1, 1,
                                    p["ws"], None)
    assert ex(A.dt_build_opts(8, 0)) == DT_EINVAL                        # unknown flag
    assert ex(A.dt_build_opts(A.DT_BUILD_BASE_CANDIDATES, 4)) == DT_EINVAL   # n_cand < k
    assert ex(A.dt_build_opts(A.DT_BUILD_BASE_CANDIDATES, 17)) == DT_EUNSUPPORTED
    assert ex(A.dt_build_opts(A.DT_BUILD_MARKOV, 0), T=-1.0) == DT_EINVAL
    assert ex(A.dt_build_opts(A.DT_BUILD_MARKOV, 0), ws=10) == DT_EWORKSPACE
    assert ex(None, k=0) == DT_EINVAL
    # the per-depth-kernel flag: same workspace, combines with the variants,
    # and every check still runs before any launch
    mk = A.dt_build_opts(A.DT_BUILD_MULTI_KERNEL, 0)
    assert L.build_supertree_ex_workspace_size(C.byref(h), 1, 16, 16, 8, C.byref(mk)) == \
        L.build_supertree_workspace_size(C.byref(h), 1, 16, 16, 8)
    assert ex(A.dt_build_opts(A.DT_BUILD_MULTI_KERNEL | A.DT_BUILD_MARKOV, 0), T=-1.0) == DT_EINVAL
    assert ex(mk, ws=10) == DT_EWORKSPACE
    assert ex(A.dt_build_opts(A.DT_BUILD_MULTI_KERNEL | 8, 0)) == DT_EINVAL
    # a small fp32 head (one-launch build) checks its workspace as well
    f = fake_head(d=64, V=1000, wdtype=A.DT_F32)
    assert L.build_supertree(C.byref(f), 1, 1, 1, 1, 6, 4, 4, 1.0, 1, 1, 1, 1, 1, 10,
                             None) == DT_EWORKSPACE


def test_pack_head_validation():
    L = A.lib()
    out = A.dt_head()
    f32 = fake_head(d=64, V=100, wdtype=A.DT_F32)
    assert L.pack_head_bytes(C.byref(f32)) == 0
    assert L.pack_head(C.byref(f32), 1, 1 << 40, C.byref(out), None) == DT_EINVAL
    h = fake_head(d=256, V=1000)
    need = L.pack_head_bytes(C.byref(h))
    assert need >= 2 * (4 * 256 * 256 * 2) + 1008 * 256 * 2
    assert L.pack_head(C.byref(h), 1, need - 1, C.byref(out), None) == DT_EWORKSPACE
    assert L.pack_head(C.byref(h), 1, need, None, None) == DT_EINVAL
    packed = fake_head(d=256, V=1000)
    packed.layout = A.DT_LAYOUT_PACKED
    assert L.pack_head(C.byref(packed), 1, need, C.byref(out), None) == DT_EINVAL
    bad = fake_head()
    bad.layout = 5
    assert build(bad) == DT_EINVAL
    f32p = fake_head(d=64, V=100, wdtype=A.DT_F32)
    f32p.layout = A.DT_LAYOUT_PACKED
    assert build(f32p, k=4) == DT_EINVAL


def test_workspace_sizes():
    L = A.lib()
    h = fake_head()
    w1 = L.build_supertree_workspace_size(C.byref(h), 1, 16, 16, 8)
    w2 = L.build_supertree_workspace_size(C.byref(h), 1, 16, 32, 8)
    assert 0 < w1 < w2
    assert L.build_supertree_workspace_size(C.byref(h), 1, 16, 16, 0) == 0
    assert L.head_step_workspace_size(C.byref(h), 16, 8) > 0
    assert L.head_step_workspace_size(C.byref(h), 0, 8) == 0
    assert L.tree_attention_workspace_size(128, 4096, 32, 8, 128) > 0
    assert L.tree_attention_workspace_size(128, 4096, 32, 8, 64) == 0
    assert L.tree_attention_workspace_size(128, 4096, 30, 8, 128) == 0


def test_prune_and_mask_validation():
    L = A.lib()
    ok = dict(R=1, D=4, W=4, B=8, beta=0.0)

    def prune(**kw):
        a = dict(ok, **kw)
        return L.prune_topB(1, 1, 1, a["R"], a["D"], a["W"], a["B"], a["beta"], 1, 1, 1, 1, None)

    assert prune(beta=0.5) == DT_EINVAL                  # Lemma 1 needs beta <= 0
    assert prune(beta=float("nan")) == DT_EINVAL
    assert prune(B=17) == DT_EINVAL                      # B > D * W
    assert prune(B=0) == DT_EINVAL
    assert prune(D=65, W=64, B=8) == DT_EUNSUPPORTED
    assert L.prune_topB(None, 1, 1, 1, 4, 4, 8, 0.0, 1, 1, 1, 1, None) == DT_EINVAL
    assert L.build_tree_mask(1, 1, 1, 0, 1, None) == DT_EINVAL
    assert L.build_tree_mask(1, 1, 1, 2048, 1, None) == DT_EUNSUPPORTED
    assert L.build_tree_mask(None, 1, 1, 8, 1, None) == DT_EINVAL


def test_stage_and_attention_validation():
    L = A.lib()
    h = fake_head()
    assert L.state_update(C.byref(h), 1, 1, 1, 0, 2, 1, 1 << 40, None) == DT_EINVAL
    assert L.state_update(C.byref(h), 1, 1, 1, 200, 2, 1, 1 << 40, None) == DT_EUNSUPPORTED
    assert L.state_update(C.byref(h), 1, 1, 1, 4, 1, 1, 1 << 40, None) == DT_EINVAL  # alias
    assert L.state_update(C.byref(h), 1, 1, 1, 4, 2, 1, 8, None) == DT_EWORKSPACE
    assert L.corrected_topk(C.byref(h), 1, 4, 8, -0.5, 1, 1, 1, 1, 1 << 40, None) == DT_EINVAL
    assert L.corrected_topk(C.byref(h), 1, 4, 17, 1.0, 1, 1, 1, 1, 1 << 40, None) == DT_EUNSUPPORTED
    args = [1, 1, 1, 1, 1, 1]
    assert L.tree_attention_verify(*args, 128, 4096, 32, 8, 64, 0.1, 1, 1, 1 << 40, None) == DT_EUNSUPPORTED
    assert L.tree_attention_verify(*args, 128, 4096, 30, 8, 128, 0.1, 1, 1, 1 << 40, None) == DT_EINVAL
    assert L.tree_attention_verify(*args, 128, 4096, 32, 8, 128, 0.1, 1, 1, 8, None) == DT_EWORKSPACE
    assert L.tree_attention_verify(None, 1, 1, 1, 1, 1, 128, 4096, 32, 8, 128, 0.1, 1, 1,
                                   1 << 40, None) == DT_EINVAL
    # key offsets of the copies are 32-bit: 2^20 prefix keys x 8 heads x 256 B is refused
    assert L.tree_attention_verify(*args, 128, 1 << 20, 32, 8, 128, 0.1, 1, 1, 1 << 40,
                                   None) == DT_EUNSUPPORTED
    # rows that fill the chip alone need no split of the key range, so no partials
    assert L.tree_attention_workspace_size(1024, 0, 32, 8, 128) == 256
    assert L.tree_attention_workspace_size(128, 4096, 32, 8, 128) > 256


def test_timing_api_without_launches():
    A.timing_reset()
    assert A.timing_read("head") == (0.0, 0)
    with pytest.raises(KeyError):
        A.timing_read("nope")
    assert A.lib().dartree_timing_read(9, C.byref(C.c_double()), C.byref(C.c_int64())) == DT_EINVAL


def test_mfma_rate_probe_validation():
    L = A.lib()
    probe = L.mfma_rate_probe
    assert probe(None, 1 << 30, 1, 1 << 20, 1 << 20, None) == DT_EINVAL          # no operands
    assert probe(1 << 20, 1 << 30, 1, None, 1 << 20, None) == DT_EINVAL          # no output
    assert probe((1 << 20) + 8, 1 << 30, 1, 1 << 21, 1 << 20, None) == DT_EINVAL  # misaligned
    assert probe(1 << 20, 1 << 30, -1, 1 << 21, 1 << 20, None) == DT_EINVAL      # negative rounds


def test_hbm_read_probe_validation():
    L = A.lib()
    probe = L.hbm_read_probe
    assert probe(1 << 20, 16, None, None) == DT_EINVAL            # no output
    assert probe(None, 16, 1 << 20, None) == DT_EINVAL            # no buffer
    assert probe(1 << 20, 12, 1 << 21, None) == DT_EINVAL         # not whole 64-bit words
    assert probe((1 << 20) + 8, 16, 1 << 21, None) == DT_EINVAL   # not 16-byte aligned
