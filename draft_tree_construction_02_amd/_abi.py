"""ctypes binding of libdartree.so (argument marshalling only).

Every function takes torch device tensors, checks dtype, device, shape and
contiguity, passes raw pointers and the current HIP stream to the C ABI
declared in include/dartree.h, and returns freshly allocated output tensors.
All computation happens in the library's HIP kernels; if the library is not
built this module raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdartree.so")

DT_F32, DT_BF16 = 0, 1
DT_LAYOUT_ROWMAJOR, DT_LAYOUT_PACKED = 0, 1
KERNEL_CLASSES = {"gemm1": 0, "gemm2": 1, "head": 2, "merge_select": 3, "reduce": 4,
                  "attention": 5, "build_small": 6, "head128": 7}

# every symbol include/dartree.h declares
EXPORTS = [
    "dartree_status_string", "dartree_version", "pack_head_bytes", "pack_head",
    "build_supertree_workspace_size", "build_supertree", "build_supertree_noalloc",
    "build_supertree_ex_workspace_size", "build_supertree_ex",
    "head_step_workspace_size", "state_update", "corrected_topk",
    "build_tree_sequential_workspace_size", "build_tree_sequential",
    "prune_topB", "build_tree_mask",
    "tree_attention_workspace_size", "tree_attention_verify",
    "accept_walk_workspace_size", "accept_walk", "hbm_read_probe", "mfma_rate_probe",
    "dartree_timing_enable", "dartree_timing_reset", "dartree_timing_read",
]


DT_BUILD_MARKOV, DT_BUILD_BASE_CANDIDATES, DT_BUILD_MULTI_KERNEL = 1, 2, 4


class dt_build_opts(C.Structure):
    _fields_ = [("flags", C.c_int32), ("n_cand", C.c_int32)]


class DartreeError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_string(code)} ({code})")


class dt_head(C.Structure):
    _fields_ = [("d", C.c_int32), ("V", C.c_int32), ("wdtype", C.c_int32),
                ("layout", C.c_int32), ("E", C.c_void_p), ("W1t", C.c_void_p),
                ("W2t", C.c_void_p), ("Ut", C.c_void_p)]


_lib_handle = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m draft_tree_construction_02_amd.build`")
        L = C.CDLL(LIB_PATH)
        vp, sz, i32, f32 = C.c_void_p, C.c_size_t, C.c_int, C.c_float
        hp = C.POINTER(dt_head)
        sig = {
            "dartree_status_string": (C.c_char_p, [i32]),
            "dartree_version": (i32, []),
            "pack_head_bytes": (sz, [hp]),
            "pack_head": (i32, [hp, vp, sz, hp, vp]),
            "build_supertree_workspace_size": (sz, [hp, i32, i32, i32, i32]),
            "build_supertree": (i32, [hp, vp, vp, vp, i32, i32, i32, i32, f32,
                                      vp, vp, vp, vp, vp, sz, vp]),
            "build_supertree_noalloc": (i32, [hp, vp, vp, vp, i32, i32, i32, i32, f32,
                                              vp, vp, vp, vp, vp]),
            "build_supertree_ex_workspace_size": (sz, [hp, i32, i32, i32, i32,
                                                       C.POINTER(dt_build_opts)]),
            "build_supertree_ex": (i32, [hp, vp, vp, vp, i32, i32, i32, i32, f32,
                                         C.POINTER(dt_build_opts), vp, vp, vp, vp, vp, sz, vp]),
            "head_step_workspace_size": (sz, [hp, i32, i32]),
            "build_tree_sequential_workspace_size": (sz, [hp, i32, i32, i32]),
            "build_tree_sequential": (i32, [hp, vp, vp, vp, i32, i32, i32, f32, f32,
                                            vp, vp, vp, vp, vp, vp, sz, vp]),
            "state_update": (i32, [hp, vp, vp, vp, i32, vp, vp, sz, vp]),
            "corrected_topk": (i32, [hp, vp, i32, i32, f32, vp, vp, vp, vp, sz, vp]),
            "prune_topB": (i32, [vp, vp, vp, i32, i32, i32, i32, f32, vp, vp, vp, vp, vp]),
            "build_tree_mask": (i32, [vp, vp, i32, i32, vp, vp]),
            "tree_attention_workspace_size": (sz, [i32, i32, i32, i32, i32]),
            "tree_attention_verify": (i32, [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                            f32, vp, vp, sz, vp]),
            "accept_walk_workspace_size": (sz, [hp, i32, i32, i32]),
            "accept_walk": (i32, [hp, vp, vp, vp, i32, i32, i32, vp, i32, vp, vp, vp, vp,
                                  vp, vp, vp, vp, sz, vp]),
            "hbm_read_probe": (i32, [vp, sz, vp, vp]),
            "mfma_rate_probe": (i32, [vp, sz, i32, vp, sz, vp]),
            "dartree_timing_enable": (i32, [i32]),
            "dartree_timing_reset": (i32, []),
            "dartree_timing_read": (i32, [i32, C.POINTER(C.c_double), C.POINTER(C.c_int64)]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib_handle = L
    return _lib_handle


def status_string(code: int) -> str:
    return lib().dartree_status_string(int(code)).decode()


def _check(code: int, where: str):
    if code != 0:
        raise DartreeError(code, where)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, dtype, name, shape=None):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _workspace(nbytes: int, device, ws=None):
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError("workspace too small")
        return ws
    return torch.empty(max(1, nbytes), dtype=torch.uint8, device=device)


class Head:
    """Device-resident correction head: E [V][d], W1t [4d][d], W2t [d][4d],
    Ut [V][d], all bfloat16 or all float32."""

    def __init__(self, E, W1t, W2t, Ut):
        dtype = E.dtype
        if dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("head weights must be bfloat16 or float32")
        V, d = E.shape
        self.E = _dev(E, dtype, "E", (V, d))
        self.W1t = _dev(W1t, dtype, "W1t", (4 * d, d))
        self.W2t = _dev(W2t, dtype, "W2t", (d, 4 * d))
        self.Ut = _dev(Ut, dtype, "Ut", (V, d))
        self.V, self.d, self.dtype = V, d, dtype
        self.device = E.device
        self.c = dt_head(d, V, DT_BF16 if dtype == torch.bfloat16 else DT_F32, 0,
                         E.data_ptr(), W1t.data_ptr(), W2t.data_ptr(), Ut.data_ptr())

    @property
    def ref(self):
        return C.byref(self.c)

    def packed(self, stream=None) -> "Head":
        """A copy of this bf16 head with W1t, W2t and Ut in the packed block
        layout (pack_head); the new head keeps the packed buffer alive."""
        if self.dtype != torch.bfloat16:
            raise ValueError("only bf16 heads are packed")
        nbytes = int(lib().pack_head_bytes(self.ref))
        buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        out = dt_head()
        _check(lib().pack_head(self.ref, _ptr(buf), nbytes, C.byref(out), _stream(stream)),
               "pack_head")
        h = Head.__new__(Head)
        h.E, h.W1t, h.W2t, h.Ut = self.E, None, None, None
        h._packed_buf = buf
        h.V, h.d, h.dtype, h.device = self.V, self.d, self.dtype, self.device
        h.c = out
        return h


def build_supertree_workspace_size(head: Head, R, D, W, k) -> int:
    return int(lib().build_supertree_workspace_size(head.ref, R, D, W, k))


def _opts(markov: bool, n_cand: int, multi_kernel: bool = False):
    if not markov and not n_cand and not multi_kernel:
        return None
    return dt_build_opts((DT_BUILD_MARKOV if markov else 0) |
                         (DT_BUILD_BASE_CANDIDATES if n_cand else 0) |
                         (DT_BUILD_MULTI_KERNEL if multi_kernel else 0), int(n_cand))


def build_supertree(head: Head, h, s0, root_tok, D: int, W: int, k: int, T: float,
                    workspace=None, out=None, stream=None, markov: bool = False,
                    n_cand: int = 0, multi_kernel: bool = False) -> dict:
    """Depth-wise batched supertree construction of R requests.

    h [R][D][d] f32, s0 [R][d] f32, root_tok [R] int32 -> dict of pool_tok,
    pool_parent, pool_score ([R][D][W]) and n_valid ([R][D]).  markov / n_cand
    select the variants of build_supertree_ex (Markov head; children among
    the depth's n_cand base-logit candidates); multi_kernel runs a small fp32
    head through the per-depth kernels instead of the one-launch build."""
    R = s0.shape[0]
    _dev(h, torch.float32, "h", (R, D, head.d))
    _dev(s0, torch.float32, "s0", (R, head.d))
    _dev(root_tok, torch.int32, "root_tok", (R,))
    dev = head.device
    if out is None:
        out = dict(pool_tok=torch.empty((R, D, W), dtype=torch.int32, device=dev),
                   pool_parent=torch.empty((R, D, W), dtype=torch.int32, device=dev),
                   pool_score=torch.empty((R, D, W), dtype=torch.float32, device=dev),
                   n_valid=torch.empty((R, D), dtype=torch.int32, device=dev))
    opts = _opts(markov, n_cand, multi_kernel)
    if opts is None:
        need = build_supertree_workspace_size(head, R, D, W, k)
        ws = _workspace(need, dev, workspace)
        rc = lib().build_supertree(head.ref, _ptr(h), _ptr(s0), _ptr(root_tok), R, D, W, k,
                                   float(T), _ptr(out["pool_tok"]), _ptr(out["pool_parent"]),
                                   _ptr(out["pool_score"]), _ptr(out["n_valid"]), _ptr(ws),
                                   ws.numel(), _stream(stream))
        _check(rc, "build_supertree")
        return out
    need = int(lib().build_supertree_ex_workspace_size(head.ref, R, D, W, k, C.byref(opts)))
    if need == 0:
        raise DartreeError(-1, "build_supertree_ex_workspace_size")
    ws = _workspace(need, dev, workspace)
    rc = lib().build_supertree_ex(head.ref, _ptr(h), _ptr(s0), _ptr(root_tok), R, D, W, k,
                                  float(T), C.byref(opts), _ptr(out["pool_tok"]),
                                  _ptr(out["pool_parent"]), _ptr(out["pool_score"]),
                                  _ptr(out["n_valid"]), _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "build_supertree_ex")
    return out


# the static device scratch of build_supertree_noalloc (DT_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


def build_supertree_noalloc(head: Head, h, s0, root_tok, D: int, W: int, k: int, T: float,
                            out: dict, stream=None) -> dict:
    """build_supertree without a workspace: the library takes its scratch from
    a static per-GPU device array, so the call allocates nothing.  The caller
    passes the outputs (``out``: pool_tok, pool_parent, pool_score, n_valid as
    build_supertree returns them).  Calls that overlap on one GPU race."""
    R = s0.shape[0]
    _dev(h, torch.float32, "h", (R, D, head.d))
    _dev(s0, torch.float32, "s0", (R, head.d))
    _dev(root_tok, torch.int32, "root_tok", (R,))
    _dev(out["pool_tok"], torch.int32, "pool_tok", (R, D, W))
    _dev(out["pool_parent"], torch.int32, "pool_parent", (R, D, W))
    _dev(out["pool_score"], torch.float32, "pool_score", (R, D, W))
    _dev(out["n_valid"], torch.int32, "n_valid", (R, D))
    rc = lib().build_supertree_noalloc(head.ref, _ptr(h), _ptr(s0), _ptr(root_tok), R, D, W, k,
                                       float(T), _ptr(out["pool_tok"]), _ptr(out["pool_parent"]),
                                       _ptr(out["pool_score"]), _ptr(out["n_valid"]),
                                       _stream(stream))
    if rc == -3:
        need = build_supertree_workspace_size(head, R, D, W, k)
        if need > NOALLOC_SCRATCH_BYTES:
            raise DartreeError(rc, f"build_supertree_noalloc: needs {need} bytes of scratch, "
                                   f"the static array holds {NOALLOC_SCRATCH_BYTES}")
    _check(rc, "build_supertree_noalloc")
    return out


def build_tree_sequential_workspace_size(head: Head, D, k, B) -> int:
    return int(lib().build_tree_sequential_workspace_size(head.ref, D, k, B))


def build_tree_sequential(head: Head, h, s0, root_tok, D: int, k: int, B: int, beta: float,
                          T: float, workspace=None, out=None, stream=None) -> dict:
    """Sequential best-first construction of one request, one head call per
    expanded node.

    h [D][d] f32, s0 [d] f32, root_tok [1] int32 -> dict of tok, parent, depth,
    score ([B], pop order) and n ([1])."""
    _dev(h, torch.float32, "h", (D, head.d))
    _dev(s0, torch.float32, "s0", (head.d,))
    _dev(root_tok, torch.int32, "root_tok", (1,))
    dev = head.device
    if out is None:
        out = dict(tok=torch.empty((B,), dtype=torch.int32, device=dev),
                   parent=torch.empty((B,), dtype=torch.int32, device=dev),
                   depth=torch.empty((B,), dtype=torch.int32, device=dev),
                   score=torch.empty((B,), dtype=torch.float32, device=dev),
                   n=torch.empty((1,), dtype=torch.int32, device=dev))
    need = build_tree_sequential_workspace_size(head, D, k, B)
    ws = _workspace(need, dev, workspace)
    rc = lib().build_tree_sequential(head.ref, _ptr(h), _ptr(s0), _ptr(root_tok), D, k, B,
                                     float(beta), float(T), _ptr(out["tok"]),
                                     _ptr(out["parent"]), _ptr(out["depth"]),
                                     _ptr(out["score"]), _ptr(out["n"]), _ptr(ws), ws.numel(),
                                     _stream(stream))
    _check(rc, "build_tree_sequential")
    return out


def head_step_workspace_size(head: Head, rows, k) -> int:
    return int(lib().head_step_workspace_size(head.ref, rows, k))


def state_update(head: Head, s_in, tok, h, workspace=None, stream=None):
    rows = s_in.shape[0]
    _dev(s_in, torch.float32, "s_in", (rows, head.d))
    _dev(tok, torch.int32, "tok", (rows,))
    _dev(h, torch.float32, "h", (head.d,))
    s_out = torch.empty_like(s_in)
    ws = _workspace(head_step_workspace_size(head, rows, 1), head.device, workspace)
    rc = lib().state_update(head.ref, _ptr(s_in), _ptr(tok), _ptr(h), rows, _ptr(s_out),
                            _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "state_update")
    return s_out


def corrected_topk(head: Head, s, k: int, T: float, workspace=None, stream=None):
    rows = s.shape[0]
    _dev(s, torch.float32, "s", (rows, head.d))
    dev = head.device
    tok = torch.empty((rows, k), dtype=torch.int32, device=dev)
    lp = torch.empty((rows, k), dtype=torch.float32, device=dev)
    lse = torch.empty((rows,), dtype=torch.float32, device=dev)
    ws = _workspace(head_step_workspace_size(head, rows, k), dev, workspace)
    rc = lib().corrected_topk(head.ref, _ptr(s), rows, k, float(T), _ptr(tok), _ptr(lp),
                              _ptr(lse), _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "corrected_topk")
    return tok, lp, lse


def prune_topB(pool_score, pool_parent, n_valid, B: int, beta: float, out=None, stream=None):
    R, D, W = pool_score.shape
    _dev(pool_score, torch.float32, "pool_score")
    _dev(pool_parent, torch.int32, "pool_parent", (R, D, W))
    _dev(n_valid, torch.int32, "n_valid", (R, D))
    dev = pool_score.device
    if out is None:
        out = dict(sel_node=torch.empty((R, B), dtype=torch.int32, device=dev),
                   sel_parent=torch.empty((R, B), dtype=torch.int32, device=dev),
                   sel_depth=torch.empty((R, B), dtype=torch.int32, device=dev),
                   n_sel=torch.empty((R,), dtype=torch.int32, device=dev))
    rc = lib().prune_topB(_ptr(pool_score), _ptr(pool_parent), _ptr(n_valid), R, D, W, B,
                          float(beta), _ptr(out["sel_node"]), _ptr(out["sel_parent"]),
                          _ptr(out["sel_depth"]), _ptr(out["n_sel"]), _stream(stream))
    _check(rc, "prune_topB")
    return out


def build_tree_mask(sel_parent, n_sel, out=None, stream=None):
    R, B = sel_parent.shape
    _dev(sel_parent, torch.int32, "sel_parent")
    _dev(n_sel, torch.int32, "n_sel", (R,))
    words = (B + 31) // 32
    if out is None:
        out = torch.empty((R, B, words), dtype=torch.int32, device=sel_parent.device)
    rc = lib().build_tree_mask(_ptr(sel_parent), _ptr(n_sel), R, B, _ptr(out), _stream(stream))
    _check(rc, "build_tree_mask")
    return out


def tree_attention_workspace_size(n_tree, P, Hq, Hkv, hd) -> int:
    return int(lib().tree_attention_workspace_size(n_tree, P, Hq, Hkv, hd))


def tree_attention_verify(q, k_prefix, v_prefix, k_tree, v_tree, mask, scale: float,
                          workspace=None, out=None, stream=None):
    """q [n][Hq][hd], k/v_prefix [P][Hkv][hd], k/v_tree [n][Hkv][hd] bf16;
    mask [n][ceil(n/32)] int32 (bit pattern) -> out [n][Hq][hd] f32."""
    n, Hq, hd = q.shape
    P, Hkv, _ = k_prefix.shape
    for t, nm in ((q, "q"), (k_prefix, "k_prefix"), (v_prefix, "v_prefix"), (k_tree, "k_tree"),
                  (v_tree, "v_tree")):
        _dev(t, torch.bfloat16, nm)
    _dev(mask, torch.int32, "mask", (n, (n + 31) // 32))
    if out is None:
        out = torch.empty((n, Hq, hd), dtype=torch.float32, device=q.device)
    ws = _workspace(tree_attention_workspace_size(n, P, Hq, Hkv, hd), q.device, workspace)
    rc = lib().tree_attention_verify(_ptr(q), _ptr(k_prefix), _ptr(v_prefix), _ptr(k_tree),
                                     _ptr(v_tree), _ptr(mask), n, P, Hq, Hkv, hd,
                                     float(scale), _ptr(out), _ptr(ws), ws.numel(),
                                     _stream(stream))
    _check(rc, "tree_attention_verify")
    return out


def accept_walk_workspace_size(target: Head, R, D, B) -> int:
    return int(lib().accept_walk_workspace_size(target.ref, R, D, B))


def accept_walk(target: Head, h, s0, root_tok, tok, parent, depth, n, tok_index=None,
                workspace=None, out=None, stream=None) -> dict:
    """Acceptance walk of R draft trees against the synthetic greedy target
    `target` (a head of its own).

    h [R][D][d] f32, s0 [R][d] f32, root_tok [R] i32; parent, depth [R][B]
    i32; n [R] i32; tok [R][B] i32, or with tok_index [R][B] i32 any
    [R][stride] i32 that tok_index indexes (build_supertree's pool_tok as
    [R][D*W] with prune_topB's sel_node).  Returns a dict of target_tok
    [R][B+1], path [R][D] and accept_len [R] (tokens per round = accept_len + 1).
    """
    R, D = h.shape[0], h.shape[1]
    B = parent.shape[1]
    _dev(h, torch.float32, "h", (R, D, target.d))
    _dev(s0, torch.float32, "s0", (R, target.d))
    _dev(root_tok, torch.int32, "root_tok", (R,))
    _dev(parent, torch.int32, "parent", (R, B))
    _dev(depth, torch.int32, "depth", (R, B))
    _dev(n, torch.int32, "n", (R,))
    if tok_index is None:
        _dev(tok, torch.int32, "tok", (R, B))
    else:
        _dev(tok_index, torch.int32, "tok_index", (R, B))
        _dev(tok, torch.int32, "tok")
        if tok.dim() != 2 or tok.shape[0] != R:
            raise ValueError("tok must be [R][stride]")
    dev = h.device
    if out is None:
        out = dict(target_tok=torch.empty((R, B + 1), dtype=torch.int32, device=dev),
                   path=torch.empty((R, D), dtype=torch.int32, device=dev),
                   accept_len=torch.empty((R,), dtype=torch.int32, device=dev))
    need = accept_walk_workspace_size(target, R, D, B)
    ws = _workspace(need, dev, workspace)
    rc = lib().accept_walk(target.ref, _ptr(h), _ptr(s0), _ptr(root_tok), R, D, B, _ptr(tok),
                           int(tok.shape[1]), _ptr(tok_index), _ptr(parent), _ptr(depth),
                           _ptr(n), _ptr(out["target_tok"]), _ptr(out["path"]),
                           _ptr(out["accept_len"]), _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "accept_walk")
    return out


def hbm_read_probe(buf, out=None, stream=None):
    """Sum of the 64-bit words of a contiguous device tensor (mod 2^64), read
    once by the streaming probe; returns a device int64 tensor of one element
    (the sum's bits)."""
    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda":
        raise ValueError("buf must be a device tensor")
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    nbytes = buf.numel() * buf.element_size()
    if out is None:
        out = torch.empty(1, dtype=torch.int64, device=buf.device)
    _dev(out, torch.int64, "out", (1,))
    rc = lib().hbm_read_probe(_ptr(buf) if nbytes else None, nbytes, _ptr(out), _stream(stream))
    _check(rc, "hbm_read_probe")
    return out


def mfma_rate_probe(operands, iters, out=None, stream=None):
    """bf16 matrix-core products with operands in registers (see the header):
    `operands` a contiguous bf16 device tensor of at least cus * 32768
    elements, `iters` rounds; returns the device float tensor of cus * 512
    per-thread accumulator sums."""
    if not isinstance(operands, torch.Tensor) or operands.device.type != "cuda":
        raise ValueError("operands must be a device tensor")
    if operands.dtype != torch.bfloat16 or not operands.is_contiguous():
        raise ValueError("operands must be contiguous bfloat16")
    cus = torch.cuda.get_device_properties(operands.device).multi_processor_count
    if out is None:
        out = torch.empty(cus * 512, dtype=torch.float32, device=operands.device)
    _dev(out, torch.float32, "out", (cus * 512,))
    rc = lib().mfma_rate_probe(_ptr(operands), operands.numel() * 2, int(iters), _ptr(out),
                               out.numel(), _stream(stream))
    _check(rc, "mfma_rate_probe")
    return out


def timing_enable(on: bool = True):
    _check(lib().dartree_timing_enable(1 if on else 0), "dartree_timing_enable")


def timing_reset():
    _check(lib().dartree_timing_reset(), "dartree_timing_reset")


def timing_read(kernel: str):
    """(total milliseconds, launches) of a kernel class since the last reset."""
    ms, n = C.c_double(0.0), C.c_int64(0)
    _check(lib().dartree_timing_read(KERNEL_CLASSES[kernel], C.byref(ms), C.byref(n)),
           "dartree_timing_read")
    return ms.value, n.value
