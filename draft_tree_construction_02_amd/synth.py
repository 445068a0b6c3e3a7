"""Seeded synthetic inputs for depth-wise batched draft-supertree construction.

This module draws random tensors and rounds them to the storage precision. It
holds none of the method's arithmetic: no state update, no logits, no softmax,
no selection. Both the fp64 oracle (through the tests) and the HIP path consume
exactly the arrays produced here.

Recipe (stated once, used everywhere):

* ``root = SeedSequence(seed)``; ``root.spawn(3)`` gives the weight stream, the
  request stream and the verification-layer stream, in that order.
* Weight stream ``spawn(4)``: E ``[V][d]``, W1t ``[4d][d]``, W2t ``[d][4d]``,
  Ut ``[V][d]``, each drawn in its storage (row-major, output-feature-major)
  layout. Each tensor is filled in flat chunks of 2**22 elements; chunk ``c``
  draws from ``PCG64(child.spawn(nchunks)[c])`` with ``standard_normal``
  (float32) and is scaled by the tensor's standard deviation.
* Request stream ``spawn(2)``: s0 ``[d]`` and h ``[D][d]`` (float32, N(0,1),
  h multiplied by ``h_scale``).
* Verification stream ``spawn(5)``: q, k_prefix, v_prefix, k_tree, v_tree,
  N(0,1).
* Target stream ``root.spawn(4)[3]`` (the first three children are the ones
  above): the synthetic greedy target of the acceptance walk shares E, W1t
  and W2t with the draft head and has Ut + sigma * (3/sqrt(d)) * N(0,1) as
  its output matrix, drawn like Ut and rounded to the storage type.
* bf16 storage is float32 rounded to nearest, ties to even, on the bit pattern.

The head follows the synthetic correction-head recipe of the workloads:
E, W1, W2 ~ N(0, 0.02^2) and U ~ N(0, (3/sqrt(d))^2).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

CHUNK = 1 << 22

# Mean per-position entropy calibration for the Qwen3-8B-shaped single-request
# build: h is multiplied by this factor so that the mean entropy of the T=1
# corrected distributions over all depths and surviving beam rows is about
# 2 nats.  Written by tests/golden/calibrate_h_scale.py, which runs the fp64
# oracle only; the value is recorded in tests/golden/h_scale_qwen3_8b.json.
H_SCALE_QWEN3_8B = 0.3473


@dataclass(frozen=True)
class Workload:
    """One synthetic supertree workload (shapes, hyper-parameters, seeds)."""
    name: str
    V: int
    d: int
    wdtype: str            # "f32" or "bf16": storage type of E, W1t, W2t, Ut
    D: int                 # draft depths
    W: int                 # layer width (surviving branches per depth)
    k: int                 # children per branch
    B: int                 # verification budget (draft nodes)
    beta: float            # depth bonus (<= 0)
    T: float               # temperature (0 = greedy limit)
    R: int = 1             # independent requests sharing the head
    seeds: tuple = (0,)    # per-request seeds (weights always from seeds[0])
    weight_seed: int = 0
    h_scale: float = 1.0
    root_tok: int = 0
    # optional verification layer (one tree-attention layer)
    attn: dict = field(default_factory=dict)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def workloads() -> dict:
    """The five workloads of the method's evaluation on synthetic Qwen3 shapes."""
    V = 151936
    w = {}
    w["tiny"] = Workload("tiny", V=1000, d=64, wdtype="f32", D=6, W=4, k=4, B=16,
                         beta=-0.1, T=1.0)
    w["qwen3_4b"] = Workload("qwen3_4b", V=V, d=2560, wdtype="bf16", D=16, W=16,
                             k=8, B=64, beta=0.0, T=1.0)
    w["qwen3_4b_t0"] = w["qwen3_4b"].with_(name="qwen3_4b_t0", T=0.0)
    w["qwen3_8b"] = Workload("qwen3_8b", V=V, d=4096, wdtype="bf16", D=16, W=32,
                             k=8, B=128, beta=-0.05, T=1.0,
                             h_scale=H_SCALE_QWEN3_8B)
    w["qwen3_8b_x8"] = Workload("qwen3_8b_x8", V=V, d=4096, wdtype="bf16", D=16,
                                W=16, k=8, B=96, beta=0.0, T=1.0, R=8,
                                seeds=tuple(range(8)))
    w["qwen3_8b_verify"] = w["qwen3_8b"].with_(
        name="qwen3_8b_verify",
        attn=dict(Hq=32, Hkv=8, hd=128, P=4096))
    return w


# ----------------------------------------------------------------------------
# drawing
# ----------------------------------------------------------------------------
def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal(ss: np.random.SeedSequence, n: int, std: float) -> np.ndarray:
    """n float32 N(0, std^2) values, drawn in 2**22-element chunks (see header)."""
    out = np.empty(n, np.float32)
    nch = max(1, (n + CHUNK - 1) // CHUNK)
    kids = ss.spawn(nch)

    def fill(c):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(kids[c]))
        g.standard_normal(out=out[lo:hi], dtype=np.float32)
        if std != 1.0:
            out[lo:hi] *= np.float32(std)

    if nch == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nch)))
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.size, np.uint16)
    nch = max(1, (flat.size + CHUNK - 1) // CHUNK)

    def conv(c):
        lo, hi = c * CHUNK, min(flat.size, (c + 1) * CHUNK)
        u = flat[lo:hi].view(np.uint32)
        r = (u >> 16) & np.uint32(1)
        out[lo:hi] = ((u + r + np.uint32(0x7FFF)) >> 16).astype(np.uint16)

    if nch == 1:
        conv(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(conv, range(nch)))
    return out.reshape(x.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class HeadWeights:
    """Correction-head weights in storage layout.

    For wdtype "bf16" the arrays are uint16 bit patterns; for "f32" float32.
    E [V][d], W1t [4d][d] (W1 transposed), W2t [d][4d], Ut [V][d] (U transposed).
    """
    wdtype: str
    V: int
    d: int
    E: np.ndarray
    W1t: np.ndarray
    W2t: np.ndarray
    Ut: np.ndarray


@dataclass
class Requests:
    s0: np.ndarray        # [R][d] float32
    h: np.ndarray         # [R][D][d] float32
    root_tok: np.ndarray  # [R] int32


def make_head(V: int, d: int, wdtype: str, seed: int = 0) -> HeadWeights:
    wss = np.random.SeedSequence(seed).spawn(3)[0]
    e_ss, w1_ss, w2_ss, u_ss = wss.spawn(4)
    E = _normal(e_ss, V * d, 0.02).reshape(V, d)
    W1t = _normal(w1_ss, 4 * d * d, 0.02).reshape(4 * d, d)
    W2t = _normal(w2_ss, d * 4 * d, 0.02).reshape(d, 4 * d)
    Ut = _normal(u_ss, V * d, 3.0 / math.sqrt(d)).reshape(V, d)
    if wdtype == "bf16":
        E, W1t, W2t, Ut = (bf16_bits(a) for a in (E, W1t, W2t, Ut))
    elif wdtype != "f32":
        raise ValueError(f"unknown wdtype {wdtype!r}")
    return HeadWeights(wdtype, V, d, E, W1t, W2t, Ut)


def make_requests(d: int, D: int, seeds, h_scale: float = 1.0,
                  root_tok: int = 0) -> Requests:
    s0 = np.empty((len(seeds), d), np.float32)
    h = np.empty((len(seeds), D, d), np.float32)
    for r, seed in enumerate(seeds):
        rss = np.random.SeedSequence(seed).spawn(3)[1]
        s_ss, h_ss = rss.spawn(2)
        s0[r] = _normal(s_ss, d, 1.0)
        h[r] = _normal(h_ss, D * d, 1.0).reshape(D, d) * np.float32(h_scale)
    return Requests(s0, h, np.full(len(seeds), root_tok, np.int32))


def make_verify_inputs(n_tree: int, P: int, Hq: int, Hkv: int, hd: int,
                       seed: int = 0) -> dict:
    """bf16 bit patterns of q [n][Hq][hd], k/v prefix [P][Hkv][hd],
    k/v tree [n][Hkv][hd]; all N(0,1) before rounding."""
    ass = np.random.SeedSequence(seed).spawn(3)[2]
    q_ss, kp_ss, vp_ss, kt_ss, vt_ss = ass.spawn(5)
    return dict(
        q=bf16_bits(_normal(q_ss, n_tree * Hq * hd, 1.0).reshape(n_tree, Hq, hd)),
        k_prefix=bf16_bits(_normal(kp_ss, P * Hkv * hd, 1.0).reshape(P, Hkv, hd)),
        v_prefix=bf16_bits(_normal(vp_ss, P * Hkv * hd, 1.0).reshape(P, Hkv, hd)),
        k_tree=bf16_bits(_normal(kt_ss, n_tree * Hkv * hd, 1.0).reshape(n_tree, Hkv, hd)),
        v_tree=bf16_bits(_normal(vt_ss, n_tree * Hkv * hd, 1.0).reshape(n_tree, Hkv, hd)),
    )


def make_target(head: HeadWeights, sigma: float, seed: int = 0) -> HeadWeights:
    """Synthetic target for the acceptance walk: the draft head with its output
    matrix perturbed by N(0, (sigma * 3/sqrt(d))^2) noise (see header)."""
    tss = np.random.SeedSequence(seed).spawn(4)[3]
    noise = _normal(tss, head.V * head.d, sigma * 3.0 / math.sqrt(head.d)).reshape(head.V, head.d)
    if head.wdtype == "bf16":
        noise += bf16_bits_to_f32(head.Ut)
        Ut = bf16_bits(noise)
    else:
        noise += head.Ut
        Ut = noise
    return HeadWeights(head.wdtype, head.V, head.d, head.E, head.W1t, head.W2t, Ut)


def make_workload_inputs(wl: Workload):
    """(HeadWeights, Requests) for a workload."""
    head = make_head(wl.V, wl.d, wl.wdtype, wl.weight_seed)
    req = make_requests(wl.d, wl.D, wl.seeds, wl.h_scale, wl.root_tok)
    return head, req
