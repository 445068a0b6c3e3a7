#!/usr/bin/env python3
"""Throughput of DARTree draft-supertree construction on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input,
with every input already resident in HBM:
  build_supertree (D depths of state update, corrected-logit head, fused
  log-softmax/top-k, beam select) -> prune_topB -> build_tree_mask ->
  tree_attention_verify (one verification layer over the pruned tree).

Prints one JSON line.  `value` is supertree builds per second (R per step).
The roofline object reports the corrected-logit head kernel: algorithmic
bytes per launch (2 d V, the bf16 output head streamed once) divided by its
average launch time measured with HIP events on the launch stream.
The cpu_baseline object times the fp64 oracle on a bounded sample.  Outside
the timed step: sequential_baseline (one head call per expanded node, same
budget) and acceptance (tokens per round of the pruned trees, and of the
sequential tree, under a synthetic greedy target; the walk's own time).

  python bench.py [--steps K] [--warmup W] [--workload qwen3_8b_x8]

The default workload is the largest one that fits one GPU: 8 independent
Qwen3-8B-shaped requests (d=4096, V=151936, D=16, W=16, k=8, B=96 each)
sharing one head, so the head streams once per depth for all 128 rows.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "supertree builds/s (D,W,k,V) + achieved HBM GB/s vs peak; oracle-exact"
HBM_PEAK_GBS = 8000.0
VERIFY = dict(Hq=32, Hkv=8, hd=128, P=4096)   # Qwen3-4B/8B attention layer shape


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def profiled_traffic(workload):
    """HBM bytes per head launch from the committed rocprofv3 counter summary
    (profiles/head_bf16_<workload>.md), or None when absent or when the
    kernel sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"head_bf16_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":", 1)[0] in ("traffic_bytes_per_launch", "source_sha256",
                                                     "sources"):
            k, v = line.split(":", 1)
            fields[k] = v.strip()
    if len(fields) != 3:
        return None
    h = hashlib.sha256()
    for f in fields["sources"].split(", "):
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return int(fields["traffic_bytes_per_launch"]) if h.hexdigest() == fields["source_sha256"] else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_8b_x8")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sequential", action="store_true",
                    help="skip the sequential best-first (one head call per node) comparison")
    ap.add_argument("--no-walk", action="store_true",
                    help="skip the acceptance walk against the synthetic target")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the timing of the step captured in a HIP graph")
    ap.add_argument("--cpu-builds", type=int, default=3,
                    help="oracle builds timed for cpu_baseline (one request per build, "
                         "cycling over the requests of the batch)")
    ap.add_argument("--cpu-budget-s", type=float, default=40.0,
                    help="stop timing further oracle builds once this much CPU time is spent")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times (reference for "
                         "hardware byte counters) and exit")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the method's "
              "hot path runs on a single device, see the design notes on sharding.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": src.numel() * 4}))
        return

    from draft_tree_construction_02_amd import _abi as A
    from draft_tree_construction_02_amd import synth

    wl = synth.workloads()[args.workload]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    t0 = time.time()
    hw, req = synth.make_workload_inputs(wl)
    log(f"[bench] inputs for {wl.name} drawn in {time.time() - t0:.1f}s")

    def up16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    def up(a):
        return up16(a) if a.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    head = A.Head(up(hw.E), up(hw.W1t), up(hw.W2t), up(hw.Ut))
    if wl.wdtype == "bf16":
        # weights are packed once, as at model load; the row-major copies are dropped
        head = head.packed()
        torch.cuda.synchronize()
    h, s0, root = (torch.from_numpy(req.h).to(dev), torch.from_numpy(req.s0).to(dev),
                   torch.from_numpy(req.root_tok).to(dev))
    R, D, W, k, B = wl.R, wl.D, wl.W, wl.k, wl.B
    vx = synth.make_verify_inputs(B, VERIFY["P"], VERIFY["Hq"], VERIFY["Hkv"], VERIFY["hd"],
                                  seed=wl.seeds[0])
    vq, vkp, vvp, vkt, vvt = (up16(vx[n]) for n in ("q", "k_prefix", "v_prefix", "k_tree",
                                                      "v_tree"))
    scale = 1.0 / math.sqrt(VERIFY["hd"])

    pool = dict(pool_tok=torch.empty((R, D, W), dtype=torch.int32, device=dev),
                pool_parent=torch.empty((R, D, W), dtype=torch.int32, device=dev),
                pool_score=torch.empty((R, D, W), dtype=torch.float32, device=dev),
                n_valid=torch.empty((R, D), dtype=torch.int32, device=dev))
    sel = dict(sel_node=torch.empty((R, B), dtype=torch.int32, device=dev),
               sel_parent=torch.empty((R, B), dtype=torch.int32, device=dev),
               sel_depth=torch.empty((R, B), dtype=torch.int32, device=dev),
               n_sel=torch.empty((R,), dtype=torch.int32, device=dev))
    mask = torch.empty((R, B, (B + 31) // 32), dtype=torch.int32, device=dev)
    ws = torch.empty(A.build_supertree_workspace_size(head, R, D, W, k), dtype=torch.uint8,
                     device=dev)
    aws = torch.empty(A.tree_attention_workspace_size(B, VERIFY["P"], VERIFY["Hq"],
                                                      VERIFY["Hkv"], VERIFY["hd"]),
                      dtype=torch.uint8, device=dev)
    aout = torch.empty((B, VERIFY["Hq"], VERIFY["hd"]), dtype=torch.float32, device=dev)

    def step():
        A.build_supertree(head, h, s0, root, D, W, k, wl.T, workspace=ws, out=pool)
        A.prune_topB(pool["pool_score"], pool["pool_parent"], pool["n_valid"], B, wl.beta,
                     out=sel)
        A.build_tree_mask(sel["sel_parent"], sel["n_sel"], out=mask)
        # verification layer over request 0's pruned tree (rows >= n_sel are empty)
        A.tree_attention_verify(vq, vkp, vvp, vkt, vvt, mask[0], scale, workspace=aws, out=aout)

    def leg(name, fn):
        # an extra measurement that fails is recorded in its field; the line still prints
        try:
            return fn()
        except Exception as exc:          # noqa: BLE001 - recorded in the line, not hidden
            log(f"[bench] {name} failed: {type(exc).__name__}: {exc}")
            return {"error": f"{type(exc).__name__}: {exc}"[:300]}

    # the matrix-core probe once before any step (and once after the timed steps, below)
    mprobe_before = leg("matrix-core probe", lambda: mfma_probe(A, torch, dev))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def build_only():
        A.build_supertree(head, h, s0, root, D, W, k, wl.T, workspace=ws, out=pool)

    def build_prune_mask():
        build_only()
        A.prune_topB(pool["pool_score"], pool["pool_parent"], pool["n_valid"], B, wl.beta,
                     out=sel)
        A.build_tree_mask(sel["sel_parent"], sel["n_sel"], out=mask)

    def timed_region(fn, per_kernel: bool):
        # events between consecutive steps give the per-step distribution;
        # the region's total (events and host wall clock) gives the throughput
        A.timing_reset()
        A.timing_enable(per_kernel)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        ev[0].record()
        for i in range(args.steps):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        A.timing_enable(False)
        per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
        return ev[0].elapsed_time(ev[-1]), wall, per

    def pct(v, q):
        return v[min(len(v) - 1, int(q * len(v)))]

    ev_ms, wall, per = timed_region(step, False)
    ms_per_step = max(ev_ms, wall * 1e3) / args.steps
    log(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step (events {ev_ms:.1f} ms, "
        f"wall {wall * 1e3:.1f} ms; median {pct(per, 0.5):.3f}, p10 {pct(per, 0.1):.3f}, "
        f"p90 {pct(per, 0.9):.3f} ms)")
    # build alone, and build + prune + mask (no verification layer)
    b_ms, b_wall, b_per = timed_region(build_only, False)
    bpm_ms, bpm_wall, bpm_per = timed_region(build_prune_mask, False)
    # the full steps again with every library launch bracketed by HIP events
    pk_ms, _, _ = timed_region(step, True)
    kern = {}
    for name in ("gemm1", "gemm2", "reduce", "head", "head128", "merge_select", "attention",
                 "build_small"):
        tot, n = A.timing_read(name)
        kern[name] = dict(launches=n, avg_us=(tot * 1e3 / n) if n else None)
    wbytes = 2 if wl.wdtype == "bf16" else 4
    one_launch = (kern["head"]["launches"] == 0 and kern["head128"]["launches"] == 0
                  and kern["build_small"]["launches"] > 0)
    # the dominant head kernel: the 128-row one when the batch has 128 rows (the
    # first depths then run at their live width on the smaller kernels)
    head_cls = "head128" if kern["head128"]["launches"] > 0 else "head"
    if one_launch:
        # a small fp32 head built in one launch: every depth reads U, W1 and W2
        head_us = kern["build_small"]["avg_us"]
        head_bytes = D * wbytes * (wl.d * wl.V + 8 * wl.d * wl.d)
    else:
        head_us = kern[head_cls]["avg_us"]
        head_bytes = wbytes * wl.d * wl.V      # the output head, streamed once per launch
    achieved = head_bytes / (head_us * 1e-6) / 1e9
    log(f"[bench] head kernel {head_us:.1f} us/launch -> {achieved:.0f} GB/s; "
        f"per-kernel timed region {pk_ms / args.steps:.3f} ms/step")

    # hipGraph on/off: the same step captured once and replayed
    graph_res = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        g_ms, g_wall, g_per = timed_region(graph.replay, False)
        g_step = max(g_ms, g_wall * 1e3) / args.steps
        graph_res = {"ms_per_step": round(g_step, 4), "builds_per_s": round(R * 1e3 / g_step, 3),
                     "median_ms": round(pct(g_per, 0.5), 4)}
        log(f"[bench] step replayed from a HIP graph: {g_step:.3f} ms/step "
            f"(eager {ms_per_step:.3f})")
        del graph
    probe = hbm_probe(A, torch, dev)
    mprobe = {"before_steps": mprobe_before,
              "after_steps": leg("matrix-core probe", lambda: mfma_probe(A, torch, dev))}
    log(f"[bench] read probe: {probe['bytes'] / 2 ** 30:.0f} GiB in {probe['us']:.1f} us "
        f"-> {probe['gbs']:.0f} GB/s")

    builds_per_s = R * 1e3 / ms_per_step
    # verification layer: QK^T and PV over prefix + tree keys for every query head
    attn_flops = 4.0 * B * (VERIFY["P"] + B) * VERIFY["hd"] * VERIFY["Hq"]
    attn_us = kern["attention"]["avg_us"]
    rows_p = next(m for m in (16, 32, 64, 128) if m >= R * W)   # padded batch rows
    if one_launch:
        head_kernel = "k_build_small: all depths of the build in one launch"
    elif head_cls == "head128":
        head_kernel = ("k_head_rows128 (one 8-wave workgroup per compute unit, operands by LDS DMA, "
                       "32x32x16 MFMA): the launches of the depths that run 128 rows")
    elif wl.wdtype != "bf16" or rows_p < 64:
        head_kernel = "k_head_bf16" if wl.wdtype == "bf16" else "k_head_f32"
    else:
        head_kernel = f"k_head_wide (64 columns per wave, {rows_p} rows)"

    # weights streamed per step: U (d V) + W1 and W2 (8 d^2) per depth, shared by R requests
    bytes_per_step = D * wbytes * (wl.d * wl.V + 8 * wl.d * wl.d)
    res = {
        "metric": METRIC,
        "value": round(builds_per_s, 3),
        "unit": "builds/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.wdtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "D": D, "W": W, "k": k, "V": wl.V, "d": wl.d, "R": R,
                   "B": B, "beta": wl.beta, "T": wl.T,
                   "verify_layer": dict(VERIFY, n_tree=B)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": profiled_traffic(wl.name),
                     "kernel": (head_kernel if one_launch
                                else f"corrected-logit head ({head_kernel})"),
                     "bytes_per_launch": head_bytes,
                     "probe_gbs": probe["gbs"],
                     "frac_of_probe": round(achieved / probe["gbs"], 4)},
        "hbm_probe": probe,
        "mfma_probe": mprobe,
        "graph": graph_res,
        "step_ms": {"mean": round(ms_per_step, 4), "median": round(pct(per, 0.5), 4),
                    "p10": round(pct(per, 0.1), 4), "p90": round(pct(per, 0.9), 4)},
        "builds_per_s_build_only": round(R * 1e3 * args.steps / max(b_ms, b_wall * 1e3), 3),
        "builds_per_s_build_prune_mask": round(R * 1e3 * args.steps / max(bpm_ms, bpm_wall * 1e3),
                                               3),
        "attention": {"us": round(attn_us, 2) if attn_us else None, "flop": attn_flops,
                      "tflops": round(attn_flops / (attn_us * 1e-6) / 1e12, 2) if attn_us else None,
                      "frac_of_bf16_dense_peak": round(attn_flops / (attn_us * 1e-6) / 2.5e15, 4)
                      if attn_us else None},
        "kernels_us": {n: (round(v["avg_us"], 2) if v["avg_us"] else None) for n, v in kern.items()},
        "weight_bytes_per_step": bytes_per_step,
        "step_weight_stream_gbs": round(bytes_per_step / (ms_per_step * 1e-3) / 1e9, 1),
    }

    # the extra legs below report beside the headline; if one of them fails,
    # the line still carries the measurement, with the failure in its field
    seq_tree = None
    if wl.R == 1 and not args.no_sequential:
        out = leg("sequential baseline", lambda: sequential_baseline(
            A, head, h, s0, root, wl, b_ms, b_wall, bpm_ms, bpm_wall, args.steps))
        if isinstance(out, tuple):
            res["sequential_baseline"], seq_tree = out
        else:
            res["sequential_baseline"] = out
    if not args.no_walk:
        res["acceptance"] = leg("acceptance walk", lambda: acceptance(
            A, synth, hw, wl, up, h, s0, root, pool, sel, seq_tree))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = leg("cpu baseline", lambda: cpu_baseline(
            wl, hw, req, max(args.cpu_builds, wl.R), args.cpu_budget_s))
    print(json.dumps(res), flush=True)


def mfma_probe(A, torch, dev, iters=297, reps=10):
    """bf16 matrix-core rate with operands in registers, for operands that
    are all 1.0 and for seeded N(0,1) operands: iters = 297 rounds are 9504
    `32x32x16` products per SIMD, the 128-row head's hi/lo products per launch
    at d = 4096, V = 151936.  Timed with events over `reps` calls; the constant
    run's sums are checked exactly.  The bench runs it before the warm-up steps
    and after the timed steps: the rate depends on the part's state."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    n = cus * 32768
    g = torch.Generator(device="cpu").manual_seed(5)
    bufs = {"constant": torch.ones(n, dtype=torch.bfloat16, device=dev),
            "random": torch.randn(n, generator=g).to(torch.bfloat16).to(dev)}
    out = torch.empty(cus * 512, dtype=torch.float32, device=dev)
    flop = cus * 8 * iters * 16 * 32768
    res = {"products_per_simd": 2 * iters * 16, "flop_per_call": flop}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for name, buf in bufs.items():
        for _ in range(2):
            A.mfma_rate_probe(buf, iters, out=out)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            A.mfma_rate_probe(buf, iters, out=out)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        if name == "constant" and not bool(torch.all(out == 4096.0 * iters)):
            raise RuntimeError("matrix-core probe returned a wrong sum")
        res[name] = {"us": round(us, 2), "tflops": round(flop / (us * 1e-6) / 1e12, 1)}
    del bufs
    return res


def hbm_probe(A, torch, dev, nbytes=2 << 30, reps=10):
    """Practical read bandwidth: the library's streaming read probe over a
    2 GiB buffer, averaged over `reps` calls timed with events on the stream it
    runs on (each call is a one-thread clear kernel plus the read)."""
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    out = torch.empty(1, dtype=torch.int64, device=dev)
    for _ in range(2):
        A.hbm_read_probe(buf, out=out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        A.hbm_read_probe(buf, out=out)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    # every 64-bit word holds two int32 ones: 2^32 + 1
    got = int(out.cpu().numpy().view("uint64")[0])
    if got != (nbytes // 8) * (2 ** 32 + 1) % 2 ** 64:
        raise RuntimeError("read probe returned a wrong sum")
    del buf
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "us": round(us, 2), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1)}


def sequential_baseline(A, head, h, s0, root, wl, b_ms, b_wall, bpm_ms, bpm_wall, steps):
    """The per-node construction the pages set against depth-wise batching:
    best-first with one head call per expanded node (same head, same B), timed
    over a few trees, next to the batched build + prune + mask of the same
    request."""
    import torch
    D, k, B = wl.D, wl.k, wl.B
    ws = torch.empty(A.build_tree_sequential_workspace_size(head, D, k, B), dtype=torch.uint8,
                     device="cuda:0")
    out = None
    h0, s00, r0 = h[0].contiguous(), s0[0].contiguous(), root[:1].contiguous()
    for _ in range(2):
        out = A.build_tree_sequential(head, h0, s00, r0, D, k, B, wl.beta, wl.T, workspace=ws,
                                      out=out)
    torch.cuda.synchronize()
    trees = 5
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for _ in range(trees):
        A.build_tree_sequential(head, h0, s00, r0, D, k, B, wl.beta, wl.T, workspace=ws, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = max(e0.elapsed_time(e1), (time.perf_counter() - w0) * 1e3) / trees
    n = int(out["n"][0].item())
    # head calls: the root plus every popped node that is neither the last one nor at depth D
    depth = out["depth"][:n].cpu().numpy()
    calls = 1 + int(sum(1 for i in range(n - 1) if depth[i] < D))
    batched_ms = max(bpm_ms, bpm_wall * 1e3) / steps / wl.R
    log(f"[bench] sequential best-first: {ms:.2f} ms/tree, {calls} head calls; batched build + "
        f"prune + mask {batched_ms:.3f} ms/tree ({ms / batched_ms:.2f}x)")
    return ({"ms_per_tree": round(ms, 3), "head_calls": calls, "nodes": n,
             "batched_ms_per_tree": round(batched_ms, 4), "batched_head_calls": D,
             "latency_ratio": round(ms / batched_ms, 3)}, out)


TARGET_SIGMA = 0.1


def acceptance(A, synth, hw, wl, up, h, s0, root, pool, sel, seq_tree):
    """Tokens per verification round of the step's pruned trees (and of the
    sequential tree of the same budget B, one request) under the synthetic
    greedy target: the draft head with its output matrix perturbed.  Not part
    of the timed step; the walk itself is timed separately."""
    import torch
    t0 = time.time()
    thw = synth.make_target(hw, TARGET_SIGMA, wl.weight_seed)
    target = A.Head(up(thw.E), up(thw.W1t), up(thw.W2t), up(thw.Ut))
    if wl.wdtype == "bf16":
        target = target.packed()
    torch.cuda.synchronize()
    R, D, W, B = wl.R, wl.D, wl.W, wl.B
    ws = torch.empty(A.accept_walk_workspace_size(target, R, D, B), dtype=torch.uint8,
                     device="cuda:0")

    def walk_pool(out=None):
        return A.accept_walk(target, h, s0, root, pool["pool_tok"].view(R, D * W),
                             sel["sel_parent"], sel["sel_depth"], sel["n_sel"],
                             tok_index=sel["sel_node"], workspace=ws, out=out)
    out = walk_pool()
    torch.cuda.synchronize()
    reps = 5
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        walk_pool(out)
    e1.record()
    torch.cuda.synchronize()
    walk_ms = e0.elapsed_time(e1) / reps
    tau_b = [int(x) + 1 for x in out["accept_len"].cpu().tolist()]
    res = {"target": f"draft head with U + N(0, ({TARGET_SIGMA} * 3/sqrt(d))^2), greedy",
           "B": B, "nodes_batched": [int(x) for x in sel["n_sel"].cpu().tolist()],
           "tau_batched": tau_b, "walk_ms": round(walk_ms, 3)}
    if seq_tree is not None:
        wsq = A.accept_walk(target, h, s0, root, seq_tree["tok"][None], seq_tree["parent"][None],
                            seq_tree["depth"][None], seq_tree["n"])
        res["nodes_sequential"] = int(seq_tree["n"][0].item())
        res["tau_sequential"] = int(wsq["accept_len"][0].item()) + 1
    log(f"[bench] acceptance walk ({time.time() - t0:.1f}s incl. target): tokens/round "
        f"batched {tau_b}" + (f", sequential {res['tau_sequential']}" if seq_tree is not None
                              else "") + f"; walk {walk_ms:.2f} ms")
    del target
    torch.cuda.empty_cache()
    return res


def cpu_baseline(wl, hw, req, nbuilds, budget_s):
    """The fp64 oracle as it stands, on this host's cores, on a bounded sample:
    full builds (all D depths) plus prune and mask of the workload's requests,
    one request per build in order (request r % R), up to `nbuilds` builds or
    until `budget_s` seconds have been spent; the value is builds per second
    of oracle time (the median build for a single request)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import dartree_oracle as O
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores, user_api="blas"):
        t0 = time.time()
        ohead = O.OracleHead(hw.wdtype, hw.E, hw.W1t, hw.W2t, hw.Ut)
        prep = time.time() - t0
        times, done = [], []
        for i in range(nbuilds):
            r = i % wl.R
            t1 = time.perf_counter()
            tree = O.build_supertree(ohead, req.h[r], req.s0[r], int(req.root_tok[r]), wl.D,
                                     wl.W, wl.k, wl.T)
            vt = O.prune_topB(tree.score, tree.parent, tree.n_valid, wl.B, wl.beta)
            O.tree_mask(vt.parent, vt.n, wl.B)
            times.append(time.perf_counter() - t1)
            done.append(r)
            if sum(times) >= budget_s:
                break
        info = threadpool_info()
    blas_threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"]
                       or [1])
    if wl.R > 1:
        value = len(times) / sum(times)
        how = (f"{len(times)} full fp64 oracle builds, requests {sorted(set(done))} of "
               f"{wl.R} ({wl.name}: D={wl.D}, W={wl.W}, k={wl.k}, d={wl.d}), each + prune + "
               f"mask; builds per second of total oracle time")
    else:
        value = 1.0 / sorted(times)[len(times) // 2]
        how = (f"{len(times)} full fp64 oracle build(s) of request 0 ({wl.name}: D={wl.D}, "
               f"W={wl.W}, k={wl.k}, d={wl.d}) + prune + mask; median")
    log(f"[bench] oracle: {len(times)} builds in {sum(times):.1f}s -> {value:.4f} builds/s "
        f"(weights widened in {prep:.1f}s), {cores} cores, {blas_threads} BLAS threads")
    return {"value": round(value, 5), "unit": "builds/s", "cores": cores, "kind": "oracle",
            "sample": how + f"; weight widening ({prep:.1f}s) excluded; budget {budget_s:.0f}s",
            "seconds": round(sum(times), 2), "blas_threads": blas_threads,
            "blas": ",".join(sorted({i.get('internal_api', '?') for i in info}))}


if __name__ == "__main__":
    main()
