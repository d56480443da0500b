"""Benchmark of one full tree-verification step on one MI355X.

A step = tree_build -> tree_mask_positions -> tree_attention -> tree_accept ->
kv_compact over one batch of synthetic inputs, all through the C ABI on one HIP
stream (by default through tree_build_meta, tree_attention, tree_accept_compact:
the same five stages in two kernel launches fewer; --unfused runs five calls).
The default workload is the largest one that fits one GPU: 64 requests over
4096-token prefixes with random trees of 8..64 nodes (depth <= 7), Llama-3-8B
attention heads 32/8/128, bf16, ~1.1 GB of K/V (the tree-build stage is the
metadata call, the trees being given); --config 1..4 selects another of the five
workloads (2: the EAGLE-2 dynamic tree at batch 1, top_k 10, depth 6, 60 draft
nodes + root over a 2048-token prefix), and
--paged N keeps the K/V cache in a paged pool of N-token blocks placed at seeded
random physical blocks (tree_attention_paged, tree_accept_compact_paged /
kv_compact_paged through the block table).

Inputs are resident in HBM before the timed region.  Input copies are rotated
(>= --rotate-mb of them) so that repeated steps stream from HBM instead of the
256 MB last-level cache.  The steps are timed twice: launched eagerly call by call
(HIP events around every attention call give the kernel's roofline figures), and
replayed from HIP graphs captured once per input copy (the headline rate; the
same kernels and arguments, without per-call host launch overhead; --no-graph
reports the eager rate instead).  Prints ONE JSON line on stdout; diagnostics go
to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 5]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
FP32_PEAK_TFLOPS = 157.3     # MI355X fp32 vector, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attention_work(w, tree_size, depth, status):
    """Algorithmic bytes and flops of one tree_attention call: each visible K/V row is
    read once per kv head, Q read and O written once, the packed mask read once;
    flops count QK^T and PV over the visible keys only (prefix + ancestors + self)."""
    eb = 2 if w.dtype == "bf16" else 4
    W = (w.T_max + 31) // 32
    nbytes = 0
    flops = 0
    for b in range(w.B):
        T = 1 if status[b] != 0 else int(tree_size[b])
        P = int(w.prefix_len[b])
        nbytes += (P + T) * w.Hkv * w.d * eb * 2 + 2 * T * w.Hq * w.d * eb + T * W * 4
        flops += sum(w.Hq * 4 * w.d * (P + int(depth[b, i]) + 1) for i in range(T))
    return nbytes, flops


def source_hash():
    """Hash of the attention source's code: // comments and blank lines are dropped,
    so an edit to comments alone keeps the counter record valid."""
    path = os.path.join(ROOT, "tree_attention_verification_amd", "csrc", "tree_attention.hip")
    with open(path) as f:
        lines = []
        for line in f.read().split("\n"):
            i = line.find("//")
            line = (line[:i] if i >= 0 else line).rstrip()
            if line:
                lines.append(line)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def machine_peaks(torch):
    """What this GPU sustains right now on plain library work, to put the roofline
    fractions next to: a 1 GiB device copy (torch) and an 8192^3 bf16 GEMM
    (torch.matmul, hipBLASLt).  Measured under the same power and clock limits as
    the step, so they sit below the published peaks."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * n * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    m = 8192
    x = torch.randn(m, m, device="cuda", dtype=torch.bfloat16)
    y = torch.randn(m, m, device="cuda", dtype=torch.bfloat16)
    torch.matmul(x, y)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        torch.matmul(x, y)
    e1.record()
    torch.cuda.synchronize()
    gemm_tf = 2 * m ** 3 * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del x, y
    torch.cuda.empty_cache()
    return {"hbm_copy_GBps": round(copy_gbs, 1), "bf16_gemm_TFLOPs": round(gemm_tf, 1),
            "what": "1 GiB device copy (read + write bytes) and 8192^3 bf16 torch.matmul on this GPU in this run"}


def measured_traffic(workload_name):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current attention source (else None)."""
    path = os.path.join(ROOT, "profiles", "attention_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get("workloads", {}).get(workload_name)
    if not ent or ent.get("source_sha") != source_hash():
        return None
    return ent.get("hbm_bytes_per_launch")


def cpu_baseline(w, seconds: float, paged=None):
    """The oracle, as it stands, on a bounded sample of the same workload (with a paged
    cache: the oracle's paged attention and compaction through the block table)."""
    from oracle import attention as oa
    from oracle import kv as okv
    from oracle import tree as ot
    from workloads import gen
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1

    def one_step(ws):
        t = ot.tree_build(ws)
        m = ot.tree_mask_positions(t["parents"], t["tree_size"], ws.prefix_len, ws.T_max, ws.dcap,
                                   t["status"] if ws.mode != "given" else None)
        tp = gen.synthetic_target_predict(ws, t["draft_tokens"], t["parents"], t["tree_size"])
        a = ot.tree_accept(t["draft_tokens"], t["parents"], t["tree_size"], tp, m["status"], ws.dcap)
        if paged is None:
            oa.tree_attention(ws.Q, ws.Kc, ws.Vc, ws.prefix_len, t["tree_size"], m["tree_mask"], status=m["status"])
            okv.kv_compact(ws.Kc, ws.Vc, ws.prefix_len, a["accept_path"], a["accept_len"])
        else:
            table = paged.block_table[:ws.B]
            oa.tree_attention_paged(ws.Q, paged.K_pool, paged.V_pool, table, paged.tokens_per_block, ws.prefix_len,
                                    t["tree_size"], m["tree_mask"], status=m["status"])
            okv.kv_compact_paged(paged.K_pool, paged.V_pool, table, paged.tokens_per_block, ws.prefix_len,
                                 a["accept_path"], a["accept_len"])
        return int(np.where(m["status"] != 0, 1, t["tree_size"]).sum())

    # sample: the first requests of the batch, as many as fit the time budget
    import copy
    nb = w.B
    sample = w
    t0 = time.perf_counter()
    nodes = one_step(sample)
    dt = time.perf_counter() - t0
    while dt > seconds and nb > 1:
        nb = max(1, nb // 2)
        sample = copy.copy(w)
        for k in ("logprobs", "root_token", "given_parents", "given_tokens", "given_size", "prefix_len", "Q", "Kc",
                  "Vc", "tgt_u", "tgt_choice", "tgt_rand"):
            v = getattr(w, k)
            if v is not None:
                setattr(sample, k, v[:nb])
        sample.B = nb
        t0 = time.perf_counter()
        nodes = one_step(sample)
        dt = time.perf_counter() - t0
    reps, total_nodes, total_t = 1, nodes, dt
    while total_t < seconds:
        t0 = time.perf_counter()
        total_nodes += one_step(sample)
        total_t += time.perf_counter() - t0
        reps += 1
    return {"value": total_nodes / total_t, "unit": "tree-nodes/s", "cores": int(threads), "kind": "oracle",
            "host_cpu_count": os.cpu_count(),
            "sample": f"{reps} full step(s) of the first {nb} of {w.B} request(s) ({total_t:.1f} s; tree ops "
                      f"single-threaded, float64 attention on {threads} BLAS thread(s))"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=5)
    ap.add_argument("--rotate-mb", type=float, default=512.0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the copy / GEMM measurement of what this GPU sustains (reported beside the roofline)")
    ap.add_argument("--unfused", action="store_true",
                    help="run the step as the five separate calls (default: tree_build_meta, tree_attention, "
                         "tree_accept_compact -- the same five stages in two kernel launches fewer)")
    ap.add_argument("--paged", type=int, default=0, metavar="N",
                    help="keep the K/V cache in a paged pool of N-token blocks (a power of two, 1..1024)")
    ap.add_argument("--layerwise", choices=["logprobs", "logits"], default=None,
                    help="build the dynamic tree one draft layer at a time (tree_build_layer x (D+1), then "
                         "tree_build_finish with the metadata), from log-prob rows or raw logits")
    ap.add_argument("--sampling", action="store_true",
                    help="accept by target-only tree rejection sampling (tree_accept_sample, then the compaction) "
                         "from synthetic target distributions instead of the greedy walk")
    ap.add_argument("--sampling-from", choices=["probs", "logits", "draft"], default="probs",
                    help="with --sampling: probs = synthetic target distributions (tree_accept_sample); logits = "
                         "synthetic target logits filtered per request (tree_sampling_probs, then "
                         "tree_accept_sample); draft = the same filtered rows sampled against synthetic drafter "
                         "distributions (tree_sampling_probs, then tree_accept_sample_draft)")
    ap.add_argument("--tree-nodes", type=int, default=None, metavar="N",
                    help="grow the trees to N nodes (65..256; T_max = N): dynamic workloads keep N - 1 draft "
                         "nodes, the random-tree workload draws sizes in [8, N]")
    ap.add_argument("--copy-mb", type=float, default=0.0,
                    help="before warmup, one device-to-device copy of this many MiB (a plain copy kernel of known "
                         "size that calibrates the HBM byte counters of a profiler run)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (requests or kv heads would be "
              "sharded across GPUs with no exchange; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from tree_attention_verification_amd import _lib
    from tree_attention_verification_amd.step import TreeVerifyStep
    from workloads import gen

    _lib.lib()
    torch.cuda.set_device(0)
    w = gen.make_workload(args.config, tree_nodes=args.tree_nodes)
    if args.tree_nodes:
        w.name = f"{w.name}+trees{args.tree_nodes}"
    paged = gen.paged_layout(w, args.paged) if args.paged else None
    kv_bytes = (w.Kc.nbytes + w.Vc.nbytes) if paged is None else (paged.K_pool.nbytes + paged.V_pool.nbytes)
    per_copy = w.Q.nbytes + kv_bytes + (w.logprobs.nbytes if w.logprobs is not None else 0)
    n_copies = max(1, min(64, math.ceil(args.rotate_mb * 2 ** 20 / per_copy)))
    workload = w.name if paged is None else f"{w.name}+paged{args.paged}"
    log(f"workload {workload}: {per_copy / 2**20:.1f} MiB of inputs per copy, {n_copies} copies rotated")
    step = TreeVerifyStep(w, n_copies=n_copies, paged=paged)
    if args.layerwise:
        if w.mode != "dynamic":
            print("--layerwise needs a dynamic-tree workload (--config 2, 3 or 4)", file=sys.stderr)
            sys.exit(2)
        rows = gen.draft_logits(w.cfg_id, w.B, w.rows_per_req, w.V) if args.layerwise == "logits" else None
        step.prepare_layers(rows=rows, logits=args.layerwise == "logits", n_copies=n_copies)
    stream = torch.cuda.current_stream()

    if args.copy_mb > 0:
        n = int(args.copy_mb * 2 ** 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {n} bytes read, {n} bytes written")
        del src, dst

    # the synthetic target's argmax needs the tree: build once and read it back (untimed)
    step.build()
    step.meta()
    torch.cuda.synchronize()
    th = step.tree_host()
    mh = step.meta_host()
    step.set_target_predict(gen.synthetic_target_predict(w, th["draft_tokens"], th["parents"], th["tree_size"]))
    if args.sampling:
        probs, uni = gen.synthetic_target_probs(w, th["draft_tokens"], th["parents"], th["tree_size"])
        step.set_target_probs(probs, uni)
        del probs
        if args.sampling_from != "probs":
            q = (gen.synthetic_draft_probs(w, th["draft_tokens"], th["parents"], th["tree_size"])
                 if args.sampling_from == "draft" else None)
            step.set_sampling_inputs(gen.synthetic_target_logits(w, th["tree_size"]), gen.sampling_params(w, w.B), q)
            del q
    torch.cuda.synchronize()
    status = mh["status"]
    nodes = int(np.where(status != 0, 1, th["tree_size"]).sum())

    def one(k, ev=None):
        step.copy = k % n_copies
        if args.layerwise:
            step.build_layers(meta=True)
        elif args.unfused:
            step.build()
            step.meta()
        else:
            step.build_meta()
        if ev is not None:
            ev[0].record(stream)
        step.attention()
        if ev is not None:
            ev[1].record(stream)
        if args.sampling:
            if ev is not None:
                ev[2].record(stream)
            if args.sampling_from != "probs":
                step.sampling_probs()
            if ev is not None:
                ev[3].record(stream)
            if args.sampling_from == "draft":
                step.accept_sample_draft()
            else:
                step.accept_sample()
            if ev is not None:
                ev[4].record(stream)
            step.compact()
        elif args.unfused:
            step.accept()
            step.compact()
        else:
            step.accept_compact()

    # eager launches, with HIP events around the attention call of every step
    for k in range(args.warmup):
        one(k)
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(5)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        one(args.warmup + k, evs[k])
    torch.cuda.synchronize()
    eager_elapsed = time.perf_counter() - t0
    attn_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    sampling_us = None
    if args.sampling:
        sampling_us = {"tree_sampling_probs": round(float(np.mean([e[2].elapsed_time(e[3]) for e in evs])) * 1e3, 2)
                       if args.sampling_from != "probs" else None,
                       ("tree_accept_sample_draft" if args.sampling_from == "draft" else "tree_accept_sample"):
                       round(float(np.mean([e[3].elapsed_time(e[4]) for e in evs])) * 1e3, 2)}
    ms_per_step_eager = eager_elapsed * 1e3 / args.steps

    # the same steps replayed from captured HIP graphs (one per input copy), the way
    # a serving loop launches a fixed-shape verification step
    ms_per_step = ms_per_step_eager
    launch = "eager"
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for k in range(3):
                one(k)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for c in range(n_copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                one(c)
            graphs.append(g)
        torch.cuda.synchronize()
        for k in range(args.warmup):
            graphs[k % n_copies].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            graphs[(args.warmup + k) % n_copies].replay()
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
        launch = "hip_graph"
        stream = torch.cuda.current_stream()

    # stage breakdown (untimed extra pass, events between every call)
    names = ["tree_build", "tree_mask_positions", "tree_attention", "tree_accept", "kv_compact"]
    reps = min(50, args.steps)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(reps)]
    for r in range(reps):
        step.copy = r % n_copies
        ev[r][0].record(stream)
        step.build(); ev[r][1].record(stream)
        step.meta(); ev[r][2].record(stream)
        step.attention(); ev[r][3].record(stream)
        step.accept(); ev[r][4].record(stream)
        step.compact(); ev[r][5].record(stream)
    torch.cuda.synchronize()
    stages = {n: round(float(np.mean([ev[r][i].elapsed_time(ev[r][i + 1]) for r in range(reps)])) * 1e3, 2)
              for i, n in enumerate(names)}

    peaks = None if args.no_peaks else machine_peaks(torch)
    nbytes, flops = attention_work(w, th["tree_size"], mh["tree_position_ids"], status)
    t_attn = attn_ms * 1e-3
    mfma_peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
    if nbytes / (HBM_PEAK_GBS * 1e9) >= flops / (mfma_peak * 1e12):
        roof = {"bound": "hbm", "achieved": round(nbytes / t_attn / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma" if w.dtype == "bf16" else "alu", "achieved": round(flops / t_attn / 1e12, 2),
                "peak": mfma_peak, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    if peaks:
        ref = peaks["hbm_copy_GBps"] if roof["unit"] == "GB/s" else peaks["bf16_gemm_TFLOPs"]
        if roof["bound"] in ("hbm", "mfma"):
            roof["frac_of_measured"] = round(roof["achieved"] / ref, 4)
    roof["traffic"] = measured_traffic(workload)
    roof["kernel"] = (("tree_attention" if paged is None else "tree_attention_paged") +
                      " call (k_attn_bf16 + k_attn_combine when the keys are split)")
    roof["algorithmic_bytes"] = int(nbytes)
    roof["algorithmic_flops"] = int(flops)
    roof["avg_us"] = round(attn_ms * 1e3, 3)

    out = {
        "metric": "tree-verify nodes/sec (batch x tree) + % of HBM/MFMA roofline, 1 MI355X",
        "value": round(nodes / (ms_per_step * 1e-3), 1),
        "unit": "tree-nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_eager": round(ms_per_step_eager, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded draft log-probs, Q/K/V and target " +
                ({"probs": "distributions", "logits": "logits and per-request sampling parameters",
                  "draft": "logits, per-request sampling parameters and drafter distributions"}[args.sampling_from]
                 if args.sampling else "argmax") + "; no weights)",
        "config": {"workload": workload, "batch": w.B, "prefix_len": [int(x) for x in w.prefix_len[:4]] +
                   (["..."] if w.B > 4 else []), "tree_nodes_per_step": nodes, "top_k": w.K, "depth": w.D,
                   "total_tokens": w.total_tokens, "Hq": w.Hq, "Hkv": w.Hkv, "head_dim": w.d, "vocab": w.V,
                   "input_copies_rotated": n_copies, "launch": launch,
                   "kv_cache": "linear" if paged is None else
                   f"paged, {args.paged} tokens per block, {paged.n_blocks} blocks in random order",
                   "calls": ", ".join([
                       f"tree_build_layer x {w.D + 1} ({args.layerwise} rows), tree_build_finish" if args.layerwise
                       else ("tree_build, tree_mask_positions" if args.unfused else "tree_build_meta"),
                       "tree_attention" + ("_paged" if paged is not None else ""),
                       (("tree_sampling_probs, " if args.sampling and args.sampling_from != "probs" else "") +
                        ("tree_accept_sample_draft, kv_compact" if args.sampling and args.sampling_from == "draft"
                         else "tree_accept_sample, kv_compact") if args.sampling else
                        "tree_accept, kv_compact" if args.unfused else "tree_accept_compact") +
                       ("_paged" if paged is not None else "")])},
        "stages_us": stages,
        **({"sampling_us": sampling_us} if sampling_us else {}),
        "roofline": roof,
    }
    if peaks:
        out["measured_peaks"] = peaks
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, paged)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
