#!/usr/bin/env python3
"""Benchmark of the prefix-shared tree-training hot path on one MI355X.

One step = the whole path over one batch of synthetic sequences:
  pack the sequences into tries (host, C++), upload the forest's metadata,
  tree attention forward (and backward when the workload trains), and the
  logprob/entropy gather when the workload has logits -- all through the C ABI.
Q/K/V/dO/logits are resident in HBM before the timed region starts.  The
packing of upcoming batches runs on two worker threads ahead of the step
that uploads them (as a data loader would), and the step re-uploads one
metadata object in place, so the host keeps ahead of the GPU.

Default workload: bimodal responses (64 prompts of 256 tokens x 4 samples,
response lengths 70 % U{50..200} and 30 % U{800..2048}, 8192-token trees,
bf16, 40 query / 8 key-value heads, head_dim 128): the 8K-token-tree
configuration whose step has all three passes, attention forward, attention
backward and the logprob/entropy gather over a 152064-token vocab.
`--workload grpo` runs the GRPO group packing (forward + gather).

Prints ONE JSON line.  `value` is the tree-attention effective TFLOP/s
(forward, plus backward when timed): algorithmic FLOPs -- 4*d*Hq per visible
(query, key) pair forward, 2.5x that backward -- over the attention kernels'
time measured with HIP events on the launch stream.  ms_per_step is the wall
clock of a whole step.  The gather's GB/s, packed tokens/s and the tree token
ratio ride along; `roofline` describes the kernel that takes the most time,
`cpu_baseline` the oracle timed on a bounded sample on the host cores.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tree-attn effective TFLOP/s (fwd/bwd) at 8K-token trees; logprob-gather GB/s"
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}   # dense MFMA peaks of MI355X
PEAK_HBM_GBPS = 8000.0


def attn_flops(pairs, hq, head_dim):
    """Algorithmic attention FLOPs: 4 d per visible (query, key) pair and
    query head forward (score and P.V products), 2.5 times that backward
    (dV, dP, dQ, dK and the recomputed scores)."""
    fwd = 4 * head_dim * hq * pairs
    return dict(fwd=fwd, bwd=2.5 * fwd, fwd_bwd=3.5 * fwd)


KDIR = os.path.join(ROOT, "prefix_shared_tree_packed_amd", "csrc", "kernels")


def kernel_sources(kernel, dtype, head_dim):
    """Source files that define `kernel` for these shapes (hashed to tie
    counter measurements to the code they were taken on)."""
    fast = dtype == "bf16" and head_dim == 128
    files = {"attn_fwd": ["attn_fwd_bf16.hip" if fast else "attn_fwd.hip"],
             "attn_bwd": ["attn_bwd_bf16.hip" if fast else "attn_bwd.hip"],
             "gather": ["gather.hip"]}[kernel]
    shared = ["common.h", "mfma.h"] + (["lds_tiles.h"] if fast and kernel != "gather" else [])
    # the metadata layout and the device work orders are built in capi.cpp;
    # the compile flags (per file too) live in build.py
    return ([os.path.join(KDIR, f) for f in files + shared] + [os.path.join(KDIR, "..", "capi.cpp")]
            + [os.path.join(KDIR, "..", "..", "build.py")])


def sources_sha256(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload, digest):
    """HBM bytes per launch recorded under profiles/ for this kernel, workload
    and source digest (read and write counters, each scaled by the copy-kernel
    calibration), or None when no record matches the current sources."""
    import glob
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as f:
            for line in f:
                if not line.startswith("traffic-record:"):
                    continue
                kv = dict(x.split("=", 1) for x in line.split(":", 1)[1].split())
                if (kv.get("kernel"), kv.get("workload"), kv.get("sources_sha256")) == \
                        (kernel, workload, digest):
                    return float(kv["bytes_per_launch"])
    return None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="bimodal",
                    help="tiny | grpo | agentic | bimodal | long | long_control")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--rope", action="store_true",
                    help="also time the tree-position rotary embedding of Q and K (in place), "
                         "reported under kernels; it stays out of value")
    ap.add_argument("--gather-bwd", action="store_true",
                    help="also time the gather backward (d logits) after the gather, reported "
                         "under kernels; it stays out of value (the wall-clock ms_per_step then "
                         "includes it)")
    ap.add_argument("--mask", action="store_true",
                    help="also time the dense uint8 mask export of every tree (per-tree metadata, "
                         "one [Np, Np] buffer reused), reported under kernels; outside the step")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample time")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run one device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import prefix_shared_tree_packed_amd as pst
    from workloads import get_workload, make_tensor, tree_tensor_seed

    pst.load()
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    w = get_workload(args.workload)
    log(f"workload {w.name}: {len(w.seqs)} sequences, {w.n_tokens} tokens")

    shape_forest = pst.build_tree(w.seqs, w.max_tokens_per_mb)
    stats = shape_forest.stats()
    sizes = [shape_forest.sizes(t) for t in range(shape_forest.n_trees)]
    n_trees = len(sizes)
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    d, hq, hkv = w.head_dim, w.hq, w.hkv

    # one buffer per tensor for the whole forest, trees back to back (the
    # layout of the forest-level metadata); each tree's rows are drawn from
    # their own seed
    Np_all = sum(s["n_padded"] for s in sizes)
    n_out_all = sum(s["n_out"] for s in sizes)

    def forest_tensor(width_shape, name, std=1.0):
        parts = [make_tensor((s["n_padded"],) + width_shape, w.dtype, tree_tensor_seed(w.seed, t, name),
                             dev, std=std) for t, s in enumerate(sizes)]
        out = torch.cat(parts) if len(parts) > 1 else parts[0]
        del parts
        return out.contiguous()

    b = {}
    b["q"] = forest_tensor((hq, d), "q")
    b["k"] = forest_tensor((hkv, d), "k")
    b["v"] = forest_tensor((hkv, d), "v")
    b["o"] = torch.empty((Np_all, hq, d), dtype=tdt, device=dev)
    b["lse"] = torch.empty((hq, Np_all), dtype=torch.float32, device=dev)
    if w.bwd:
        b["do"] = forest_tensor((hq, d), "do")
        b["dq"] = torch.empty_like(b["q"])
        b["dk"] = torch.empty_like(b["k"])
        b["dv"] = torch.empty_like(b["v"])
        shape_meta = pst.forest_meta_create(shape_forest)
        ws_bytes = pst.tree_attn_bwd_workspace_bytes(shape_meta, hq, hkv, d, w.dtype)
        torch.cuda.synchronize()
        shape_meta.destroy()
        b["ws"] = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if w.gather:
        b["logits"] = forest_tensor((w.vocab,), "logits", std=w.logit_std)
        b["lp"] = torch.empty(n_out_all, dtype=torch.float32, device=dev)
        b["ent"] = torch.empty(n_out_all, dtype=torch.float32, device=dev)
        if args.gather_bwd:
            # (lse, entropy) per row, written by the forward gather, read by the backward
            b["row_stats"] = torch.empty((Np_all, 2), dtype=torch.float32, device=dev)
            gen = torch.Generator(device=dev).manual_seed(w.seed + 99)
            b["dlp"] = torch.randn(n_out_all, generator=gen, device=dev)
            b["dent"] = torch.randn(n_out_all, generator=gen, device=dev)
            b["dlogits"] = torch.empty_like(b["logits"])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    # Host side of a step: the batch's forest is packed on worker threads
    # (the C++ builder runs with the interpreter lock released), up to
    # `ahead` batches before the step that uploads it, as a training data
    # loader would; the step itself re-uploads the one metadata object in
    # place (pst_forest_meta_update: no allocation, stream-ordered behind
    # the previous step's kernels) and queues the kernels.  Every step
    # still packs and uploads its own batch inside the timed region.
    from concurrent.futures import ThreadPoolExecutor

    def build():
        return pst.build_tree(w.seqs, w.max_tokens_per_mb)

    pool = ThreadPoolExecutor(max_workers=2)
    ahead = 3
    queued = [pool.submit(build) for _ in range(ahead)]
    meta = pst.forest_meta_create(shape_forest, stream)

    def step(record):
        forest = queued.pop(0).result()
        queued.append(pool.submit(build))
        meta.update(forest, stream)
        forest.close()
        m = meta
        e = [torch.cuda.Event(enable_timing=True) for _ in range(8)] if record else None
        if record:
            # When the host only just keeps ahead (short steps, e.g. grpo's
            # 0.6 ms), the GPU can reach e[0] idle and wait there for the
            # forward's submission, timing the launch latency as kernel
            # time.  A short spin (~0.05 ms of GPU time, counted in
            # ms_per_step) lets the host queue the forward first.
            torch.cuda._sleep(100000)
            e[0].record(stream)
        pst.tree_attn_fwd(b["q"], b["k"], b["v"], m, out=b["o"], lse=b["lse"], stream=stream)
        if record:
            e[1].record(stream)
        if w.bwd:
            pst.tree_attn_bwd(b["q"], b["k"], b["v"], b["o"], b["lse"], b["do"], m,
                              dq=b["dq"], dk=b["dk"], dv=b["dv"], workspace=b["ws"], stream=stream)
        if record:
            e[2].record(stream)
        if w.gather:
            pst.gather_tree_logprobs_entropy(b["logits"], m, logprobs=b["lp"], entropy=b["ent"],
                                             row_stats=b.get("row_stats"), stream=stream)
        if record:
            e[3].record(stream)
        if args.rope:
            if record:
                e[6].record(stream)
            pst.tree_rope(b["q"], m, stream=stream)
            pst.tree_rope(b["k"], m, stream=stream)
            if record:
                e[7].record(stream)
        if w.gather and args.gather_bwd:
            # outside the timed path of the step (its own event pair)
            if record:
                e[4].record(stream)
            pst.gather_tree_logprobs_entropy_bwd(b["logits"], m, b["dlp"], b["dent"],
                                                 dlogits=b["dlogits"], row_stats=b["row_stats"],
                                                 stream=stream)
            if record:
                e[5].record(stream)
        return e

    log(f"{n_trees} trees; warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()

    # host packing alone, for the record
    t0 = time.perf_counter()
    for _ in range(5):
        pst.build_tree(w.seqs, w.max_tokens_per_mb).close()
    host_build_ms = (time.perf_counter() - t0) / 5 * 1e3

    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    events = [step(True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) / args.steps * 1e3
    for f in queued:
        f.result().close()
    pool.shutdown()

    fwd_ms, bwd_ms, gat_ms, gbw_ms, rope_ms = [], [], [], [], []
    for e in events:
        fwd_ms.append(e[0].elapsed_time(e[1]))
        bwd_ms.append(e[1].elapsed_time(e[2]))
        gat_ms.append(e[2].elapsed_time(e[3]))
        if w.gather and args.gather_bwd:
            gbw_ms.append(e[4].elapsed_time(e[5]))
        if args.rope:
            rope_ms.append(e[6].elapsed_time(e[7]))
    meta.destroy()

    if args.mask:
        mask_t, mask_bytes = time_dense_mask(pst, torch, shape_forest, sizes, stream, args.steps)
        mask_entry = {"ms_per_step": mask_t * 1e3, "GB/s": mask_bytes / mask_t / 1e9,
                      "launches_per_step": n_trees, "in_step": False}

    K = args.steps
    pairs = stats["n_pairs"]
    flops = attn_flops(pairs, hq, d)
    fwd_flops = float(flops["fwd"])
    bwd_flops = float(flops["bwd"]) if w.bwd else 0.0
    fwd_t = sum(fwd_ms) / K * 1e-3           # seconds of forward kernels per step
    bwd_t = sum(bwd_ms) / K * 1e-3 if w.bwd else 0.0  # (no kernel between the events otherwise)
    gat_t = sum(gat_ms) / K * 1e-3
    attn_tflops = (fwd_flops + bwd_flops) / (fwd_t + bwd_t) / 1e12
    kernels = {"attn_fwd": {"ms_per_step": fwd_t * 1e3, "TFLOP/s": fwd_flops / fwd_t / 1e12,
                            "launches_per_step": 1}}
    if w.bwd:
        kernels["attn_bwd"] = {"ms_per_step": bwd_t * 1e3, "TFLOP/s": bwd_flops / bwd_t / 1e12,
                               "launches_per_step": 1}
    if args.rope:
        rope_t = sum(rope_ms) / K * 1e-3
        esz_qk = 4 if w.dtype == "f32" else 2
        # real rows of Q and K read and written once, the row pointers and depths
        rope_bytes = 2 * stats["tree_tokens"] * (hq + hkv) * d * esz_qk + 2 * 2 * 4 * (Np_all + 1)
        kernels["rope_qk"] = {"ms_per_step": rope_t * 1e3, "GB/s": rope_bytes / rope_t / 1e9,
                              "launches_per_step": 2, "in_step": False}
    if args.mask:
        kernels["dense_mask_u8"] = mask_entry
    gather_bytes = 0
    if w.gather:
        esz = 4 if w.dtype == "f32" else 2
        n_out = sum(s["n_out"] for s in sizes)
        n_real = stats["tree_tokens"]
        # logits of every real row once + per output two fp32 writes and its
        # slot and target reads + the row pointer of every row
        gather_bytes = n_real * w.vocab * esz + n_out * (4 + 4 + 4 + 4) + 4 * (Np_all + 1)
        kernels["gather"] = {"ms_per_step": gat_t * 1e3, "GB/s": gather_bytes / gat_t / 1e9,
                             "launches_per_step": 1}
        if args.gather_bwd:
            gbw_t = sum(gbw_ms) / K * 1e-3
            # real rows read once + every row of d logits written + per output
            # its two gradients, slot and target + the rows' saved statistics
            gbw_bytes = (n_real + Np_all) * w.vocab * esz + n_out * 16 + 4 * (Np_all + 1) + 8 * n_real
            kernels["gather_bwd"] = {"ms_per_step": gbw_t * 1e3, "GB/s": gbw_bytes / gbw_t / 1e9,
                                     "launches_per_step": 1, "in_step": False}

    # roofline of the kernel that takes the most time
    cands = [("attn_fwd", fwd_t), ("attn_bwd", bwd_t), ("gather", gat_t)]
    dom = max((c for c in cands if c[0] in kernels), key=lambda c: c[1])[0]
    if dom == "gather":
        ach = gather_bytes / gat_t / 1e9
        roof = {"kernel": "gather", "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": ach / PEAK_HBM_GBPS, "traffic": None,
                "algorithmic_per_launch": gather_bytes}
    else:
        fl, tt = (fwd_flops, fwd_t) if dom == "attn_fwd" else (bwd_flops, bwd_t)
        ach = fl / tt / 1e12
        peak = PEAK_TFLOPS[w.dtype]
        roof = {"kernel": dom, "bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                "frac": ach / peak, "traffic": None, "algorithmic_per_launch": fl}

    digest = sources_sha256(kernel_sources(roof["kernel"], w.dtype, d))
    roof["sources_sha256"] = digest
    roof["traffic"] = measured_traffic(roof["kernel"], w.name, digest)

    out = {
        "metric": METRIC,
        "value": attn_tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "sequences": len(w.seqs), "orig_tokens": stats["orig_tokens"],
            "max_tokens_per_mb": w.max_tokens_per_mb, "trees": n_trees,
            "hq": hq, "hkv": hkv, "head_dim": d, "vocab": w.vocab,
            "passes": "+".join(p for p, on in (("fwd", w.fwd), ("bwd", w.bwd), ("gather", w.gather)) if on),
        },
        "tree_token_ratio": stats["tree_token_ratio"],
        "packed_tokens_per_s": stats["tree_tokens"] / (ms_per_step * 1e-3),
        "gather_GBps": kernels["gather"]["GB/s"] if w.gather else None,
        "visible_pairs": pairs,
        "causal_pairs": stats["causal_pairs"],
        "tiles": stats["n_tiles"],
        "tile_utilisation": pairs / (stats["n_tiles"] * 128 * 128),
        "block_utilisation": pairs / (blocks32(shape_forest) * 32 * 32),
        "host_build_ms": host_build_ms,
        "kernels": kernels,
        "roofline": roof,
        "cpu_baseline": None,
    }

    out["host_packing"] = host_packing(pst, w, shape_forest)

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        bcopy = torch.empty_like(a)
        torch.cuda.synchronize()
        bcopy.copy_(a)                    # runtime blit kernel
        torch.mul(a, 1.0, out=bcopy)      # elementwise kernel, same bytes
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = n * 4
        del a, bcopy

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, sizes, b, args.cpu_seconds)

    print(json.dumps(out), flush=True)


def time_dense_mask(pst, torch, forest, sizes, stream, steps):
    """Seconds per pass of the uint8 dense-mask export over every tree, and
    the algorithmic bytes of a pass (Np^2 mask bytes + the subtree ends)."""
    metas = [pst.tree_meta_create(forest, t, stream) for t in range(len(sizes))]
    npmax = max(s["n_padded"] for s in sizes)
    buf = torch.empty(npmax * npmax, dtype=torch.uint8, device="cuda")
    outs = [buf[:s["n_padded"] ** 2].view(s["n_padded"], s["n_padded"]) for s in sizes]

    def one_pass():
        for m, o in zip(metas, outs):
            pst.tree_dense_mask(m, "u8", out=o, stream=stream)

    one_pass()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        one_pass()
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / steps * 1e-3
    for m in metas:
        m.destroy()
    del buf
    return t, sum(s["n_padded"] ** 2 + 4 * s["n_padded"] for s in sizes)


def blocks32(forest):
    """Non-empty 32x32 blocks over all trees: the granularity at which the
    attention kernels execute MFMAs (2-bit classes packed in each 128-tile)."""
    import numpy as np

    n = 0
    for t in range(forest.n_trees):
        cls = forest.export(t)["q_cls"].view(np.uint32)
        n += sum(int(np.count_nonzero((cls >> (2 * i)) & 3)) for i in range(16))
    return n


def host_packing(pst, w, forest, ranks=8, reps=5):
    """Host allocation timings: the workload's sequence lengths into
    micro-batches of its capacity (FFD and KK, with KK's fallback flag), the
    same lengths balanced over `ranks` ranks, and the trees balanced over the
    ranks by visible pairs; best of `reps` runs each, with the spread."""
    import numpy as np
    lens = np.array([len(s) for s in w.seqs], dtype=np.int64)
    res = {"items": int(lens.size), "ranks": ranks}

    def timed(fn):
        best, r = float("inf"), None
        for _ in range(reps):
            t0 = time.perf_counter()
            r = fn()
            best = min(best, time.perf_counter() - t0)
        return r, best * 1e3

    for alg in ("ffd", "kk"):
        (g, fb), ms = timed(lambda: pst.pack_allocate(lens, w.max_tokens_per_mb, 1, 1, alg))
        m = pst.packing_metrics(lens, g, w.max_tokens_per_mb)
        res[f"mb_{alg}"] = {"ms": ms, "groups": len(g), "fell_back": fb, "spread": m["spread"],
                            "utilization": m["utilization"]}
        (g, fb), ms = timed(lambda: pst.pack_allocate(lens, 1 << 62, ranks, 1, alg))
        m = pst.packing_metrics(lens, g, 1 << 62)
        res[f"ranks_{alg}"] = {"ms": ms, "spread": m["spread"], "imbalance_ratio": m["imbalance_ratio"]}
        rank, ms = timed(lambda: pst.assign_trees(forest, ranks, cost="pairs", algorithm=alg))
        pairs = np.array([forest.sizes(t)["n_pairs"] for t in range(forest.n_trees)])
        loads = np.bincount(rank, weights=pairs, minlength=ranks)
        res[f"trees_{alg}"] = {"ms": ms, "max_pairs": int(loads.max()), "min_pairs": int(loads.min())}
    return res


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, sizes, fb, target_s):
    """The oracle, as it stands, on a bounded sample of the same workload:
    the dense-mask float64 forward of tree 0 for as many query heads of the
    first key/value group as fit in about `target_s` seconds (at least one),
    reported in the same algorithmic-FLOP unit as `value`."""
    import numpy as np
    import torch

    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    ref = oracle.build_forest(w.seqs, w.max_tokens_per_mb)
    tree = ref.trees[0]
    G = w.hq // w.hkv
    # tree 0 occupies the first rows of the forest buffers
    n0 = tree.n_padded
    b = {key: fb[key][:n0] for key in ("q", "k", "v", "logits") if key in fb}
    h64 = lambda x: x.detach().to("cpu", torch.float64).numpy()  # noqa: E731
    mask = oracle.dense_mask(tree)
    # whole key/value groups of query heads (group g serves heads g*G .. g*G+G-1)
    # until the projected time passes target_s
    elapsed, groups = 0.0, 0
    while groups < w.hkv and (groups == 0 or elapsed * (groups + 1) / groups < target_s):
        qq = h64(b["q"][:, groups * G:(groups + 1) * G])
        kk = h64(b["k"][:, groups:groups + 1])
        vv = h64(b["v"][:, groups:groups + 1])
        s0 = time.perf_counter()
        oracle.attn_fwd(tree, qq, kk, vv, mask=mask)
        elapsed += time.perf_counter() - s0
        groups += 1
    heads = groups * G
    flops = 4.0 * w.head_dim * heads * tree.n_pairs
    res = {
        "value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": f"dense-mask float64 forward of tree 0 ({tree.n_tokens} tokens), "
                  f"{heads} of {w.hq} query heads, {elapsed:.1f} s",
        "host_cpus": os.cpu_count(),
        "cpu_model": cpu_model(),
    }
    if w.gather:
        sids = tree.seq_ids[:2]
        rows = np.concatenate([tree.seq_index[s] for s in sids])
        uniq = np.unique(rows)
        x = h64(b["logits"][torch.as_tensor(uniq, device=b["logits"].device)])
        sub = oracle.Tree(**{**tree.__dict__, "seq_ids": sids,
                             "seq_index": {s: np.searchsorted(uniq, tree.seq_index[s]) for s in sids}})
        s0 = time.perf_counter()
        oracle.gather_logprobs_entropy(sub, w.seqs, x)
        gs = time.perf_counter() - s0
        res["gather_GBps"] = len(rows) * w.vocab * (4 if w.dtype == "f32" else 2) / gs / 1e9
        res["gather_sample"] = f"{len(sids)} sequences ({len(rows)} rows of {w.vocab} logits), {gs:.2f} s"
    return res


if __name__ == "__main__":
    main()
