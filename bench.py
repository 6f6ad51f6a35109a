#!/usr/bin/env python3
"""Benchmark of one tree-verification step on one MI355X.

A step is the whole hot path over one batch: tree_mask_build ->
tree_verify_attn -> tree_accept. The default workload is the Graft-shaped
60-node tree (batch 1, 2048-token prefix, Qwen3-8B attention: 32 query / 8 kv
heads, head_dim 128, bf16, 16-token pages). Inputs are seeded synthetic data
resident in HBM; R copies of Q/K/V are rotated so that consecutive steps do
not find their KV in the 256 MB last-level cache. The K timed steps are
replayed from a HIP graph captured from the library's own launches.

Prints one JSON line: throughput in verified tree-tokens/s, the attention
kernel's achieved HBM bandwidth against the 8 TB/s peak (HIP events over the
timed region), and the CPU oracle's rate on the host as a reported baseline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verified tree-tokens/s and achieved HBM TB/s (% of peak), Qwen3-8B-shaped 60-node tree"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
VALU_FP32_PEAK_TFLOPS = 157.3


PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ("tv_attn.hip", "tv_internal.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    """sha256 over the attention kernel's sources (ties counter data to a build)."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "tree_verification_attention_mask_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per tree_verify_attn call from the committed counter summary
    (rocprofv3 FETCH_SIZE / WRITE_SIZE passes scaled by a copy of known size),
    or None when there is none or the kernel sources changed since."""
    path = os.path.join(PROFILES, "tree_verify_attn_%s_hbm_counters.md" % workload)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel source sha256") != kernel_source_hash():
        return None
    try:
        return float(fields["hbm bytes per call"])
    except (KeyError, ValueError):
        return None


def depths(parent, cu):
    d = [0] * len(parent)
    for b in range(len(cu) - 1):
        for i in range(int(cu[b]) + 1, int(cu[b + 1])):
            d[i] = d[int(cu[b]) + int(parent[i])] + 1
    return d


def algorithmic_work(w):
    """Bytes: Q read once, every prefix and tree K/V row read once, O written
    once. FLOPs: 4 * head_dim per visible (row, key) pair (QK^T and PV)."""
    import numpy as np
    elt = 2 if w.dtype == "bf16" else 4
    n, hq, hkv, d = w.total_nodes, w.num_q_heads, w.num_kv_heads, w.head_dim
    kv_rows = int(np.sum(w.prefix_len.astype(np.int64) + w.nodes_per_request))
    bytes_ = 2 * n * hq * d * elt + 2 * kv_rows * hkv * d * elt
    dep = depths(w.parent, w.cu_nodes)
    pairs = 0
    for b in range(w.batch):
        for i in range(int(w.cu_nodes[b]), int(w.cu_nodes[b + 1])):
            pairs += int(w.prefix_len[b]) + dep[i] + 1
    flops = 4 * d * hq * pairs
    return bytes_, flops


def cpu_baseline(w, seconds):
    """The oracle, as it is, over whole steps of the same workload, single thread."""
    import numpy as np
    import oracle
    q = w.q.float().numpy()
    k = w.k_cache.float().numpy()
    v = w.v_cache.float().numpy()
    reps = 0
    t0 = time.perf_counter()
    while True:
        if w.mask_kind == "bits":
            oracle.mask_bits(w.parent, w.cu_nodes, w.words_per_node)
        else:
            oracle.mask_anchor(w.parent, w.cu_nodes)
        oracle.tree_attn(q, k, v, w.block_table, w.prefix_len, w.cu_nodes, w.parent,
                         w.num_q_heads, w.num_kv_heads, w.scale)
        if w.draft_tok is not None:
            oracle.accept(w.parent, w.draft_tok, w.target_tok, w.cu_nodes, w.max_depth)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    del q, k, v, np
    return {"value": reps * w.total_nodes / el, "unit": "tree-tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": "%d whole steps of %s (mask + fp64 attention over all %d x %d rows + "
                      "acceptance) in %.1f s, one thread of %s (%d in this process's "
                      "affinity set)" % (reps, w.name, w.total_nodes, w.num_q_heads, el,
                                         cpu_model(), len(os.sched_getaffinity(0)))}


def cpu_baseline_threads(w, seconds):
    """The same oracle over whole steps, the attention rows split into equal
    parts over host threads (one part each; the C routine runs outside the
    interpreter lock), at most 16 threads and no more than the affinity set."""
    import numpy as np
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    q = w.q.float().numpy()
    k = w.k_cache.float().numpy()
    v = w.v_cache.float().numpy()
    rows = np.stack(np.meshgrid(np.arange(w.total_nodes), np.arange(w.num_q_heads),
                                indexing="ij"), -1).reshape(-1, 2).astype(np.int32)
    parts = [c for c in np.array_split(rows, threads) if len(c)]

    def part(c):
        oracle.tree_attn(q, k, v, w.block_table, w.prefix_len, w.cu_nodes, w.parent,
                         w.num_q_heads, w.num_kv_heads, w.scale, rows=c)

    reps = 0
    with ThreadPoolExecutor(len(parts)) as ex:
        t0 = time.perf_counter()
        while True:
            if w.mask_kind == "bits":
                oracle.mask_bits(w.parent, w.cu_nodes, w.words_per_node)
            else:
                oracle.mask_anchor(w.parent, w.cu_nodes)
            list(ex.map(part, parts))
            if w.draft_tok is not None:
                oracle.accept(w.parent, w.draft_tok, w.target_tok, w.cu_nodes, w.max_depth)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return {"value": reps * w.total_nodes / el, "unit": "tree-tokens/s", "cores": len(parts),
            "kind": "oracle",
            "sample": "%d whole steps of %s in %.1f s, the %d x %d attention rows in %d equal "
                      "parts on %d threads of %s (%d in this process's affinity set)"
                      % (reps, w.name, el, w.total_nodes, w.num_q_heads, len(parts), len(parts),
                         cpu_model(), len(os.sched_getaffinity(0)))}


def measure_other(cfg, steps, dev):
    """tree_verify_attn on another workload, timed like the headline's
    attention figure: HIP-graph replays of at least 8 back-to-back calls over
    rotating buffer sets (R sets with R x working set >= 512 MB), HIP events
    on the launch stream, one warm replay first; plus the whole step (mask,
    attention, acceptance) the same way. Returns the figures against the
    roofline that bounds the workload: HBM for KV-bound shapes, MFMA for the
    long-context and SpecOPD shapes."""
    import torch

    import tree_verification_attention_mask_amd as tv
    import workloads as W
    w = W.make(cfg)
    alg_bytes, alg_flops = algorithmic_work(w)
    set_bytes = 2 * w.k_cache.numel() * w.k_cache.element_size() + 2 * w.q.numel() * w.q.element_size()
    R = max(1, min(64, math.ceil(512e6 / set_bytes)))
    parent = torch.from_numpy(w.parent).to(dev)
    cu = torch.from_numpy(w.cu_nodes).to(dev)
    prefix = torch.from_numpy(w.prefix_len).to(dev)
    table = torch.from_numpy(w.block_table).to(dev)
    qs = [w.q.to(dev)]
    ks = [w.k_cache.to(dev)]
    vs = [w.v_cache.to(dev)]
    w.q = w.k_cache = w.v_cache = None
    for _ in range(R - 1):
        qs.append(qs[0].clone())
        ks.append(ks[0].clone())
        vs.append(vs[0].clone())
    outs = [torch.empty_like(qs[0]) for _ in range(R)]
    lses = [torch.empty(qs[0].shape[:2], dtype=torch.float32, device=dev) for _ in range(R)]
    need = tv.verify_attn_workspace_size(w.batch, w.total_nodes, w.max_nodes, w.max_prefix_len,
                                         w.num_q_heads, w.num_kv_heads, w.head_dim, qs[0].dtype)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
    m = tv.tree_mask_build(parent, cu, w.max_nodes, kind=w.mask_kind)
    mk = {k_: v_ for k_, v_ in m.items()}
    has_tok = w.draft_tok is not None
    draft = torch.from_numpy(w.draft_tok).to(dev) if has_tok else None
    target = torch.from_numpy(w.target_tok).to(dev) if has_tok else None
    acc = {}
    if has_tok:
        al, path, bonus = tv.tree_accept(parent, draft, target, cu, w.max_nodes, w.max_depth)
        acc = {"accept_len": al, "path": path, "bonus": bonus}

    def attn(s_):
        tv.tree_verify_attn(qs[s_], ks[s_], vs[s_], table, prefix, cu, mk, w.max_nodes,
                            w.max_prefix_len, scale=w.scale, out=outs[s_], lse=lses[s_],
                            workspace=ws)

    def step(s_):
        tv.tree_mask_build(parent, cu, w.max_nodes, kind=w.mask_kind, out=mk)
        attn(s_)
        if has_tok:
            tv.tree_accept(parent, draft, target, cu, w.max_nodes, w.max_depth, out=acc)

    for i in range(2 * R):
        step(i % R)
    torch.cuda.synchronize()
    RG = max(R, 8)

    def timed(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s_ in range(RG):
                fn(s_ % R)
        g.replay()
        torch.cuda.synchronize()
        reps = max(2, steps // RG)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * RG)

    us = timed(attn)
    us_step = timed(step)
    gbs = alg_bytes / (us * 1e-6) / 1e9
    tfl = alg_flops / (us * 1e-6) / 1e12
    bound = "mfma" if cfg in (4, 5) else "hbm"
    pl = tv.verify_attn_plan(w.batch, w.total_nodes, w.max_nodes, w.max_prefix_len,
                             w.num_q_heads, w.num_kv_heads, w.head_dim, qs[0].dtype)
    res = {"workload": w.name, "tree_nodes": w.total_nodes, "batch": w.batch,
           "max_prefix_len": w.max_prefix_len, "rotating_buffer_sets": R,
           "us_per_call": us, "step_us": us_step,
           "tree_tokens_per_s": w.total_nodes / (us_step * 1e-6),
           "algorithmic_bytes_per_launch": alg_bytes, "algorithmic_flops_per_launch": alg_flops,
           "achieved_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
           "achieved_tflops": tfl, "mfma_frac": tfl / MFMA_BF16_PEAK_TFLOPS,
           "bound": bound, "frac": (tfl / MFMA_BF16_PEAK_TFLOPS) if bound == "mfma"
           else (gbs / HBM_PEAK_GBS),
           "traffic": measured_traffic(w.name),
           "plan": {k_: pl[k_] for k_ in ("rows_per_block", "row_blocks", "splits",
                                          "keys_per_split")}}
    del qs, ks, vs, outs, lses, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def cpu_model():
    """The host CPU's model name (for the CPU baseline's record)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, help="workload 1..5 (default 2, the headline)")
    ap.add_argument("--rot", type=int, default=0, help="rotating buffer sets (0 = auto)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--other-configs", default="3,4,5",
                    help="comma-separated workloads whose tree_verify_attn call (and whole step) "
                         "is also timed and reported under 'configs' ('' = none)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="before timing, copy this many MiB device to device three times "
                         "(a plain copy of known size that hardware-counter passes use to "
                         "scale FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode (requests, kv-head "
              "groups or key ranges would shard with no exchange but one LSE merge). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import tree_verification_attention_mask_amd as tv
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    dev = "cuda:0"
    w = W.make(args.config)
    log("workload", w.name, "nodes", w.total_nodes, "max prefix", w.max_prefix_len)
    alg_bytes, alg_flops = algorithmic_work(w)
    kv_bytes = 2 * w.k_cache.numel() * w.k_cache.element_size()
    set_bytes = kv_bytes + 2 * w.q.numel() * w.q.element_size()
    R = args.rot or max(1, min(64, math.ceil(512e6 / set_bytes)))

    parent = torch.from_numpy(w.parent).to(dev)
    cu = torch.from_numpy(w.cu_nodes).to(dev)
    prefix = torch.from_numpy(w.prefix_len).to(dev)
    table = torch.from_numpy(w.block_table).to(dev)
    has_tok = w.draft_tok is not None
    draft = torch.from_numpy(w.draft_tok).to(dev) if has_tok else None
    target = torch.from_numpy(w.target_tok).to(dev) if has_tok else None
    q0, k0, v0 = w.q.to(dev), w.k_cache.to(dev), w.v_cache.to(dev)
    qs = [q0] + [q0.clone() for _ in range(R - 1)]
    ks = [k0] + [k0.clone() for _ in range(R - 1)]
    vs = [v0] + [v0.clone() for _ in range(R - 1)]
    outs = [torch.empty_like(q0) for _ in range(R)]
    lses = [torch.empty(q0.shape[:2], dtype=torch.float32, device=dev) for _ in range(R)]
    need = tv.verify_attn_workspace_size(w.batch, w.total_nodes, w.max_nodes, w.max_prefix_len,
                                         w.num_q_heads, w.num_kv_heads, w.head_dim, q0.dtype)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
    mask_out = {}
    acc_out = {}
    m = tv.tree_mask_build(parent, cu, w.max_nodes, kind=w.mask_kind)
    mask_out = {k_: v_ for k_, v_ in m.items() if isinstance(v_, torch.Tensor)}
    if has_tok:
        al, path, bonus = tv.tree_accept(parent, draft, target, cu, w.max_nodes, w.max_depth)
        acc_out = {"accept_len": al, "path": path, "bonus": bonus}

    def mask_call():
        return tv.tree_mask_build(parent, cu, w.max_nodes, kind=w.mask_kind, out=mask_out)

    def attn_call(s, mk):
        tv.tree_verify_attn(qs[s], ks[s], vs[s], table, prefix, cu, mk, w.max_nodes,
                            w.max_prefix_len, scale=w.scale, out=outs[s], lse=lses[s],
                            workspace=ws)

    def accept_call():
        if has_tok:
            tv.tree_accept(parent, draft, target, cu, w.max_nodes, w.max_depth, out=acc_out)

    def step(s):
        mk = mask_call()
        attn_call(s, mk)
        accept_call()

    if args.copy_probe_mb > 0:
        src = torch.empty(args.copy_probe_mb << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("copy probe: 3 x %d MiB device-to-device" % args.copy_probe_mb)

    for i in range(args.warmup):
        step(i % R)
    torch.cuda.synchronize()
    eager_out = outs[0].clone()
    eager_acc = [t.clone() for t in acc_out.values()]

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    # a replay runs RG >= 8 steps back to back, cycling over the R buffer
    # sets, so that graph-launch overhead stays out of the per-step figures
    # also when one set already defeats the last-level cache (R = 1)
    RG = max(R, 8)
    g_full = capture(lambda: [step(s % R) for s in range(RG)])
    rem = args.steps % RG
    g_rem = capture(lambda: [step(s % R) for s in range(rem)]) if rem else None
    g_attn = capture(lambda: [attn_call(s % R, mask_out | {"kind": w.mask_kind,
                                                          "words_per_node": m["words_per_node"]})
                              for s in range(RG)])
    # the small calls read the same few KB every time: a graph of at least 32
    # back-to-back calls keeps graph-launch overhead out of their figures
    RS = max(R, 32)
    g_mask = capture(lambda: [mask_call() for _ in range(RS)])
    g_acc = capture(lambda: [accept_call() for _ in range(RS)]) if has_tok else None
    # a replay reproduces the eager results bit for bit
    outs[0].zero_()
    g_full.replay()
    torch.cuda.synchronize()
    assert torch.equal(outs[0], eager_out), "graph replay differs from eager run"
    assert all(torch.equal(a, b) for a, b in zip(acc_out.values(), eager_acc))
    # every graph the timed region replays has been replayed once before it
    if g_rem is not None:
        g_rem.replay()
    torch.cuda.synchronize()

    reps_full = args.steps // RG
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record()
    for _ in range(reps_full):
        g_full.replay()
    if g_rem is not None:
        g_rem.replay()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps
    log("timed %d steps: %.3f ms (events), %.3f s wall" % (args.steps, ms_total, wall))

    # spread over replays: each replay of the R-step graph timed on its own
    # (after the timed region, which it does not touch)
    per_replay = []
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(max(10, min(reps_full, 200)))]
    for a_, b_ in evs:
        a_.record()
        g_full.replay()
        b_.record()
    torch.cuda.synchronize()
    per_replay = np.array([a_.elapsed_time(b_) * 1e3 / RG for a_, b_ in evs])
    spread = {"unit": "us per step, mean of one replay of %d steps" % RG,
              "replays": len(evs), "p10": float(np.percentile(per_replay, 10)),
              "median": float(np.median(per_replay)), "p90": float(np.percentile(per_replay, 90))}

    def time_graph(g, calls_per_replay):
        reps = max(1, args.steps // RG)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g.replay()
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * calls_per_replay)  # us per call

    us_attn = time_graph(g_attn, RG)
    us_mask = time_graph(g_mask, RS)
    us_acc = time_graph(g_acc, RS) if g_acc is not None else 0.0

    # D-cut budget selection (the step that shapes this workload's chains),
    # timed the same way when the workload carries draft confidences
    next_rows = {}
    if "confidence" in (w.meta or {}):
        conf_d = torch.from_numpy(np.asarray(w.meta["confidence"], np.float32)).to(dev)
        tok_d = torch.zeros((conf_d.shape[0], conf_d.shape[1] + 1), dtype=torch.int32, device=dev)
        nb, kb = conf_d.shape[0], w.meta["budget"]
        dc_out = {"n_keep": torch.empty(nb, dtype=torch.int32, device=dev),
                  "cu_nodes": torch.empty(nb + 1, dtype=torch.int32, device=dev),
                  "parent": torch.empty(kb, dtype=torch.int32, device=dev),
                  "packed_tokens": torch.empty(kb, dtype=torch.int32, device=dev)}
        tv.dcut_select(conf_d, tok_d, kb, out=dc_out)
        g_dcut = capture(lambda: [tv.dcut_select(conf_d, tok_d, kb, out=dc_out)
                                  for _ in range(RS)])
        next_rows["dcut_select_us"] = time_graph(g_dcut, RS)
        next_rows["dcut_select_shape"] = "batch %d, draft_len %d, budget %d" % (
            conf_d.shape[0], conf_d.shape[1], w.meta["budget"])
    # SpecOPD E2E-TV statistics over the branch nodes (needs both models'
    # logits: seeded synthetic ones, target ~ N(0, 3^2), draft = target + N(0, 1))
    if "anchors" in (w.meta or {}):
        nb_nodes = w.total_nodes - int(w.meta["trunk"])
        vocab = W.QWEN3_VOCAB
        gen = torch.Generator(device=dev).manual_seed(args.config)
        tl = (torch.randn((nb_nodes, vocab), generator=gen, device=dev) * 3.0).to(torch.bfloat16)
        dl = (tl.float() + torch.randn((nb_nodes, vocab), generator=gen, device=dev)).to(torch.bfloat16)
        width = nb_nodes // len(w.meta["anchors"])
        cu_b = torch.arange(0, nb_nodes + 1, width, dtype=torch.int32, device=dev)
        tv.e2e_tv_stats(tl, dl, cu_b)
        g_tv = capture(lambda: [tv.e2e_tv_stats(tl, dl, cu_b) for _ in range(8)])
        us_tv = time_graph(g_tv, 8)
        tv_bytes = 2 * tl.numel() * tl.element_size()
        next_rows["e2e_tv_stats_us"] = us_tv
        next_rows["e2e_tv_stats_shape"] = "%d branch nodes x %d vocab, bf16 logits" % (nb_nodes, vocab)
        next_rows["e2e_tv_stats_gbs"] = tv_bytes / (us_tv * 1e-6) / 1e9
        next_rows["e2e_tv_stats_hbm_frac"] = next_rows["e2e_tv_stats_gbs"] / HBM_PEAK_GBS
    # Graft's retrieval table for the Graft-shaped tree: the online update from
    # the target's logits at the 60 verified nodes (seeded synthetic logits,
    # N(0, 3^2)) and the 20-slot retrieval template under the graft point
    if w.name == W.CONFIG_NAMES[2]:
        vocab, k_adj = W.QWEN3_VOCAB, 8
        gen = torch.Generator(device=dev).manual_seed(args.config)
        adj = torch.randint(0, vocab, (vocab, k_adj), generator=gen, device=dev, dtype=torch.int32)
        lg = (torch.randn((w.total_nodes, vocab), generator=gen, device=dev) * 3.0).to(torch.bfloat16)
        node_tok = torch.randint(0, vocab, (w.total_nodes,), generator=gen, device=dev,
                                 dtype=torch.int32)
        par_t, rank_t, seen, kids = [], [], {W.GRAFT_TREE_PARENT[40]: -1}, {}
        for j in range(40, 60):
            seen[j] = j - 40
            pp = seen[W.GRAFT_TREE_PARENT[j]]
            kids[pp] = kids.get(pp, 0) + 1
            par_t.append(pp)
            rank_t.append(kids[pp] - 1)
        roots = node_tok[:1].clone()
        ret_out = torch.empty((1, len(par_t)), dtype=torch.int32, device=dev)
        ws_up = torch.empty(max(1, tv.graft_update_workspace_size(w.total_nodes, vocab, k_adj)),
                            dtype=torch.uint8, device=dev)
        tv.graft_update(adj, lg, node_tok, workspace=ws_up)
        tv.graft_retrieve(adj, roots, par_t, rank_t, out=ret_out)
        g_up = capture(lambda: [tv.graft_update(adj, lg, node_tok, workspace=ws_up)
                                for _ in range(RS)])
        g_ret = capture(lambda: [tv.graft_retrieve(adj, roots, par_t, rank_t, out=ret_out)
                                 for _ in range(RS)])
        us_up = time_graph(g_up, RS)
        next_rows["graft_update_us"] = us_up
        next_rows["graft_update_gbs"] = 2 * lg.numel() / (us_up * 1e-6) / 1e9
        next_rows["graft_update_shape"] = "%d verified nodes x %d vocab bf16 logits, k %d" % (
            w.total_nodes, vocab, k_adj)
        next_rows["graft_retrieve_us"] = time_graph(g_ret, RS)
        next_rows["graft_retrieve_shape"] = "1 request, 20-slot template (depth %d)" % 5
    # Stochastic verification of the same tree at temperature 1: seeded target
    # and draft logits (N(0, 3^2), draft = target + N(0, 1)), children drawn
    # from the draft without replacement, seeded uniforms
    if w.name == W.CONFIG_NAMES[2]:
        si = W.sampled_inputs(np.random.default_rng(args.config), [list(W.GRAFT_TREE_PARENT)],
                              W.QWEN3_VOCAB)
        s_par = torch.from_numpy(si.parent).to(dev)
        s_tok = torch.from_numpy(si.draft_tok).to(dev)
        s_cu = torch.from_numpy(si.cu_nodes).to(dev)
        s_tl = torch.from_numpy(si.target_logits).to(torch.bfloat16).to(dev)
        s_dl = torch.from_numpy(si.draft_logits).to(torch.bfloat16).to(dev)
        s_ua = torch.from_numpy(si.u_accept).to(dev)
        s_ub = torch.from_numpy(si.u_bonus).to(dev)
        s_ws = torch.empty(max(1, tv.tree_accept_sampled_workspace_size(
            len(si.parent), si.max_children, W.QWEN3_VOCAB)),
                           dtype=torch.uint8, device=dev)
        s_out = {"accept_len": torch.empty(1, dtype=torch.int32, device=dev),
                 "path": torch.empty((1, si.max_depth + 1), dtype=torch.int32, device=dev),
                 "bonus": torch.empty(1, dtype=torch.int32, device=dev)}

        def sampled_call():
            tv.tree_accept_sampled(s_par, s_tok, s_cu, s_tl, s_dl, s_ua, s_ub, len(si.parent),
                                   si.max_children, si.max_depth, 1.0, workspace=s_ws, out=s_out)
        sampled_call()
        g_s = capture(lambda: [sampled_call() for _ in range(8)])
        next_rows["accept_sampled_us"] = time_graph(g_s, 8)
        next_rows["accept_sampled_len"] = int(s_out["accept_len"].item())
        next_rows["accept_sampled_shape"] = (
            "60-node Graft tree, 151936-vocab bf16 target and draft logits, T = 1")
    achieved_gbs = alg_bytes / (us_attn * 1e-6) / 1e9
    achieved_tflops = alg_flops / (us_attn * 1e-6) / 1e12
    plan_splits = (need > 0)
    # the long-context and trunk-sharing workloads are bound by the matrix
    # cores (their arithmetic intensity is far above the ridge point), the
    # others by HBM bandwidth and latency
    mfma_bound = args.config in (4, 5)

    result = {
        "metric": METRIC,
        "value": w.total_nodes / (ms_per_step * 1e-3),
        "unit": "tree-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) Q/K/V, generated tree and tokens)",
        "config": {"workload": w.name, "batch": w.batch, "tree_nodes": w.total_nodes,
                   "max_prefix_len": w.max_prefix_len, "q_heads": w.num_q_heads,
                   "kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "page_size": w.page_size,
                   "mask": w.mask_kind, "rotating_buffer_sets": R, "hip_graph": True},
        "roofline": ({"bound": "mfma", "achieved": achieved_tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                      "unit": "TFLOP/s", "frac": achieved_tflops / MFMA_BF16_PEAK_TFLOPS}
                     if mfma_bound else
                     {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS,
                      "unit": "GB/s", "frac": achieved_gbs / HBM_PEAK_GBS}) | {
                     "traffic": measured_traffic(w.name),
                     "kernel_source_sha256": kernel_source_hash(),
                     "kernel": "tree_verify_attn (attn_bf16_kernel%s)" %
                               (" + combine_kernel" if plan_splits else ""),
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "us_per_launch": us_attn},
        "mfma": {"achieved_tflops": achieved_tflops, "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                 "frac": achieved_tflops / MFMA_BF16_PEAK_TFLOPS,
                 "algorithmic_flops_per_launch": alg_flops},
        "hbm": {"achieved_gbs": achieved_gbs, "peak_gbs": HBM_PEAK_GBS,
                "frac": achieved_gbs / HBM_PEAK_GBS},
        "breakdown_us": {"tree_mask_build": us_mask, "tree_verify_attn": us_attn,
                         "tree_accept": us_acc, "step": ms_per_step * 1e3},
        "step_spread_us": spread,
    }
    if next_rows:
        result["next_rows"] = next_rows
    others = [int(c) for c in args.other_configs.split(",") if c.strip()]
    others = [c for c in others if c != args.config]
    if others:
        del qs, ks, vs, outs, g_full, g_rem, g_attn
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        result["configs"] = []
        for c in others:
            log("timing tree_verify_attn on workload", W.CONFIG_NAMES[c])
            result["configs"].append(measure_other(c, args.steps, dev))
    if not args.no_cpu_baseline:
        log("timing the CPU oracle (about %.0f s)" % args.cpu_seconds)
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        log("timing the CPU oracle on host threads (about %.0f s)" % args.cpu_seconds)
        result["cpu_baseline_threads"] = cpu_baseline_threads(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
