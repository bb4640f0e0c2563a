"""Decode-step benchmark of the sparse decode library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

A step is one whole decode step (index scan + top-k + sparse attention) of
the named workload over one batch of synthetic inputs already resident in
HBM, enqueued through the C ABI on one stream (``--graph``: replayed as a
captured HIP graph instead, measured about 2.5 % slower here).  Two input sets
with different seeds alternate so that the timed window never re-reads a
set that the 256 MB last-level cache could hold.  Prints ONE JSON line.

The default workload is the lightning-indexer decode at 128K context: batch
32, 131072 cached tokens, 64 index heads over an fp8 K-index with per-token
scales, top-2048, 128-head MLA attention over 576-wide bf16 latent rows in
64-token pages.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
PREQUEUE_CYCLES = 4_000_000  # spin ahead of the timed steps (about 2 ms of shader clock)
METRIC = "sparse decode steps/s (score+top-k+attn) at 128K ctx; % of HBM peak BW"


def algorithmic_bytes(w, bits=None) -> dict:
    """Bytes the method must move per step (no score scratch).  bits: the
    planes read per key of the Fathom scan (default: the bit budget)."""
    B, n, k = w.B, w.n, w.k
    bits = w.budget if bits is None else bits
    out = {}
    if w.kind == "lightning":
        out["k_index"] = B * n * (w.idx_dim + 4)            # fp8 key + fp32 scale
        out["selected_kv"] = B * k * w.d_qk * 2             # latent rows, read once
        out["q_w"] = B * w.idx_heads * (w.idx_dim * 2 + 4) + B * w.hq * w.d_qk * 2
        out["out"] = B * w.hq * (w.d_v + 1) * 4
        out["idx_pt"] = B * k * 4 * 2                       # top-k ids + page-table reads
    elif w.kind == "block":
        out["k_index"] = B * n * w.idx_dim * 2
        out["selected_kv"] = w.layers * B * k * w.block * w.hkv * (w.d_qk + w.d_v) * 2
        out["q_w"] = B * w.idx_heads * w.idx_dim * 2 + w.layers * B * w.hq * w.d_qk * 2
        out["out"] = w.layers * B * w.hq * (w.d_v + 1) * 4
        out["idx_pt"] = B * k * 4
    elif w.kind == "fathom":
        out["k_index"] = B * w.hkv * (bits * n // 8 + w.d_qk * 12)  # planes read + zero/scale/var
        out["selected_kv"] = B * w.hkv * k * (w.d_qk + w.d_v) * 2
        out["q_w"] = B * w.hq * w.d_qk * 2
        out["out"] = B * w.hq * (w.d_v + 1) * 4
        out["idx_pt"] = B * w.hkv * k * 4
    elif w.kind == "dot":
        out["k_index"] = B * n * w.d_qk * 4
        out["selected_kv"] = B * k * w.hkv * (w.d_qk + w.d_v) * 4
        out["q_w"] = B * w.hq * w.d_qk * 4
        out["out"] = B * w.hq * (w.d_v + 1) * 4
        out["idx_pt"] = B * k * 4
    out["total"] = sum(out.values())
    return out


def compute_dtype(w) -> str:
    """The arithmetic type of the step's contractions: fp32 for the fp32
    workload; otherwise bf16 MFMA with fp32 accumulation (the fp8 K-index
    and the 4-bit planes are widened exactly before they are used)."""
    return "f32" if w.dtype == "f32" else "bf16"


def score_kernel_bytes(w, bits=None) -> int:
    """Algorithmic bytes of one launch of the index-scan kernel."""
    bits = w.budget if bits is None else bits
    if w.kind == "lightning":
        return w.B * w.n * (w.idx_dim + 4)
    if w.kind == "block":
        return w.B * w.n * w.idx_dim * 2
    if w.kind == "fathom":
        return w.B * w.hkv * bits * w.n // 8
    return w.B * w.n * w.d_qk * 4


ROOT = os.path.dirname(os.path.abspath(__file__))
SCORE_SOURCES = ("indexer_top_sparse_amd/csrc/score.hip", "indexer_top_sparse_amd/csrc/common.hpp")


def score_source_digest() -> str:
    """sha256 over the sources the index-scan kernels are built from."""
    h = hashlib.sha256()
    for rel in SCORE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profiled_traffic(w):
    """HBM bytes per index-scan launch from the committed counter summary of
    this workload (FETCH_SIZE and WRITE_SIZE, each scaled by what the same
    counter reads for a plain copy of known size), or None when there is no
    summary or the kernel sources have changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"score_{w.kind}_{w.name}_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln:
                key, _, val = ln.partition(":")
                fields[key.strip()] = val.strip()
    if fields.get("kernel_source_sha256") != score_source_digest():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def calibrate_copy() -> int:
    """A plain 256 MiB device-to-device copy, five times: the known-size
    kernel that FETCH_SIZE and WRITE_SIZE are scaled against."""
    import torch

    n = 256 * 1024 * 1024
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}), flush=True)
    return 0


def cpu_baseline(w, inp, requests: int) -> dict:
    """The oracle (as it stands) on a bounded sample of the same workload."""
    import numpy as np
    import torch

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import synth  # noqa: F401
    from oracle import step as S

    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = 1
    p = {"n": w.n, "k": w.k, "hq": w.hq, "hkv": w.hkv, "dtype": w.dtype,
         "seq_lens": w.seq_lens, "page": w.page, "block": w.block, "budget": w.budget,
         "d_qk": w.d_qk, "d_v": w.d_v}
    reqs = list(range(min(requests, w.B)))
    if w.kind != "lightning":
        raise ValueError("cpu baseline sample is defined for the lightning workload")
    t_total = 0.0
    for b in reqs:
        # request b's inputs only; its pages renumbered 0..n_pages-1
        pt = inp["page_table"][b].long()
        arr = {
            "q_idx": synth.host_view(inp["q_idx"][b:b + 1]),
            "head_w": synth.host_view(inp["head_w"][b:b + 1]),
            "k8": synth.host_view(inp["k8"][b:b + 1]),
            "k_scale": synth.host_view(inp["k_scale"][b:b + 1]),
            "q": synth.host_view(inp["q"][b:b + 1]),
            "kv_pool": synth.host_view(inp["kv_pool"].index_select(0, pt)),
            "page_table": np.arange(pt.numel(), dtype=np.int32)[None, :],
        }
        t0 = time.perf_counter()
        S.lightning_step(arr, p)
        t_total += time.perf_counter() - t0
    per_req = t_total / len(reqs)
    return {"value": 1.0 / (per_req * w.B), "unit": "steps/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(reqs)} of {w.B} requests at full context "
                      f"(n={w.n}, k={w.k}), oracle seconds scaled by {w.B}/{len(reqs)}; "
                      f"host cpu_count={os.cpu_count()}, "
                      f"affinity={len(os.sched_getaffinity(0))}, BLAS threads={threads}"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="lightning_128k")
    ap.add_argument("--graph", action="store_true",
                    help="capture each input set's step in a HIP graph and time the replays")
    ap.add_argument("--no-graph", action="store_true",
                    help="enqueue the step directly (the default)")
    ap.add_argument("--cpu-requests", type=int, default=4)
    ap.add_argument("--no-prequeue", action="store_true",
                    help="start the timed steps on an empty queue (no spin kernel ahead of them)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--misses", type=int, default=1,
                    help="hot-buffer workloads: 1 = the workload's miss rate, 0 = none")
    ap.add_argument("--miss-rate", type=float, default=None,
                    help="hot-buffer workloads: this fixed miss rate (e.g. 0.4)")
    ap.add_argument("--fixed-depth", type=int, default=None, metavar="BITS",
                    help="Fathom workloads: a fixed allocation of BITS planes per key "
                         "(the same for every query) instead of the water-filling")
    ap.add_argument("--host-planes", action="store_true",
                    help="Fathom workloads: bit planes read in place from pinned host memory")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run the known-size copy that hardware byte counters are scaled by")
    ap.add_argument("--policy", choices=["lru"], default=None,
                    help="hot-buffer workloads: evolve the hot buffer with the least-recently-used "
                         "replacement (sparse_hot_update) over steps whose index queries drift")
    ap.add_argument("--drift", type=float, default=0.1,
                    help="--policy: per-step query drift q <- (1 - a) q + a noise")
    ap.add_argument("--prefetch", type=int, default=0,
                    help="--policy: after each update, prefetch the M tokens ranked just "
                         "below the top-k (a top-(k+M) of the same scores)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(requests would shard by batch with no exchange between GPUs)",
              file=sys.stderr)
        return 2

    if args.calibrate_copy:
        return calibrate_copy()
    if args.policy:
        return run_policy(args)

    import torch

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import synth
    from synth.gen import build_hot_buffer
    import indexer_top_sparse_amd as isa
    from indexer_top_sparse_amd.runner import StepRunner

    isa.lib()  # fail loudly if the HIP library is missing
    w = synth.get(args.config)
    miss_rate = (args.miss_rate if args.miss_rate is not None
                 else (w.miss_rate if args.misses else 0.0))
    dev = "cuda"
    print(f"[bench] generating inputs for {w.name}", file=sys.stderr, flush=True)
    sets = []
    # two input sets alternate; the hot-buffer workloads (whose K-index alone
    # is far larger than the last-level cache) use one to bound pinned memory
    for s in range(1 if w.hot else 2):
        ws = w.with_(seed=w.seed + 100 * s)
        inp = synth.make_inputs(ws, dev)
        if w.kind == "fathom" and args.fixed_depth is not None:
            inp["depth_in"] = synth.fixed_depths(ws, args.fixed_depth, dev)
        if w.kind == "fathom" and args.host_planes:
            inp["planes"] = synth.pinned_copy(inp["planes"])
        hot = None
        if w.hot:
            # the selection the step will make decides which rows are hot
            sel = _selection_for_hot(inp, ws, dev)
            hw = ws.with_(miss_rate=miss_rate)
            hot = build_hot_buffer(dict(inp, workload=hw), sel, dev)
        sets.append((inp, StepRunner(inp, hot=hot)))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    # warmup (eager), then capture one graph per input set
    ns = len(sets)
    for i in range(max(args.warmup, 1)):
        sets[i % ns][1].run()
    torch.cuda.synchronize()
    graphs = []
    if args.graph and not args.no_graph:
        for _, r in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                r.run()
            graphs.append(g)
        for i in range(max(args.warmup, 1)):
            graphs[i % ns].replay()
    torch.cuda.synchronize()

    # dominant kernel: the index scan, one launch at a time between HIP events
    # on the stream it runs on, each launch preceded by a whole step over the
    # other input set so that the caches are in the state the step leaves.
    # It runs before the timed steps, so those start on a GPU that has been
    # busy for a while (a short run straight after a few warm-up steps is a
    # few percent slower than the steady state)
    reps = 20
    sets[0][1].index_scores()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(evs):
        if graphs:
            graphs[(i + 1) % ns].replay()
        else:
            sets[(i + 1) % ns][1].run()
        e0.record(stream)
        sets[i % ns][1].index_scores()
        e1.record(stream)
    torch.cuda.synchronize()
    score_ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / reps
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    # HIP events on the stream the steps run on bracket exactly the K timed
    # steps, inside a synchronize on both sides; the host clock around the
    # same region (less the spin ahead of it) is reported beside it (it adds
    # the fixed cost of draining the queue, which a short run does not
    # amortise)
    t_beg = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_pre = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_pre.record(stream)
    if not args.no_prequeue:
        # The host takes longer to enqueue a step than the GPU takes to start
        # it once the queue is empty, so on an idle GPU the first steps would
        # wait for their own launches.  A spin kernel of about 2 ms ahead of
        # the timed region lets the host queue the steps behind it; the events
        # after it then see only the GPU running the K steps.
        torch.cuda._sleep(PREQUEUE_CYCLES)
    t_beg.record(stream)
    for i in range(args.steps):
        if graphs:
            graphs[i % ns].replay()
        else:
            sets[i % ns][1].run()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0 - t_pre.elapsed_time(t_beg) * 1e-3
    elapsed = t_beg.elapsed_time(t_end) * 1e-3
    ms = 1e3 * elapsed / args.steps
    steps_s = args.steps / elapsed

    bits = args.fixed_depth if (w.kind == "fathom" and args.fixed_depth is not None) else None
    kb = score_kernel_bytes(w, bits)
    achieved = kb / (score_ms * 1e-3) / 1e9
    traffic = profiled_traffic(w)

    ab = algorithmic_bytes(w, bits)
    line = {
        "metric": METRIC,
        "value": round(steps_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": compute_dtype(w),
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "context": w.n, "top_k": w.k,
                   "index_heads": w.idx_heads, "attn_heads": w.hq, "kv_heads": w.hkv,
                   "d_qk": w.d_qk, "d_v": w.d_v, "page": w.page, "block": w.block,
                   "bit_budget": w.budget, "hot_tokens": w.hot,
                   "miss_rate": miss_rate if w.hot else None,
                   "fixed_depth_bits": bits, "host_planes": bool(args.host_planes and w.kind == "fathom"),
                   "graph": bool(graphs)},
        "host_wall_ms_per_step": round(1e3 * wall / args.steps, 5),
        "step_bytes": ab["total"],
        "step_GBps": round(ab["total"] / (ms * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(ab["total"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {"kernel": f"index scan ({w.kind})", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "avg_launch_ms": round(score_ms, 5),
                     "bytes_per_launch": kb},
    }
    if not args.no_cpu and w.kind == "lightning" and not w.hot:
        print("[bench] timing the oracle on a sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, sets[0][0], args.cpu_requests)
    line["append"] = time_append(w, sets[-1][1], stream)
    print(json.dumps(line), flush=True)
    return 0


def time_append(w, r, stream) -> dict:
    """The decode-side append of one new token per request (index entry and
    KV rows) into the last input set, timed with HIP events (last, since it
    changes that set's inputs)."""
    import torch
    import indexer_top_sparse_amd as isa

    dev = r.topk.device
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed * 1000 + 99)
    pos = torch.tensor([min(w.valid(b), w.n - 1) for b in range(w.B)], dtype=torch.int32,
                       device=dev)
    aa, _ = r.layer_args[0]
    kd = w.idx_dim if w.kind in ("lightning", "block") else w.d_qk
    key_shape = (w.B, w.hkv, kd) if w.kind == "fathom" else (w.B, kd)
    key_new = torch.randn(key_shape, generator=g, device=dev)
    kvh = 1 if w.kind == "lightning" else w.hkv
    cdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    k_new = torch.randn((w.B, kvh, w.d_qk), generator=g, device=dev).to(cdt)
    v_new = None
    if aa.c.v_cache:
        v_new = torch.randn((w.B, kvh, w.d_v), generator=g, device=dev).to(cdt)
    reps = 20
    for _ in range(3):
        isa.sparse_append_token(r.ia, aa, pos, key_new, k_new, v_new, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        isa.sparse_append_token(r.ia, aa, pos, key_new, k_new, v_new, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    return {"us_per_call": round(e0.elapsed_time(e1) / reps * 1e3, 2), "tokens": w.B}


def run_policy(args) -> int:
    """Hot-buffer workloads with the replacement policy: steps (eager, since
    each update carries its own step number) whose index queries drift, each
    followed by sparse_hot_update and, with --prefetch M, by
    sparse_hot_prefetch of the M tokens ranked just below the top-k.
    Reports steps/s of step + update (+ prefetch), the update's and the
    prefetch's own times and the miss rate the policy leaves."""
    import torch

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import synth
    from synth.gen import build_hot_buffer
    import indexer_top_sparse_amd as isa
    from indexer_top_sparse_amd.runner import StepRunner

    isa.lib()
    w = synth.get(args.config)
    if not w.hot:
        print("--policy needs a hot-buffer workload", file=sys.stderr)
        return 2
    dev = "cuda"
    inp = synth.make_inputs(w, dev)
    # the starting buffer: the first selection, at the workload's miss rate
    hot = build_hot_buffer(inp, _selection_for_hot(inp, w, dev), dev)
    r = StepRunner(inp, hot=hot)
    S = w.hot
    hs = hot["hot_slot"]
    toks = torch.full((w.B, S), -1, dtype=torch.int32, device=dev)
    bi, ti = torch.nonzero(hs >= 0, as_tuple=True)
    toks[bi, hs[bi, ti].long()] = ti.to(torch.int32)
    stamps = torch.zeros((w.B, S), dtype=torch.int32, device=dev)
    aa = r.layer_args[0][0]
    q = inp["q_idx"]
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 555)
    args.warmup = max(args.warmup, 1)
    total = args.warmup + args.steps
    qs = []
    for _ in range(total):
        noise = torch.randn(q.shape, generator=g, device=dev, dtype=torch.float32)
        q.copy_(((1.0 - args.drift) * q.float() + args.drift * noise).to(q.dtype))
        qs.append(q.clone())
    misses = torch.zeros((), dtype=torch.int64, device=dev)
    selected = torch.zeros((), dtype=torch.int64, device=dev)
    # missed rows of every step (warm-up included, in dispatch order), so that
    # a kernel trace's miss-fetch durations pair with the bytes each moved
    miss_log = torch.zeros(total, dtype=torch.int64, device=dev)
    seq = inp.get("seq_lens")
    vl = (seq if seq is not None else torch.full((w.B,), w.n, device=dev)).view(-1, 1)
    upd = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]

    M = args.prefetch
    if M:
        # the decomposed step keeps the scores, whose top-(k+M) names the
        # prefetch candidates; its top-k runs in a workspace of its own so
        # that the staged rows survive until the update
        r.index_scores()
        ws_t = isa.workspace(isa.sparse_topk_workspace_size(w.B, w.n, w.k + M))
        cand = torch.empty((w.B, w.k + M), dtype=torch.int32, device=dev)
        pf = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]

    def step(i, timed):
        q.copy_(qs[i])
        if M:
            sc = r.index_scores()[:, 0]
            isa.sparse_topk(sc, w.k, r.topk[:, 0], None, seq, 1, ws_t)
            isa.sparse_gather_attn_decode(aa, r.topk, 1, w.k, 1, r.outs[0], r.lses[0], r.ws)
        else:
            r.run()
        sel = r.topk[:, 0]
        ok = (sel >= 0) & (sel < vl)
        hit = torch.gather(hs, 1, sel.clamp(min=0).long()) >= 0
        miss_log[i] = (ok & ~hit).sum()
        misses.add_(miss_log[i])
        selected.add_(ok.sum())
        if timed:
            upd[i - args.warmup][0].record()
        isa.sparse_hot_update(None if M else r.ia, aa, r.topk, w.k, 1, S, i + 1, toks,
                              stamps, r.ws)
        if timed:
            upd[i - args.warmup][1].record()
        if M:
            isa.sparse_topk(sc, w.k + M, cand, None, seq, 1, ws_t)
            if timed:
                pf[i - args.warmup][0].record()
            isa.sparse_hot_prefetch(aa, cand, w.k + M, S, i + 1, toks, stamps)
            if timed:
                pf[i - args.warmup][1].record()

    print(f"[bench] {w.name}: {args.warmup} + {args.steps} steps with LRU replacement",
          file=sys.stderr, flush=True)
    # warm-up steps run every kernel the timed ones do (first launches load code)
    for i in range(max(args.warmup, 1)):
        step(i, False)
    torch.cuda.synchronize()
    misses.zero_()
    selected.zero_()
    # timed steps; the miss count (three small reductions per step) and the
    # update's events ride along
    t0 = time.perf_counter()
    for i in range(args.warmup, total):
        step(i, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    upd_us = sum(a.elapsed_time(b) for a, b in upd) / len(upd) * 1e3
    pf_us = sum(a.elapsed_time(b) for a, b in pf) / len(pf) * 1e3 if M else None
    line = {
        "metric": METRIC + " (hot buffer with LRU replacement)",
        "value": round(args.steps / elapsed, 2), "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(1e3 * elapsed / args.steps, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": compute_dtype(w), "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "context": w.n, "top_k": w.k,
                   "hot_tokens": S, "policy": args.policy, "drift": args.drift,
                   "start_miss_rate": w.miss_rate, "prefetch": M, "graph": False},
        "measured_miss_rate": round(misses.item() / max(selected.item(), 1), 4),
        "miss_rows_per_step": miss_log.cpu().tolist(),
        "row_bytes": w.d_qk * 2,
        "update_us_per_call": round(upd_us, 2),
        "prefetch_us_per_call": round(pf_us, 2) if M else None,
    }
    print(json.dumps(line), flush=True)
    return 0


def _selection_for_hot(inp, w, dev):
    """The step's own selection (indexer + top-k through the library), used
    only to decide which rows start in the hot buffer."""
    import torch
    import indexer_top_sparse_amd as isa

    ia = isa.lightning_index_args(inp["q_idx"], inp["head_w"], inp["k8"], inp["k_scale"],
                                  inp.get("seq_lens"))
    scores = torch.empty((w.B, w.n), dtype=torch.float32, device=dev)
    ws = isa.workspace(max(isa.sparse_workspace_size(ia, None, w.k),
                           isa.sparse_topk_workspace_size(w.B, w.n, w.k)), dev)
    isa.sparse_index_score(ia, scores, ws)
    sel = torch.empty((w.B, w.k), dtype=torch.int32, device=dev)
    isa.sparse_topk(scores, w.k, sel, None, inp.get("seq_lens"), 1, ws)
    torch.cuda.synchronize()
    return sel


if __name__ == "__main__":
    sys.exit(main())
