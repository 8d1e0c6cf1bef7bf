"""HGA forward + backward throughput on one MI355X.

One step = the whole hot path over one batch of the 16K-context workload: chunk
and group summaries of K, two-level routing, exact-token attention forward, and
the backward (dQ, then dK/dV).  Workload: a 2048-query segment at the end of a
16384-token history, 32 query / 8 kv heads, head_dim 128, chunk 64, group 8,
top-k 16 chunks, top-g 64 groups, bf16, seeded synthetic inputs.  Inputs are
resident in HBM before the timed region.

The timed region replays the step from a HIP graph (the kernels allocate and
clear nothing, so a replay is the eager step without host launch gaps); the
eager step time is reported beside it.  Per-phase times come from HIP events
around each kernel in an eager pass (each includes its launch gap).  The
roofline kernel's duration comes from 20 back-to-back launches of that kernel
alone in one graph, with HIP events on the replay stream.

Prints one JSON line: throughput in query tokens/s, per-phase kernel times, the
roofline of the dominant kernel, and the CPU oracle timed on a bounded sample
of the same workload.  --decode and --segments select the other two workloads.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HGA fwd+bwd query tokens/sec at 16K ctx, 1 MI355X; % HBM / % MFMA peak"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = {
    "summaries": ["summaries.hip"],
    "route": ["route.hip"],
    "attend_fwd": ["attend_fwd.hip"],
    "attend_bwd_dq": ["attend_bwd.hip"],
    "attend_bwd_dkdv": ["attend_bwd_dkdv.hip", "bwd_common.h"],
    "attend_bwd_dkdv_order": ["attend_bwd_dkdv.hip", "bwd_common.h"],
    "decode_route": ["route.hip"],
    "decode_attend": ["decode.hip"],
}


def source_hash(phase: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "hierarchical_routed_sparse_amd", "csrc")
    for f in KERNEL_SOURCES[phase] + ["hga_device.h", "../build_lib.py"]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="segment_2k_over_16k",
                    help="segment_2k_over_16k (the headline), causal_16k, fwd_bwd_b2_4k, "
                         "qwen3_8b_2k, segment_2k_over_64k_ties, tiny_fp32_1k")
    ap.add_argument("--side-by-side-bwd", action="store_true",
                    help="time the backward as the preparation pass, then dQ on a second "
                         "stream beside dK/dV (default: dQ, then dK/dV on one stream)")
    ap.add_argument("--fwd-only", action="store_true",
                    help="time the forward step only (summaries, routing, attention)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle leg (profiling runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--segments", action="store_true",
                    help="segment-wise mode: the 16384-token sequence as 8 segments of 2048, "
                         "each forward + backward with the history detached")
    ap.add_argument("--host-kv", action="store_true",
                    help="with --segments or --decode: keep the keys and values in pinned "
                         "host memory")
    ap.add_argument("--stage", action="store_true",
                    help="with --segments: stage each segment's routed working set (the "
                         "distinct kept history groups and the segment's rows) into HBM")
    ap.add_argument("--seg-on-device", action="store_true",
                    help="with --segments --stage: each segment's keys and values are also "
                         "given in device memory (the active segment), and staged from there")
    ap.add_argument("--causal", action="store_true",
                    help="strictly causal routing (block j routed with the 64 queries before it)")
    ap.add_argument("--decode", action="store_true",
                    help="decode mode: 64 new tokens per sequence (one block) over a 16K "
                         "cache, batch 16; with --causal the block is routed once")
    return ap.parse_args()


def algorithmic_work(w, pairs: int) -> dict:
    """Per-launch algorithmic bytes or flops of each phase (one launch per
    step).  Flops count the products the method needs, 2*D per attended pair
    and product: the forward's two (Q.K^T, P.V), the backward's five
    (Q.K^T and dO.V^T for P and dP, then dS.K for dQ, P^T.dO for dV and
    dS^T.Q for dK), of which the dQ call needs the first three and the dK/dV
    call the last two.  The recomputation of Q.K^T and dO.V^T in the dK/dV
    kernel is not counted here (see executed_work)."""
    B, Hq, Hkv, D, Sq, Skv = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.q_len, w.kv_len
    esz = 2 if w.dtype == "bf16" else 4
    means = B * Hkv * (Skv // 64 + Skv // 8) * D * 4
    idx = B * Hq * (Sq // 64) * (w.top_k + w.top_g) * 4
    return {
        # read K once, write the fp32 chunk and group means once
        "summaries": ("hbm", B * Hkv * Skv * D * esz + means),
        # read Q once and the means once, write the indices
        "route": ("hbm", B * Hq * Sq * D * esz + means + idx),
        # 2 products (Q.K^T, P.V) of 2*D flops per attended pair
        "attend_fwd": ("mfma", 4 * D * pairs),
        # Q.K^T, dO.V^T, dS.K
        "attend_bwd_dq": ("mfma", 6 * D * pairs),
        # P^T.dO, dS^T.Q
        "attend_bwd_dkdv": ("mfma", 4 * D * pairs),
    }


def executed_work(group_idx, D: int) -> dict:
    """MFMA flops the attention kernels issue per launch, counted from their
    tiling and the routing: the forward and dQ kernels walk 32-key tiles (the
    own chunk as two tiles, then the kept groups four per tile) for the 64
    queries of a routing row, 2*D flops per (query, key) slot and product (2
    products forward, 3 for dQ); the dK/dV kernel takes, for every (routing
    row, chunk) it attends, the 16-key slices (group pairs) with a kept group
    (all four for the own chunk) against the 64 queries, with 4 products
    (Q.K^T and dO.V^T recomputed, then P^T.dO and dS^T.Q).  Masked slots
    count: this is what the matrix cores execute, not the method's work."""
    import numpy as np
    gi = group_idx.reshape(-1, group_idx.shape[-1])
    kept = (gi >= 0).sum(axis=1)
    tiles = 2 + (kept + 3) // 4
    slots = int(tiles.sum()) * 32 * 64
    g = np.where(gi >= 0, gi, -1)
    # distinct (chunk, group pair) per row: (g >> 1) identifies the pair
    pairs = 0
    for row in g:
        v = row[row >= 0]
        pairs += len(np.unique(v >> 1))
    slices = pairs + 4 * gi.shape[0]
    return {
        "attend_fwd": 4 * D * slots,
        "attend_bwd_dq": 6 * D * slots,
        "attend_bwd_dkdv": 8 * D * slices * 16 * 64,
    }


def attended_pairs(group_idx) -> int:
    """Attended (query, key) pairs: 64*8 per kept group plus 64*65/2 causal
    pairs of the own chunk, for every routing row."""
    kept = int((group_idx >= 0).sum().item())
    rows = group_idx.shape[0] * group_idx.shape[1] * group_idx.shape[2]
    return 64 * 8 * kept + rows * (64 * 65 // 2)


# the kernels one call of a phase launches, in order, where there are several
# (none at present: the dK/dV work order of the whole range is computed inside
# the dQ call; only a chunk sub-range call adds dkdv_order_kernel)
PHASE_KERNELS = {}
KERNEL_NAMES = {
    "summaries": "summaries_kernel", "route": "route_kernel", "attend_fwd": "attend_fwd_kernel",
    "attend_bwd_dq": "attend_bwd_dq_kernel", "attend_bwd_dkdv": "attend_bwd_dkdv_kernel",
    "attend_bwd_dkdv_order": "dkdv_order_kernel", "decode_route": "route_kernel",
    "decode_attend": "decode_kernel",
}


def load_traffic(phase: str, workload: str):
    """HBM bytes per call of `phase` at `workload`, summed over the kernels the
    call launches, from the stored counter runs (profiles/hbm_traffic.json,
    keyed by workload, then phase); None when any of them is missing or its
    sources changed since."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    total = 0.0
    for k in PHASE_KERNELS.get(phase, [phase]):
        r = rec.get("workloads", {}).get(workload, {}).get(k)
        if not r or r.get("source_sha") != source_hash(k):
            return None
        total += r.get("hbm_bytes_per_launch")
    return total


def cpu_host():
    """The host's CPU model and the threads this process may use (capped at
    16, the CPU share of one GPU on the measurement boxes)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return model, n, min(n, 16)


def cpu_baseline(w, x, budget_s: float = 12.0, causal: bool = False, fwd_only: bool = False,
                 parallel_s: float = 4.0, span: int = 8):
    """The CPU oracle on the same inputs, timed two ways.

    Work unit: the routing rows of one (b, kv head) over `span` consecutive
    64-query blocks (all of the kv head's query heads), run as the oracle's
    segment at the end of its own prefix of the history: routing over the
    prefix's summaries, attention forward and, unless `fwd_only`, the
    backward.  That is exactly those rows' share of the layer's work (the
    unit's dK/dV are partial sums of the layer's).  Units are taken in a
    seeded random order.  The summaries of every kv head are timed once in
    full.  Single thread: units one after another until `budget_s` seconds;
    all cores: the same units on a pool of host threads (the oracle is C,
    called through ctypes, which releases the interpreter lock) until
    `parallel_s` seconds of wall time.  Each rate is scaled from its sample
    of units to the whole layer."""
    import concurrent.futures as cf
    import threading
    import numpy as np
    import oracle
    from hierarchical_routed_sparse_amd import synthetic as syn
    oracle.build(force=False)
    B, Hq, Hkv = w.batch, w.n_q_heads, w.n_kv_heads
    r, nblk, q0 = Hq // Hkv, w.q_len // 64, w.kv_len - w.q_len
    span = min(span, nblk)
    Kf = syn.to_f64(x["K"], w.dtype)
    Vf = syn.to_f64(x["V"], w.dtype)
    t0 = time.perf_counter()
    cm, gm = oracle.summaries(Kf)
    t_summ = time.perf_counter() - t0
    units = [(b, hk, j) for b in range(B) for hk in range(Hkv) for j in range(0, nblk, span)]
    order = np.random.default_rng(0).permutation(len(units))

    def prep(i):
        b, hk, j = units[i]
        hs = slice(hk * r, (hk + 1) * r)
        n = min(span, nblk - j)
        end = q0 + 64 * (j + n)    # the unit's prefix: keys up to its last block's chunk
        qs = slice(64 * j, 64 * (j + n))
        u = {"Q": syn.to_f64(x["Q"][b:b + 1, hs, qs], w.dtype)}
        if not fwd_only:
            u["dO"] = syn.to_f64(x["dO"][b:b + 1, hs, qs], w.dtype)
        if causal:
            u["Qprev"] = syn.to_f64(x["Q"][b:b + 1, hs, 64 * (j - 1):64 * j], w.dtype) \
                if j > 0 else syn.to_f64(x["Qprev"][b:b + 1, hs], w.dtype)
        return u, Kf[b:b + 1, hk:hk + 1, :end], Vf[b:b + 1, hk:hk + 1, :end], \
            cm[b:b + 1, hk:hk + 1, :end // 64], gm[b:b + 1, hk:hk + 1, :end // 8], end

    def work(u, K, V, c, g, end):
        _, gi = oracle.route(u["Q"], c, g, end, w.top_k, w.top_g, causal=causal,
                             Qprev=u.get("Qprev"))
        oracle.attend_fwd(u["Q"], K, V, gi)
        if not fwd_only:
            oracle.attend_bwd(u["Q"], K, V, gi, u["dO"])

    done, dt = 0, 0.0
    for i in order:
        args = prep(i)
        t0 = time.perf_counter()
        work(*args)
        dt += time.perf_counter() - t0
        done += 1
        if dt >= budget_s:
            break
    t_layer = t_summ + dt * len(units) / done
    model, avail, threads = cpu_host()
    what = "routing, attention forward" + ("" if fwd_only else " and backward")
    res = {
        "value": w.batch * w.q_len / t_layer,
        "unit": "query tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{done} of the {len(units)} units of {span} query blocks x {r} query heads "
                   f"(seeded random order), each the oracle's segment over its own history "
                   f"prefix ({what}, fp64), {dt:.1f} s single-threaded, scaled "
                   f"x{len(units) / done:.2f} to the layer, plus the summaries of the whole "
                   f"layer ({t_summ:.2f} s)"),
        "cpu_model": model,
        "host_threads_available": avail,
    }
    # all cores: a pool of threads pulling prepared units until the wall-time
    # budget (the units' inputs are sliced before the timed region)
    need = min(len(units), int(1.5 * threads * parallel_s * done / dt) + threads)
    ready = [prep(i) for i in order[:need]]
    nxt = iter(ready)
    lock = threading.Lock()
    counts = []
    deadline = time.perf_counter() + parallel_s

    def worker():
        n = 0
        while time.perf_counter() < deadline:
            with lock:
                a = next(nxt, None)
            if a is None:
                break
            work(*a)
            n += 1
        counts.append(n)

    t0 = time.perf_counter()
    deadline = t0 + parallel_s
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        for f in [ex.submit(worker) for _ in range(threads)]:
            f.result()
    wall = time.perf_counter() - t0
    pdone = sum(counts)
    t_par = t_summ / threads + wall * len(units) / max(pdone, 1)
    res["all_cores"] = {
        "value": w.batch * w.q_len / t_par,
        "unit": "query tokens/s",
        "cores": threads,
        "sample": (f"{pdone} units (the same unit work) on {threads} threads in {wall:.1f} s "
                   f"wall, scaled x{len(units) / max(pdone, 1):.2f} to the layer; summaries "
                   f"counted as split over the threads"),
    }
    return res


def segments_main(args):
    """Segment-wise training step of one layer: a 16384-token sequence cut into
    8 segments of 2048 tokens, each running summaries (appended), routing,
    attention forward and the backward (dQ; dK, dV of the segment's own keys
    only) in order.  Reports the whole sequence's rate and each segment's time
    against its offset."""
    import torch
    from hierarchical_routed_sparse_amd import synthetic as syn
    from hierarchical_routed_sparse_amd.segments import SegmentRunner

    L, S = 16384, 2048
    w = syn.Workload("sequence_16k", 1, 32, 8, 128, L, L, 16, 64, "bf16", 5,
                     1 / (128 ** 0.5), backward=True)
    x = syn.make_inputs(w, with_grad_output=True)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    t = {k: syn.to_torch(v, w.dtype, dev) for k, v in x.items()}
    run = SegmentRunner(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, L, S, w.top_k, w.top_g,
                        dtype=w.dtype, device=dev, kv_on_host=args.host_kv, stage=args.stage)
    run.k_history.copy_(t["K"].cpu() if args.host_kv else t["K"])
    run.v_history.copy_(t["V"].cpu() if args.host_kv else t["V"])
    nseg = L // S
    Qs = [t["Q"][:, :, i * S:(i + 1) * S].contiguous() for i in range(nseg)]
    dOs = [t["dO"][:, :, i * S:(i + 1) * S].contiguous() for i in range(nseg)]
    stream = torch.cuda.current_stream()

    # --seg-on-device: each segment's keys and values also in device memory, as
    # a projection produces them (the active segment in VRAM); the staging then
    # takes the segment's rows from there
    Ks = Vs = [None] * nseg
    if args.seg_on_device:
        Ks = [t["K"][:, :, i * S:(i + 1) * S].contiguous() for i in range(nseg)]
        Vs = [t["V"][:, :, i * S:(i + 1) * S].contiguous() for i in range(nseg)]

    def one_pass(ev=None):
        for i in range(nseg):
            if ev: ev[i][0].record(stream)
            run.step(i, Qs[i], dOs[i], stream=stream, K_seg=Ks[i], V_seg=Vs[i])
            if ev: ev[i][1].record(stream)

    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(nseg)]
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        one_pass(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_pass = wall * 1e3 / args.steps
    seg = [{"offset": i * S, "kv_len": (i + 1) * S,
            "ms": round(sum(e[i][0].elapsed_time(e[i][1]) for e in evs) / args.steps, 4)}
           for i in range(nseg)]
    # key/value rows each segment reads (one untimed pass): the forward and the
    # dQ pass each gather every row's kept groups and own chunk; summaries and
    # dK/dV read the segment's own keys (and values)
    row_bytes = w.head_dim * 2
    for i in range(nseg):
        run.forward(i, Qs[i], stream=stream, K_seg=Ks[i], V_seg=Vs[i])
        kept = int((run.group_idx >= 0).sum().item())
        rows = w.batch * w.n_q_heads * (S // 64)
        gather = (kept * 8 + rows * 64) * row_bytes * 2
        own = w.batch * w.n_kv_heads * S * row_bytes
        if args.stage:
            # staged: the distinct kept history groups and the segment's rows
            # (K and V); a group the previous segment's staging held is copied
            # from there in device memory, the rest from the history, which
            # the summaries read too (the segment's keys)
            import torch as _t
            sg = run.stage_groups[i]
            nbh = w.batch * w.n_kv_heads
            lb = -(-(nbh * sg * 4) // 256) * 256
            ws = run.stage_wss[i % 2]
            cnt = ws[lb:lb + 4 * nbh].view(_t.int32).cpu()
            src = ws[lb + (-(-(4 * nbh) // 256) * 256):][:4 * nbh * sg].view(_t.int32).cpu()
            src = src.view(nbh, sg)
            union = int(cnt.sum().item())
            from_hist = sum(int((src[k, :int(cnt[k])] < 0).sum().item()) for k in range(nbh))
            seg[i]["union_groups"] = union
            seg[i]["union_groups_from_history"] = from_hist
            seg[i]["staged_bytes_from_history"] = \
                (from_hist * 8 * row_bytes + (0 if args.seg_on_device else own)) * 2 + own
            seg[i]["history_GBs"] = round(seg[i]["staged_bytes_from_history"]
                                          / (seg[i]["ms"] * 1e-3) / 1e9, 1)
        seg[i]["kv_bytes_read"] = 2 * gather + own + 2 * own
        seg[i]["kv_GBs"] = round(seg[i]["kv_bytes_read"] / (seg[i]["ms"] * 1e-3) / 1e9, 1)
    out = {
        "metric": "HGA segment-wise fwd+bwd query tokens/sec, 16K sequence as 8 x 2048 segments "
                  "(history detached" + (", K/V in pinned host memory" if args.host_kv else "")
                  + (", routed working set staged in HBM per segment" if args.stage else "")
                  + (", active segment in HBM" if args.seg_on_device else "")
                  + "), 1 MI355X",
        "value": w.batch * L / (ms_pass * 1e-3),
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_pass,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded clustered keys, N(0,1)/sqrt(128) queries and values)",
        "config": {"workload": "sequence_16k as 8 segments of 2048, fwd+bwd per segment",
                   "batch": 1, "q_heads": 32, "kv_heads": 8, "head_dim": 128, "seq_len": L,
                   "segment": S, "top_k": 16, "top_g": 64},
        "segments": seg,
    }
    print(json.dumps(out))


def graph_of(fn, copies: int = 1):
    """`fn` (which launches on the current stream) captured `copies` times into
    one HIP graph (torch.cuda.CUDAGraph).  The kernels allocate nothing and
    clear nothing with memset, so a replay repeats the eager work exactly."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(copies):
            fn()
    torch.cuda.synchronize()
    return g


def timed_replays(g, steps: int, warmup: int) -> float:
    """Milliseconds per replay of `g` over `steps` replays (after `warmup`),
    bracketed by device synchronisations."""
    import torch
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def kernel_us(fn, launches: int = 20, reps: int = 5) -> float:
    """Average duration of one launch of `fn`: `launches` back-to-back copies in
    one graph (no host launch gaps), HIP events around each replay on the
    replay stream, averaged over `reps` replays."""
    import torch
    g = graph_of(fn, launches)
    g.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    tot = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        g.replay()
        e1.record(st)
        torch.cuda.synchronize()
        tot += e0.elapsed_time(e1)
    return tot * 1e3 / (reps * launches)


def calibration_copy(dev):
    """One plain 256 MiB device-to-device copy (a known read and write volume
    for scaling the memory counters)."""
    import torch
    src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def replay_percentiles(g, steps: int) -> dict:
    """Per-step time distribution of `steps` further replays of `g`, each
    bracketed by HIP events on the replay stream (after the timed region, so
    the events do not touch it): p10, median, p90 in ms."""
    import torch
    st = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record(st)
        g.replay()
        b.record(st)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    q = lambda f: t[min(len(t) - 1, int(f * (len(t) - 1) + 0.5))]
    return {"p10": round(q(0.1), 4), "p50": round(q(0.5), 4), "p90": round(q(0.9), 4)}


def device_measured(dev) -> dict:
    """What this GPU reports and sustains, beside the published peaks the
    rooflines use: device properties, the rate of a plain 1 GiB device copy
    (read plus write bytes over time), and the rate of a large dense bf16
    matrix product through the vendor library (torch.matmul, 8192^3)."""
    import torch
    p = torch.cuda.get_device_properties(dev)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", ""),
            "compute_units": p.multi_processor_count,
            "memory_GB": round(p.total_memory / 1e9, 1),
            "l2_MB": round(getattr(p, "L2_cache_size", 0) / 2 ** 20, 1)}
    st = torch.cuda.current_stream()

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        for _ in range(reps):
            fn()
        b.record(st)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / reps

    src = torch.empty(2 ** 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    sec = timed(lambda: dst.copy_(src), 10)
    info["copy_GBs"] = round(2 * 2 ** 30 / sec / 1e9, 1)
    del src, dst
    n = 8192
    x = torch.randn(n, n, device=dev).to(torch.bfloat16)
    y = torch.randn(n, n, device=dev).to(torch.bfloat16)
    sec = timed(lambda: torch.matmul(x, y), 10)
    info["bf16_gemm_TFLOPs"] = round(2 * n ** 3 / sec / 1e12, 1)
    del x, y
    torch.cuda.empty_cache()
    return info


def decode_work(w, kept_groups: int) -> dict:
    """Per-launch algorithmic bytes of the two decode kernels.  Routing: the
    queries, the chunk summaries before the own chunk (read once for the query
    heads of a kv head), the group summaries of every row's kept chunks, the
    indices written.  Attention: per row the query, its group indices, the key
    and value rows of its kept groups and of its own chunk up to the token, the
    output row and lse."""
    B, Hq, Hkv, D, L = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.kv_len
    p = L - 1
    cp = p // 64
    kk = min(w.top_k, cp)
    rows = B * Hq
    route = rows * D * 2 + B * Hkv * cp * D * 4 + rows * kk * 8 * D * 4 + rows * (w.top_k + w.top_g) * 4
    own = p - 64 * cp + 1
    attend = rows * (D * 2 + D * 2 + 4) + kept_groups * 4 + (kept_groups * 8 + rows * own) * D * 2 * 2
    return {"decode_route": route, "decode_attend": attend}


def cpu_baseline_decode(w, x, cm, gm, causal=False, budget_s: float = 12.0):
    """The CPU oracle on the same decode work, single thread, one sequence at
    a time, cycling over four of the batch's sequences until `budget_s`
    seconds of work are done.  Block routing: one token's decode (routing over
    the resident summaries and attention, fp64).  Strictly causal routing: one
    block of 64 tokens (the block's routing once, then the attention of its
    64 tokens, which equals the forward over the block)."""
    import oracle
    from hierarchical_routed_sparse_amd import synthetic as syn
    oracle.build(force=False)
    seqs = []
    for b in range(min(4, w.batch)):
        f = {k: syn.to_f64(v[b:b + 1], w.dtype) for k, v in x.items()}
        seqs.append((f, cm[b:b + 1], gm[b:b + 1]))
    done, toks, dt = 0, 0, 0.0
    while dt < budget_s:
        f, c, g = seqs[done % len(seqs)]
        t0 = time.perf_counter()
        if causal:
            _, gi = oracle.route(f["Q"], c, g, f["K"].shape[2], w.top_k, w.top_g, causal=True,
                                 Qprev=f["Qprev"])
            oracle.attend_fwd(f["Q"], f["K"], f["V"], gi)
            toks += f["Q"].shape[2]
        else:
            oracle.decode(f["Q"][:, :, 0], f["K"], f["V"], c, g, w.top_k, w.top_g)
            toks += 1
        dt += time.perf_counter() - t0
        done += 1
    what = ("blocks of 64 tokens (routing once, attention of every token)" if causal
            else "single-token decode steps (routing over the resident summaries and attention)")
    return {
        "value": toks / dt,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{done} single-sequence {what}, all {w.n_q_heads} query heads, fp64, "
                   f"cycling over {len(seqs)} of the {w.batch} sequences, {dt:.1f} s "
                   f"single-threaded"),
    }


def decode_main(args):
    """Decode of one layer: 64 consecutive new tokens (positions 16384-16447,
    one block) for each of 16 sequences over a cache of capacity 16448; the
    summaries of the 256 complete chunks before the block are resident (a
    decoder appends one chunk's summary every 64 tokens).  Block routing: each
    token is routed with its own query, then attended (2 kernels per token).
    With --causal (strictly causal routing): the block is routed once from the
    previous block's 64 queries, then each token is attended (1 kernel per
    token).  The 64 steps are captured as one graph; a step is one token per
    sequence.  The roofline kernel is the attention at position 16423."""
    import numpy as np
    import torch
    import hierarchical_routed_sparse_amd as hga
    from hierarchical_routed_sparse_amd import synthetic as syn

    w = syn.WORKLOADS["decode_b16_16k"]            # kv_len 16424: the roofline position
    T, j = 64, 256                                  # tokens 64j .. 64j + 63
    cap = 64 * (j + 1)
    wi = syn.scaled_workload(w, q_len=T, kv_len=cap)
    x = syn.make_inputs(wi, with_qprev=args.causal)  # Q: the 64 tokens' queries
    dev = "cuda:0"
    torch.cuda.set_device(0)
    B, Hq, Hkv, D = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    shapes = [hga.make_shape(B, Hq, Hkv, D, 1, 64 * j + t + 1, w.top_k, w.top_g,
                             dtype=w.dtype, kv_capacity=cap) for t in range(T)]
    edt = torch.bfloat16
    K = syn.to_torch(x["K"], w.dtype, dev)
    V = syn.to_torch(x["V"], w.dtype, dev)
    Qt = syn.to_torch(x["Q"], w.dtype, dev)
    Qs = [Qt[:, :, t].contiguous() for t in range(T)]
    Qprev = syn.to_torch(x["Qprev"], w.dtype, dev) if args.causal else None
    cm = torch.zeros(B, Hkv, cap // 64, D, device=dev)
    gm = torch.zeros(B, Hkv, cap // 8, D, device=dev)
    hga.hga_build_summaries(shapes[0], K, cm, gm, 0, j)
    if args.host_kv:
        torch.cuda.synchronize()
        Kh = torch.empty(K.shape, dtype=edt, pin_memory=True)
        Vh = torch.empty(V.shape, dtype=edt, pin_memory=True)
        Kh.copy_(K)
        Vh.copy_(V)
        K, V = Kh, Vh
    ci = torch.empty(B, Hq, w.top_k, dtype=torch.int32, device=dev)
    gi = torch.empty(B, Hq, w.top_g, dtype=torch.int32, device=dev)
    O = torch.empty(B, Hq, D, dtype=edt, device=dev)
    lse = torch.empty(B, Hq, device=dev)
    # host-resident K/V: pass their GPU addresses (resolved once, outside any capture)
    Ka, Va = (hga._ptr(K, "K", host_ok=True), hga._ptr(V, "V", host_ok=True)) if args.host_kv \
        else (K, V)

    def route(t):
        if args.causal:
            hga.hga_decode_route_causal(shapes[0], Qprev, cm, gm, ci, gi)
        else:
            hga.hga_decode_route(shapes[t], Qs[t], cm, gm, ci, gi)

    def attend(t):
        hga.hga_decode_attend(shapes[t], Qs[t], Ka, Va, gi, O, lse)

    def block(acc=None):
        # acc: [route_ms, attend_ms] accumulated from HIP events (eager pass)
        stream = torch.cuda.current_stream()
        for t in range(T):
            if acc is not None:
                e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                e[0].record(stream)
            if t == 0 or not args.causal:
                route(t)
            if acc is not None:
                e[1].record(stream)
            attend(t)
            if acc is not None:
                e[2].record(stream)
                acc.append(e)

    for _ in range(args.warmup):
        block()
    torch.cuda.synchronize()
    if args.calibrate_copy:
        calibration_copy(dev)
    nblocks = max(1, -(-args.steps // T))   # whole blocks of 64 steps
    evs = []
    t0 = time.perf_counter()
    for _ in range(nblocks):
        block(evs)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / (nblocks * T)
    route_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / (nblocks * T)
    attend_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / (nblocks * T)
    # the block of 64 steps captured into a HIP graph before the kernel
    # timings, and timed right after them (the GPU at its working clocks, as
    # in the headline step)
    g_block = graph_of(block)

    # roofline kernel: the attention at position 16423 (token 39 of the block)
    tr = 39
    route(tr)
    torch.cuda.synchronize()
    kept = int((gi >= 0).sum().item())
    work = decode_work(w, kept)
    rep = {}
    for p, fn in (("decode_route", lambda: route(tr)), ("decode_attend", lambda: attend(tr))):
        us = kernel_us(fn)
        ach = work[p] / (us * 1e-6) / 1e9
        rep[p] = {"kernel_us": round(us, 2), "bound": "hbm",
                  "algorithmic_bytes": work[p], "achieved_GBs": round(ach, 1),
                  "frac": round(ach / PEAK_HBM_GBS, 4)}
    # the timed region: `nblocks` replays of the block (64 steps each)
    ms_step = timed_replays(g_block, nblocks, 1) / T
    rep["decode_route"]["us_per_token_in_step"] = round(route_ms * 1e3, 2)
    rep["decode_attend"]["us_per_token_in_step"] = round(attend_ms * 1e3, 2)
    dom = "decode_attend"
    us = rep[dom]["kernel_us"]
    ach = work[dom] / (us * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": ach / PEAK_HBM_GBS, "traffic": None if args.host_kv else load_traffic(dom, w.name),
            "kernel": dom, "kernel_us": us, "algorithmic_per_launch": work[dom]}
    base = None
    if not args.no_cpu_baseline:
        cmh = cm.cpu().numpy().astype(np.float64)
        gmh = gm.cpu().numpy().astype(np.float64)
        if args.causal:
            base = cpu_baseline_decode(wi, x, cmh, gmh, causal=True)
        else:
            xd = {"Q": x["Q"][:, :, tr:tr + 1], "K": x["K"][:, :, :w.kv_len],
                  "V": x["V"][:, :, :w.kv_len]}
            base = cpu_baseline_decode(w, xd, cmh[:, :, :w.kv_len // 64],
                                       gmh[:, :, :8 * (w.kv_len // 64)])
    form = "strictly causal routing, routed once per 64-token block" if args.causal \
        else "each token routed with its own query"
    out = {
        "metric": "HGA decode tokens/sec at 16K ctx (batch 16, " + form
                  + (", K/V in pinned host memory" if args.host_kv else "") + "), 1 MI355X",
        "value": B / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": nblocks * T,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "eager_ms_per_step": eager_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded clustered keys, N(0,1)/sqrt(128) queries and values)",
        "config": {"workload": f"{w.name}: 64 decode steps per sequence at positions "
                               f"{64 * j}-{64 * j + T - 1}, cache capacity {cap}, {form}",
                   "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
                   "chunk": 64, "group": 8, "top_k": w.top_k, "top_g": w.top_g,
                   "kept_groups_at_16423": kept},
        "roofline": roof,
        "phases": rep,
        "cpu_baseline": base,
    }
    print(json.dumps(out))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(the layer shards by kv head with no exchange between the shards).",
              file=sys.stderr)
        sys.exit(2)

    if args.segments:
        segments_main(args)
        return
    if args.decode:
        decode_main(args)
        return

    import numpy as np
    import torch
    import hierarchical_routed_sparse_amd as hga
    from hierarchical_routed_sparse_amd import synthetic as syn

    w = syn.WORKLOADS[args.workload]
    fwd_only = args.fwd_only
    x = syn.make_inputs(w, with_grad_output=not fwd_only, with_qprev=args.causal)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    t = {k: syn.to_torch(v, w.dtype, dev) for k, v in x.items()}
    s = hga.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.q_len, w.kv_len,
                       w.top_k, w.top_g, dtype=w.dtype)
    sz = hga._sizes(s)
    f32, i32 = torch.float32, torch.int32
    edt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    cm = torch.empty(sz["cm"], dtype=f32, device=dev)
    gm = torch.empty(sz["gm"], dtype=f32, device=dev)
    ci = torch.empty(sz["ci"], dtype=i32, device=dev)
    gi = torch.empty(sz["gi"], dtype=i32, device=dev)
    O = torch.empty(sz["q"], dtype=edt, device=dev)
    lse = torch.empty(sz["lse"], dtype=f32, device=dev)
    phases = ["summaries", "route", "attend_fwd"]
    calls = {
        "summaries": lambda: hga.hga_build_summaries(s, t["K"], cm, gm),
        "route": (lambda: hga.hga_route_causal(s, t["Q"], t["Qprev"], cm, gm, ci, gi))
        if args.causal else (lambda: hga.hga_route(s, t["Q"], cm, gm, ci, gi)),
        "attend_fwd": lambda: hga.hga_attend_fwd(s, t["Q"], t["K"], t["V"], gi, O, lse),
    }
    if not fwd_only:
        dQ = torch.empty(sz["q"], dtype=edt, device=dev)
        dK = torch.empty(sz["kv"], dtype=edt, device=dev)
        dV = torch.empty(sz["kv"], dtype=edt, device=dev)
        ws = torch.empty(hga.hga_attend_bwd_workspace(s), dtype=torch.uint8, device=dev)
        phases += ["attend_bwd_dq", "attend_bwd_dkdv"]
        calls["attend_bwd_dq"] = lambda: hga.hga_attend_bwd_dq(
            s, t["Q"], t["K"], t["V"], O, lse, t["dO"], gi, dQ, ws)
        calls["attend_bwd_dkdv"] = lambda: hga.hga_attend_bwd_dkdv(
            s, t["Q"], t["K"], t["V"], lse, t["dO"], gi, dK, dV, ws)

    def step(ev=None):
        # every call launches on the current stream (the capture stream inside
        # a graph capture); the backward in sequence: dQ (writing the dK/dV
        # metadata into the workspace), then dK/dV
        stream = torch.cuda.current_stream()
        for i, p in enumerate(phases):
            if ev: ev[i].record(stream)
            calls[p]()
        if ev: ev[len(phases)].record(stream)

    side = torch.cuda.Stream()

    def step_side_by_side():
        # the backward's metadata from its preparation pass, then dQ on a
        # second stream beside dK/dV on the first (forked and joined by events,
        # which a graph capture records as its dependencies)
        main = torch.cuda.current_stream()
        for p in phases[:3]:
            calls[p]()
        hga.hga_attend_bwd_prep(s, O, t["dO"], gi, ws)
        side.wait_stream(main)
        with torch.cuda.stream(side):
            hga.hga_attend_bwd_dq(s, t["Q"], t["K"], t["V"], O, lse, t["dO"], gi, dQ, None)
        calls["attend_bwd_dkdv"]()
        main.wait_stream(side)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.calibrate_copy:
        calibration_copy(dev)

    # eager pass: per-phase HIP events (each phase includes its launch gap)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    phase_ms = {p: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / args.steps
                for i, p in enumerate(phases)}
    # the step captured into a HIP graph (with --side-by-side-bwd also the form
    # with dQ beside dK/dV after the preparation pass).  The captures come
    # before the kernel timings below, and the timed replays right after them:
    # a capture is host work during which the GPU idles and its clocks drop,
    # while the timings keep it busy, so the timed steps run at the GPU's
    # working clocks, as they do inside a training loop.
    g_serial = graph_of(step)
    g_side = None
    if not fwd_only and args.side_by_side_bwd:
        for _ in range(args.warmup):
            step_side_by_side()
        torch.cuda.synchronize()
        g_side = graph_of(step_side_by_side)
    pairs = attended_pairs(gi)
    work = algorithmic_work(w, pairs)
    executed = executed_work(gi.cpu().numpy(), w.head_dim)
    phase_rep = {}
    for p in phases:
        kind, amount = work[p]
        sec = phase_ms[p] * 1e-3
        if kind == "hbm":
            ach = amount / sec / 1e9
            phase_rep[p] = {"us": round(phase_ms[p] * 1e3, 2), "bound": "hbm",
                            "algorithmic_bytes": amount,
                            "achieved_GBs": round(ach, 1), "frac": round(ach / PEAK_HBM_GBS, 4)}
        else:
            ach = amount / sec / 1e12
            phase_rep[p] = {"us": round(phase_ms[p] * 1e3, 2), "bound": "mfma",
                            "algorithmic_flop": amount,
                            "achieved_TFLOPs": round(ach, 1),
                            "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                            "executed_flop": executed[p],
                            "executed_TFLOPs": round(executed[p] / sec / 1e12, 1)}
    # kernel-only durations of every phase (back-to-back launches in a graph)
    for p in phases:
        phase_rep[p]["kernel_us"] = round(kernel_us(calls[p]), 2)
    if not fwd_only:
        phase_rep["attend_bwd_prep"] = {"kernel_us": round(kernel_us(
            lambda: hga.hga_attend_bwd_prep(s, O, t["dO"], gi, ws)), 2),
            "note": "delta, group-mask map and dK/dV work order for the side-by-side "
                    "backward (the serial backward has dQ write them)"}
    # the timed region: `steps` replays of the step's graph (after `warmup`)
    ms_serial = timed_replays(g_serial, args.steps, args.warmup)
    ms_step = ms_serial
    if g_side is not None:
        ms_step = timed_replays(g_side, args.steps, args.warmup)
    step_pct = replay_percentiles(g_side if g_side is not None else g_serial, args.steps)

    dom = max(phases, key=lambda p: phase_rep[p]["kernel_us"])
    kind, amount = work[dom]
    dom_us = phase_rep[dom]["kernel_us"]
    sec = dom_us * 1e-6
    if kind == "hbm":
        roof = {"bound": "hbm", "achieved": amount / sec / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": amount / sec / 1e12, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = load_traffic(dom, w.name)
    roof["kernel"] = dom
    roof["launches"] = " + ".join(KERNEL_NAMES[k] for k in PHASE_KERNELS.get(dom, [dom]))
    roof["kernel_us"] = dom_us
    roof["algorithmic_per_launch"] = amount
    if kind == "mfma":
        roof["executed_per_launch"] = executed[dom]
        roof["executed_TFLOPs"] = executed[dom] / sec / 1e12
    # routing against HBM peak: summaries + route on their kernel times
    rb = work["summaries"][1] + work["route"][1]
    rt = phase_rep["summaries"]["kernel_us"] + phase_rep["route"]["kernel_us"]
    phase_rep["routing_total"] = {"kernel_us": round(rt, 2), "algorithmic_bytes": rb,
                                  "achieved_GBs": round(rb / (rt * 1e-6) / 1e9, 1),
                                  "frac": round(rb / (rt * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    # the gather: the K/V rows the forward and dQ kernels move into LDS (every
    # kept group and the own chunk, per routing row) and the Q/dO rows the
    # dK/dV kernel moves (per (routing row, chunk) it attends), over each
    # kernel's whole time with its products: a lower bound on the rate the
    # gather itself sustains.  Logical bytes count a row each time it is
    # gathered; most are served from the GPU's caches, so the logical rate may
    # exceed the HBM peak.  The HBM bytes the kernels move are the counter
    # figures (`traffic`).
    kept = int((gi >= 0).sum().item())
    nrows = gi.shape[0] * gi.shape[1] * gi.shape[2]
    esz = 2 if w.dtype == "bf16" else 4
    gnp = gi.cpu().numpy()
    kv_logical = (kept * 8 + nrows * 64) * w.head_dim * esz * 2
    unique = 0
    r = w.n_q_heads // w.n_kv_heads
    own = (w.kv_len - w.q_len) // 8 + np.arange(8 * (w.q_len // 64))
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            sel = gnp[b, h * r:(h + 1) * r]
            unique += len(np.union1d(np.unique(sel[sel >= 0]), own)) * 8
    unique *= w.head_dim * esz * 2
    gather = {"kv_rows_logical_bytes": kv_logical, "kv_rows_unique_bytes": unique}
    kernels = ["attend_fwd"] + ([] if fwd_only else ["attend_bwd_dq", "attend_bwd_dkdv"])
    for k in kernels:
        if k == "attend_bwd_dkdv":
            entries = 0
            for row in gnp.reshape(-1, gnp.shape[-1]):
                v = row[row >= 0]
                entries += len(np.unique(v >> 3)) + 1
            logical = entries * 64 * (2 * w.head_dim * esz + 8)
        else:
            logical = kv_logical
        us = phase_rep[k]["kernel_us"]
        ach = logical / (us * 1e-6) / 1e9
        gather[k] = {"logical_bytes": logical, "kernel_us": us, "achieved_GBs": round(ach, 1),
                     "frac_of_hbm_peak": round(ach / PEAK_HBM_GBS, 4),
                     "hbm_traffic": load_traffic(k, w.name)}
    phase_rep["gather"] = gather

    base = None
    if not args.no_cpu_baseline:
        base = cpu_baseline(w, x, causal=args.causal, fwd_only=fwd_only)

    what = "fwd" if fwd_only else "fwd+bwd"
    metric = METRIC if (w.name == "segment_2k_over_16k" and not fwd_only) else \
        f"HGA {what} query tokens/sec, {w.name}, 1 MI355X; % HBM / % MFMA peak"
    out = {
        "metric": metric + (" (strictly causal routing)" if args.causal else ""),
        "value": w.batch * w.q_len / (ms_step * 1e-3),
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "one_stream_ms_per_step": ms_serial,
        "eager_ms_per_step": eager_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded clustered keys, N(0,1)/sqrt(128) queries and values)",
        "config": {
            "backward_schedule": None if fwd_only else (
                "prep, then dQ on a second stream beside dK/dV" if args.side_by_side_bwd
                else "dQ, then dK/dV on one stream"),
            "workload": f"{w.name} {what}" + (", strictly causal routing" if args.causal else ""),
            "batch": w.batch, "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads,
            "head_dim": w.head_dim, "q_len": w.q_len, "kv_len": w.kv_len,
            "chunk": 64, "group": 8, "top_k": w.top_k, "top_g": w.top_g,
            "attended_pairs": pairs,
        },
        "roofline": roof,
        "phases": phase_rep,
        "step_ms_percentiles": step_pct,
        # (not in the counter runs, whose calibration copy must be the only large one)
        "device": None if args.calibrate_copy else device_measured(dev),
        "cpu_baseline": base,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
