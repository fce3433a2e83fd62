#!/usr/bin/env python3
"""Throughput of the fused equivariant convolution on one MI355X.

One step = the whole hot path over one batch of the workload: the fused
spherical harmonics -> Clebsch-Gordan product -> destination sum
(eqtp_conv_fused), then the per-l channel linear (eqtp_linear).  The default
workload is "mid": 10,000 atoms in a periodic box at 0.1 atoms/A^3, radius
cut-off 4 A (266,116 directed edges), lmax 3, C = 64, parity path set (23
paths, 353 coefficients), bf16-operand 64x64 linear.  Inputs are synthetic
(seeded) and resident in device memory before timing starts.

Prints one JSON line (see the "metric" field); diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 (matrix and packed vector)
METRIC = "edges/sec fused SH+CG-TP+aggregate (10k atoms, C=64, L=3); % of roofline"

GRAPH_STEPS = 20  # at most this many steps captured per HIP graph with --graph

WORKLOAD_TEXT = {
    "tiny": "tiny: 64 atoms, 6 A cube (open boundaries), r_c=3 A, both directions, L=2, C=8, conv",
    "typical": "typical: 1000 atoms, periodic 0.1/A^3, k=20 nearest, L=3, C=32, conv + fp32 32x32 per-l linear",
    "mid": "mid: 10k atoms, periodic 0.1/A^3, r_c=4 A, L=3, C=64, conv + bf16 64x64 per-l linear",
    "large": "large: 100k atoms, periodic 0.1/A^3, r_c=5 A, L=3, C=32, conv (dst-sorted)",
    "radial": "radial: 50k atoms, periodic 0.1/A^3, r_c=5 A, L=3, C=128, radial-weighted conv",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def count_terms(lmax, path_set):
    """Non-zero coupling coefficients (2*nnz*C flops per edge) from the library's tables."""
    import re

    gen = os.path.join(ROOT, "spherical_harmonic_cg_amd", "csrc", "generated")
    tag = "L%d_%s" % (lmax, "parity" if path_set == 0 else "so3")
    m = re.search(r"constexpr int kNumTerms_%s = (\d+);" % tag, open(os.path.join(gen, "cg_tables.inc")).read())
    if m:
        return int(m.group(1))
    m = re.search(r"lmax = %d, %s path set: \d+ paths, \d+ edge-aligned terms \(full coupling: (\d+)\)" % (
        lmax, "parity" if path_set == 0 else "so3"), open(os.path.join(gen, "so2_tables.inc")).read())
    return int(m.group(1))


def so2_ops(lmax, path_set):
    """Arithmetic instructions per edge and channel of the edge-aligned kernel,
    from its tables: two frame rotations (4 per (m cos, m sin) pair for each of
    the two pair rotations, one per non-zero of J and of J^T) and the sparse
    coupling (one per term plus one per (path, output) run)."""
    import re

    txt = open(os.path.join(ROOT, "spherical_harmonic_cg_amd", "csrc", "generated", "so2_tables.inc")).read()
    K = (lmax + 1) ** 2
    starts = [int(v) for v in re.search(r"kJRowStart\[\d+\] = \{([^}]*)\}", txt).group(1).split(",")]
    nnz_j = starts[K]
    pairs = lmax * (lmax + 1) // 2
    tag = "L%d_%s" % (lmax, "parity" if path_set == 0 else "so3")
    body = re.search(r"kSo2Terms_%s\[\d+\] = \{(.*?)\n\};" % tag, txt, re.S).group(1)
    terms = [tuple(int(v) for v in ln.strip().strip("{").split(",")[:3]) for ln in body.strip().splitlines()]
    runs = len({(p, mu3) for (p, _, mu3) in terms})
    return 2 * (2 * 4 * pairs + 2 * nnz_j) + len(terms) + runs


KERNEL_SOURCES = ("spherical_harmonic_cg_amd/csrc/conv_node.hip", "spherical_harmonic_cg_amd/csrc/eqtp_device.hpp",
                  "spherical_harmonic_cg_amd/csrc/generated/cg_tables.inc")


def kernel_source_hash(sources=KERNEL_SOURCES):
    import hashlib

    h = hashlib.sha256()
    for rel in sources:
        h.update(open(os.path.join(ROOT, rel), "rb").read())
    return h.hexdigest()[:16]


def graph_steps(K):
    """Steps captured per HIP graph with --graph: the largest divisor of K up to
    GRAPH_STEPS, so that whole replays run exactly K steps."""
    return max(d for d in range(1, min(GRAPH_STEPS, K) + 1) if K % d == 0)


def measured_traffic(config, atom_order, unsorted, algo, path_set="parity", x_bf16=False, sort_edges=False):
    """HBM-side bytes per launch of the conv kernel from the committed counter
    summary (profiles/traffic.json), or None when that summary was taken on
    different kernel sources or another workload."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except ValueError:
        return None
    order = ("unsorted+gpusort" if sort_edges else "unsorted") if unsorted else "sorted"
    key = "%s/%s/%s/%d" % (config, atom_order, order, algo)
    if path_set != "parity":
        key += "/" + path_set
    if x_bf16:
        key += "/xbf16"
    ent = rec.get(key)
    # each entry names the sources of the kernel it was taken on (default: the node kernel's)
    if not ent or ent.get("source_sha256_16") != kernel_source_hash(tuple(ent.get("sources", KERNEL_SOURCES))):
        return None
    return ent["read_bytes"] + ent["write_bytes"]


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline(wl, budget_s):
    """The fp64 oracle on the same workload, on the host.

    The oracle shares the destination rows out over its OpenMP threads (OMP_NUM_THREADS, else every
    core of the process); the result does not depend on the thread count.  Bounded sample: a first run
    over 200 destination rows sizes the sample so that one timed run takes about ``budget_s`` seconds
    (the whole workload if it fits); the all-thread figure is the median of three runs (one if a run
    exceeds 30 s).  A one-thread run over a sample of the same rows is reported beside it."""
    import oracle

    def run(rows):
        e = int(wl.row_ptr[rows])
        t = time.perf_counter()
        h = oracle.conv(wl.N, wl.vec[:e], wl.src[:e], wl.dst[:e], wl.x, wl.weights, wl.lmax,
                        path_set=wl.path_set, weight_mode=wl.weight_mode, r_cut=wl.r_cut)
        if wl.w_lin is not None:
            oracle.linear(h[:rows].astype(np.float32), wl.w_lin, wl.lmax, bf16=wl.linear_bf16)
        return time.perf_counter() - t, e

    def sized(budget, threads):
        oracle.set_threads(threads)
        probe_rows = min(wl.N, 200)
        dt, e = run(probe_rows)
        per_edge = dt / max(e, 1)
        rows = wl.N
        if per_edge * wl.E > budget:
            rows = int(np.searchsorted(wl.row_ptr, budget / per_edge))
            rows = max(probe_rows, min(rows, wl.N))
        return rows

    rows = sized(budget_s, 0)
    threads = oracle.num_threads()
    runs = []
    for _ in range(3):
        runs.append(run(rows))
        if runs[-1][0] > 30.0:
            break
    dt = float(np.median([r[0] for r in runs]))
    e = runs[0][1]
    rows1 = sized(budget_s / 3.0, 1)
    dt1, e1 = run(rows1)
    oracle.set_threads(0)
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 0
    what = "conv%s" % (" + per-l linear" if wl.w_lin is not None else "")
    return {"value": round(e / dt, 1), "unit": "edges/s", "cores": threads, "kind": "oracle",
            "sample": "fp64 oracle, %d threads (%d cores in the process affinity, %s), on the first %d of %d "
                      "destination rows (%d of %d edges) of the same workload: %s, median of %d runs, %.2f s"
                      % (threads, affinity, _cpu_model(), rows, wl.N, e, wl.E, what, len(runs), dt),
            "single_thread": {"value": round(e1 / dt1, 1), "unit": "edges/s", "cores": 1,
                              "sample": "first %d destination rows (%d edges), %.2f s" % (rows1, e1, dt1)}}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="mid", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--algo", type=int, default=0, help="0 auto, 1 node/matrix cores, 2 edge/vector ALUs")
    ap.add_argument("--unsorted", action="store_true", help="random edge order (atomic path)")
    ap.add_argument("--sort-edges", action="store_true",
                    help="with --unsorted: each step groups the edges by destination on the GPU "
                         "(eqtp_sort_edges) and runs the dst-sorted conv on them, instead of the atomic path")
    ap.add_argument("--ws", action="store_true",
                    help="with --unsorted: eqtp_conv_fused_ws, which groups the edges by destination in a "
                         "workspace (rows in input order) and runs the dst-sorted kernels, inside each step")
    ap.add_argument("--atom-order", default="generation", choices=("generation", "cell"),
                    help="'cell': spatially coherent atom numbering (a labelled extra, not the headline)")
    ap.add_argument("--path-set", default="parity", choices=("parity", "so3"),
                    help="'so3': the 34-path SO(3) set (a labelled extra, not the headline)")
    ap.add_argument("--out-bf16", action="store_true",
                    help="with --unsorted: bfloat16 conv output summed with packed bf16 atomics; the linear then "
                         "reads it in bf16 storage")
    ap.add_argument("--x-bf16", action="store_true",
                    help="bfloat16 node features (a labelled extra: halves the gathered bytes)")
    ap.add_argument("--lmax", type=int, default=None,
                    help="instead of --config: the mid graph (10k atoms, r_c=4 A, C=64) with features of degree "
                         "up to LMAX (4..6 run the edge-aligned kernel; a labelled extra, not the headline)")
    ap.add_argument("--graph", action="store_true",
                    help="time the step as one captured HIP graph replayed K times (sorted edges, no GPU sort)")
    ap.add_argument("--prewarm-s", type=float, default=0.3,
                    help="seconds of untimed steps before the warmup steps (device clock ramp)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--backward", action="store_true",
                    help="also time eqtp_conv_backward (all three gradients) on the same inputs (an extra field)")
    ap.add_argument("--messages", action="store_true",
                    help="also time eqtp_conv_messages (per-edge [E,C,K] output, the page's kernel) (an extra field)")
    ap.add_argument("--interaction", action="store_true",
                    help="also time eqtp_interaction (channel linear, radial network, convolution with the "
                         "network's path weights, channel linear) on the same graph and features (an extra field)")
    ap.add_argument("--sh", action="store_true",
                    help="also time eqtp_sh (standalone harmonics [E,K] of the workload's edges) (an extra field)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after timing, run one 256 MiB device copy (counter calibration)")
    args = ap.parse_args()

    if args.sort_edges and not args.unsorted:
        ap.error("--sort-edges needs --unsorted")
    if args.ws and (not args.unsorted or args.sort_edges):
        ap.error("--ws needs --unsorted (and replaces --sort-edges)")
    if args.out_bf16 and (not args.unsorted or args.sort_edges or args.ws):
        ap.error("--out-bf16 needs --unsorted (atomics into the output; not with --sort-edges or --ws)")
    if args.graph and args.unsorted:
        ap.error("--graph times dst-sorted edges only")
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path (a split into CSR "
              "row ranges with a halo exchange of source features is not built); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import spherical_harmonic_cg_amd as eq
    from spherical_harmonic_cg_amd import synth

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    eq.load_library()
    torch.cuda.set_device(0)

    t_gen = time.perf_counter()
    if args.lmax is not None:
        wl = synth.lmax_graph(args.lmax, 64, seed=2026, n=10000, path_set=1 if args.path_set == "so3" else 0)
    else:
        wl = synth.make_config(args.config, atom_order=args.atom_order,
                               path_set=1 if args.path_set == "so3" else 0)
    log("workload %s: N=%d E=%d C=%d lmax=%d P=%d (generated in %.1fs)" % (wl.name, wl.N, wl.E, wl.C, wl.lmax,
                                                                            wl.P, time.perf_counter() - t_gen))
    dev = torch.device("cuda:0")
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    if args.unsorted:
        pvec, psrc, pdst = synth.random_permutation(wl)
        vec, src, dst, row_ptr = T(pvec), T(psrc), T(pdst), None
    else:
        vec, src, dst, row_ptr = T(wl.vec), T(wl.src), None, T(wl.row_ptr)
    x = T(wl.x)
    if args.x_bf16:
        x = x.to(torch.bfloat16)
    w = T(wl.weights)
    out = torch.empty(x.shape, dtype=torch.bfloat16 if args.out_bf16 else torch.float32, device=dev)
    w_lin = T(wl.w_lin) if wl.w_lin is not None else None
    out2 = torch.empty(x.shape, dtype=torch.float32, device=dev) if w_lin is not None else None
    lin_dtype = eq.EQTP_BF16 if (wl.linear_bf16 or args.out_bf16) else eq.EQTP_F32
    if args.out_bf16 and w_lin is not None:
        w_lin = w_lin.to(torch.bfloat16)  # bf16 h needs bf16 W (bf16 storage for both)
    out_dtype = eq.EQTP_BF16 if args.out_bf16 else eq.EQTP_F32
    stream = torch.cuda.current_stream()

    sort_out = None
    if args.sort_edges:
        sort_out = (torch.empty(wl.N + 1, dtype=torch.int32, device=dev), torch.empty_like(src),
                    torch.empty_like(vec), torch.empty_like(src))

    def sort():
        if sort_out is not None:
            eq.eqtp_sort_edges(dst, wl.N, vec=vec, src=src, out=sort_out)

    ws_buf = None
    if args.ws:
        ws_buf = torch.empty(eq.eqtp_conv_workspace_bytes(wl.N, wl.E, wl.lmax, wl.C, weight_mode=wl.weight_mode,
                                                          path_set=wl.path_set), dtype=torch.uint8, device=dev)

    def conv():
        if ws_buf is not None:
            eq.eqtp_conv_fused_ws(vec, src, x, w, wl.lmax, dst=dst, path_set=wl.path_set, weight_mode=wl.weight_mode,
                                  r_cut=wl.r_cut, algo=args.algo, out=out, workspace=ws_buf)
            return
        if sort_out is not None:
            rp_s, _, vec_s, src_s = sort_out
            eq.eqtp_conv_fused(vec_s, src_s, x, w, wl.lmax, row_ptr=rp_s, path_set=wl.path_set,
                               weight_mode=wl.weight_mode, r_cut=wl.r_cut, algo=args.algo, out=out)
            return
        eq.eqtp_conv_fused(vec, src, x, w, wl.lmax, row_ptr=row_ptr, dst=dst, path_set=wl.path_set,
                           weight_mode=wl.weight_mode, r_cut=wl.r_cut, algo=args.algo, out=out, out_dtype=out_dtype)

    def linear():
        if w_lin is not None:
            eq.eqtp_linear(out, w_lin, wl.lmax, lin_dtype, out=out2)

    # the clocks of a device that was idle take tens of milliseconds of sustained work to ramp: run the
    # step for --prewarm-s seconds first (untimed, like the warmup steps that follow)
    prewarm_steps = 0
    t_pre = time.perf_counter()
    while time.perf_counter() - t_pre < args.prewarm_s:
        for _ in range(10):
            sort()
            conv()
            linear()
        prewarm_steps += 10
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        sort()
        conv()
        linear()
    torch.cuda.synchronize()

    K = args.steps
    # 1. the step rate: K back-to-back steps between two events (nothing else on the stream)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(K):
        sort()
        conv()
        linear()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / K
    graph_note = None
    if args.graph:
        # the same step captured as a HIP graph, GRAPH_STEPS steps per graph (one graph launch costs about
        # as much as a few kernel launches, so a one-step graph gains nothing), replayed until K steps ran:
        # what the step costs without the host's per-launch work (the eager rate is kept in the record)
        eager_ms = ms_per_step
        per_graph = graph_steps(K)
        reps = K // per_graph
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            conv()
            linear()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                conv()
                linear()
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        t_start.record(stream)
        for i in range(reps):
            g.replay()
        t_end.record(stream)
        torch.cuda.synchronize()
        ms_per_step = t_start.elapsed_time(t_end) / (reps * per_graph)
        graph_note = {"eager_ms_per_step": round(eager_ms, 5), "graph_ms_per_step": round(ms_per_step, 5),
                      "steps_per_graph": per_graph, "graph_replays": reps}
        log("graph replay: %.4f ms/step (%d steps per graph, %d replays; eager %.4f)" % (
            ms_per_step, per_graph, reps, eager_ms))
    # 2. per-launch durations: the same K steps again with an event pair around every launch (the
    #    events add gaps between the kernels, so this pass does not give the step rate)
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        ev[i][0].record(stream)
        sort()
        ev[i][1].record(stream)
        conv()
        ev[i][2].record(stream)
        linear()
        ev[i][3].record(stream)
    torch.cuda.synchronize()
    sort_ms = np.array([a.elapsed_time(b) for a, b, _, _ in ev])
    conv_ms = np.array([b.elapsed_time(c) for _, b, c, _ in ev])
    lin_ms = np.array([c.elapsed_time(d) for _, _, c, d in ev])
    log("timed %d steps: %.4f ms/step (events), wall %.4f ms/step; per launch (second pass): conv avg %.4f ms "
        "(p10 %.4f p90 %.4f), linear avg %.4f ms" % (K, ms_per_step, 1e3 * wall / K, conv_ms.mean(),
                                                      np.percentile(conv_ms, 10), np.percentile(conv_ms, 90),
                                                      lin_ms.mean()))
    if sort_out is not None:
        log("edge sort (eqtp_sort_edges) avg %.4f ms per step, inside the step" % sort_ms.mean())

    backward = None
    if args.backward:
        if args.x_bf16:
            log("backward: fp32 features only; skipped for this workload")
        elif wl.weight_mode == 1:
            gout = torch.randn(out.shape, dtype=torch.float32, device=dev)
            bkw = dict(dst=dst) if args.unsorted else dict(row_ptr=row_ptr)
            bvec, bsrc = vec, src
            if sort_out is not None:
                bkw = dict(row_ptr=sort_out[0])
                bvec, bsrc = sort_out[2], sort_out[3]

            def bwd_rad():
                eq.eqtp_conv_backward(bvec, bsrc, x, w, gout, wl.lmax, path_set=wl.path_set, weight_mode=1,
                                      r_cut=wl.r_cut, **bkw)

            # grouped by source on the GPU, then one pass for all three (what the autograd wrapper runs)
            E_ = wl.E
            rows = torch.empty(E_, dtype=torch.int32, device=dev) if "row_ptr" in bkw else None
            grp = (torch.empty(wl.N + 1, dtype=torch.int32, device=dev), torch.empty(E_, dtype=torch.int32, device=dev),
                   torch.empty((E_, 3), dtype=torch.float32, device=dev), torch.empty(E_, dtype=torch.int32, device=dev))
            sws = torch.empty(max(16, eq.eqtp_sort_workspace_bytes(wl.N, E_)), dtype=torch.uint8, device=dev)

            def bwd_rad_src():
                d_ = eq.eqtp_edge_rows(bkw["row_ptr"], E_, out=rows) if "row_ptr" in bkw else bkw["dst"]
                eq.eqtp_sort_edges_stable(bsrc, wl.N, vec=bvec, src=d_, out=grp, workspace=sws)
                eq.eqtp_conv_backward_by_source(grp[2], grp[3], grp[0], x, w, gout, wl.lmax, path_set=wl.path_set,
                                                need_vec=True, perm=grp[1], weight_mode=1, r_cut=wl.r_cut)

            def timed_r(fn):
                for _ in range(3):
                    fn()
                torch.cuda.synchronize()
                kb = max(5, K // 4)
                b0 = torch.cuda.Event(enable_timing=True)
                b1 = torch.cuda.Event(enable_timing=True)
                b0.record(stream)
                for _ in range(kb):
                    fn()
                b1.record(stream)
                torch.cuda.synchronize()
                return b0.elapsed_time(b1) / kb, kb

            rms, kb = timed_r(bwd_rad)
            sms, _ = timed_r(bwd_rad_src)
            backward = {"ms": round(sms, 5), "edges_per_s": round(wl.E / (sms * 1e-3), 1), "launches": kb,
                        "what": "grad_x, grad_W [8, P*C] and grad_vec of the radial-weight conv: source grouping "
                                "on the GPU (eqtp_edge_rows + eqtp_sort_edges_stable), then eqtp_conv_backward_by_source "
                                "with EQTP_W_RADIAL (one pass, grad_x without atomics)",
                        "edge_path_ms": round(rms, 5),
                        "edge_path_what": "eqtp_conv_backward with EQTP_W_RADIAL on the edges as given (zero fills "
                                          "+ one kernel, grad_x by fp32 atomics)"}
            log("backward (radial weights): by source %.4f ms (%.3e edges/s); edge path %.4f ms" % (
                sms, wl.E / (sms * 1e-3), rms))
        else:
            gout = torch.randn(out.shape, dtype=torch.float32, device=dev)
            bkw = dict(dst=dst) if args.unsorted else dict(row_ptr=row_ptr)
            bvec, bsrc = vec, src
            if sort_out is not None:
                bkw = dict(row_ptr=sort_out[0])
                bvec, bsrc = sort_out[2], sort_out[3]

            def bwd():  # the coupling walk (grad_vec of sorted edges on the matrix cores)
                eq.eqtp_conv_backward(bvec, bsrc, x, w, gout, wl.lmax, path_set=wl.path_set,
                                      algo=eq.EQTP_ALGO_NODE_MFMA, **bkw)

            def bwd_so2():  # the default: the edge-aligned form
                eq.eqtp_conv_backward(bvec, bsrc, x, w, gout, wl.lmax, path_set=wl.path_set, **bkw)

            # by source: destinations of the CSR, sort by source, grad_x and grad_w on
            # the matrix cores, grad_vec edge by edge (what the autograd wrapper runs)
            E_ = wl.E
            if "row_ptr" in bkw:
                rows = torch.empty(E_, dtype=torch.int32, device=dev)
            grp = (torch.empty(wl.N + 1, dtype=torch.int32, device=dev), torch.empty(E_, dtype=torch.int32, device=dev),
                   torch.empty((E_, 3), dtype=torch.float32, device=dev), torch.empty(E_, dtype=torch.int32, device=dev))
            sws = torch.empty(max(16, eq.eqtp_sort_workspace_bytes(wl.N, E_)), dtype=torch.uint8, device=dev)

            def bwd_src():
                d_ = eq.eqtp_edge_rows(bkw["row_ptr"], E_, out=rows) if "row_ptr" in bkw else bkw["dst"]
                eq.eqtp_sort_edges_stable(bsrc, wl.N, vec=bvec, src=d_, out=grp, workspace=sws)
                eq.eqtp_conv_backward_by_source(grp[2], grp[3], grp[0], x, w, gout, wl.lmax, path_set=wl.path_set)
                eq.eqtp_conv_backward(bvec, bsrc, x, w, gout, wl.lmax, path_set=wl.path_set, need_x=False,
                                      need_w=False, need_vec=True, **bkw)

            def timed(fn):
                for _ in range(max(3, args.warmup // 4)):
                    fn()
                torch.cuda.synchronize()
                kb = max(5, K // 4)
                b0 = torch.cuda.Event(enable_timing=True)
                b1 = torch.cuda.Event(enable_timing=True)
                b0.record(stream)
                for _ in range(kb):
                    fn()
                b1.record(stream)
                torch.cuda.synchronize()
                return b0.elapsed_time(b1) / kb, kb

            if wl.lmax > 3:
                def bwd_so2_src():
                    d_ = eq.eqtp_edge_rows(bkw["row_ptr"], E_, out=rows) if "row_ptr" in bkw else bkw["dst"]
                    eq.eqtp_sort_edges_stable(bsrc, wl.N, vec=bvec, src=d_, out=grp, workspace=sws)
                    eq.eqtp_conv_backward_by_source(grp[2], grp[3], grp[0], x, w, gout, wl.lmax,
                                                    path_set=wl.path_set, need_vec=True, perm=grp[1])

                oms, kb = timed(bwd_so2)
                sms, _ = timed(bwd_so2_src)
                backward = {"ms": round(sms, 5), "edges_per_s": round(wl.E / (sms * 1e-3), 1), "launches": kb,
                            "what": "grad_x, grad_w and grad_vec of the conv in the edge-aligned form: source "
                                    "grouping on the GPU (eqtp_edge_rows + eqtp_sort_edges_stable), then "
                                    "eqtp_conv_backward_by_source (one pass, grad_x without atomics)",
                            "edge_path_ms": round(oms, 5),
                            "edge_path_what": "eqtp_conv_backward on the edges as given (zero fills + one kernel, "
                                              "fp32 atomics for grad_x)"}
                log("backward (edge-aligned form): by source %.4f ms (%.3e edges/s); edge path %.4f ms" % (
                    sms, wl.E / (sms * 1e-3), oms))
            else:
                bms, kb = timed(bwd)
                sms, _ = timed(bwd_src)
                oms, _ = timed(bwd_so2)
                backward = {"ms": round(sms, 5), "edges_per_s": round(wl.E / (sms * 1e-3), 1), "launches": kb,
                            "what": "grad_x, grad_w and grad_vec of the conv: source grouping on the GPU "
                                    "(eqtp_edge_rows + eqtp_sort_edges_stable), eqtp_conv_backward_by_source (grad_x, "
                                    "grad_w), eqtp_conv_backward (grad_vec)",
                            "edge_path_ms": round(oms, 5),
                            "edge_path_what": "all three from eqtp_conv_backward with the default algorithm (the "
                                              "edge-aligned form, fp32 atomics for grad_x)",
                            "coupling_walk_ms": round(bms, 5),
                            "coupling_walk_what": "all three from eqtp_conv_backward with EQTP_ALGO_NODE_MFMA"}
                log("backward: by source %.4f ms (%.3e edges/s); edge path (edge-aligned) %.4f ms; coupling walk "
                    "%.4f ms" % (sms, wl.E / (sms * 1e-3), oms, bms))

    interaction = None
    if args.interaction:
        if args.unsorted or args.x_bf16 or wl.lmax > 3 or wl.C % 16 != 0:
            log("interaction: dst-sorted fp32 features, lmax <= 3, C a multiple of 16 only; skipped")
        else:
            iw = synth.interaction_weights(wl.lmax, wl.C, wl.path_set)
            it = [T(a) for a in (iw.W_up, iw.W1, iw.W2, iw.W3, iw.W_out)]
            norm = wl.E / wl.N
            ix_r_cut = wl.r_cut if wl.r_cut > 0 else 5.0
            ws = torch.empty(eq.eqtp_interaction_workspace_bytes(wl.N, wl.E, wl.lmax, wl.C, ix_r_cut, norm,
                                                                 wl.path_set), dtype=torch.uint8, device=dev)
            ix_out = torch.empty_like(x)

            def ix():
                eq.eqtp_interaction(vec, src, row_ptr, x, *it, wl.lmax, ix_r_cut, norm=norm, path_set=wl.path_set,
                                    workspace=ws, out=ix_out)

            for _ in range(3):
                ix()
            torch.cuda.synchronize()
            kb = max(5, K // 4)
            b0 = torch.cuda.Event(enable_timing=True)
            b1 = torch.cuda.Event(enable_timing=True)
            b0.record(stream)
            for _ in range(kb):
                ix()
            b1.record(stream)
            torch.cuda.synchronize()
            ims = b0.elapsed_time(b1) / kb
            P_ = wl.P
            interaction = {"ms": round(ims, 5), "edges_per_s": round(wl.E / (ims * 1e-3), 1), "launches": kb,
                           "hidden": 64, "r_cut": ix_r_cut, "norm": round(norm, 4),
                           "path_weight_tflops": round(2.0 * 64 * P_ * wl.C * wl.E / (ims * 1e-3) / 1e12, 3),
                           "what": "eqtp_interaction: linear_up, radial network 8->64->64 (SiLU), convolution with "
                                   "path weights phi_e W3 (last layer on the matrix cores), linear_out / norm"}
            log("interaction layer: %.4f ms (%.3e edges/s)" % (ims, wl.E / (ims * 1e-3)))

    messages = None
    if args.messages and args.x_bf16:
        log("messages: fp32 features only; skipped")
    elif args.messages:
        msg_out = torch.empty((wl.E, wl.C, wl.K), dtype=torch.float32, device=dev)

        def msg():
            eq.eqtp_conv_messages(vec, src, x, w, wl.lmax, path_set=wl.path_set, weight_mode=wl.weight_mode,
                                  r_cut=wl.r_cut, out=msg_out)

        for _ in range(3):
            msg()
        torch.cuda.synchronize()
        km = max(5, K // 4)
        m0 = torch.cuda.Event(enable_timing=True)
        m1 = torch.cuda.Event(enable_timing=True)
        m0.record(stream)
        for _ in range(km):
            msg()
        m1.record(stream)
        torch.cuda.synchronize()
        mms = m0.elapsed_time(m1) / km
        wbytes = wl.E * wl.C * wl.K * 4
        messages = {"ms": round(mms, 5), "edges_per_s": round(wl.E / (mms * 1e-3), 1), "launches": km,
                    "write_GBps": round(wbytes / (mms * 1e-3) / 1e9, 1),
                    "what": "per-edge messages [E,C,K] (one launch of eqtp_conv_messages)"}
        del msg_out
        log("messages: %.4f ms (%.3e edges/s, %.0f GB/s written)" % (mms, wl.E / (mms * 1e-3),
                                                                      wbytes / (mms * 1e-3) / 1e9))

    sh = None
    if args.sh:
        Y = torch.empty((wl.E, wl.K), dtype=torch.float32, device=dev)
        for _ in range(3):
            eq.eqtp_sh(vec, wl.lmax, Y=Y)
        torch.cuda.synchronize()
        ks = max(20, K // 2)
        s0 = torch.cuda.Event(enable_timing=True)
        s1 = torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for _ in range(ks):
            eq.eqtp_sh(vec, wl.lmax, Y=Y)
        s1.record(stream)
        torch.cuda.synchronize()
        sms = s0.elapsed_time(s1) / ks
        sbytes = wl.E * (12 + 4 * wl.K)
        sh = {"ms": round(sms, 5), "launches": ks, "bytes": sbytes, "GBps": round(sbytes / (sms * 1e-3) / 1e9, 1),
              "frac_hbm": round(sbytes / (sms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
              "what": "eqtp_sh: 12 B in and 4*K B out per edge, back-to-back launches between two events"}
        del Y
        log("sh: %.4f ms (%.0f GB/s, %.3f of HBM peak)" % (sms, sh["GBps"], sh["frac_hbm"]))

    if args.calib_copy:
        a = torch.empty(64 << 20, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        a.fill_(1.0)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log("calibration copy: 256 MiB read + 256 MiB written")

    edges_per_s = wl.E / (ms_per_step * 1e-3)
    nnz = count_terms(wl.lmax, wl.path_set)
    flop_edge = 2 * nnz * wl.C + (2 * 8 * wl.P * wl.C if wl.weight_mode == 1 else 0)
    conv_s = float(conv_ms.mean()) * 1e-3
    achieved_tflops = flop_edge * wl.E / conv_s / 1e12
    cfg_key = args.config if args.lmax is None else "lmax%d" % args.lmax
    # which kernel ran: the node kernel (fixed weights, dst-sorted, lmax <= 3) is bound by the fp32 matrix
    # cores; every other form by the fp32 vector ALUs (the radial edge-aligned kernel forms its radial
    # weights on the matrix cores but spends most of its time in the vector coupling)
    sorted_edges = not args.unsorted or args.sort_edges or args.ws
    node_kernel = wl.weight_mode == 0 and sorted_edges and wl.lmax <= 3 and args.algo in (0, 1)
    roofline = {"bound": "mfma" if node_kernel else "alu", "achieved": round(achieved_tflops, 3),
                "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved_tflops / PEAK_FP32_TFLOPS, 4),
                "traffic": None if args.out_bf16 else measured_traffic(cfg_key, args.atom_order, args.unsorted,
                                                                        args.algo, args.path_set, args.x_bf16,
                                                                        args.sort_edges)}
    if wl.weight_mode == 1:
        roofline["counted"] = ("2*nnz*C coupling flop (nnz=%d) + 2*8*P*C radial flop per edge, whichever form "
                               "the kernel computes them in" % nnz)
    elif args.algo == 3 or wl.lmax > 3:
        # edge-aligned kernel: vector-ALU bound; flop = 2 per arithmetic instruction lane it executes
        ops = so2_ops(wl.lmax, wl.path_set)
        so2_tflops = 2 * ops * wl.C * wl.E / conv_s / 1e12
        roofline = {"bound": "alu", "achieved": round(so2_tflops, 3), "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(so2_tflops / PEAK_FP32_TFLOPS, 4), "traffic": None,
                    "counted": "%d arithmetic ops per edge and channel (two frame rotations + sparse coupling), "
                               "2 flop each; the coupling form would count 2*%d" % (ops, nnz)}
    alg_bytes = 2 * wl.N * wl.C * wl.K * 4 + wl.E * 16 + (wl.N + 1) * 4 + wl.weights.size * 4
    log("conv: %.3e counted flop (2*nnz*C per edge), %.1f MB algorithmic bytes -> %.1f GB/s" % (
        flop_edge * wl.E, alg_bytes / 1e6, alg_bytes / conv_s / 1e9))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_budget_s)
        log("cpu baseline: %.1f edges/s (%s); one thread %.1f edges/s (%s)" % (
            cpu["value"], cpu["sample"], cpu["single_thread"]["value"], cpu["single_thread"]["sample"]))

    rec = {
        "metric": METRIC,
        "value": round(edges_per_s, 1),
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": (WORKLOAD_TEXT[args.config] if args.lmax is None else
                                "mid graph at lmax %d: 10k atoms, periodic 0.1/A^3, r_c=4 A, L=%d, C=64, conv"
                                % (wl.lmax, wl.lmax))
                   + (" (random edge order)" if args.unsorted else "")
                   + (" (sorted by destination on the GPU inside each step)" if args.sort_edges else "")
                   + (" (grouped by destination in a workspace inside each step, eqtp_conv_fused_ws)" if args.ws else "")
                   + (" (cell-sorted atom numbering)" if args.atom_order == "cell" else "")
                   + (" (SO(3) path set)" if args.path_set == "so3" else "")
                   + (" (bfloat16 node features)" if args.x_bf16 else "")
                   + (" (bfloat16 output, packed bf16 atomics; the linear reads it in bf16)" if args.out_bf16
                      else "")
                   + (" (step replayed as one HIP graph)" if args.graph else ""),
                   "atoms": wl.N, "edges": wl.E, "channels": wl.C, "lmax": wl.lmax, "paths": wl.P,
                   "coupling_nnz": nnz, "algo": args.algo},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "prewarm": {"seconds": args.prewarm_s, "steps": prewarm_steps,
                    "what": "untimed steps run before the warmup steps so that the device clocks have ramped"},
    }
    if sort_out is not None:
        rec["edge_sort"] = {"ms": round(float(sort_ms.mean()), 5),
                            "what": "eqtp_sort_edges (counting sort by destination), inside ms_per_step"}
    if graph_note is not None:
        rec["graph"] = graph_note
    if backward is not None:
        rec["backward"] = backward
    if messages is not None:
        rec["messages"] = messages
    if interaction is not None:
        rec["interaction"] = interaction
    if sh is not None:
        rec["sh"] = sh
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
