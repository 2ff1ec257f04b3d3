#!/usr/bin/env python3
"""Decode-step benchmark of the N:M bitmask SpMV against the same-GPU dense bf16 GEMV.

A step is one decode token (batch B, default 1) through a stack of synthetic decoder
layers -- every projection of every layer is one nm_spmv call on its own packed
weights -- for each N:M pattern of the workload.  The dense baseline runs the same
stack with dense_gemv on the unpruned weights.  Inputs are generated and packed on
the GPU before the timed region (column norms -> N:M select + pack), spot-checked
against the CPU oracle, and every timed launch reads weights already resident in HBM.

The headline step runs the projections that read the same x as one launch each --
q|k|v through nm_spmv_multi, gate|up through nm_spmv_swiglu (silu(g) * u written by the
epilogue), o and down alone -- against the same grouping of dense launches; the step
with one nm_spmv call per projection is reported beside it.

Printed (one JSON line on stdout): effective GB/s of the step (algorithmic bytes:
packed values + masks of every matrix, x once per launch, the launch's outputs), a
per-projection and per-fused-launch table (us, GB/s, % of the 8 TB/s HBM peak, dense
us, speedup, hipBLASLt us), the bitmask / uint8-offset / int32-index comparison, the
roofline of the step's dominant launch and the CPU oracle timed on the host cores.

Cache defeat: every per-projection timing rotates over >= 512 MB of distinct buffers
(twice the 256 MB Infinity Cache), and the step itself walks all layers of all
patterns in decode order (several GB between reuses).

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config 8b] [--layers 8]
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

HBM_PEAK_GBS = 8000.0
FP64_MFMA_PEAK_TFLOPS = 78.6
ROTATE_BYTES = 512e6
# Launches per timed graph: a rotation pool is cycled (buffer i % pool) in whole passes
# up to at least this many launches, so the cost of starting a graph replay is spread
# over as many dispatches as the pages' protocol times (50), and every buffer -- also
# across back-to-back replays -- is re-read only after the whole pool (>= 512 MB).
TIMED_LAUNCHES = 64
TIMED_REPLAYS = 5
METRIC = "nm_spmv GB/s and % HBM peak per layer; speedup vs dense bf16 GEMV, batch 1"

# Layer shapes (rows R = outputs, K = inputs) of the models the pages evaluate.
# group = which activation feeds the projection (projections of one group share x).
CONFIGS = {
    "tiny": dict(workload="tiny: one 256x512 matrix, 2:4", batch=(1,),
                 projs=[("w", 256, 512, "in")], patterns=[(2, 4)]),
    "8b": dict(workload="Llama-3.1-8B-shaped decode layer set, 2:4 and 16:32",
               projs=[("q", 4096, 4096, "attn"), ("k", 1024, 4096, "attn"), ("v", 1024, 4096, "attn"),
                      ("o", 4096, 4096, "attn_out"), ("gate", 14336, 4096, "mlp"), ("up", 14336, 4096, "mlp"),
                      ("down", 4096, 14336, "mlp_mid")],
               patterns=[(2, 4), (16, 32)], batch=(1,)),
    "8b-sweep": dict(workload="Llama-3.1-8B-shaped decode layer set, all four 50% patterns",
                     projs=None, patterns=[(2, 4), (4, 8), (8, 16), (16, 32)], batch=(1,), base="8b"),
    "qwen14b": dict(workload="Qwen3-14B-shaped layers, 4:8",
                    projs=[("q", 5120, 5120, "attn"), ("gate", 17408, 5120, "mlp"), ("up", 17408, 5120, "mlp"),
                           ("down", 5120, 17408, "mlp_mid")], patterns=[(4, 8)], batch=(1,)),
    "qwen32b": dict(workload="Qwen3-32B-shaped layers, 4:8",
                    projs=[("q", 8192, 5120, "attn"), ("gate", 25600, 5120, "mlp"), ("up", 25600, 5120, "mlp"),
                           ("down", 5120, 25600, "mlp_mid")], patterns=[(4, 8)], batch=(1,)),
    "70b": dict(workload="Llama-3.3-70B-shaped single-GPU layers, 8:16",
                projs=[("q", 8192, 8192, "attn"), ("k", 1024, 8192, "attn"), ("v", 1024, 8192, "attn"),
                       ("o", 8192, 8192, "attn_out"), ("gate", 28672, 8192, "mlp"), ("up", 28672, 8192, "mlp"),
                       ("down", 8192, 28672, "mlp_mid")], patterns=[(8, 16)], batch=(1, 2, 4, 8)),
}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def sparse_bytes(R, K, B):
    """Algorithmic bytes of one nm_spmv call: values R*K + masks R*K/8 + x 2BK + y 2BR."""
    return R * K + R * K // 8 + 2 * B * K + 2 * B * R


META_BYTES_PER_KEPT = {"bitmask": 0.25, "u8_offset": 1, "i32_index": 4}


def meta_format_bytes(fmt, R, K, B):
    """Algorithmic bytes of one SpMV call with the given metadata format."""
    return R * K + int(META_BYTES_PER_KEPT[fmt] * R * K // 2) + 2 * B * K + 2 * B * R


def dense_bytes(R, K, B):
    return 2 * R * K + 2 * B * K + 2 * B * R


def is_glu(grp):
    return [pr[0] for pr in grp] == ["gate", "up"]


def group_label(grp):
    return "|".join(pr[0] for pr in grp) + ("+swiglu" if is_glu(grp) else "")


def group_bytes(grp, B, dense):
    """Algorithmic bytes of one fused launch: every matrix of the group once, x once, and
    the outputs (one h of R rows for the gated MLP, else every matrix's y)."""
    K = grp[0][2]
    w = sum((2 if dense else 1.125) * R * K for _, R, _, _ in grp)
    outs = grp[0][1] if is_glu(grp) else sum(R for _, R, _, _ in grp)
    return int(w) + 2 * B * K + 2 * B * outs


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="8b", choices=sorted(CONFIGS))
    ap.add_argument("--layers", type=int, default=8, help="decoder layers of distinct buffers in a step")
    ap.add_argument("--batch", type=int, default=1, help="tokens per step (B)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall time of the oracle sample on all host cores (half of it again on one core)")
    ap.add_argument("--skip-check", action="store_true", help="skip the oracle spot check")
    ap.add_argument("--no-meta-formats", action="store_true",
                    help="skip the bitmask vs uint8-offset vs int32-index comparison table")
    ap.add_argument("--no-solver", action="store_true", help="skip the OBS / SparseGPT solver measurement")
    ap.add_argument("--solver-tokens", type=int, default=4096, help="calibration tokens for the solver")
    ap.add_argument("--no-unstructured", action="store_true",
                    help="skip the 50%% unstructured vs N:M comparison table")
    ap.add_argument("--profile-proj", default=None,
                    help="with --profile-kernel: launch this projection alone through nm_spmv (e.g. gate) "
                         "instead of the dominant launch")
    ap.add_argument("--profile-kernel", action="store_true",
                    help="counter-collection mode: only the dominant launch shape (eager, rotated) plus a "
                         "plain 256 MiB device copy used to calibrate the byte counters")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="host-only: turn two rocprofv3 --pmc runs of --profile-kernel (FETCH_SIZE, "
                         "WRITE_SIZE) into profiles/traffic.json")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="host-only: print a per-kernel / per-launch-shape summary of a rocprofv3 "
                         "--kernel-trace --stats run")
    return ap.parse_args()


class Timer:
    """HIP events on the current stream."""

    def __init__(self, torch):
        self.torch = torch

    def time_graph(self, g, reps):
        t = self.torch
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        t.cuda.synchronize()
        return e0.elapsed_time(e1) / reps  # ms per replay


def time_launches(torch, timer, fns):
    """Average µs per launch of a rotation: one graph of whole passes over the pool's
    launches (at least TIMED_LAUNCHES), replayed once untimed, then the median of
    TIMED_REPLAYS event-timed replays."""
    n = -(-TIMED_LAUNCHES // len(fns)) * len(fns)
    g = capture(torch, [fns[i % len(fns)] for i in range(n)])
    g.replay()
    t = sorted(timer.time_graph(g, 1) for _ in range(TIMED_REPLAYS))
    del g
    return t[len(t) // 2] * 1e3 / n


def capture(torch, fns):
    """Capture a list of launches into one HIP graph (launch overhead off the clock)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in fns:  # eager pass: first-call setup happens outside the capture
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for f in fns:
            f()
    torch.cuda.synchronize()
    return g


def main():
    args = parse()
    if args.ingest_pmc:
        return ingest_pmc(args, *args.ingest_pmc)
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bitmask_spmv_amd as nm
    import synth

    assert torch.cuda.is_available(), "bench.py needs a HIP GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    cfg = dict(CONFIGS[args.config])
    if cfg.get("projs") is None:
        cfg["projs"] = CONFIGS[cfg["base"]]["projs"]
    B = args.batch
    L = args.layers
    projs, patterns = cfg["projs"], cfg["patterns"]
    props = torch.cuda.get_device_properties(0)
    log(f"device {props.name} CUs={props.multi_processor_count} config={args.config} layers={L} B={B}")
    if args.profile_kernel:
        return profile_kernel(args, torch, nm, synth, cfg, dev)

    # ---------------------------------------------------------------- inputs
    # Per projection a pool of distinct weight buffers of >= 512 MB (and >= L); the
    # step uses the first L of each pool as the L decoder layers.
    t0 = time.time()
    pool_sparse = {}  # (pattern, proj) -> list of (masks, values)
    pool_dense = {}   # proj -> list of W
    pack_ms = 0.0
    pack_bytes = 0
    norm_ms = 0.0
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for pi, (name, R, K, group) in enumerate(projs):
        ns = max(L, math.ceil(ROTATE_BYTES / sparse_bytes(R, K, B)))
        nd = max(L, math.ceil(ROTATE_BYTES / dense_bytes(R, K, B)))
        for (N, M) in patterns:
            pool_sparse[(N, M), name] = []
        pool_dense[name] = []
        for c in range(max(ns, nd)):
            W = synth.device_weights(R, K, args.seed, 100 + pi, c)
            X = synth.device_calib_acts(K, args.seed, 200 + pi, c)
            ev0.record()
            n = nm.nm_col_norm(X)
            ev1.record()
            torch.cuda.synchronize()
            norm_ms += ev0.elapsed_time(ev1)
            for (N, M) in patterns:
                if c < ns:
                    ev0.record()
                    pk = nm.nm_prune_pack(W, n, N, M)
                    ev1.record()
                    torch.cuda.synchronize()
                    pack_ms += ev0.elapsed_time(ev1)
                    pack_bytes += 2 * R * K + sparse_bytes(R, K, 0)
                    pool_sparse[(N, M), name].append(pk)
            if c < nd:
                pool_dense[name].append(W)
            del X, n
    xs = {}
    for gi, group in enumerate(sorted({p[3] for p in projs})):
        K = [p[2] for p in projs if p[3] == group][0]
        xs[group] = [synth.device_decode_x(B, K, args.seed, 300 + gi, l) for l in range(L)]
    ys = {name: torch.empty((B, R), dtype=torch.bfloat16, device=dev) for name, R, K, _ in projs}
    ws_bytes = max([nm.nm_spmv_workspace_bytes(R, K, B) for _, R, K, _ in projs]
                   + [nm.dense_gemv_workspace_bytes(R, K, B) for _, R, K, _ in projs]
                   + [nm.nm_spmv_swiglu_workspace_bytes(R, K, B) for _, R, K, _ in projs]
                   + [nm.dense_gemv_swiglu_workspace_bytes(R, K, B) for _, R, K, _ in projs]
                   + [nm.nm_spmv_multi_workspace_bytes([R] * 3, K, B) for _, R, K, _ in projs]
                   + [nm.dense_gemv_multi_workspace_bytes([R] * 3, K, B) for _, R, K, _ in projs]
                   + [nm.nm_spmv_unstructured_workspace_bytes(R, K, B) for _, R, K, _ in projs] + [4])
    ws = torch.empty((ws_bytes + 3) // 4, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"inputs generated and packed in {time.time() - t0:.1f}s "
        f"(pack {pack_bytes / pack_ms / 1e6:.0f} GB/s, col_norm {norm_ms:.2f} ms total)")

    # ---------------------------------------------------------------- oracle spot check
    parity = "skipped"
    if not args.skip_check:
        import oracle

        def host_u16(t):
            return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

        g = np.random.default_rng(args.seed)
        for pi, (name, R, K, group) in enumerate(projs):
            rows = np.unique(np.concatenate([[0, R - 1], g.choice(R, size=min(R, 6), replace=False)]))
            ridx = torch.from_numpy(rows).to(dev)
            W = pool_dense[name][0]
            X = synth.device_calib_acts(K, args.seed, 200 + pi, 0)
            nref = oracle.col_norm(host_u16(X))
            assert (nm.nm_col_norm(X).cpu().numpy().view(np.uint32) == nref.view(np.uint32)).all(), "col_norm"
            Ws = host_u16(W.index_select(0, ridx))
            x = xs[group][0]
            xh = host_u16(x)
            for (N, M) in patterns:
                masks, values = pool_sparse[(N, M), name][0]
                mref, vref = oracle.prune_pack(Ws, nref, N, M)
                assert (masks.index_select(0, ridx).cpu().numpy().view(np.uint32) == mref).all(), f"masks {name}"
                assert (host_u16(values.index_select(0, ridx)) == vref).all(), f"values {name}"
                y = nm.nm_spmv(masks, values, x, workspace=ws)
                yref, absum = oracle.spmv(mref, vref, xh, K)
                yg = (host_u16(y)[:, rows].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
                assert oracle.within_tolerance(yg, yref, absum).all(), f"spmv {name} {N}:{M}"
            yd = nm.dense_gemv(W, x, workspace=ws)
            ydref, dabs = oracle.dense(Ws, xh)
            ydg = (host_u16(yd)[:, rows].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            assert oracle.within_tolerance(ydg, ydref, dabs).all(), f"dense {name}"
        parity = "ok"
        log("oracle spot check ok (col_norm, masks, values bit-exact; spmv/dense within tolerance)")

    # ---------------------------------------------------------------- step graphs
    def spmv_call(pk, x, y):
        m, v = pk
        return lambda: nm.nm_spmv(m, v, x, out=y, workspace=ws)

    def dense_call(W, x, y):
        return lambda: nm.dense_gemv(W, x, out=y, workspace=ws)

    sparse_fns, dense_fns = [], []
    step_sparse_bytes = 0
    step_dense_bytes = 0
    for (N, M) in patterns:
        for l in range(L):
            for name, R, K, group in projs:
                sparse_fns.append(spmv_call(pool_sparse[(N, M), name][l], xs[group][l], ys[name]))
                step_sparse_bytes += sparse_bytes(R, K, B)
    for l in range(L):
        for name, R, K, group in projs:
            dense_fns.append(dense_call(pool_dense[name][l], xs[group][l], ys[name]))
            step_dense_bytes += dense_bytes(R, K, B)
    g_sparse = capture(torch, sparse_fns)
    g_dense = capture(torch, dense_fns)
    timer = Timer(torch)

    # The same step with projections that read the same x (q|k|v, gate|up) fused into one
    # launch each (nm_spmv_multi / dense_gemv_multi): x is staged once per group.
    groups = []  # list of lists of projection tuples, in layer order
    for proj in projs:
        if groups and groups[-1][0][3] == proj[3]:
            groups[-1].append(proj)
        else:
            groups.append([proj])
    fused_fns, fused_dense_fns = [], []
    fused_sparse_bytes = L * len(patterns) * sum(group_bytes(grp, B, False) for grp in groups)
    fused_dense_bytes = L * sum(group_bytes(grp, B, True) for grp in groups)
    for (N, M) in patterns:
        for l in range(L):
            for grp in groups:
                if len(grp) == 1:
                    name = grp[0][0]
                    fused_fns.append(spmv_call(pool_sparse[(N, M), name][l], xs[grp[0][3]][l], ys[name]))
                elif [pr[0] for pr in grp] == ["gate", "up"]:
                    # gated MLP: h = silu(gate x) * (up x) written by the launch's epilogue
                    fused_fns.append(lambda g=pool_sparse[(N, M), "gate"][l], u=pool_sparse[(N, M), "up"][l],
                                     x=xs[grp[0][3]][l]: nm.nm_spmv_swiglu(g, u, x, out=ys["gate"], workspace=ws))
                else:
                    pk = [pool_sparse[(N, M), pr[0]][l] for pr in grp]
                    outs = [ys[pr[0]] for pr in grp]
                    fused_fns.append(lambda pk=pk, x=xs[grp[0][3]][l], outs=outs:
                                     nm.nm_spmv_multi(pk, x, outs=outs, workspace=ws))
    for l in range(L):
        for grp in groups:
            if [pr[0] for pr in grp] == ["gate", "up"]:
                fused_dense_fns.append(lambda g=pool_dense["gate"][l], u=pool_dense["up"][l], x=xs[grp[0][3]][l]:
                                       nm.dense_gemv_swiglu(g, u, x, out=ys["gate"], workspace=ws))
                continue
            Wl = [pool_dense[pr[0]][l] for pr in grp]
            outs = [ys[pr[0]] for pr in grp]
            fused_dense_fns.append(lambda Wl=Wl, x=xs[grp[0][3]][l], outs=outs:
                                   nm.dense_gemv_multi(Wl, x, outs=outs, workspace=ws))
    g_fused = capture(torch, fused_fns)
    g_fused_dense = capture(torch, fused_dense_fns)

    for _ in range(args.warmup):
        g_sparse.replay()
        g_dense.replay()
    torch.cuda.synchronize()
    ms_sparse = timer.time_graph(g_sparse, args.steps)
    ms_dense = timer.time_graph(g_dense, args.steps)
    for _ in range(args.warmup):
        g_fused.replay()
        g_fused_dense.replay()
    torch.cuda.synchronize()
    ms_fused = timer.time_graph(g_fused, args.steps)
    ms_fused_dense = timer.time_graph(g_fused_dense, args.steps)
    log(f"fused step: sparse {ms_fused * 1e3:.1f} us ({len(fused_fns)} launches), dense "
        f"{ms_fused_dense * 1e3:.1f} us ({len(fused_dense_fns)} launches)")
    log(f"step: sparse {ms_sparse * 1e3:.1f} us ({len(sparse_fns)} launches), dense {ms_dense * 1e3:.1f} us "
        f"({len(dense_fns)} launches, {len(patterns)} pattern(s) share it)")

    # ---------------------------------------------------------------- per projection
    per = {}
    for (N, M) in patterns:
        for name, R, K, group in projs:
            pool = pool_sparse[(N, M), name]
            fns = [spmv_call(pk, xs[group][i % L], ys[name]) for i, pk in enumerate(pool)]
            us = time_launches(torch, timer, fns)
            per.setdefault(name, {"R": R, "K": K})[f"{N}:{M}"] = {
                "us": round(us, 2), "GBs": round(sparse_bytes(R, K, B) / us / 1e3, 1),
                "pct_peak": round(100 * sparse_bytes(R, K, B) / us / 1e3 / HBM_PEAK_GBS, 1),
                "rotation_MB": round(len(fns) * sparse_bytes(R, K, B) / 1e6)}
    for name, R, K, group in projs:
        pool = pool_dense[name]
        fns = [dense_call(W, xs[group][i % L], ys[name]) for i, W in enumerate(pool)]
        us = time_launches(torch, timer, fns)
        lin = [(lambda W=W, x=xs[group][i % L]: torch.nn.functional.linear(x, W)) for i, W in enumerate(pool)]
        us_lin = time_launches(torch, timer, lin)
        d = per[name]
        d["dense_us"] = round(us, 2)
        d["dense_GBs"] = round(dense_bytes(R, K, B) / us / 1e3, 1)
        d["hipblaslt_us"] = round(us_lin, 2)
        for (N, M) in patterns:
            d[f"{N}:{M}"]["speedup_vs_dense"] = round(us / d[f"{N}:{M}"]["us"], 3)
            d[f"{N}:{M}"]["speedup_vs_hipblaslt"] = round(us_lin / d[f"{N}:{M}"]["us"], 3)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- fused launches
    # Every group of projections that read the same x as one launch (q|k|v through
    # nm_spmv_multi, gate|up through nm_spmv_swiglu whose epilogue writes silu(g) * u),
    # timed over >= 512 MB of distinct buffers like the table above.
    def fused_call(grp, i, N=None, M=None):
        x = xs[grp[0][3]][i % L]
        if N is None:
            Ws = [pool_dense[pr[0]][i % len(pool_dense[pr[0]])] for pr in grp]
            if is_glu(grp):
                return lambda: nm.dense_gemv_swiglu(Ws[0], Ws[1], x, out=ys["gate"], workspace=ws)
            outs = [ys[pr[0]] for pr in grp]
            return lambda: nm.dense_gemv_multi(Ws, x, outs=outs, workspace=ws)
        pk = [pool_sparse[(N, M), pr[0]][i % len(pool_sparse[(N, M), pr[0]])] for pr in grp]
        if is_glu(grp):
            return lambda: nm.nm_spmv_swiglu(pk[0], pk[1], x, out=ys["gate"], workspace=ws)
        outs = [ys[pr[0]] for pr in grp]
        return lambda: nm.nm_spmv_multi(pk, x, outs=outs, workspace=ws)

    for grp in groups:
        if len(grp) == 1:
            continue
        label = group_label(grp)
        fb, fdb = group_bytes(grp, B, False), group_bytes(grp, B, True)
        d = per.setdefault(label, {"R": [pr[1] for pr in grp], "K": grp[0][2]})
        for (N, M) in patterns:
            n_rot = min(len(pool_sparse[(N, M), pr[0]]) for pr in grp)
            us = time_launches(torch, timer, [fused_call(grp, i, N, M) for i in range(n_rot)])
            d[f"{N}:{M}"] = {"us": round(us, 2), "GBs": round(fb / us / 1e3, 1),
                             "pct_peak": round(100 * fb / us / 1e3 / HBM_PEAK_GBS, 1),
                             "rotation_MB": round(n_rot * fb / 1e6)}
        n_rot = min(len(pool_dense[pr[0]]) for pr in grp)
        us = time_launches(torch, timer, [fused_call(grp, i) for i in range(n_rot)])
        d["dense_us"] = round(us, 2)
        d["dense_GBs"] = round(fdb / us / 1e3, 1)
        for (N, M) in patterns:
            d[f"{N}:{M}"]["speedup_vs_dense"] = round(us / d[f"{N}:{M}"]["us"], 3)
        torch.cuda.synchronize()
        log(f"{label}: " + ", ".join(f"{k} {v['us']} us ({v['pct_peak']}%)" for k, v in d.items()
                                     if isinstance(v, dict)) + f"; dense {d['dense_us']} us")

    # ---------------------------------------------------------------- achievable read
    # What a launch that only streams reaches on the same byte count under the same
    # rotation (nm_stream_read over >= 512 MB of distinct buffers of that size): the rate
    # each launch's % of the 8 TB/s peak is read against.
    stream_us = {}

    def time_stream_read(nbytes):
        nbytes = (int(nbytes) + 15) // 16 * 16
        if nbytes not in stream_us:
            cnt = max(2, math.ceil(ROTATE_BYTES / nbytes))
            bufs = [torch.empty(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(cnt)]
            sink = torch.empty(nm.nm_stream_read_sink_words(nbytes), dtype=torch.int32, device=dev)
            stream_us[nbytes] = time_launches(torch, timer, [(lambda b=b: nm.nm_stream_read(b, sink=sink))
                                                             for b in bufs])
            del bufs
        return nbytes, stream_us[nbytes]

    first_pat = f"{patterns[0][0]}:{patterns[0][1]}"
    stream_log = []
    for grp in [[pr] for pr in projs] + [grp for grp in groups if len(grp) > 1]:
        label = grp[0][0] if len(grp) == 1 else group_label(grp)
        nbytes, us = time_stream_read(group_bytes(grp, B, False))
        d = per[label]
        d["stream_read"] = {"us": round(us, 2), "GBs": round(nbytes / us / 1e3, 1),
                            "pct_peak": round(100 * nbytes / us / 1e3 / HBM_PEAK_GBS, 1),
                            "spmv_over_stream_time": round(d[first_pat]["us"] / us, 3)}
        stream_log.append(f"{label} {round(us, 2)} us ({d['stream_read']['pct_peak']}%)")
    torch.cuda.synchronize()
    log("stream read of the same bytes (achievable): " + ", ".join(stream_log))

    # ---------------------------------------------------------------- metadata formats
    # The same product over the first pattern's packs with the metadata as uint8 offsets
    # and int32 column indices (converted on the device from the masks), each timed over
    # >= 512 MB of distinct buffers like the table above.
    meta_table = None
    if not args.no_meta_formats:
        meta_table = {}
        (N, M) = patterns[0]
        fmts = (("u8_offset", nm.NM_META_U8_OFFSET), ("i32_index", nm.NM_META_I32_INDEX))
        for name, R, K, group in projs:
            d = meta_table.setdefault(name, {"R": R, "K": K, "pattern": f"{N}:{M}"})
            bm = per[name][f"{N}:{M}"]
            d["bitmask"] = {"us": bm["us"], "GBs": bm["GBs"], "bytes": meta_format_bytes("bitmask", R, K, B)}
            for key, fmt in fmts:
                nb = meta_format_bytes(key, R, K, B)
                cnt = min(len(pool_sparse[(N, M), name]), max(2, math.ceil(ROTATE_BYTES / nb)))
                pool = [(nm.nm_meta_from_mask(mk, fmt), v) for mk, v in pool_sparse[(N, M), name][:cnt]]
                if fmt == nm.NM_META_U8_OFFSET:
                    # same lanes and summation order as the word-per-lane bitmask kernel:
                    # identical bits; the bitmask launch runs on the matrix cores instead
                    # for B >= 5 and K a multiple of 1024 (other order: agreement only)
                    mk0, v0 = pool_sparse[(N, M), name][0]
                    yb = nm.nm_spmv(mk0, v0, xs[group][0], workspace=ws)
                    ym = nm.nm_spmv_meta(pool[0][0], fmt, v0, xs[group][0], workspace=ws)
                    if B < 5 or K % 1024:
                        assert torch.equal(yb.view(torch.int16), ym.view(torch.int16)), f"{key} {name} != bitmask"
                    else:
                        yf, mf = yb.float(), ym.float()
                        assert float((yf - mf).abs().max()) <= 1e-2 * float(yf.abs().max()), f"{key} {name} != bitmask"
                fns = [(lambda mt=mt, v=v, x=xs[group][i % L]:
                        nm.nm_spmv_meta(mt, fmt, v, x, out=ys[name], workspace=ws)) for i, (mt, v) in enumerate(pool)]
                us = time_launches(torch, timer, fns)
                d[key] = {"us": round(us, 2), "GBs": round(nb / us / 1e3, 1), "bytes": nb,
                          "slowdown_vs_bitmask": round(us / bm["us"], 3),
                          "rotation_MB": round(len(fns) * nb / 1e6)}
                del pool, fns
            torch.cuda.synchronize()
        log("metadata formats (us): " + "; ".join(
            f"{n} bitmask {d['bitmask']['us']} u8 {d['u8_offset']['us']} i32 {d['i32_index']['us']}"
            for n, d in meta_table.items()))

    # ---------------------------------------------------------------- 50% unstructured rows
    # The pages' other 50% setting: each row keeps its K/2 highest scores, same encoding,
    # a varying number of set bits per word.  Packed on the device from the same weights
    # and timed like the N:M table (>= 512 MB of distinct buffers).
    unstructured = None
    if not args.no_unstructured:
        import oracle

        unstructured = {}
        (N, M) = patterns[0]
        for pi, (name, R, K, group) in enumerate(projs):
            nb_ = sparse_bytes(R, K, B)
            cnt = max(2, math.ceil(ROTATE_BYTES / nb_))
            pool = []
            for c in range(cnt):
                W = synth.device_weights(R, K, args.seed, 100 + pi, c)
                n = nm.nm_col_norm(synth.device_calib_acts(K, args.seed, 200 + pi, c))
                pool.append(nm.nm_prune_pack_unstructured(W, n))
                if c == 0:
                    # spot check: masks/values bit-exact and the product within tolerance on sampled rows
                    g = np.random.default_rng(args.seed + pi)
                    rows = np.unique(np.concatenate([[0, R - 1], g.choice(R, size=min(R, 6), replace=False)]))
                    ridx = torch.from_numpy(rows).to(dev)
                    hu = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                    nref = oracle.col_norm(hu(synth.device_calib_acts(K, args.seed, 200 + pi, c)))
                    ms, vs = oracle.prune_pack_unstructured(hu(W.index_select(0, ridx)), nref)
                    mk, vl = pool[0]
                    assert (mk.index_select(0, ridx).cpu().numpy().view(np.uint32) == ms).all(), f"u masks {name}"
                    assert (hu(vl.index_select(0, ridx)) == vs).all(), f"u values {name}"
                    yu = nm.nm_spmv_unstructured(mk, vl, xs[group][0], workspace=ws)
                    yref, absum = oracle.spmv_unstructured(ms, vs, hu(xs[group][0]), K)
                    yg = (hu(yu)[:, rows].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
                    assert oracle.within_tolerance(yg, yref, absum).all(), f"unstructured spmv {name}"
                del W, n
            fns = [(lambda mk=mk, vl=vl, x=xs[group][i % L]:
                    nm.nm_spmv_unstructured(mk, vl, x, out=ys[name], workspace=ws)) for i, (mk, vl) in enumerate(pool)]
            us = time_launches(torch, timer, fns)
            nmus = per[name][f"{N}:{M}"]["us"]
            unstructured[name] = {"R": R, "K": K, "us": round(us, 2), "GBs": round(nb_ / us / 1e3, 1),
                                  "pct_peak": round(100 * nb_ / us / 1e3 / HBM_PEAK_GBS, 1),
                                  f"nm_{N}:{M}_us": nmus, "slowdown_vs_nm": round(us / nmus, 3),
                                  "speedup_vs_dense": round(per[name]["dense_us"] / us, 3),
                                  "rotation_MB": round(len(fns) * nb_ / 1e6)}
            del pool, fns
            torch.cuda.synchronize()
        log("unstructured 50% (us): " + "; ".join(f"{n} {d['us']} (N:M {d[f'nm_{N}:{M}_us']}, dense "
                                                   f"x{d['speedup_vs_dense']})" for n, d in unstructured.items()))

    # ---------------------------------------------------------------- OBS / SparseGPT solver
    # Offline: the Hessian of T synthetic calibration tokens (fp64 MFMA), the damped
    # inverse factor and the column-sequential N:M solve of the largest MLP projection;
    # quality as the relative reconstruction error on the calibration tokens, against
    # the Wanda selection of the same weights.
    solver = None
    if not args.no_solver:
        name_s, R_s, K_s, _ = max(projs, key=lambda p: p[1] * p[2])
        T_s = args.solver_tokens
        (N, M) = patterns[0]
        W_s = synth.device_weights(R_s, K_s, args.seed, 600)
        X_s = synth.device_calib_acts(K_s, args.seed, 601, T=T_s)

        def timed(fn, reps=1):
            fn()
            torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record()
            for _ in range(reps):
                out = fn()
            ev[1].record()
            torch.cuda.synchronize()
            return ev[0].elapsed_time(ev[1]) / reps, out

        h_ms, H_s = timed(lambda: nm.nm_hessian(X_s), reps=5)
        f_ms, _ = timed(lambda: nm.nm_obs_inverse_factor(H_s, 0.01))
        sg_ms, (m_s, v_s) = timed(lambda: nm.nm_sparsegpt_prune_pack(W_s, H_s, N, M, 0.01))
        n_s = nm.nm_col_norm(X_s)
        mw, vw = nm.nm_prune_pack(W_s, n_s, N, M)

        def rel_err(mk, vl):
            Wp = nm.nm_unpack(mk, vl).float()
            Wf = W_s.float()
            Xf = X_s.float()
            num = ((Wf - Wp) @ Xf.T).pow(2).sum()
            den = (Wf @ Xf.T).pow(2).sum()
            return float(num / den)

        # H is symmetric: the kernel computes the 64x64 tiles on and above the diagonal
        # (g(g+1)/2 of them, g = ceil(K/64)) on the fp64 matrix cores; those are the flops
        # it executes and the ones held against the peak.
        g_t = -(-K_s // 64)
        flops = 2.0 * (g_t * (g_t + 1) // 2) * 64 * 64 * T_s
        solver = {"shape": f"{name_s} {R_s}x{K_s}", "pattern": f"{N}:{M}", "tokens": T_s,
                  "hessian_ms": round(h_ms, 3), "hessian_TFLOPs": round(flops / h_ms / 1e9, 2),
                  "hessian_tflop_executed": round(flops / 1e12, 4),
                  "hessian_frac_fp64_mfma_peak": round(flops / h_ms / 1e9 / FP64_MFMA_PEAK_TFLOPS, 4),
                  "inverse_factor_ms": round(f_ms, 2), "prune_pack_ms": round(sg_ms, 2),
                  "rel_recon_error": {"wanda": rel_err(mw, vw), "sparsegpt": rel_err(m_s, v_s)}}
        log(f"solver on {solver['shape']} {N}:{M}, {T_s} tokens: hessian {h_ms:.2f} ms "
            f"({solver['hessian_TFLOPs']} TFLOP/s fp64), inverse factor {f_ms:.1f} ms, solve+pack {sg_ms:.1f} ms; "
            f"rel. error wanda {solver['rel_recon_error']['wanda']:.4f} vs sparsegpt "
            f"{solver['rel_recon_error']['sparsegpt']:.4f}")
        del W_s, X_s, H_s, m_s, v_s, mw, vw
        torch.cuda.synchronize()

    # Dominant kernel: the launch of the (fused) step whose launches take the largest share
    # of it; its algorithmic bytes over its average launch time is the roofline's achieved.
    share = {}
    for grp in groups:
        label = grp[0][0] if len(grp) == 1 else group_label(grp)
        share[label] = sum(per[label][f"{N}:{M}"]["us"] for (N, M) in patterns)
    dom = max(share, key=share.get)
    dom_grp = next(grp for grp in groups if (grp[0][0] if len(grp) == 1 else group_label(grp)) == dom)
    dom_us = share[dom] / len(patterns)
    dom_bytes = group_bytes(dom_grp, B, False)
    achieved = dom_bytes / dom_us / 1e3  # GB/s
    traffic = None
    tf = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tf):
        try:
            with open(tf) as f:
                tj = json.load(f)
            key = f"{args.config}:{dom}:B{B}"
            if key in tj and tj[key].get("kernel_sha") == kernel_fingerprint():
                traffic = tj[key]["bytes_per_launch"]
        except (OSError, ValueError, KeyError):
            traffic = None
    dom_desc = (f"{'nm_spmv_swiglu' if is_glu(dom_grp) else ('nm_spmv_multi' if len(dom_grp) > 1 else 'nm_spmv')} "
                f"on {dom} ({' + '.join(f'{pr[1]}x{pr[2]}' for pr in dom_grp)}), B={B}")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": dom_desc, "algorithmic_bytes_per_launch": dom_bytes,
                "avg_launch_us": round(dom_us, 3)}

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        cores = len(os.sched_getaffinity(0))
        (N, M) = patterns[0]
        host = []
        sb = 0
        for name, R, K, group in projs:
            masks, values = pool_sparse[(N, M), name][0]
            host.append((masks.cpu().numpy().view(np.uint32), values.contiguous().view(torch.int16).cpu().numpy()
                         .view(np.uint16), xs[group][0].contiguous().view(torch.int16).cpu().numpy().view(np.uint16), K))
            sb += sparse_bytes(R, K, B)
        def run_for(seconds, nthreads):
            """Whole passes over the layer until `seconds` of wall time have gone by."""
            reps, t1 = 0, time.time()
            while reps == 0 or time.time() - t1 < seconds:
                for m_h, v_h, x_h, K in host:
                    oracle.spmv(m_h, v_h, x_h, K, nthreads=nthreads)
                reps += 1
            return reps, time.time() - t1

        reps, dt = run_for(args.cpu_seconds, cores)
        reps1, dt1 = run_for(args.cpu_seconds / 2, 1)  # the same sample on one core
        model = ""
        try:
            with open("/proc/cpuinfo") as f:
                model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
        except OSError:
            pass
        cpu = {"value": round(sb * reps / dt / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
               "sample": f"layer 0 of the set ({', '.join(p[0] for p in projs)}), {N}:{M}, B={B}, "
                         f"x{reps} reps, {dt:.1f}s wall",
               "one_core": {"value": round(sb * reps1 / dt1 / 1e9, 3), "unit": "GB/s",
                            "sample": f"the same layer, x{reps1} reps, {dt1:.1f}s wall"},
               "cpu_model": model}

    value = fused_sparse_bytes / (ms_fused * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_fused, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg["workload"], "layers": L, "batch": B,
                   "patterns": [f"{N}:{M}" for N, M in patterns], "parallelism": "single GPU"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1),
        "step": {"launches": len(fused_fns), "groups": [group_label(grp) for grp in groups],
                 "bytes": fused_sparse_bytes,
                 "dense_ms": round(ms_fused_dense, 4),
                 "dense_GBs": round(fused_dense_bytes / (ms_fused_dense * 1e-3) / 1e9, 1),
                 "speedup_vs_dense": round(ms_fused_dense * len(patterns) / ms_fused, 3)},
        "unfused_step": {"launches": len(sparse_fns), "ms": round(ms_sparse, 4), "bytes": step_sparse_bytes,
                         "GBs": round(step_sparse_bytes / (ms_sparse * 1e-3) / 1e9, 1),
                         "pct_hbm_peak": round(100 * step_sparse_bytes / (ms_sparse * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
                         "dense_ms": round(ms_dense, 4),
                         "speedup_vs_dense": round(ms_dense * len(patterns) / ms_sparse, 3)},
        "per_layer": per,
        "metadata_formats": meta_table,
        "unstructured_50": unstructured,
        "solver": solver,
        "pack_GBs": round(pack_bytes / pack_ms / 1e6, 1),
        "parity": parity,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


COPY_BYTES = 256 << 20


def profile_kernel(args, torch, nm, synth, cfg, dev):
    """Eager launches of the step's dominant launch (gate|up through nm_spmv_swiglu when the
    layer set has them, else the largest single projection), first pattern, rotated over
    >= 512 MB of distinct packed buffers, then one plain device-to-device copy of
    COPY_BYTES: the reference for the counters."""
    projs = cfg["projs"]
    names = [p[0] for p in projs]
    N, M = cfg["patterns"][0]
    B = args.batch
    glu = "gate" in names and "up" in names and args.profile_proj is None
    if args.profile_proj is not None:
        if args.profile_proj not in names:
            raise SystemExit(f"--profile-proj: no projection {args.profile_proj!r} in {names}")
        _, R, K, _ = projs[names.index(args.profile_proj)]
        label, mats = args.profile_proj, 1
    elif glu:
        _, R, K, _ = projs[names.index("gate")]
        label, mats = "gate|up+swiglu", 2
    else:
        _, R, K, _ = max(projs, key=lambda p: p[1] * p[2])
        label, mats = max(projs, key=lambda p: p[1] * p[2])[0], 1
    per_launch = mats * (R * K + R * K // 8)
    n_pool = max(2, math.ceil(ROTATE_BYTES / per_launch))
    pool = []
    for c in range(n_pool):
        n = nm.nm_col_norm(synth.device_calib_acts(K, args.seed, 401, c))
        packs = []
        for m in range(mats):
            W = synth.device_weights(R, K, args.seed, 400 + m, c)
            packs.append(nm.nm_prune_pack(W, n, N, M))
            del W
        pool.append(packs)
    x = synth.device_decode_x(B, K, args.seed, 402)
    y = torch.empty((B, R), dtype=torch.bfloat16, device=dev)
    wsb = nm.nm_spmv_swiglu_workspace_bytes(R, K, B) if glu else nm.nm_spmv_workspace_bytes(R, K, B)
    ws = torch.empty(max(1, wsb // 4), dtype=torch.float32, device=dev)
    src = torch.empty(COPY_BYTES // 2, dtype=torch.int16, device=dev).random_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for i in range(args.steps):
        packs = pool[i % n_pool]
        if glu:
            nm.nm_spmv_swiglu(packs[0], packs[1], x, out=y, workspace=ws)
        else:
            nm.nm_spmv(*packs[0], x, out=y, workspace=ws)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"profile_kernel": f"{label} {mats}x {R}x{K} {N}:{M} B={B}", "label": label,
                      "launches": args.steps, "copy_bytes": COPY_BYTES}), flush=True)


def _pmc_rows(d):
    import csv
    import glob

    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            key = (r["Dispatch_Id"], r["Kernel_Name"], r["Grid_Size"], r["Counter_Name"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return per


def ingest_pmc(args, fetch_dir, write_dir):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the dominant SpMV launches, scaled by
    what the same counters report for the plain copy of COPY_BYTES (which moves exactly
    COPY_BYTES each way).  Writes profiles/traffic.json."""
    cfg = dict(CONFIGS[args.config])
    if cfg.get("projs") is None:
        cfg["projs"] = CONFIGS[cfg["base"]]["projs"]
    names = [p[0] for p in cfg["projs"]]
    if "gate" in names and "up" in names:
        _, R, K, _ = cfg["projs"][names.index("gate")]
        name, mats = "gate|up+swiglu", 2
        grp = [p for p in cfg["projs"] if p[0] in ("gate", "up")]
    else:
        big = max(cfg["projs"], key=lambda p: p[1] * p[2])
        name, R, K, mats, grp = big[0], big[1], big[2], 1, [big]
    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = _pmc_rows(d)
        spmv = [v for (disp, kn, grid, cn), v in per.items() if cn == counter and "spmv_kernel" in kn]
        copies = [v for (disp, kn, grid, cn), v in per.items()
                  if cn == counter and "copy" in kn.lower() and "nmk" not in kn]
        if not spmv or not copies:
            raise SystemExit(f"{counter}: missing spmv ({len(spmv)}) or copy ({len(copies)}) dispatches")
        copy_kib = max(copies)  # the 256 MiB copy is the largest copy dispatch
        factor = COPY_BYTES / (copy_kib * 1024.0)
        spmv.sort()
        med = spmv[len(spmv) // 2]
        out[counter] = {"counter_kib_median": med, "copy_counter_kib": copy_kib, "scale": factor,
                        "bytes_per_launch": med * 1024.0 * factor, "dispatches": len(spmv)}
    total = out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"]
    key = f"{args.config}:{name}:B{args.batch}"
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = {}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    data[key] = {"kernel": f"{name} {mats}x {R}x{K}", "bytes_per_launch": round(total),
                 "algorithmic_bytes": group_bytes(grp, args.batch, False), "kernel_sha": kernel_fingerprint(),
                 "fetch": out["FETCH_SIZE"], "write": out["WRITE_SIZE"]}
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")
    print(json.dumps(data[key]))


def summarize_trace(d):
    import csv
    import glob
    import statistics

    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {d}")
    groups = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            kn = r["Kernel_Name"]
            if "nmk::" in kn:
                short = kn.replace("void ", "", 1) if kn.startswith("void ") else kn
                short = short.replace("nmk::(anonymous namespace)::", "").split("(")[0]
            else:
                short = "torch/other: " + kn[:40]
            wg = int(r["Workgroup_Size_X"]) * int(r.get("Workgroup_Size_Y", 1) or 1)
            grid = (int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y", 1) or 1)) // max(wg, 1)
            groups.setdefault((short, grid), []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    def pct(v, q):  # nearest-rank percentile
        s = sorted(v)
        return s[min(len(s) - 1, max(0, int(round(q / 100 * len(s) + 0.5)) - 1))]

    print("| kernel | workgroups | dispatches | avg us | median us | p10 us | p90 us | min us | total ms |")
    print("|---|---|---|---|---|---|---|---|---|")
    for (k, g), v in sorted(groups.items(), key=lambda kv: -sum(kv[1]))[:25]:
        print(f"| {k} | {g} | {len(v)} | {statistics.mean(v):.2f} | {statistics.median(v):.2f} | {pct(v, 10):.2f} | "
              f"{pct(v, 90):.2f} | {min(v):.2f} | {sum(v) / 1e3:.2f} |")


def kernel_fingerprint() -> str:
    """Hash of the SpMV kernel source (kernel, shared staging/dot helpers, device helpers):
    counters recorded for an older kernel are not reused."""
    import hashlib

    h = hashlib.sha256()
    for f in ("nm_spmv.hip", "nm_spmv_common.h", "nm_device.h"):
        with open(os.path.join(ROOT, "bitmask_spmv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
