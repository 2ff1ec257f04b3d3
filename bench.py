#!/usr/bin/env python3
"""Decode-step benchmark of the N:M bitmask SpMV against the same-GPU dense bf16 GEMV.

A step is one decode token (batch B, default 1) through a stack of synthetic decoder
layers -- every projection of every layer is one pruned linear on its own packed
weights -- for each N:M pattern of the workload.  The dense baseline runs the same
stack with dense_gemv on the unpruned weights.  Inputs are generated and packed on
the GPU before the timed region (column norms -> N:M select + pack), spot-checked
against the CPU oracle, and every timed launch reads weights already resident in HBM.

The headline (value, roofline) is the Llama-3.1-8B layer set at B = 1 with 2:4 and 16:32:
the projections that read the same x run as one launch each -- q|k|v through
nm_spmv_multi, gate|up through nm_spmv_swiglu (silu(g) * u written by the epilogue), o
and down alone -- against the same grouping of dense launches; the step with one
nm_spmv call per projection is reported beside it.

Beside it, in the same JSON line (`configs`), the other workloads: the 8B set swept over
the four 50% patterns with 32 decoder layers of distinct buffers, Qwen3-14B/32B layers
at 4:8, and Llama-3.3-70B layers at 8:16 with 1, 2, 4 and 8 tokens.

Per-layer timing (every projection and every fused launch): one HIP graph of whole
passes over a pool of distinct buffers (>= 512 MB, twice the 256 MB Infinity Cache, and
at least 64 launches), replayed 10 times untimed (>= 50 warmup launches), then 50 timed
replays; the per-launch time of each replay gives the median and its p10/p90 (the
pages' protocol times the median of 50 iterations after 50 warmup ones).

Printed (one JSON line on stdout): effective GB/s of the step (algorithmic bytes:
packed values + masks of every matrix, x once per launch, the launch's outputs), the
per-layer tables (us with p10/p90, GB/s, % of the 8 TB/s HBM peak, dense us, speedup,
hipBLASLt us, the achievable streaming read of the same bytes), the per-layer check
against >= 70 % of peak and >= 1.5x dense, the bitmask / uint8-offset / int32-index
comparison, the roofline of the step's dominant launch and the CPU oracle timed on the
host cores.

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
# up to at least this many launches, and every buffer -- also across back-to-back
# replays -- is re-read only after the whole pool (>= 512 MB) has been.
TIMED_LAUNCHES = 64
WARM_REPLAYS = 10
WARM_MS = 25.0  # and at least this much replay time before the timed replays
SETTLE_S = 0.5   # step replays before each further workload's timings (see settle)
TIMED_REPLAYS = 50
TARGET_PCT, TARGET_SPEEDUP = 70.0, 1.5
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
# The other workloads measured beside the headline in the default run: (config, decoder
# layers in the step, batch sizes).
OTHER_CONFIGS = [("8b-sweep", 32, (1,)), ("qwen14b", 4, (1,)), ("qwen32b", 4, (1,)), ("70b", 4, (1, 2, 4, 8))]


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
    return grp[0][0] if len(grp) == 1 else "|".join(pr[0] for pr in grp) + ("+swiglu" if is_glu(grp) else "")


def group_bytes(grp, B, dense):
    """Algorithmic bytes of one (fused) launch: every matrix of the group once, x once, and
    the outputs (one h of R rows for the gated MLP, else every matrix's y)."""
    K = grp[0][2]
    w = sum((2 if dense else 1.125) * R * K for _, R, _, _ in grp)
    outs = grp[0][1] if is_glu(grp) else sum(R for _, R, _, _ in grp)
    return int(w) + 2 * B * K + 2 * B * outs


def layer_groups(projs):
    """Projections in layer order, consecutive ones that share x grouped into one launch."""
    groups = []
    for proj in projs:
        if groups and groups[-1][0][3] == proj[3]:
            groups[-1].append(proj)
        else:
            groups.append([proj])
    return groups


def best_dense_launch_sum(per, projs, patterns):
    """The fused step's launches from the per-launch table, against the faster dense
    baseline per launch: for each launch group, min(this repository's dense launch,
    hipBLASLt's single projections summed -- no fused equivalent there, so the gated MLP's
    SiLU-multiply is left out in its favour).  Returns {"sparse_us", "best_dense_us",
    "speedup"} for the first pattern, or None when hipBLASLt was not measured."""
    N, M = patterns[0]
    sp = bd = 0.0
    for grp in layer_groups(projs):
        d = per.get(group_label(grp))
        if not d or f"{N}:{M}" not in d or "dense_us" not in d:
            return None
        hip = [per.get(pr[0], {}).get("hipblaslt_us") for pr in grp]
        if any(h is None for h in hip):
            return None
        sp += d[f"{N}:{M}"]["us"]
        bd += min(d["dense_us"], sum(hip))
    return {"sparse_us": round(sp, 3), "best_dense_us": round(bd, 3), "speedup": round(bd / sp, 3)}


def pctl(v, q):
    """Nearest-rank percentile."""
    s = sorted(v)
    return s[min(len(s) - 1, max(0, int(math.ceil(q / 100 * len(s))) - 1))]


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
    ap.add_argument("--no-other-configs", action="store_true",
                    help="measure only the headline workload (skip the 8B pattern sweep, Qwen3 and 70B sets)")
    ap.add_argument("--profile-proj", default=None,
                    help="with --profile-kernel: launch this projection alone through nm_spmv (e.g. gate) "
                         "instead of the dominant launch")
    ap.add_argument("--profile-kernel", action="store_true",
                    help="profiling mode: only the dominant launch shape, rotated and timed as the "
                         "per-launch tables time it, plus a plain 256 MiB device copy used to calibrate the "
                         "byte counters")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="host-only: turn two rocprofv3 --pmc runs of --profile-kernel (FETCH_SIZE, "
                         "WRITE_SIZE) into profiles/traffic.json")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="host-only: print a per-kernel / per-launch-shape summary of a rocprofv3 "
                         "--kernel-trace --stats run")
    return ap.parse_args()


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


def time_graph(torch, g, reps):
    """Average ms per replay over `reps` back-to-back replays (HIP events on the stream the
    graph replays on)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def time_launches(torch, fns):
    """Per-launch µs of a rotation: one graph of whole passes over the pool's launches (at
    least TIMED_LAUNCHES), untimed replays (WARM_REPLAYS and at least WARM_MS of them, so
    that clocks settle after host-side work whatever ran before), then TIMED_REPLAYS replays
    timed one by one; returns the median and p10/p90 of the per-launch time of a replay."""
    n = -(-TIMED_LAUNCHES // len(fns)) * len(fns)
    g = capture(torch, [fns[i % len(fns)] for i in range(n)])
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record()
    g.replay()
    w1.record()
    torch.cuda.synchronize()
    for _ in range(max(WARM_REPLAYS - 1, math.ceil(WARM_MS / max(w0.elapsed_time(w1), 1e-3)))):
        g.replay()
    e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(TIMED_REPLAYS)]
    for e0, e1 in e:
        e0.record()
        g.replay()
        e1.record()
    torch.cuda.synchronize()
    t = [e0.elapsed_time(e1) * 1e3 / n for e0, e1 in e]
    del g
    return {"us": round(pctl(t, 50), 3), "p10": round(pctl(t, 10), 3), "p90": round(pctl(t, 90), 3),
            "launches": n * TIMED_REPLAYS}


def rate(nbytes, t):
    """GB/s and % of the HBM peak of nbytes per t['us']."""
    gbs = nbytes / t["us"] / 1e3
    return {"GBs": round(gbs, 1), "pct_peak": round(100 * gbs / HBM_PEAK_GBS, 1)}


class Ctx:
    """Device, library handles and one shared workspace (grown on demand)."""

    def __init__(self, args):
        import numpy as np
        import torch

        import bitmask_spmv_amd as nm
        import synth

        self.np, self.torch, self.nm, self.synth, self.args = np, torch, nm, synth, args
        self.dev = torch.device("cuda", 0)
        self.ws = torch.empty(1, dtype=torch.float32, device=self.dev)

    def workspace(self, projs, B):
        nm = self.nm
        need = max([nm.nm_spmv_workspace_bytes(R, K, B) for _, R, K, _ in projs]
                   + [nm.dense_gemv_workspace_bytes(R, K, B) for _, R, K, _ in projs]
                   + [nm.nm_spmv_swiglu_workspace_bytes(R, K, B) for _, R, K, _ in projs]
                   + [nm.dense_gemv_swiglu_workspace_bytes(R, K, B) for _, R, K, _ in projs]
                   + [nm.nm_spmv_multi_workspace_bytes([R] * 3, K, B) for _, R, K, _ in projs]
                   + [nm.dense_gemv_multi_workspace_bytes([R] * 3, K, B) for _, R, K, _ in projs]
                   + [nm.nm_spmv_unstructured_workspace_bytes(R, K, B) for _, R, K, _ in projs] + [4])
        if self.ws.numel() * 4 < need:
            self.ws = self.torch.empty((need + 3) // 4, dtype=self.torch.float32, device=self.dev)
        return self.ws


def build_pools(c, projs, patterns, L, seed, with_dense=True):
    """Per projection a pool of distinct packed buffers of >= 512 MB (and >= L) per pattern,
    and the same for the dense weights; the step uses the first L of each pool as its L
    decoder layers.  Returns (pool_sparse, pool_dense, stats)."""
    torch, nm, synth = c.torch, c.nm, c.synth
    pool_sparse, pool_dense = {}, {}
    pack_ms = norm_ms = 0.0
    pack_bytes = 0
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for pi, (name, R, K, group) in enumerate(projs):
        ns = max(L, math.ceil(ROTATE_BYTES / sparse_bytes(R, K, 1)))
        nd = max(L, math.ceil(ROTATE_BYTES / dense_bytes(R, K, 1))) if with_dense else 0
        for (N, M) in patterns:
            pool_sparse[(N, M), name] = []
        pool_dense[name] = []
        for i in range(max(ns, nd)):
            W = synth.device_weights(R, K, seed, 100 + pi, i)
            X = synth.device_calib_acts(K, seed, 200 + pi, i)
            ev0.record()
            n = nm.nm_col_norm(X)
            ev1.record()
            torch.cuda.synchronize()
            norm_ms += ev0.elapsed_time(ev1)
            for (N, M) in patterns:
                if i < ns:
                    # outputs allocated first: the events time the pack kernel, not the allocator
                    mk = torch.empty((R, K // 32), dtype=torch.int32, device=c.dev)
                    vl = torch.empty((R, K // 2), dtype=torch.bfloat16, device=c.dev)
                    ev0.record()
                    pk = nm.nm_prune_pack(W, n, N, M, masks=mk, values=vl)
                    ev1.record()
                    torch.cuda.synchronize()
                    pack_ms += ev0.elapsed_time(ev1)
                    pack_bytes += 2 * R * K + sparse_bytes(R, K, 0)
                    pool_sparse[(N, M), name].append(pk)
            if i < nd:
                pool_dense[name].append(W)
            del X, n, W
    return pool_sparse, pool_dense, {"pack_ms": pack_ms, "pack_bytes": pack_bytes, "norm_ms": norm_ms}


def make_inputs(c, projs, B, L, seed):
    """L decode inputs per activation group (one per decoder layer) and one output per
    projection."""
    synth, torch = c.synth, c.torch
    xs = {}
    for gi, group in enumerate(sorted({p[3] for p in projs})):
        K = [p[2] for p in projs if p[3] == group][0]
        xs[group] = [synth.device_decode_x(B, K, seed, 300 + gi, B, l) for l in range(L)]
    ys = {name: torch.empty((B, R), dtype=torch.bfloat16, device=c.dev) for name, R, K, _ in projs}
    return xs, ys


def spot_check(c, projs, patterns, pool_sparse, pool_dense, xs, seed):
    """Column norms, masks and values bit-exact and spmv / dense within tolerance on a
    sample of rows of layer 0 of every projection, against the CPU oracle."""
    import oracle

    np, torch, nm, synth = c.np, c.torch, c.nm, c.synth

    def host_u16(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    g = np.random.default_rng(seed)
    for pi, (name, R, K, group) in enumerate(projs):
        rows = np.unique(np.concatenate([[0, R - 1], g.choice(R, size=min(R, 6), replace=False)]))
        ridx = torch.from_numpy(rows).to(c.dev)
        X = synth.device_calib_acts(K, seed, 200 + pi, 0)
        nref = oracle.col_norm(host_u16(X))
        assert (nm.nm_col_norm(X).cpu().numpy().view(np.uint32) == nref.view(np.uint32)).all(), "col_norm"
        W = pool_dense[name][0] if pool_dense.get(name) else synth.device_weights(R, K, seed, 100 + pi, 0)
        Ws = host_u16(W.index_select(0, ridx))
        x = xs[group][0]
        xh = host_u16(x)
        for (N, M) in patterns:
            masks, values = pool_sparse[(N, M), name][0]
            mref, vref = oracle.prune_pack(Ws, nref, N, M)
            assert (masks.index_select(0, ridx).cpu().numpy().view(np.uint32) == mref).all(), f"masks {name}"
            assert (host_u16(values.index_select(0, ridx)) == vref).all(), f"values {name}"
            y = nm.nm_spmv(masks, values, x, workspace=c.ws)
            yref, absum = oracle.spmv(mref, vref, xh, K)
            yg = (host_u16(y)[:, rows].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            assert oracle.within_tolerance(yg, yref, absum).all(), f"spmv {name} {N}:{M}"
        yd = nm.dense_gemv(W, x, workspace=c.ws)
        ydref, dabs = oracle.dense(Ws, xh)
        ydg = (host_u16(yd)[:, rows].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert oracle.within_tolerance(ydg, ydref, dabs).all(), f"dense {name}"


def group_call(c, grp, pk, x, ys, dense=False):
    """One launch of a group: nm_spmv / nm_spmv_multi / nm_spmv_swiglu (pk: packs), or the
    dense counterparts (pk: weights)."""
    nm, ws = c.nm, c.ws
    if dense:
        if len(grp) == 1:
            return lambda: nm.dense_gemv(pk[0], x, out=ys[grp[0][0]], workspace=ws)
        if is_glu(grp):
            return lambda: nm.dense_gemv_swiglu(pk[0], pk[1], x, out=ys["gate"], workspace=ws)
        outs = [ys[pr[0]] for pr in grp]
        return lambda: nm.dense_gemv_multi(pk, x, outs=outs, workspace=ws)
    if len(grp) == 1:
        m, v = pk[0]
        return lambda: nm.nm_spmv(m, v, x, out=ys[grp[0][0]], workspace=ws)
    if is_glu(grp):
        return lambda: nm.nm_spmv_swiglu(pk[0], pk[1], x, out=ys["gate"], workspace=ws)
    outs = [ys[pr[0]] for pr in grp]
    return lambda: nm.nm_spmv_multi(pk, x, outs=outs, workspace=ws)


def step_graphs(c, projs, patterns, pool_sparse, pool_dense, xs, ys, L, B):
    """The fused decode step: L decoder layers of every pattern in decode order, each layer
    its groups as one launch each; the dense step runs the same grouping once."""
    groups = layer_groups(projs)
    sparse, dense = [], []
    for (N, M) in patterns:
        for l in range(L):
            for grp in groups:
                sparse.append(group_call(c, grp, [pool_sparse[(N, M), pr[0]][l] for pr in grp], xs[grp[0][3]][l], ys))
    for l in range(L):
        for grp in groups:
            dense.append(group_call(c, grp, [pool_dense[pr[0]][l] for pr in grp], xs[grp[0][3]][l], ys, dense=True))
    sb = L * len(patterns) * sum(group_bytes(grp, B, False) for grp in groups)
    db = L * sum(group_bytes(grp, B, True) for grp in groups)
    return sparse, dense, sb, db


def settle(c, fns, seconds=SETTLE_S):
    """Replays of one step for about `seconds` (untimed) before a workload's timings, so
    that they start from the clocks of sustained decoding.  After the pools of a workload
    are built the first ~0.35 s of launches ran up to 8% slow (70B q at B = 1: 14.6 us,
    then 13.5 us), whatever was launched; after a pause of 1 s the 8B step read 2% slow
    again (0.761 ms against 0.746 ms right after these replays)."""
    g = capture(c.torch, fns)
    t0 = time.time()
    while time.time() - t0 < seconds:
        g.replay()
        c.torch.cuda.synchronize()
    del g


def time_step(c, fns, steps, warmup):
    g = capture(c.torch, fns)
    for _ in range(warmup):
        g.replay()
    c.torch.cuda.synchronize()
    ms = time_graph(c.torch, g, steps)
    del g
    return ms


def per_layer_table(c, projs, patterns, pool_sparse, pool_dense, xs, ys, L, B, hipblaslt=False):
    """Every projection and every fused group timed alone over its rotation pool: sparse per
    pattern, dense, speedup (and hipBLASLt's torch.nn.functional.linear for single
    projections when asked, with the speedup against the faster of the two dense
    baselines)."""
    torch = c.torch
    per = {}
    for grp in [[p] for p in projs] + [grp for grp in layer_groups(projs) if len(grp) > 1]:
        label = group_label(grp)
        K = grp[0][2]
        d = per.setdefault(label, {"R": grp[0][1] if len(grp) == 1 else [pr[1] for pr in grp], "K": K})
        nb, ndb = group_bytes(grp, B, False), group_bytes(grp, B, True)
        for (N, M) in patterns:
            n_rot = min(len(pool_sparse[(N, M), pr[0]]) for pr in grp)
            fns = [group_call(c, grp, [pool_sparse[(N, M), pr[0]][i] for pr in grp], xs[grp[0][3]][i % L], ys)
                   for i in range(n_rot)]
            t = time_launches(torch, fns)
            d[f"{N}:{M}"] = dict(t, **rate(nb, t), rotation_MB=round(n_rot * nb / 1e6))
        if pool_dense.get(grp[0][0]):
            n_rot = min(len(pool_dense[pr[0]]) for pr in grp)
            fns = [group_call(c, grp, [pool_dense[pr[0]][i] for pr in grp], xs[grp[0][3]][i % L], ys, dense=True)
                   for i in range(n_rot)]
            t = time_launches(torch, fns)
            d["dense_us"], d["dense_p10"], d["dense_p90"] = t["us"], t["p10"], t["p90"]
            d["dense_GBs"] = rate(ndb, t)["GBs"]
            for (N, M) in patterns:
                d[f"{N}:{M}"]["speedup_vs_dense"] = round(t["us"] / d[f"{N}:{M}"]["us"], 3)
            if hipblaslt and len(grp) == 1:
                lin = [(lambda W=pool_dense[grp[0][0]][i], x=xs[grp[0][3]][i % L]: torch.nn.functional.linear(x, W))
                       for i in range(n_rot)]
                tl = time_launches(torch, lin)
                d["hipblaslt_us"] = tl["us"]
                for (N, M) in patterns:
                    d[f"{N}:{M}"]["speedup_vs_hipblaslt"] = round(tl["us"] / d[f"{N}:{M}"]["us"], 3)
                    # against the faster of the two dense baselines
                    d[f"{N}:{M}"]["speedup_vs_best_dense"] = round(min(tl["us"], t["us"]) / d[f"{N}:{M}"]["us"], 3)
        torch.cuda.synchronize()
    return per


def target_check(per, patterns):
    """Each launch of the table against the per-layer target: >= 70 % of the HBM peak and
    >= 1.5x the same-GPU dense GEMV; with the achievable streaming read of its bytes."""
    out = {}
    for label, d in per.items():
        for (N, M) in patterns:
            e = d.get(f"{N}:{M}")
            if not e or "speedup_vs_dense" not in e:
                continue
            row = {"pct_peak": e["pct_peak"], "speedup_vs_dense": e["speedup_vs_dense"],
                   "pct_ok": e["pct_peak"] >= TARGET_PCT, "speedup_ok": e["speedup_vs_dense"] >= TARGET_SPEEDUP}
            if "stream_read" in d:
                # a plain read of the launch's bytes below the bar: no kernel of this size
                # can reach it, whatever its walk costs
                row["stream_read_pct_peak"] = d["stream_read"]["pct_peak"]
                row["pct_reachable_by_plain_read"] = d["stream_read"]["pct_peak"] >= TARGET_PCT
            out[f"{label} {N}:{M}"] = row
    return out


def measure_other(c, name, L, batches, steps, warmup, seed, check):
    """One of the other workloads: per-layer table and fused step for each batch size."""
    torch = c.torch
    cfg = dict(CONFIGS[name])
    projs = cfg.get("projs") or CONFIGS[cfg["base"]]["projs"]
    patterns = cfg["patterns"]
    t0 = time.time()
    pool_sparse, pool_dense, _ = build_pools(c, projs, patterns, L, seed + 17)
    out = {"workload": cfg["workload"], "layers": L, "patterns": [f"{N}:{M}" for N, M in patterns], "by_batch": {}}
    for B in batches:
        xs, ys = make_inputs(c, projs, B, L, seed + 17)
        c.workspace(projs, B)
        if check and B == batches[0]:
            spot_check(c, projs, patterns, pool_sparse, pool_dense, xs, seed + 17)
        sparse, dense, sb, db = step_graphs(c, projs, patterns, pool_sparse, pool_dense, xs, ys, L, B)
        settle(c, sparse)
        ms = time_step(c, sparse, steps, warmup)
        msd = time_step(c, dense, steps, warmup)
        per = per_layer_table(c, projs, patterns, pool_sparse, pool_dense, xs, ys, L, B, hipblaslt=True)
        gbs = sb / (ms * 1e-3) / 1e9
        out["by_batch"][f"B{B}"] = {
            "step": {"launches": len(sparse), "ms": round(ms, 4), "GBs": round(gbs, 1),
                     "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1), "dense_ms": round(msd, 4),
                     "speedup_vs_dense": round(msd * len(patterns) / ms, 3),
                     "launch_sum_vs_best_dense": best_dense_launch_sum(per, projs, patterns)},
            "per_layer": per}
        lsum = out["by_batch"][f"B{B}"]["step"]["launch_sum_vs_best_dense"]
        log(f"{name} B={B}: step {ms * 1e3:.1f} us ({100 * gbs / HBM_PEAK_GBS:.1f}% of peak, "
            f"{msd * len(patterns) / ms:.2f}x dense"
            + (f", launches {lsum['speedup']:.2f}x the faster dense per launch" if lsum else "") + "); " + ", ".join(
                f"{k} {v[p]['us']} us ({v[p]['pct_peak']}%)" for k, v in per.items()
                for p in [f"{N}:{M}" for N, M in patterns[:1]]))
        del xs, ys, sparse, dense
    del pool_sparse, pool_dense
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    out["seconds"] = round(time.time() - t0, 1)
    return out


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

    import torch

    assert torch.cuda.is_available(), "bench.py needs a HIP GPU"
    torch.cuda.set_device(0)
    c = Ctx(args)
    np, nm, synth = c.np, c.nm, c.synth
    cfg = dict(CONFIGS[args.config])
    if cfg.get("projs") is None:
        cfg["projs"] = CONFIGS[cfg["base"]]["projs"]
    B = args.batch
    L = args.layers
    projs, patterns = cfg["projs"], cfg["patterns"]
    props = torch.cuda.get_device_properties(0)
    log(f"device {props.name} CUs={props.multi_processor_count} config={args.config} layers={L} B={B}")
    if args.profile_kernel:
        return profile_kernel(args, torch, nm, synth, cfg, c.dev)

    # ---------------------------------------------------------------- inputs
    t0 = time.time()
    pool_sparse, pool_dense, st = build_pools(c, projs, patterns, L, args.seed)
    xs, ys = make_inputs(c, projs, B, L, args.seed)
    ws = c.workspace(projs, B)
    torch.cuda.synchronize()
    log(f"inputs generated and packed in {time.time() - t0:.1f}s "
        f"(pack {st['pack_bytes'] / st['pack_ms'] / 1e6:.0f} GB/s, col_norm {st['norm_ms']:.2f} ms total)")

    # ---------------------------------------------------------------- oracle spot check
    parity = "skipped"
    if not args.skip_check:
        spot_check(c, projs, patterns, pool_sparse, pool_dense, xs, args.seed)
        parity = "ok"
        log("oracle spot check ok (col_norm, masks, values bit-exact; spmv/dense within tolerance)")

    # ---------------------------------------------------------------- steps
    groups = layer_groups(projs)
    fused_fns, fused_dense_fns, fused_sparse_bytes, fused_dense_bytes = step_graphs(
        c, projs, patterns, pool_sparse, pool_dense, xs, ys, L, B)
    # steady state first (untimed): then the W warm-up steps and exactly K timed steps
    settle(c, fused_fns)
    ms_fused = time_step(c, fused_fns, args.steps, args.warmup)
    ms_fused_dense = time_step(c, fused_dense_fns, args.steps, args.warmup)
    # the same step with one nm_spmv call per projection
    single = [[p] for p in projs]
    sparse_fns = [group_call(c, grp, [pool_sparse[(N, M), grp[0][0]][l]], xs[grp[0][3]][l], ys)
                  for (N, M) in patterns for l in range(L) for grp in single]
    dense_fns = [group_call(c, grp, [pool_dense[grp[0][0]][l]], xs[grp[0][3]][l], ys, dense=True)
                 for l in range(L) for grp in single]
    step_sparse_bytes = L * len(patterns) * sum(sparse_bytes(R, K, B) for _, R, K, _ in projs)
    ms_sparse = time_step(c, sparse_fns, args.steps, args.warmup)
    ms_dense = time_step(c, dense_fns, args.steps, args.warmup)
    log(f"fused step: sparse {ms_fused * 1e3:.1f} us ({len(fused_fns)} launches), dense "
        f"{ms_fused_dense * 1e3:.1f} us ({len(fused_dense_fns)} launches)")
    log(f"step: sparse {ms_sparse * 1e3:.1f} us ({len(sparse_fns)} launches), dense {ms_dense * 1e3:.1f} us "
        f"({len(dense_fns)} launches, {len(patterns)} pattern(s) share it)")

    # ---------------------------------------------------------------- per layer
    per = per_layer_table(c, projs, patterns, pool_sparse, pool_dense, xs, ys, L, B, hipblaslt=True)
    for label, d in per.items():
        log(f"{label}: " + ", ".join(f"{k} {v['us']} us [{v['p10']}-{v['p90']}] ({v['pct_peak']}%, "
                                     f"x{v.get('speedup_vs_dense')})" for k, v in d.items()
                                     if isinstance(v, dict)) + f"; dense {d.get('dense_us')} us")

    # ---------------------------------------------------------------- achievable read
    # What a launch that only streams reaches on the same byte count under the same
    # rotation (nm_stream_read over >= 512 MB of distinct buffers of that size): the rate
    # each launch's % of the 8 TB/s peak is read against.
    stream_t = {}

    def time_stream_read(nbytes):
        nbytes = (int(nbytes) + 15) // 16 * 16
        if nbytes not in stream_t:
            cnt = max(2, math.ceil(ROTATE_BYTES / nbytes))
            g = torch.Generator(device=c.dev)
            g.manual_seed(nbytes)
            bufs = [torch.randint(-(1 << 31), 1 << 31, (nbytes // 4,), dtype=torch.int32, device=c.dev, generator=g)
                    for _ in range(cnt)]
            sink = torch.empty(nm.nm_stream_read_sink_words(nbytes), dtype=torch.int32, device=c.dev)
            stream_t[nbytes] = time_launches(torch, [(lambda b=b: nm.nm_stream_read(b, sink=sink)) for b in bufs])
            del bufs
        return nbytes, stream_t[nbytes]

    first_pat = f"{patterns[0][0]}:{patterns[0][1]}"
    stream_log = []
    for grp in [[pr] for pr in projs] + [grp for grp in groups if len(grp) > 1]:
        label = group_label(grp)
        nbytes, t = time_stream_read(group_bytes(grp, B, False))
        d = per[label]
        d["stream_read"] = dict(t, **rate(nbytes, t), spmv_over_stream_time=round(d[first_pat]["us"] / t["us"], 3))
        stream_log.append(f"{label} {t['us']} us ({d['stream_read']['pct_peak']}%)")
    torch.cuda.synchronize()
    log("stream read of the same bytes (achievable): " + ", ".join(stream_log))
    check = target_check(per, patterns)
    log("per-layer target (>= 70% of peak, >= 1.5x dense): " + ", ".join(
        f"{k} {'pass' if v['pct_ok'] and v['speedup_ok'] else 'FAIL'}"
        + ("" if v.get("pct_reachable_by_plain_read", True) else f" (plain read {v['stream_read_pct_peak']}%)")
        for k, v in check.items()))

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
                    if nm.nm_spmv_plan(R, K, B)["kernel"] == nm.NM_KERNEL_WORD:
                        assert torch.equal(yb.view(torch.int16), ym.view(torch.int16)), f"{key} {name} != bitmask"
                    else:
                        yf, mf = yb.float(), ym.float()
                        assert float((yf - mf).abs().max()) <= 1e-2 * float(yf.abs().max()), f"{key} {name} != bitmask"
                fns = [(lambda mt=mt, v=v, x=xs[group][i % L]:
                        nm.nm_spmv_meta(mt, fmt, v, x, out=ys[name], workspace=ws)) for i, (mt, v) in enumerate(pool)]
                t = time_launches(torch, fns)
                d[key] = dict(t, GBs=rate(nb, t)["GBs"], bytes=nb, slowdown_vs_bitmask=round(t["us"] / bm["us"], 3),
                              rotation_MB=round(len(fns) * nb / 1e6))
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
            for i in range(cnt):
                W = synth.device_weights(R, K, args.seed, 100 + pi, i)
                n = nm.nm_col_norm(synth.device_calib_acts(K, args.seed, 200 + pi, i))
                pool.append(nm.nm_prune_pack_unstructured(W, n))
                if i == 0:
                    # spot check: masks/values bit-exact and the product within tolerance on sampled rows
                    g = np.random.default_rng(args.seed + pi)
                    rows = np.unique(np.concatenate([[0, R - 1], g.choice(R, size=min(R, 6), replace=False)]))
                    ridx = torch.from_numpy(rows).to(c.dev)
                    hu = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)  # noqa: E731
                    nref = oracle.col_norm(hu(synth.device_calib_acts(K, args.seed, 200 + pi, i)))
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
            t = time_launches(torch, fns)
            nmus = per[name][f"{N}:{M}"]["us"]
            unstructured[name] = dict(t, R=R, K=K, **rate(nb_, t), **{f"nm_{N}:{M}_us": nmus},
                                      slowdown_vs_nm=round(t["us"] / nmus, 3),
                                      speedup_vs_dense=round(per[name]["dense_us"] / t["us"], 3),
                                      rotation_MB=round(len(fns) * nb_ / 1e6))
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
    # of it; its algorithmic bytes over its median launch time is the roofline's achieved.
    share = {}
    for grp in groups:
        share[group_label(grp)] = sum(per[group_label(grp)][f"{N}:{M}"]["us"] for (N, M) in patterns)
    dom = max(share, key=share.get)
    dom_grp = next(grp for grp in groups if group_label(grp) == dom)
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
                "avg_launch_us": round(dom_us, 3), "timing": "median of 50 replays of a >= 64-launch graph"}

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

    # ---------------------------------------------------------------- the other workloads
    n_fused, n_unfused = len(fused_fns), len(sparse_fns)
    others = None
    if not args.no_other_configs and args.config == "8b":
        del pool_sparse, pool_dense, fused_fns, fused_dense_fns, sparse_fns, dense_fns
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        others = {}
        for name, layers, batches in OTHER_CONFIGS:
            others[name] = measure_other(c, name, layers, batches, args.steps, args.warmup, args.seed,
                                         not args.skip_check)

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
        "step": {"launches": n_fused,
                 "groups": [group_label(grp) for grp in groups],
                 "bytes": fused_sparse_bytes,
                 "dense_ms": round(ms_fused_dense, 4),
                 "dense_GBs": round(fused_dense_bytes / (ms_fused_dense * 1e-3) / 1e9, 1),
                 "speedup_vs_dense": round(ms_fused_dense * len(patterns) / ms_fused, 3),
                 "launch_sum_vs_best_dense": best_dense_launch_sum(per, projs, patterns)},
        "unfused_step": {"launches": n_unfused, "ms": round(ms_sparse, 4),
                         "bytes": step_sparse_bytes,
                         "GBs": round(step_sparse_bytes / (ms_sparse * 1e-3) / 1e9, 1),
                         "pct_hbm_peak": round(100 * step_sparse_bytes / (ms_sparse * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
                         "dense_ms": round(ms_dense, 4),
                         "speedup_vs_dense": round(ms_dense * len(patterns) / ms_sparse, 3)},
        "per_layer": per,
        "per_layer_target": {"criterion": f">= {TARGET_PCT:.0f}% of the 8 TB/s HBM peak and >= {TARGET_SPEEDUP}x "
                                          "the same-GPU dense GEMV, per launch", "launches": check},
        "configs": others,
        "metadata_formats": meta_table,
        "unstructured_50": unstructured,
        "solver": solver,
        "pack_GBs": round(st["pack_bytes"] / st["pack_ms"] / 1e6, 1),
        "parity": parity,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


COPY_BYTES = 256 << 20


def profile_kernel(args, torch, nm, synth, cfg, dev):
    """The step's dominant launch (gate|up through nm_spmv_swiglu when the layer set has
    them, else the largest single projection), first pattern, rotated over >= 512 MB of
    distinct packed buffers and timed exactly as the per-launch tables time it (printed:
    per-launch µs by HIP events), then one plain device-to-device copy of COPY_BYTES: the
    reference for the counters."""
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

    def launch(packs):
        if glu:
            return lambda: nm.nm_spmv_swiglu(packs[0], packs[1], x, out=y, workspace=ws)
        return lambda: nm.nm_spmv(*packs[0], x, out=y, workspace=ws)

    # the bench's own timing of this launch (one graph of whole passes over the pool,
    # warm-up and timed replays): the dispatches a profiler sees are those of the table
    t = time_launches(torch, [launch(p) for p in pool])
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"profile_kernel": f"{label} {mats}x {R}x{K} {N}:{M} B={B}", "label": label,
                      "per_launch_us_events": t, "copy_bytes": COPY_BYTES}), flush=True)


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
        spmv = [v for (disp, kn, grid, cn), v in per.items()
                if cn == counter and ("spmv_kernel" in kn or "spmv_tile" in kn)]
        # the calibration copy: the runtime's buffer copy, the last dispatch of the command
        # (torch's own elementwise copy kernels, e.g. dtype conversions, do not count)
        copies = [(int(disp), v) for (disp, kn, grid, cn), v in per.items()
                  if cn == counter and "rocclr_copybuffer" in kn.lower()]
        if not spmv or not copies:
            raise SystemExit(f"{counter}: missing spmv ({len(spmv)}) or copy ({len(copies)}) dispatches")
        copy_kib = max(copies)[1]
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
    for f in ("nm_spmv.hip", "nm_spmv_tile.hip", "nm_spmv_common.h", "nm_device.h"):
        with open(os.path.join(ROOT, "bitmask_spmv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
