#!/usr/bin/env python3
"""MoE-layer benchmark on one MI355X.

A step is one forward of the whole layer (q8 of x, router + top-k, gate/up,
SwiGLU, down + routing-weighted combine + shared expert) for one chunk of
synthetic tokens. The headline workload is the Qwen3.6-35B-A3B-shaped decode
layer (H 2048, 256 experts, top-8 softmax + shared expert, F 512, Q4_K, one
token). Steps rotate over layer copies at distinct HBM addresses (the model's
40 layers) and over a pool of 64 inputs, so expert weights come from HBM, not
from the 256 MB Infinity Cache or the L2s.

Headline timed region: exactly K steps, replayed from HIP graphs that hold
whole rotations over the layer copies (the copy a step reads is the least
recently used one), bracketed by synchronizes. Per-kernel durations for the
roofline come from start/stop events that each kernel's dispatch records on
the library's stream (moe_layer_forward_timed). The other workloads (gpt-oss,
DeepSeek-V4-Flash and Kimi-K2 shapes) are timed in the same run as medians of
graph replays and reported under detail.workloads. Measured ceilings: a
non-temporal streaming read over 4 GiB and an int8 MFMA issue loop. The CPU
baseline is the fp64 oracle on a bounded sample of tokens, on one host thread
and on all of them.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, AMD published
I8_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA, AMD published (5.0 POP/s)
FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 MFMA, AMD published (5.0 PFLOP/s)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--workload", default="qwen3.6-35b-a3b")
    p.add_argument("--extra", default="gpt-oss-20b,deepseek-v4-flash,kimi-k2,gpt-oss-20b-t16,"
                                      "gpt-oss-20b-mx8",
                   help="further workloads timed in the same run (comma list; '' for none)")
    p.add_argument("--extra-reps", type=int, default=5, help="graph replays per extra workload")
    p.add_argument("--copies", type=int, default=None, help="layer copies rotated in HBM")
    p.add_argument("--tokens", type=int, default=None,
                   help="tokens per step of the headline workload (default: the workload's)")
    p.add_argument("--x-pool", type=int, default=64)
    p.add_argument("--stage-iters", type=int, default=400)
    p.add_argument("--cpu-baseline", type=int, default=1)
    p.add_argument("--cpu-seconds", type=float, default=8.0,
                   help="target wall time of each CPU-baseline leg")
    p.add_argument("--threads", type=int, default=None)
    p.add_argument("--probes", type=int, default=1, help="measure the read wall and MFMA peak")
    p.add_argument("--pool-layers", type=int, default=8,
                   help="layers of the expert-pool decode leg (0: skip it)")
    p.add_argument("--pool-frac", type=float, default=0.25,
                   help="device slots of the pool leg as a fraction of its experts")
    p.add_argument("--pool-steps", type=int, default=96)
    p.add_argument("--pool-warmup", type=int, default=96)
    p.add_argument("--wall-gib", type=int, default=4)
    p.add_argument("--crossover", default="",
                   help="comma list of workloads: time each on both expert-FFN paths at "
                        "--crossover-tokens chunk sizes (reported under detail.crossover)")
    p.add_argument("--crossover-tokens", default="1,2,3,4,6,8,12,16")
    p.add_argument("--layout", default="auto", choices=("auto", "rows", "tile64", "mx16"),
                   help="order of the expert blocks on the device: auto = MX16 rows for "
                        "MXFP4 layers on the per-pair path, 64-row tiles for layers that take "
                        "the grouped path at every chunk size (an expert of 8 MB or more), row "
                        "order otherwise")
    p.add_argument("--calib-copy-mb", type=int, default=0,
                   help="run a plain device copy of this many MiB (counter calibration)")
    return p.parse_args()


DEFAULT_COPIES = {"tiny": 1, "qwen3.6-35b-a3b": 40, "gpt-oss-20b": 24, "deepseek-v4-flash": 4,
                  "kimi-k2": 2, "qwen3.6-35b-a3b-q5k": 40, "qwen3.6-35b-a3b-q2k": 40,
                  "gpt-oss-20b-t16": 8, "gpt-oss-20b-mx8": 8}


def rotation(copies: int) -> int:
    """Forwards per graph: whole rotations over the copies, at least 64."""
    return copies * ((64 + copies - 1) // copies)


# ------------------------------------------------------------------ probes
def measure_probes(M, torch, wall_gib: int):
    """Streaming read wall (GB/s) and int8 MFMA rates (TOPS) on this GPU."""
    out = {}
    stream = torch.cuda.Stream()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    nbytes = wall_gib << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    best = 0.0
    per = {}
    for nwg in (2048, 4096, 8192):
        ts = []
        for _ in range(6):
            a, b = M.HipEvent(), M.HipEvent()
            a.record(stream)
            M.moe_probe_read_wall(buf, nbytes, nwg, sink, stream)
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_ms(b))
        ts = sorted(ts[1:])
        gbs = nbytes / (ts[len(ts) // 2] * 1e-3) / 1e9
        per[nwg] = round(gbs, 1)
        best = max(best, gbs)
    out["read_wall_GBps"] = round(best, 1)
    out["read_wall_detail"] = {"bytes": nbytes, "GBps_by_workgroups": per,
                               "kernel": "k_read_wall (non-temporal dwordx4, 8 in flight/lane)"}
    del buf
    # launch-chain floor: per forward of n empty kernels, replayed from a graph
    # of 64 forwards as the layer timing is (n = the layer call's kernels)
    chain = {}
    s = torch.cuda.Stream()
    for n in (3, 4, 7):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for _ in range(64):
                M.moe_probe_empty_chain(n, s)
        ts = []
        with torch.cuda.stream(s):
            g.replay()
            for _ in range(6):
                a, b = M.HipEvent(), M.HipEvent()
                a.record(s)
                g.replay()
                b.record(s)
                b.synchronize()
                ts.append(a.elapsed_ms(b) * 1e3 / 64)
        ts = sorted(ts[1:])
        chain[str(n)] = round(ts[len(ts) // 2], 3)
        del g
    out["empty_chain_us_per_forward"] = chain
    for k64, name in ((0, "mfma_i32_16x16x32_i8"), (1, "mfma_i32_16x16x64_i8")):
        nwg, iters = 2048, 400
        ops = nwg * 4 * iters * 8 * 16 * 16 * (64 if k64 else 32) * 2
        ts = []
        for _ in range(5):
            a, b = M.HipEvent(), M.HipEvent()
            a.record(stream)
            M.moe_probe_mfma_i8(k64, iters, nwg, sink, stream)
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_ms(b))
        ts = sorted(ts[1:])
        out[f"{name}_TOPS"] = round(ops / (ts[len(ts) // 2] * 1e-3) / 1e12, 1)
    torch.cuda.synchronize()
    return out


# --------------------------------------------------------------- workloads
def pick_layout(args, cfg) -> int:
    """moe_layout of a workload's expert matrices (see --layout)."""
    import gen
    if args.layout == "rows":
        return 0
    tiles_ok = (cfg.fmt_gu == gen.Q4_K and cfg.fmt_d in (gen.Q4_K, gen.Q6_K) and not cfg.biases
                and not cfg.act_quant)
    # MX16: MXFP4 rows with aligned nibble fields, for the per-pair MXFP4 kernels
    mx16_ok = (cfg.fmt_gu == gen.MXFP4 and cfg.fmt_d == gen.MXFP4 and not cfg.act_quant
               and cfg.H <= 32 * 256 and cfg.F <= 32 * 256)
    if args.layout == "tile64":
        return 1 if tiles_ok else 0
    if args.layout == "mx16":
        return 2 if mx16_ok else 0
    if mx16_ok:
        return 2
    return 1 if tiles_ok and cfg.expert_algo_bytes >= 8e6 else 0


def run_workload(args, name: str, headline: bool, probes: dict, th: int):
    import numpy as np
    import torch

    import gen
    import quantized_moe_expert_route_amd as M
    from gen.device import DeviceLayer, x_to_device

    cfg = gen.CONFIGS[name]
    if headline and args.tokens:
        cfg = cfg.with_(T=args.tokens, description=f"{cfg.description}; {args.tokens}-token chunk")
    copies = (args.copies if headline and args.copies else None) or DEFAULT_COPIES[name]
    cfg = cfg.with_(layout=pick_layout(args, cfg))
    t0 = time.time()
    data = gen.make_layer(cfg, threads=th)
    dl = DeviceLayer(data, copies=copies)
    T = cfg.T
    xs = []
    for i in range(args.x_pool):
        x, xb = gen.make_x(cfg, T=T, x_index=i)
        xs.append(x_to_device(data, x, xb)[0])
    dtype = M.MOE_DTYPE_BF16 if cfg.x_bf16 else M.MOE_DTYPE_F32
    ws = dl.workspace(T)
    y = torch.empty((T, cfg.H), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
    setup_s = time.time() - t0

    def fwd(i, stream=None):
        M.moe_layer_forward(dl.descs[i % copies], xs[i % args.x_pool], dtype, T, y, ids, w, ws,
                            ws.numel(), stream)

    stream = torch.cuda.Stream()
    warm = args.warmup if headline else min(args.warmup, 2 * rotation(copies))
    with torch.cuda.stream(stream):
        for i in range(warm):
            fwd(i)
    torch.cuda.synchronize()

    G = rotation(copies)

    def graph_of(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for j in range(n):
                fwd(j)
        return g

    full = graph_of(G)
    for _ in range(2):
        full.replay()
    torch.cuda.synchronize()
    res = {"workload": cfg.description, "tokens_per_step": T, "layer_copies": copies,
           "x_pool": args.x_pool, "forwards_per_graph": G,
           "expert_layout": ("rows", "tile64", "mx16")[cfg.layout]}
    if headline:
        # exactly K steps: whole rotations, then the first K mod G forwards of
        # one (their copies are the least recently used ones at that point)
        K = args.steps
        tail = graph_of(K % G) if K % G else None
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for _ in range(K // G):
            full.replay()
        if tail is not None:
            tail.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_start
        res["ms_per_step"] = elapsed * 1e3 / K
        res["tokens_per_s"] = T * K / elapsed
        res["steps_timed"] = K
        res["copies_touched"] = min(copies, K)
    else:
        per = []
        with torch.cuda.stream(stream):  # replay() launches on the current stream
            for _ in range(args.extra_reps):
                a, b = M.HipEvent(), M.HipEvent()
                a.record(stream)
                full.replay()
                b.record(stream)
                b.synchronize()
                per.append(a.elapsed_ms(b) / G)
        med = float(np.median(per))
        res["ms_per_step"] = med
        res["tokens_per_s"] = T / (med * 1e-3)
        res["timing"] = f"median of {args.extra_reps} replays of a {G}-forward graph"
    del full

    # per-kernel durations: start/stop events recorded by each kernel's dispatch
    n_st = M.moe_layer_stage_count(dl.desc, T)
    names = [M.moe_layer_stage_name(dl.desc, T, i) for i in range(n_st)]
    R = args.stage_iters if headline else max(32, min(args.stage_iters, 4 * G))
    evs = [[M.HipEvent() for _ in range(2 * n_st)] for _ in range(R)]
    with torch.cuda.stream(stream):
        for i in range(R):
            M.moe_layer_forward_timed(dl.descs[i % copies], xs[i % args.x_pool], dtype, T, y, ids,
                                      w, ws, ws.numel(), stream, [e.handle for e in evs[i]])
    torch.cuda.synchronize()
    stage_ms = np.zeros((R, n_st))
    for i in range(R):
        for s in range(n_st):
            stage_ms[i, s] = evs[i][2 * s].elapsed_ms(evs[i][2 * s + 1])
    skip = min(20, R // 4)
    stage_avg_us = {names[s]: float(stage_ms[skip:, s].mean() * 1e3) for s in range(n_st)}

    # realized routing of the pool inputs on copy 0: unique experts per step
    realized = []
    for i in range(args.x_pool):
        M.moe_layer_forward(dl.descs[0], xs[i], dtype, T, y, ids, w, ws, ws.numel())
        torch.cuda.synchronize()
        realized.append(ids.cpu().numpy().copy())
    uniq = [len(np.unique(r)) + (1 if cfg.shared else 0) for r in realized]
    uniq_mean = float(np.mean(uniq))
    sel_bytes = uniq_mean * cfg.expert_algo_bytes
    path = ("grouped_mx" if cfg.act_quant else "grouped") if n_st == 7 else "gemv"
    algo = algo_bytes(cfg, path, uniq_mean)
    kn = kernel_names(cfg, path)
    dom = max(("gateup", "down"), key=lambda k: stage_avg_us.get(k, 0.0))
    dom_us = stage_avg_us[dom]
    expert_us = stage_avg_us.get("gateup", 0) + stage_avg_us.get("down", 0)
    achieved = algo[dom] / (dom_us * 1e-6) / 1e9
    wall = probes.get("read_wall_GBps")
    roof = {
        "kernel": kn[dom],
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": _traffic_for(kn[dom], name, path),
        "measured_wall": wall,
        "frac_of_measured_wall": round(achieved / wall, 4) if wall else None,
        # the same number of empty kernels, replayed the same way: the time a
        # forward of this schedule cannot go below whatever the kernels do
        "launch_chain_floor_us": probes.get("empty_chain_us_per_forward", {}).get(str(n_st)),
        "algo_bytes_per_launch": round(algo[dom]),
        "avg_launch_us": round(dom_us, 3),
    }
    res.update({
        "path": path,
        "roofline": roof,
        "selected_expert_bytes_per_step": round(sel_bytes),
        "unique_experts_per_step": uniq_mean,
        "layer_GBps_selected_experts": round(sel_bytes / (res["ms_per_step"] * 1e-3) / 1e9, 1),
        "layer_hbm_frac": round(sel_bytes / (res["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "expert_kernels_us": round(expert_us, 3),
        "expert_GBps": round(sel_bytes / (expert_us * 1e-6) / 1e9, 1) if expert_us else None,
        "kernel_source_hash": kernel_source_hash(path),
        "stage_avg_us": {k: round(v, 3) for k, v in stage_avg_us.items()},
        "setup_s": round(setup_s, 1),
    })
    for k in ("gateup", "down"):
        res[f"{k}_GBps"] = round(algo[k] / (stage_avg_us[k] * 1e-6) / 1e9, 1)
        res[f"{k}_kernel"] = kn[k]
    if path in ("grouped", "grouped_mx"):
        # routed tokens per active expert in a chunk (realized histogram)
        cnt = np.concatenate([np.bincount(r.ravel(), minlength=cfg.E) for r in realized])
        act = cnt[cnt > 0]
        res["tokens_per_active_expert"] = {
            "mean": round(float(act.mean()), 2), "max": int(act.max()),
            "hist_1_2_3_4-7_8-15_16+": [int((act == 1).sum()), int((act == 2).sum()),
                                        int((act == 3).sum()),
                                        int(((act >= 4) & (act < 8)).sum()),
                                        int(((act >= 8) & (act < 16)).sum()),
                                        int((act >= 16).sum())]}
        # MFMA work of the tile kernels: 2 H F per routed (token, slot) pair
        # and matrix (algorithmic; padded tile rows are not counted). int8 MFMA
        # on the q8 path; block-scaled fp8 x fp4 MFMA (priced at the dense fp8
        # peak) on the MX path
        P = T * cfg.k + (T if cfg.shared else 0)
        ops = {"gateup": P * 2 * 2 * cfg.H * cfg.F, "down": P * 2 * cfg.H * cfg.F}
        peak = FP8_PEAK_TFLOPS if path == "grouped_mx" else I8_PEAK_TOPS
        mf = {}
        for k in ("gateup", "down"):
            tops = ops[k] / (stage_avg_us[k] * 1e-6) / 1e12
            mf[k] = {"kernel": kn[k], "ops_per_launch": ops[k], "achieved_T_per_s": round(tops, 1),
                     "frac_of_peak": round(tops / peak, 4)}
        res["mfma"] = {"op": "f8f6f4 block-scaled" if path == "grouped_mx" else "int8",
                       "peak_T_per_s": peak,
                       "measured_int8_TOPS_16x16x32": probes.get("mfma_i32_16x16x32_i8_TOPS"),
                       "measured_int8_TOPS_16x16x64": probes.get("mfma_i32_16x16x64_i8_TOPS"),
                       **mf}
    keep = (data, cfg)
    del dl, xs, ws, y, ids, w, evs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, keep


def crossover(args, name: str, th: int) -> dict:
    """Per-forward time of one workload on the per-pair GEMV path and on the
    expert-grouped path (forced through the descriptor's path field) at several
    chunk sizes, and the path the automatic rule picks."""
    import numpy as np
    import torch

    import gen
    import quantized_moe_expert_route_amd as M
    from gen.device import DeviceLayer, x_to_device

    cfg0 = gen.CONFIGS[name]
    copies = min(DEFAULT_COPIES[name], 24)
    data = gen.make_layer(cfg0, threads=th)
    dl = DeviceLayer(data, copies=copies)
    out = {}
    for T in [int(v) for v in args.crossover_tokens.split(",") if v]:
        cfg = cfg0.with_(T=T)
        xs = [x_to_device(data, *gen.make_x(cfg, T=T, x_index=i))[0] for i in range(16)]
        dt = M.MOE_DTYPE_BF16 if cfg.x_bf16 else M.MOE_DTYPE_F32
        y = torch.empty((T, cfg.H), dtype=torch.float32, device="cuda")
        ids = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
        row = {}
        for pname, path in (("auto", M.MOE_PATH_AUTO), ("gemv", M.MOE_PATH_GEMV),
                            ("grouped", M.MOE_PATH_GROUPED)):
            for d in dl.descs:
                d.path = path
            if pname == "auto":
                row["auto_path"] = "grouped" if M.moe_layer_stage_count(dl.desc, T) == 7 else "gemv"
                continue
            ws = dl.workspace(T)
            s = torch.cuda.Stream()
            G = rotation(copies)

            def fwd(i):
                M.moe_layer_forward(dl.descs[i % copies], xs[i % 16], dt, T, y, ids, w, ws,
                                    ws.numel(), s)

            with torch.cuda.stream(s):
                for i in range(G):
                    fwd(i)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for i in range(G):
                    fwd(i)
            per = []
            with torch.cuda.stream(s):
                g.replay()
                for _ in range(5):
                    a, b = M.HipEvent(), M.HipEvent()
                    a.record(s)
                    g.replay()
                    b.record(s)
                    b.synchronize()
                    per.append(a.elapsed_ms(b) * 1e3 / G)
            row[f"{pname}_us"] = round(float(np.median(per)), 2)
            del g, ws
        out[T] = row
    for d in dl.descs:
        d.path = M.MOE_PATH_AUTO
    del dl
    torch.cuda.empty_cache()
    return {"workload": cfg0.description, "layer_copies": copies, "per_forward": out}


def pool_leg(args, th: int) -> dict:
    """A decode stack larger than its device arena: L Qwen3.6-shaped layers
    (own routers, Zipf(1.1) selection skew, one set of expert bytes reused by
    every layer) whose routed experts live in the pool's pinned host tier; the
    arena holds a fraction of them. Per step and layer: moe_pool_layer_step
    (route, ids to the host, resolve, optional prefetch of the next layer's
    predicted experts, quantize, expert FFN), then x += y. Compared with the same
    stack fully resident (moe_layer_forward per layer, no host round trip), and
    with an arena that holds every expert (the round-trip cost alone)."""
    import ctypes as C

    import torch

    import gen
    import quantized_moe_expert_route_amd as M
    from gen.device import DeviceLayer

    L = args.pool_layers
    cfg = gen.CONFIGS["qwen3.6-35b-a3b"].with_(zipf_s=1.1, T=1)
    t0 = time.time()
    data0 = gen.make_layer(cfg, threads=th)
    layers = []
    for l in range(L):
        r = data0 if l == 0 else gen.make_layer(cfg.with_(seed=cfg.seed + 97 * l), experts=[])
        layers.append(gen.LayerData(cfg, r.w_router, r.sel_bias, data0.pool, None, None, None,
                                    data0.x, None))
    dls = [DeviceLayer(d) for d in layers]
    del layers
    E, k, H = cfg.E, cfg.k, cfg.H
    n_trans = 64
    state = {}

    def new_pool(n_slots):
        pool = M.Pool(L, E, cfg.expert_bytes, cfg.gate_bytes, 2 * cfg.gate_bytes, n_slots, n_trans)
        for l in range(L):
            for e in range(E):
                pool.host_slab(l, e)[:] = data0.pool[e]
        descs = []
        for l, dl in enumerate(dls):
            d = M.MoeLayerDesc()
            C.pointer(d)[0] = dl.desc
            d.gate, d.up, d.down = pool.tables(l)
            descs.append(d)
        state["pool"], state["descs"] = pool, descs
        return pool

    setup_s = time.time() - t0
    T = 1
    stream = torch.cuda.Stream()
    ws_n = max(M.moe_pool_step_workspace(dl.desc, T) for dl in dls)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    xs = [torch.from_numpy(gen.make_x(cfg, T=T, x_index=i)[0]).cuda() for i in range(256)]

    def step_resident(x):
        for l in range(L):
            M.moe_layer_forward(dls[l].desc, x, M.MOE_DTYPE_F32, T, y, ids, w, ws, ws_n, stream)
            x = x + y
        return x

    def step_pool(x, prefetch):
        pool, descs = state["pool"], state["descs"]
        for l in range(L):
            nd = descs[l + 1] if prefetch and l + 1 < L else None
            pool.layer_step(l, descs[l], nd, x, M.MOE_DTYPE_F32, T, ids, w, y, ws, ws_n, stream)
            x = x + y
        return x

    W = args.pool_warmup

    def timed(fn, steps, pool):
        # warm-up steps fill the hot set; the timed ones use inputs not seen in it
        with torch.cuda.stream(stream):
            for i in range(W):
                fn(xs[i % len(xs)])
            torch.cuda.synchronize()
            st0 = pool.stats() if pool else None
            t = time.perf_counter()
            for i in range(steps):
                fn(xs[(W + i) % len(xs)])
            torch.cuda.synchronize()
            dt = time.perf_counter() - t
        if not pool:
            return dt, None
        st1 = pool.stats()
        return dt, {kk: st1[kk] - st0[kk] for kk in st1}

    S = args.pool_steps
    res = {"workload": f"{L}-layer stack of {cfg.description}, Zipf(1.1) selection skew, "
                       f"decode (1 token), 256 distinct inputs",
           "layers": L, "experts_total": L * E, "expert_bytes": cfg.expert_algo_bytes,
           "host_tier_GB": round(L * E * cfg.expert_bytes / 1e9, 2),
           "transient_slots": n_trans, "steps": S, "warmup_steps": W,
           "setup_s": round(setup_s, 1),
           "step": "moe_pool_layer_step per layer (route, ids to host, resolve, optional "
                   "next-layer prefetch, quantize, expert FFN), then x += y"}
    dt, _ = timed(step_resident, S, None)
    res["resident_tokens_per_s"] = round(S / dt, 1)
    res["resident_us_per_layer"] = round(dt / (S * L) * 1e6, 2)
    for name, frac, pf in (("pool_all_fit", 1.0, False), ("pool", args.pool_frac, False),
                           ("pool_prefetch", args.pool_frac, True)):
        slots = L * E + n_trans if frac >= 1.0 else max(n_trans + 8, int(frac * L * E))
        pool = new_pool(slots)
        dt, st = timed(lambda x: step_pool(x, pf), S, pool)
        req = max(1, st["requests"])
        res[name] = {
            "arena_slots": slots, "arena_frac": round(slots / (L * E), 3),
            "tokens_per_s": round(S / dt, 1),
            "us_per_layer": round(dt / (S * L) * 1e6, 2),
            "hit_rate": round((st["hits_resident"] + st["hits_transient"]) / req, 4),
            "h2d_GB_per_s": round(st["bytes_h2d"] / dt / 1e9, 2),
            "h2d_bytes_per_token": round(st["bytes_h2d"] / S),
            "stats": st,
        }
        pool.close()
        state.clear()
    del dls, ws
    torch.cuda.empty_cache()
    return res


def cpu_model() -> str:
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(args, data, cfg, th: int):
    """The oracle, unchanged, on a bounded sample of tokens of the workload:
    one host thread, then all of them."""
    import numpy as np

    import gen
    import oracle

    L = oracle.Layer(data)
    T = cfg.T
    tok_s = _oracle_token_s(cfg)

    def sample(n):
        return np.concatenate([gen.make_x(cfg, T=T, x_index=i)[0]
                               for i in range((n + T - 1) // T)])[:n]

    n1 = max(4, int(args.cpu_seconds / tok_s))
    x1 = sample(n1)
    t = time.perf_counter()
    ref = L.forward(x1, threads=1)
    s1 = time.perf_counter() - t
    parity = parity_vs_oracle(data, cfg, x1, ref)
    nn = max(16, int(args.cpu_seconds * th / tok_s))
    xn = sample(nn)
    t = time.perf_counter()
    L.forward(xn, threads=th)
    sn = time.perf_counter() - t
    return {"value": round(nn / sn, 2), "unit": "tokens/s", "cores": th, "kind": "oracle",
            "sample": f"{nn} tokens of the same workload (x pool members), whole layer per token, "
                      f"fp64 oracle on {th} host threads, {sn:.1f} s wall; and {n1} tokens on one "
                      f"thread, {s1:.1f} s",
            "single_thread_value": round(n1 / s1, 2),
            "nproc": os.cpu_count(), "threads_available": th, "cpu_model": cpu_model(),
            "parity": parity}


def parity_vs_oracle(data, cfg, x, ref):
    """The single-thread sample's tokens through the library (chunks of the
    workload's T on one layer copy, the benchmark's path and expert order)
    against the oracle's outputs for them: q8 of x bitwise, expert ids exact,
    routing weights and per-token max |dy| / ||y_ref||."""
    import numpy as np
    import torch

    import gen
    import quantized_moe_expert_route_amd as M
    from gen.device import DeviceLayer, x_to_device

    dl = DeviceLayer(data)
    T = cfg.T
    n = (x.shape[0] // T) * T
    if n == 0:
        return None
    ys, idss, ws_ = [], [], []
    y = torch.empty((T, cfg.H), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
    wsp = dl.workspace(T)
    for t0 in range(0, n, T):
        xc = np.ascontiguousarray(x[t0:t0 + T])
        xt, dt = x_to_device(data, xc, gen.round_bf16(xc) if cfg.x_bf16 else None)
        M.moe_layer_forward(dl.desc, xt, dt, T, y, ids, w, wsp, wsp.numel())
        torch.cuda.synchronize()
        ys.append(y.cpu().numpy().copy())
        idss.append(ids.cpu().numpy().copy())
        ws_.append(w.cpu().numpy().copy())
    yg, ig, wg = np.concatenate(ys), np.concatenate(idss), np.concatenate(ws_)
    yr = ref["y"][:n]
    # q8 of x (the q8 format the gate/up rows consume; MXFP8 layers have their
    # own quantizer): the library's quantizer against the oracle's, bitwise
    q8_exact = None
    if not cfg.act_quant:
        import oracle
        B = gen.BLOCK_ELEMS[cfg.fmt_gu]
        afmt = M.MOE_AFMT_Q8_K if B == 256 else M.MOE_AFMT_Q8_32
        H = cfg.H
        qs = torch.empty((n, H), dtype=torch.int8, device="cuda")
        qd = torch.empty((n, H // B), dtype=torch.float32, device="cuda")
        qb = torch.empty((n, H // 16), dtype=torch.int16, device="cuda")
        xin = np.ascontiguousarray(x[:n])
        xt, dt = x_to_device(data, xin, gen.round_bf16(xin) if cfg.x_bf16 else None)
        M.moe_quantize_act_q8k(xt, dt, n, H, afmt, M.qact(qs, qd, qb if B == 256 else None, afmt, n, H))
        torch.cuda.synchronize()
        gq, gd, gb = qs.cpu().numpy(), qd.cpu().numpy(), qb.cpu().numpy()
        q8_exact = True
        for t in range(n):
            a, b, c = oracle.quantize_q8(xin[t], B)
            q8_exact &= bool(np.array_equal(gq[t], a) and np.array_equal(gd[t].view(np.uint32), b.view(np.uint32))
                             and (c is None or np.array_equal(gb[t], c)))
    err = np.abs(yg.astype(np.float64) - yr).max(axis=1) / np.maximum(np.linalg.norm(yr, axis=1), 1e-30)
    return {"tokens": int(n), "q8_x_bitexact": q8_exact,
            "ids_exact": bool(np.array_equal(ig, ref["ids"][:n])),
            "w_max_abs_err": float(np.abs(wg - ref["w"][:n]).max()),
            "y_max_rel_err": float(err.max()), "y_tolerance": 2e-3,
            "pass": bool(np.array_equal(ig, ref["ids"][:n]) and err.max() <= 2e-3)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU; --gpus {args.gpus} is not supported "
              "(expert-parallel sharding over several GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)
    import torch

    import gen
    import quantized_moe_expert_route_amd as M

    torch.cuda.set_device(0)
    th = args.threads or gen.default_threads()
    if args.calib_copy_mb:
        # fp32 -> fp16 conversion: reads 4 B and writes 2 B per element (known traffic)
        n = (args.calib_copy_mb << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty(n, dtype=torch.float16, device="cuda")
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    probes = measure_probes(M, torch, args.wall_gib) if args.probes else {}
    head, (data, cfg) = run_workload(args, args.workload, True, probes, th)
    cpu = cpu_baseline(args, data, cfg, th) if args.cpu_baseline else None
    del data
    extras = {}
    for name in [n for n in args.extra.split(",") if n and n != args.workload]:
        r, _ = run_workload(args, name, False, probes, th)
        extras[name] = r
    xover = {n: crossover(args, n, th) for n in args.crossover.split(",") if n}
    pool = pool_leg(args, th) if args.pool_layers > 0 else None
    out = {
        "metric": "MoE-layer decode tokens/s and achieved HBM GB/s (% of peak), 1 MI355X",
        "value": round(head["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {
            "workload": head["workload"],
            "tokens_per_step": head["tokens_per_step"],
            "layer_copies": head["layer_copies"],
            "x_pool": head["x_pool"],
            "path": head["path"],
            "expert_layout": head["expert_layout"],
        },
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "detail": {
            **{k: v for k, v in head.items() if k not in (
                "workload", "tokens_per_step", "layer_copies", "x_pool", "path", "expert_layout",
                "roofline",
                "tokens_per_s", "ms_per_step")},
            "probes": probes,
            **({"crossover": xover} if xover else {}),
            **({"expert_pool": pool} if pool else {}),
            "workloads": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv)
                              for kk, vv in v.items()} for k, v in extras.items()},
        },
    }
    print(json.dumps(out), flush=True)


def algo_bytes(cfg, path: str, unique_experts: float) -> dict:
    """Algorithmic bytes per launch of the two expert kernels and the router. The
    per-pair path streams every (token, slot) pair's expert rows (T k + shared
    pairs); the grouped path each selected expert's rows once (unique experts
    + shared). Padding bytes of a row are not counted. The router reads W_r and
    x."""
    pairs = cfg.T * cfg.k + (cfg.T if cfg.shared else 0)
    units = unique_experts if path in ("grouped", "grouped_mx") else pairs
    return {
        "gateup": units * 2 * cfg.F * gen_row_bytes(cfg.fmt_gu, cfg.H),
        "down": units * cfg.H * gen_row_bytes(cfg.fmt_d, cfg.F),
        # router weights and the activations they are dotted with
        "router": 4 * cfg.E * cfg.H + (2 if cfg.x_bf16 else 4) * cfg.T * cfg.H,
    }


def gen_row_bytes(fmt, K):
    import gen
    return gen.row_bytes(fmt, K)


def kernel_names(cfg, path: str) -> dict:
    """Kernel (as rocprofv3 names it) of each stage of a layer forward (MXFP4
    layers: the per-pair MXFP4 kernels, whose LDS budget every workload here
    fits; rows in either order)."""
    import gen
    if path == "gemv":
        mx = gen.MXFP4
        gu = "k_gateup_mx" if cfg.fmt_gu == mx else "k_gateup"
        if cfg.fmt_d in (gen.Q4_K, gen.Q5_K, gen.Q2_K):  # rows staged through LDS
            dn = "k_down_lds"
        else:
            dn = "k_down_mx" if cfg.fmt_d == mx else "k_down"
        return {"router": "k_router", "gateup": gu, "down": dn}
    rt = "k_router_mfma22" if cfg.T > 16 and cfg.E + 1 > 16 else "k_router_mfma"  # 2 x 2 blocked
    if path == "grouped_mx":
        return {"router": rt, "gateup": "k_gmx<0>", "down": "k_gmx<1>"}
    nb = cfg.biases
    gu = "k_glds_q4k<0>" if cfg.fmt_gu == gen.Q4_K and not nb else "k_gu_grouped"
    if cfg.fmt_d == gen.Q4_K and not nb:
        dn = "k_glds_q4k<1>"
    elif cfg.fmt_d == gen.Q6_K and not nb:
        dn = "k_glds_q6k_down"
    else:
        dn = "k_down_grouped"
    return {"router": rt, "gateup": gu, "down": dn}


_PATH_SOURCES = {
    "gemv": ("moe_kernels.hip", "moe_device.h", "moe_internal.h"),
    "grouped": ("moe_grouped.hip", "moe_device.h", "moe_internal.h"),
    "grouped_mx": ("moe_mx.hip", "moe_grouped.hip", "moe_device.h", "moe_internal.h"),
}


def kernel_source_hash(path: str) -> str:
    """Hash of the kernel sources of one path (a committed counter measurement
    stays valid while they are unchanged)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_moe_expert_route_amd", "csrc")
    for n in _PATH_SOURCES[path]:
        h.update(open(os.path.join(csrc, n), "rb").read())
    return h.hexdigest()[:16]


def _traffic_for(kernel: str, workload: str, path: str):
    """HBM bytes per launch from the committed PMC summary, if it was taken on
    the current kernel sources of the path (else null)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(p))
    except Exception:
        return None
    ent = rec.get("kernels", {}).get(f"{workload}:{kernel}")
    if ent is None or ent.get("source_hash") != kernel_source_hash(path):
        return None
    return ent.get("hbm_bytes_per_launch")


def _oracle_token_s(cfg) -> float:
    """Rough single-thread oracle seconds per token (measured: ~1.1 ns per weight
    for K-quants, ~16 ns for MXFP4); sizes the CPU sample."""
    macs = (cfg.k + (1 if cfg.shared else 0)) * 3 * cfg.H * cfg.F
    ns_per_mac = 16.0 if cfg.fmt_gu == 2 else 1.1
    return macs * ns_per_mac * 1e-9


if __name__ == "__main__":
    main()
