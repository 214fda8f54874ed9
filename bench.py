#!/usr/bin/env python3
"""MoE-layer decode benchmark on one MI355X.

A step is one forward of the whole layer (q8 of x, router + top-k, gate/up,
SwiGLU, down + routing-weighted combine + shared expert) for one chunk of
synthetic tokens. The default workload is the Qwen3.6-35B-A3B-shaped decode
layer (H 2048, 256 experts, top-8 softmax + shared expert, F 512, Q4_K, one
token). Steps rotate over layer copies at distinct HBM addresses (the model's
40 layers) and over a pool of 64 inputs, so expert weights come from HBM, not
from the 256 MB Infinity Cache or the L2s.

Timed region: K steps replayed from a HIP graph, bracketed by synchronizes.
Per-kernel durations for the roofline come from HIP events recorded between
the layer's kernels on the library's stream (moe_layer_forward_timed).
The CPU baseline is the fp64 oracle on a bounded sample of tokens.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--workload", default="qwen3.6-35b-a3b")
    p.add_argument("--copies", type=int, default=None, help="layer copies rotated in HBM")
    p.add_argument("--x-pool", type=int, default=64)
    p.add_argument("--stage-iters", type=int, default=400)
    p.add_argument("--cpu-baseline", type=int, default=1)
    p.add_argument("--cpu-tokens", type=int, default=None)
    p.add_argument("--threads", type=int, default=None)
    p.add_argument("--calib-copy-mb", type=int, default=0,
                   help="run a plain device copy of this many MiB (counter calibration)")
    return p.parse_args()


DEFAULT_COPIES = {"tiny": 1, "qwen3.6-35b-a3b": 40, "gpt-oss-20b": 24, "deepseek-v4-flash": 4,
                  "kimi-k2": 2, "qwen3.6-35b-a3b-q5k": 40, "qwen3.6-35b-a3b-q2k": 40}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU; --gpus {args.gpus} is not supported "
              "(expert-parallel sharding over several GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import gen
    import quantized_moe_expert_route_amd as M
    from gen.device import DeviceLayer, x_to_device

    torch.cuda.set_device(0)
    cfg = gen.CONFIGS[args.workload]
    th = args.threads or gen.default_threads()
    copies = args.copies or DEFAULT_COPIES[args.workload]
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
    if args.calib_copy_mb:
        # fp32 -> fp16 conversion: reads 4 B and writes 2 B per element (known traffic)
        n = (args.calib_copy_mb << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty(n, dtype=torch.float16, device="cuda")
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # ---- warmup (eager) and realized routing per copy
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            fwd(i)
    torch.cuda.synchronize()

    # ---- graph of G forwards; K steps = (K // G) replays + a tail graph
    K = args.steps
    G = min(K, max(copies, 64))
    graphs = {}

    def graph_of(n, start):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for j in range(n):
                fwd(start + j)
        return g

    graphs["full"] = graph_of(G, 0)
    tail = K % G
    if tail:
        graphs["tail"] = graph_of(tail, 0)
    for _ in range(2):
        graphs["full"].replay()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(K // G):
        graphs["full"].replay()
    if tail:
        graphs["tail"].replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / K
    tokens_per_s = T * K / elapsed

    # ---- per-kernel durations: start/stop events recorded by each kernel's dispatch
    n_st = M.moe_layer_stage_count(dl.desc, T)
    names = [M.moe_layer_stage_name(dl.desc, T, i) for i in range(n_st)]
    R = args.stage_iters
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

    # ---- bytes: selected experts (realized routing of the pool inputs on copy 0)
    realized = []
    for i in range(args.x_pool):
        M.moe_layer_forward(dl.descs[0], xs[i], dtype, T, y, ids, w, ws, ws.numel())
        torch.cuda.synchronize()
        realized.append(ids.cpu().numpy().copy())
    uniq = [len(np.unique(r)) + (1 if cfg.shared else 0) for r in realized]
    uniq_mean = float(np.mean(uniq))
    sel_bytes = uniq_mean * cfg.expert_algo_bytes
    path = "grouped" if n_st == 7 else "gemv"
    algo = algo_bytes(cfg, path, uniq_mean)
    kern_names = kernel_names(cfg, path)
    dom = max(("gateup", "down"), key=lambda k: stage_avg_us.get(k, 0.0))
    dom_us = stage_avg_us[dom]
    expert_us = stage_avg_us.get("gateup", 0) + stage_avg_us.get("down", 0)
    achieved = algo[dom] / (dom_us * 1e-6) / 1e9
    traffic = _traffic_for(kern_names[dom], args.workload, path)
    roofline = {
        "kernel": kern_names[dom],
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "algo_bytes_per_launch": round(algo[dom]),
        "avg_launch_us": round(dom_us, 3),
    }

    # ---- CPU baseline: the oracle on a bounded sample of tokens
    cpu = None
    if args.cpu_baseline:
        import oracle
        L = oracle.Layer(data)
        n_tok = args.cpu_tokens or max(16, min(1024, int(20.0 / _oracle_token_s(cfg))))
        xs_np = np.concatenate([gen.make_x(cfg, T=T, x_index=i)[0] for i in range(
            (n_tok + T - 1) // T)])[:n_tok]
        t1 = time.perf_counter()
        L.forward(xs_np, threads=th)
        cpu_s = time.perf_counter() - t1
        cpu = {"value": round(n_tok / cpu_s, 2), "unit": "tokens/s", "cores": th, "kind": "oracle",
               "sample": f"{n_tok} tokens of the same workload (x pool members), whole layer per "
                         f"token, fp64 oracle, {th} host threads, {cpu_s:.1f} s wall "
                         f"(~{cpu_s * th:.0f} thread-seconds of CPU work)"}

    out = {
        "metric": "MoE-layer decode tokens/s and achieved HBM GB/s (% of peak), 1 MI355X",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {
            "workload": cfg.description,
            "tokens_per_step": T,
            "layer_copies": copies,
            "x_pool": args.x_pool,
            "path": path,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "detail": {
            "selected_expert_bytes_per_step": round(sel_bytes),
            "unique_experts_per_step": uniq_mean,
            "layer_GBps_selected_experts": round(sel_bytes / (ms_per_step * 1e-3) / 1e9, 1),
            "layer_hbm_frac": round(sel_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "expert_kernels_us": round(expert_us, 3),
            "kernel_source_hash": kernel_source_hash(path),
            "expert_GBps": round(sel_bytes / (expert_us * 1e-6) / 1e9, 1) if expert_us else None,
            "stage_avg_us": {k: round(v, 3) for k, v in stage_avg_us.items()},
            "setup_s": round(setup_s, 1),
        },
    }
    print(json.dumps(out), flush=True)


def algo_bytes(cfg, path: str, unique_experts: float) -> dict:
    """Algorithmic bytes per launch of the two expert kernels. The per-pair path
    streams every (token, slot) pair's expert rows (T k + shared pairs); the
    grouped path each selected expert's rows once (unique experts + shared).
    Padding bytes of a row are not counted."""
    pairs = cfg.T * cfg.k + (cfg.T if cfg.shared else 0)
    units = unique_experts if path == "grouped" else pairs
    return {
        "gateup": units * 2 * cfg.F * gen_row_bytes(cfg.fmt_gu, cfg.H),
        "down": units * cfg.H * gen_row_bytes(cfg.fmt_d, cfg.F),
        "router": 4 * cfg.E * cfg.H,
    }


def gen_row_bytes(fmt, K):
    import gen
    return gen.row_bytes(fmt, K)


def kernel_names(cfg, path: str) -> dict:
    """Kernel (as rocprofv3 names it) of each stage of a layer forward (MXFP4
    layers: the realigning kernels, whose LDS budget every workload here fits)."""
    import gen
    if path == "gemv":
        mx = gen.MXFP4
        gu = "k_gateup_mx" if cfg.fmt_gu == mx else "k_gateup"
        if cfg.fmt_d in (gen.Q4_K, gen.Q5_K, gen.Q2_K):  # rows staged through LDS
            dn = "k_down_lds"
        else:
            dn = "k_down_mx" if cfg.fmt_d == mx else "k_down"
        return {"router": "k_router", "gateup": gu, "down": dn}
    nb = cfg.biases
    gu = "k_glds_q4k<0>" if cfg.fmt_gu == gen.Q4_K and not nb else "k_gu_grouped"
    if cfg.fmt_d == gen.Q4_K and not nb:
        dn = "k_glds_q4k<1>"
    elif cfg.fmt_d == gen.Q6_K and not nb:
        dn = "k_glds_q6k_down"
    else:
        dn = "k_down_grouped"
    rt = "k_router_mfma22" if cfg.T > 16 and cfg.E + 1 > 16 else "k_router_mfma"  # 2 x 2 blocked
    return {"router": rt, "gateup": gu, "down": dn}


_PATH_SOURCES = {
    "gemv": ("moe_kernels.hip", "moe_device.h", "moe_internal.h"),
    "grouped": ("moe_grouped.hip", "moe_device.h", "moe_internal.h"),
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
    for K-quants, ~16 ns for MXFP4); sizes the CPU sample to about 20 s of CPU
    work."""
    macs = (cfg.k + (1 if cfg.shared else 0)) * 3 * cfg.H * cfg.F
    ns_per_mac = 16.0 if cfg.fmt_gu == 2 else 1.1
    return macs * ns_per_mac * 1e-9


if __name__ == "__main__":
    main()
