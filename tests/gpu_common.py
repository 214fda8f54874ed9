"""Shared helpers of the GPU parity tests (HIP path vs the oracle)."""
import sys

import numpy as np
import torch

import gen
import oracle
import quantized_moe_expert_route_amd as M
from gen.device import DeviceLayer, x_to_device

Y_TOL = 2e-3  # per token: max |dy| / ||y_ref||_2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(y_gpu: np.ndarray, y_ref: np.ndarray) -> np.ndarray:
    """Per-token max |dy| / ||y_ref||_2."""
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    num = np.abs(y_gpu - y_ref).max(axis=-1)
    den = np.maximum(np.linalg.norm(y_ref, axis=-1), 1e-30)
    return num / den


def run_layer(dl: DeviceLayer, xt: torch.Tensor, dtype: int, T: int, copy: int = 0):
    cfg = dl.cfg
    y = torch.empty((T, cfg.H), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
    ws = dl.workspace(T)
    M.moe_layer_forward(dl.descs[copy], xt, dtype, T, y, ids, w, ws, ws.numel())
    torch.cuda.synchronize()
    return y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


def check_layer(cfg, data=None, T=None, x_index=0, tokens=None, present=None, tol=Y_TOL,
                sh_gate_vec=None, threads=8):
    """Run the whole layer on the GPU and compare with the oracle on `tokens`."""
    data = data or gen.make_layer(cfg)
    T = cfg.T if T is None else T
    x, xb = gen.make_x(cfg, T=T, x_index=x_index)
    dl = DeviceLayer(data, present=present, sh_gate_vec=sh_gate_vec)
    xt, dt = x_to_device(data, x, xb)
    say(f"layer {cfg.name} T={T} x_index={x_index}")
    y, ids, w = run_layer(dl, xt, dt, T)
    L = oracle.Layer(data, present=present, sh_gate_vec=sh_gate_vec)
    tokens = list(range(T)) if tokens is None else list(tokens)
    ref = L.forward(x, tokens=tokens, threads=threads)
    assert np.array_equal(ids[tokens], ref["ids"]), "expert ids differ"
    assert np.abs(w[tokens] - ref["w"]).max() <= 1e-6
    err = rel_err(y[tokens], ref["y"])
    say(f"  max rel err {err.max():.3e} over {len(tokens)} tokens")
    assert err.max() <= tol, err
    return y, ids, w, ref
