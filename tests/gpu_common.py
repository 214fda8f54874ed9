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
                sh_gate_vec=None, threads=8, path=0, interleaved=False, layout=None):
    """Run the whole layer on the GPU and compare with the oracle on `tokens`."""
    data = data or gen.make_layer(cfg)
    T = cfg.T if T is None else T
    x, xb = gen.make_x(cfg, T=T, x_index=x_index)
    dl = DeviceLayer(data, present=present, sh_gate_vec=sh_gate_vec, path=path,
                     interleaved=interleaved, layout=layout)
    xt, dt = x_to_device(data, x, xb)
    say(f"layer {cfg.name} T={T} x_index={x_index} path={path} interleaved={interleaved} "
        f"layout={dl.layout}")
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


def x_cases(T, H, seed):
    x = gen.normal(seed, gen.T_X, 77, T, H, 1.0)
    if T > 1:
        x[1] = 0.0                       # all-zero row
    if T > 2:
        x[2, :32] = 0.0                  # a zero block
        x[2, min(40, H - 1)] = 1e4       # a spike
    if T > 3:
        x[3] *= 1e-6
    return x


def upload_q8(x_rows, B):
    T, K = x_rows.shape
    qs = np.zeros((T, K), np.int8)
    d = np.zeros((T, K // B), np.float32)
    bs = np.zeros((T, K // 16), np.int16)
    for t in range(T):
        a, b, c = oracle.quantize_q8(x_rows[t], B)
        qs[t], d[t] = a, b
        if c is not None:
            bs[t] = c
    tq, td, tb = (torch.from_numpy(v).cuda() for v in (qs, d, bs))
    afmt = M.MOE_AFMT_Q8_K if B == 256 else M.MOE_AFMT_Q8_32
    return (qs, d, bs), M.qact(tq, td, tb if B == 256 else None, afmt, T, K), (tq, td, tb)


def random_blocks(fmt, n_rows, K, rng):
    """Blocks with arbitrary field values (negative Q6_K scales, every MXFP4 code,
    negative Q5_1 minimums, every Q3_K scale)."""
    nb = K // gen.BLOCK_ELEMS[fmt]
    rows = []
    for r in range(n_rows):
        row = []
        for b in range(nb):
            if fmt == gen.Q4_K:
                row.append(gen.pack_q4k(int(rng.integers(0x0400, 0x3C00)),
                                        int(rng.integers(0x0400, 0x3C00)),
                                        rng.integers(0, 64, 8), rng.integers(0, 64, 8),
                                        rng.integers(0, 16, 256)))
            elif fmt == gen.Q5_K:
                row.append(gen.pack_q5k(int(rng.integers(0x0400, 0x3C00)),
                                        int(rng.integers(0x0400, 0x3C00)),
                                        rng.integers(0, 64, 8), rng.integers(0, 64, 8),
                                        rng.integers(0, 32, 256)))
            elif fmt == gen.Q2_K:
                row.append(gen.pack_q2k(int(rng.integers(0x0400, 0x3C00)),
                                        int(rng.integers(0x0400, 0x3C00)),
                                        rng.integers(0, 16, 16), rng.integers(0, 16, 16),
                                        rng.integers(0, 4, 256)))
            elif fmt == gen.Q6_K:
                row.append(gen.pack_q6k(int(rng.integers(0x0400, 0x3C00)),
                                        rng.integers(-128, 128, 16).astype(np.int8),
                                        rng.integers(0, 64, 256)))
            elif fmt == gen.Q3_K:
                row.append(gen.pack_q3k(int(rng.integers(0x0400, 0x3C00)), rng.integers(0, 64, 16),
                                        rng.integers(-4, 4, 256)))
            elif fmt == gen.Q4_0:
                row.append(gen.pack_q40(int(rng.integers(0x0400, 0x3C00)), rng.integers(0, 16, 32)))
            elif fmt == gen.Q5_1:
                row.append(gen.pack_q51(int(rng.integers(0x0400, 0x3C00)),
                                        int(rng.integers(0x0400, 0x3C00)) | (rng.integers(2) << 15),
                                        rng.integers(0, 32, 32)))
            else:
                row.append(gen.pack_mxfp4(int(rng.integers(100, 150)), rng.integers(0, 16, 32)))
        rows.append(np.concatenate(row))
    return np.stack(rows)
