"""Seeded random layers against the oracle (q8 activations, and MXFP4 layers with
MXFP8 activations on the block-scaled MFMA path): formats (gate/up and down each of
the eight), widths, expert counts, top-k up to 16, chunk sizes, routers, shared
experts, biases, activations, bf16 inputs, row orders (rows, 64-row tiles,
MX16) and forced paths, combined at random within what the boundary accepts.
Each case draws its configuration from its own seed, so a failure names a
reproducible layer. Configurations the host refuses (MOE_EUNSUPPORTED: GEMV
shapes past the kernels' LDS budget in formats without tile kernels, MX16
widths past its kernels) are checked to be refused and skipped.
Only the experts the tokens select are generated (the oracle routes first)."""
import numpy as np
import pytest
import torch

import gen
import oracle
import quantized_moe_expert_route_amd as M
from gen.device import DeviceLayer, x_to_device
from tests.gpu_common import Y_TOL, rel_err, run_layer, say

pytestmark = pytest.mark.gpu

FMTS = [gen.Q4_K, gen.Q6_K, gen.MXFP4, gen.Q5_K, gen.Q2_K, gen.Q3_K, gen.Q4_0, gen.Q5_1]
N_CASES = 120


def draw(case: int):
    rng = np.random.default_rng(7919 * case + 13)
    kind = case % 6  # 0, 1: tile-capable formats (grouped path); 2: MXFP4; else any
    if kind < 2:
        fgu, fd = gen.Q4_K, int(rng.choice([gen.Q4_K, gen.Q6_K]))
    elif kind == 2:
        fgu = fd = gen.MXFP4
    else:
        fgu, fd = int(rng.choice(FMTS)), int(rng.choice(FMTS))
    bgu, bd = gen.BLOCK_ELEMS[fgu], gen.BLOCK_ELEMS[fd]
    H = int(rng.integers(1, 3072 // bgu + 1)) * bgu
    F = int(rng.integers(1, 3072 // bd + 1)) * bd
    E = int(rng.choice([1, 2, 5, 8, 16, 31, 64, 100, 256]))
    # at most ~400 MB of expert blocks (the host holds the whole pool)
    eb = 2 * F * gen.row_stride(fgu, H) + H * gen.row_stride(fd, F)
    E = max(1, min(E, (400 << 20) // eb - 1))
    k = int(rng.integers(1, min(E, 16) + 1))
    T = int(rng.choice([1, 1, 2, 3, 4, 5, 7, 9, 12, 16]))
    while T * k > 64 and T > 1:
        T -= 1
    mx = fgu == gen.MXFP4 and fd == gen.MXFP4
    cfg = gen.LayerConfig(
        f"rand{case}", H=H, F=F, E=E, k=k, T=T, seed=100 + case,
        router=int(rng.integers(0, 2)), norm_topk=int(rng.integers(0, 2)),
        route_scale=float(rng.choice([1.0, 1.0, 2.5])), fmt_gu=fgu, fmt_d=fd,
        shared=bool(rng.integers(0, 2)), act=int(rng.integers(0, 2)),
        biases=bool(rng.integers(0, 3) == 0), x_bf16=bool(rng.integers(0, 3) == 0),
        zipf_s=float(rng.choice([0.0, 0.0, 1.1])))
    layout = 0
    if mx and rng.integers(0, 2):
        layout = M.MOE_LAYOUT_MX16
    tiles_ok = fgu == gen.Q4_K and fd in (gen.Q4_K, gen.Q6_K) and not cfg.biases
    if tiles_ok and rng.integers(0, 3) == 0:
        layout = M.MOE_LAYOUT_TILE64
    path = int(rng.choice([M.MOE_PATH_AUTO, M.MOE_PATH_AUTO, M.MOE_PATH_GEMV,
                           M.MOE_PATH_GROUPED]))
    if layout == M.MOE_LAYOUT_TILE64 and path == M.MOE_PATH_GEMV:
        path = M.MOE_PATH_AUTO
    if layout == M.MOE_LAYOUT_MX16 and path == M.MOE_PATH_GROUPED:
        path = M.MOE_PATH_AUTO
    return cfg, layout, path


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_layer(case):
    cfg, layout, path = draw(case)
    if cfg.n_pool * cfg.expert_bytes > (512 << 20):
        pytest.skip("host pool over 512 MB")
    say(f"random case {case}: H={cfg.H} F={cfg.F} E={cfg.E} k={cfg.k} T={cfg.T} "
        f"fmt={cfg.fmt_gu}/{cfg.fmt_d} router={cfg.router} norm={cfg.norm_topk} "
        f"shared={cfg.shared} act={cfg.act} biases={cfg.biases} bf16={cfg.x_bf16} "
        f"zipf={cfg.zipf_s} layout={layout} path={path}")
    base = gen.make_layer(cfg, experts=[])
    x, xb = gen.make_x(cfg, T=cfg.T, x_index=case)
    used = set()
    for t in range(cfg.T):
        lg = oracle.router_logits(base.w_router, x[t])
        used |= {int(e) for e in oracle.topk(lg, cfg.k, base.sel_bias)}
    if cfg.shared:
        used.add(cfg.E)
    data = gen.make_layer(cfg, experts=sorted(used))
    dl = DeviceLayer(data, path=path, layout=layout)
    if M.moe_workspace_size(dl.desc, cfg.T) == 0:
        xt, dt = x_to_device(data, x, xb)
        y = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device="cuda")
        ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
        with pytest.raises(M.MoeError) as ei:
            M.moe_layer_forward(dl.desc, xt, dt, cfg.T, y, None, None, ws, ws.numel())
        assert ei.value.status == M.MOE_EUNSUPPORTED
        pytest.skip("refused by the boundary (MOE_EUNSUPPORTED)")
    xt, dt = x_to_device(data, x, xb)
    try:
        y, ids, w = run_layer(dl, xt, dt, cfg.T)
    except M.MoeError as err:
        # a valid layer whose per-pair shape no GEMV kernel takes (LDS budget)
        # and whose formats have no tile kernels: routing only
        tiles = cfg.fmt_gu in (gen.Q4_K, gen.Q6_K) and cfg.fmt_d in (gen.Q4_K, gen.Q6_K)
        assert err.status == M.MOE_EUNSUPPORTED and (not tiles or path == M.MOE_PATH_GEMV)
        assert M.moe_layer_stage_count(dl.desc, cfg.T) != 7
        pytest.skip("expert FFN refused (MOE_EUNSUPPORTED): routing only")
    ref = oracle.Layer(data).forward(x, threads=8)
    assert np.array_equal(ids, ref["ids"]), "expert ids differ"
    assert np.abs(w - ref["w"]).max() <= 2e-6
    err = rel_err(y, ref["y"])
    say(f"  max rel err {err.max():.3e}")
    assert err.max() <= Y_TOL, err


def draw_mx8(case: int):
    """MXFP4 layers with MXFP8 activations (the block-scaled MFMA path at every T)."""
    rng = np.random.default_rng(104729 * case + 7)
    H = int(rng.integers(1, 96 + 1)) * 32
    F = int(rng.integers(1, 96 + 1)) * 32
    E = int(rng.choice([1, 2, 4, 8, 16, 32, 64, 128]))
    k = int(rng.integers(1, min(E, 16) + 1))
    T = int(rng.choice([1, 2, 3, 5, 8, 16, 17, 33]))
    while T * k > 96 and T > 1:
        T -= 1
    return gen.LayerConfig(
        f"randmx{case}", H=H, F=F, E=E, k=k, T=T, seed=300 + case,
        router=int(rng.integers(0, 2)), norm_topk=int(rng.integers(0, 2)),
        fmt_gu=gen.MXFP4, fmt_d=gen.MXFP4, shared=bool(rng.integers(0, 2)),
        act=int(rng.integers(0, 2)), biases=bool(rng.integers(0, 2)),
        x_bf16=bool(rng.integers(0, 2)), act_quant=1)


@pytest.mark.parametrize("case", range(24))
def test_random_layer_mx8(case):
    cfg = draw_mx8(case)
    say(f"random mx8 case {case}: H={cfg.H} F={cfg.F} E={cfg.E} k={cfg.k} T={cfg.T} "
        f"router={cfg.router} norm={cfg.norm_topk} shared={cfg.shared} act={cfg.act} "
        f"biases={cfg.biases} bf16={cfg.x_bf16}")
    base = gen.make_layer(cfg, experts=[])
    x, xb = gen.make_x(cfg, T=cfg.T, x_index=case)
    used = set()
    for t in range(cfg.T):
        lg = oracle.router_logits(base.w_router, x[t])
        used |= {int(e) for e in oracle.topk(lg, cfg.k, base.sel_bias)}
    if cfg.shared:
        used.add(cfg.E)
    data = gen.make_layer(cfg, experts=sorted(used))
    dl = DeviceLayer(data)
    assert M.moe_layer_stage_count(dl.desc, cfg.T) == 7
    xt, dt = x_to_device(data, x, xb)
    y, ids, w = run_layer(dl, xt, dt, cfg.T)
    ref = oracle.Layer(data).forward(x, threads=8)
    assert np.array_equal(ids, ref["ids"]), "expert ids differ"
    assert np.abs(w - ref["w"]).max() <= 2e-6
    err = rel_err(y, ref["y"])
    say(f"  max rel err {err.max():.3e}")
    assert err.max() <= Y_TOL, err
