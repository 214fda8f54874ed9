"""GPU parity of the whole layer against the oracle: ids exact, outputs within
2e-3 of ||y||_2 per token; NULL-mask partition, determinism, edge cases."""
import numpy as np
import pytest
import torch

import gen
import oracle
import quantized_moe_expert_route_amd as M
from gen.device import DeviceLayer, x_to_device
from tests.gpu_common import Y_TOL, check_layer, rel_err, run_layer, say
from tests.shrunk import SHRUNK

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", list(SHRUNK))
def test_layer_shrunk(name):
    check_layer(SHRUNK[name])


@pytest.mark.parametrize("name,T", [("tiny", 1), ("tiny", 13), ("qwen3.6-35b-a3b", 1),
                                    ("qwen3.6-35b-a3b", 4), ("gpt-oss-20b", 1),
                                    ("gpt-oss-20b", 3), ("gpt-oss-20b", 16)])
def test_layer_full_decode(name, T):
    """Full-size layers through the per-pair path; the gpt-oss shape also at 16
    tokens (MXFP4 layers take it at every T: 64 gate/up pairs, 16 down rows of
    workgroups)."""
    check_layer(gen.CONFIGS[name], T=T, x_index=T, threads=16)


@pytest.mark.parametrize("H,F,k,shared", [(1024, 2048, 4, False), (2048, 1024, 8, True),
                                          (3584, 512, 2, False), (6144, 256, 2, True),
                                          (2048, 2048, 8, True)])
def test_layer_mxfp4_shapes(H, F, k, shared):
    """MXFP4 layers whose rows take each plan of the realigned GEMV kernels (one
    to nine 16-byte pieces per lane and row pair, one to four blocks per lane;
    up to nine slots in the down kernel). At F = 2048 with nine slots the
    activation images exceed the LDS budget and the down projection takes the
    register-staged kernel instead."""
    cfg = gen.CONFIGS["gpt-oss-20b"].with_(name=f"mx-{H}-{F}-{k}", E=16, H=H, F=F, k=k,
                                           shared=shared, T=2)
    check_layer(cfg)


@pytest.mark.parametrize("name,fmt_gu,fmt_d,T", [
    ("qwen3.6-35b-a3b", "Q5_K", "Q5_K", 1), ("qwen3.6-35b-a3b", "Q5_K", "Q5_K", 6),
    ("deepseek-v4-flash", "Q5_K", "Q6_K", 3), ("deepseek-v4-flash", "Q4_K", "Q5_K", 16),
    ("qwen-full", "Q5_K", "Q5_K", 1)])
def test_layer_q5k(name, fmt_gu, fmt_d, T):
    """Q5_K experts (gate/up, down or both) through the per-pair GEMV kernels,
    which every chunk of a Q5_K layer takes (no MFMA tile kernel for it): the
    shrunk Qwen3.6 and DeepSeek-V4-Flash shapes, up to a 16-token chunk, and the
    full Qwen3.6 shape at one token."""
    f = {"Q4_K": gen.Q4_K, "Q5_K": gen.Q5_K, "Q6_K": gen.Q6_K}
    base = gen.CONFIGS["qwen3.6-35b-a3b"] if name == "qwen-full" else SHRUNK[name]
    cfg = base.with_(name=f"{base.name}-{fmt_gu}-{fmt_d}", fmt_gu=f[fmt_gu], fmt_d=f[fmt_d], T=T)
    check_layer(cfg, x_index=T)


@pytest.mark.parametrize("name,fmt_gu,fmt_d,T", [
    ("qwen3.6-35b-a3b", "Q2_K", "Q2_K", 1), ("qwen3.6-35b-a3b", "Q2_K", "Q2_K", 6),
    ("deepseek-v4-flash", "Q2_K", "Q6_K", 3), ("kimi-k2", "Q4_K", "Q2_K", 7),
    ("qwen-full", "Q2_K", "Q5_K", 1)])
def test_layer_q2k(name, fmt_gu, fmt_d, T):
    """Q2_K experts through the per-pair GEMV kernels (every chunk of a Q2_K
    layer takes them), alone and mixed with Q4_K, Q5_K and Q6_K matrices."""
    f = {"Q4_K": gen.Q4_K, "Q5_K": gen.Q5_K, "Q6_K": gen.Q6_K, "Q2_K": gen.Q2_K}
    base = gen.CONFIGS["qwen3.6-35b-a3b"] if name == "qwen-full" else SHRUNK[name]
    cfg = base.with_(name=f"{base.name}-{fmt_gu}-{fmt_d}", fmt_gu=f[fmt_gu], fmt_d=f[fmt_d], T=T)
    check_layer(cfg, x_index=T)


FMTS = {"Q4_K": gen.Q4_K, "Q6_K": gen.Q6_K, "Q5_K": gen.Q5_K, "Q2_K": gen.Q2_K,
        "Q3_K": gen.Q3_K, "Q4_0": gen.Q4_0, "Q5_1": gen.Q5_1}


@pytest.mark.parametrize("name,fmt_gu,fmt_d,T", [
    ("qwen3.6-35b-a3b", "Q3_K", "Q3_K", 1), ("qwen3.6-35b-a3b", "Q3_K", "Q3_K", 6),
    ("deepseek-v4-flash", "Q3_K", "Q6_K", 3), ("kimi-k2", "Q4_K", "Q3_K", 7),
    ("qwen3.6-35b-a3b", "Q4_0", "Q4_0", 1), ("qwen3.6-35b-a3b", "Q4_0", "Q4_0", 5),
    ("gpt-oss-20b", "Q4_0", "Q5_1", 3), ("kimi-k2", "Q5_1", "Q5_1", 7),
    ("deepseek-v4-flash", "Q5_1", "Q4_K", 4), ("kimi-k2", "Q4_K", "Q4_0", 2),
    ("qwen-full", "Q3_K", "Q4_0", 1), ("gptoss-full", "Q5_1", "Q4_0", 1)])
def test_layer_q3k_q40_q51(name, fmt_gu, fmt_d, T):
    """Q3_K (256-weight blocks, q8_K activations) and Q4_0 / Q5_1 (32-weight
    blocks, int8 q8_32 activations) experts through the per-pair GEMV kernels,
    alone and mixed with each other and with Q4_K and Q6_K: the shrunk shapes
    (gpt-oss's 320 / 288 widths are 10 and 9 blocks of 32, with biases and the
    clamped SwiGLU), up to a 7-token chunk, and the full Qwen3.6 and gpt-oss
    shapes at one token."""
    base = (gen.CONFIGS["qwen3.6-35b-a3b"] if name == "qwen-full"
            else gen.CONFIGS["gpt-oss-20b"] if name == "gptoss-full" else SHRUNK[name])
    cfg = base.with_(name=f"{base.name}-{fmt_gu}-{fmt_d}", fmt_gu=FMTS[fmt_gu],
                     fmt_d=FMTS[fmt_d], T=T)
    check_layer(cfg, x_index=T)


@pytest.mark.parametrize("name,T,path", [
    ("qwen3.6-35b-a3b", 1, M.MOE_PATH_GEMV), ("qwen3.6-35b-a3b", 16, M.MOE_PATH_GROUPED),
    ("deepseek-v4-flash", 5, M.MOE_PATH_GROUPED), ("gpt-oss-20b", 3, M.MOE_PATH_AUTO),
    ("kimi-k2", 7, M.MOE_PATH_GEMV)])
def test_fused_gate_up_interleaved(name, T, path):
    """Experts stored with one fused gate_up tensor of alternating gate and up
    rows: the descriptor's up pointer is one row past the gate pointer and both
    strides are two rows. Same outputs as the stacked layout (bitwise) and the
    oracle, on the per-pair GEMV and the expert-grouped paths."""
    cfg = SHRUNK[name].with_(T=T)
    data = gen.make_layer(cfg)
    y, ids, w, _ = check_layer(cfg, data=data, x_index=T, path=path, interleaved=True)
    x, xb = gen.make_x(cfg, T=T, x_index=T)
    dl = DeviceLayer(data, path=path)
    xt, dt = x_to_device(data, x, xb)
    y2, ids2, w2 = run_layer(dl, xt, dt, T)
    assert np.array_equal(ids, ids2) and np.array_equal(w, w2)
    assert np.array_equal(y, y2)


@pytest.mark.parametrize("fmt_gu,fmt_d,F,T", [
    ("Q4_K", "Q4_0", 1440, 1), ("Q4_K", "Q5_1", 1440, 4), ("Q6_K", "Q4_0", 352, 3),
    ("Q5_1", "Q5_1", 1440, 2), ("MXFP4", "MXFP4", 1440, 2)])
def test_expert_width_not_multiple_of_256(fmt_gu, fmt_d, F, T):
    """Expert widths F that are not multiples of 256 (1440 = 45 blocks of 32,
    352 = 11): gate/up rows of any format are F rows, and the down rows of
    width F take a 32-weight format."""
    f = dict(FMTS, MXFP4=gen.MXFP4)
    base = SHRUNK["qwen3.6-35b-a3b"]
    cfg = base.with_(name=f"qwen-F{F}-{fmt_gu}-{fmt_d}", fmt_gu=f[fmt_gu], fmt_d=f[fmt_d],
                     F=F, T=T)
    check_layer(cfg, x_index=T)


def _routed_layer(cfg, T, x_index):
    """The full-size layer with only the experts the oracle routes these tokens
    to (plus the shared expert) generated; the others stay zero and unused."""
    base = gen.make_layer(cfg, experts=[])
    x, _ = gen.make_x(cfg, T=T, x_index=x_index)
    used = set()
    for t in range(T):
        used |= {int(e) for e in oracle.topk(oracle.router_logits(base.w_router, x[t]), cfg.k,
                                             base.sel_bias)}
    if cfg.shared:
        used.add(cfg.E)  # the shared expert's pool slot
    return gen.make_layer(cfg, experts=sorted(used))


@pytest.mark.parametrize("name,T,path", [
    ("deepseek-v4-flash", 1, M.MOE_PATH_GEMV), ("deepseek-v4-flash", 3, M.MOE_PATH_GEMV),
    ("deepseek-v4-flash", 1, M.MOE_PATH_AUTO), ("deepseek-v4-flash", 3, M.MOE_PATH_AUTO),
    ("kimi-k2", 1, M.MOE_PATH_GEMV), ("kimi-k2", 2, M.MOE_PATH_GEMV),
    ("kimi-k2", 1, M.MOE_PATH_AUTO), ("kimi-k2", 2, M.MOE_PATH_AUTO),
    ("deepseek-v4-flash", 1, "tile64"), ("kimi-k2", 2, "tile64")])
def test_layer_full_decode_routed(name, T, path):
    """Full-size DeepSeek-V4-Flash and Kimi-K2 layers at one to three tokens:
    the per-pair path (sigmoid routers, DeepSeek with selection bias; E = 384,
    16 candidates per lane in the top-k; Q6_K down rows in registers and Q4_K
    down rows through LDS at H = 7168), and the same small chunks on the path
    the automatic rule picks for them (expert-grouped: their experts hold 8 MB
    or more of blocks), also with the experts in 64-row tiles."""
    cfg = gen.CONFIGS[name]
    layout = M.MOE_LAYOUT_TILE64 if path == "tile64" else M.MOE_LAYOUT_ROWS
    path = M.MOE_PATH_AUTO if path == "tile64" else path
    check_layer(cfg, data=_routed_layer(cfg, T, 30 + T), T=T, x_index=30 + T, path=path,
                layout=layout)


def test_layer_full_verify_chunk_sampled():
    """DeepSeek-V4-Flash-shaped 16-token chunk at full size, experts in 64-row
    tiles as the benchmark runs it; the oracle checks every token. The same
    chunk over row-order experts gives the same bytes."""
    cfg = gen.CONFIGS["deepseek-v4-flash"]
    data = gen.make_layer(cfg)
    y, ids, w, _ = check_layer(cfg, data=data, tokens=range(16), threads=16,
                               layout=M.MOE_LAYOUT_TILE64)
    x, xb = gen.make_x(cfg, T=cfg.T, x_index=0)
    dr = DeviceLayer(data, layout=M.MOE_LAYOUT_ROWS)
    xt, dt = x_to_device(data, x, xb)
    yr, idr, wr = run_layer(dr, xt, dt, cfg.T)
    assert np.array_equal(ids, idr) and np.array_equal(w, wr)
    assert np.array_equal(y.view(np.uint32), yr.view(np.uint32))


@pytest.mark.parametrize("path", [M.MOE_PATH_GEMV, M.MOE_PATH_GROUPED])
def test_expert_ffn_given_routing(path):
    cfg = SHRUNK["kimi-k2"]
    data = gen.make_layer(cfg)
    T = cfg.T
    x, _ = gen.make_x(cfg, T=T, x_index=3)
    rng = np.random.default_rng(0)
    ids = np.stack([rng.choice(cfg.E, cfg.k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[0] = ids[1]  # tokens sharing experts
    w = rng.random((T, cfg.k)).astype(np.float32)
    dl = DeviceLayer(data, path=path)
    qs = torch.empty((T, cfg.H), dtype=torch.int8, device="cuda")
    d = torch.empty((T, cfg.H // 256), dtype=torch.float32, device="cuda")
    bs = torch.empty((T, cfg.H // 16), dtype=torch.int16, device="cuda")
    q = M.qact(qs, d, bs, M.MOE_AFMT_Q8_K, T, cfg.H)
    xt = torch.from_numpy(x).cuda()
    M.moe_quantize_act_q8k(xt, M.MOE_DTYPE_F32, T, cfg.H, M.MOE_AFMT_Q8_K, q)
    y = torch.empty((T, cfg.H), dtype=torch.float32, device="cuda")
    ws = dl.workspace(T)
    M.moe_expert_ffn(dl.desc, q, xt, M.MOE_DTYPE_F32, T, torch.from_numpy(ids).cuda(),
                     torch.from_numpy(w).cuda(), y, ws, ws.numel())
    torch.cuda.synchronize()
    L = oracle.Layer(data)
    for t in range(T):
        ref = L.expert_part(x[t], ids[t], w[t])
        assert rel_err(y[t].cpu().numpy(), ref) <= Y_TOL


@pytest.mark.parametrize("name,path", [("qwen3.6-35b-a3b", 0), ("gpt-oss-20b", 0),
                                       ("deepseek-v4-flash", 0),
                                       ("deepseek-v4-flash", M.MOE_PATH_GROUPED)])
def test_null_mask_partition(name, path):
    """Experts split over two 'devices' by NULL pointers: the partial outputs sum
    to the full output (the expert-parallel sharding pattern on one GPU)."""
    cfg = SHRUNK[name].with_(shared=False)
    data = gen.make_layer(cfg)
    T = cfg.T
    x, xb = gen.make_x(cfg, T=T, x_index=2)
    mask = np.random.default_rng(7).random(cfg.E) < 0.5
    outs = []
    for present in (None, mask, ~mask):
        dl = DeviceLayer(data, present=present, path=path)
        xt, dt = x_to_device(data, x, xb)
        outs.append(run_layer(dl, xt, dt, T))
    (yf, idf, wf), (ya, ida, wa), (yb, idb, wb) = outs
    assert np.array_equal(idf, ida) and np.array_equal(idf, idb)
    assert np.array_equal(wf, wa)
    assert rel_err(ya + yb, yf).max() <= 1e-5
    L = oracle.Layer(data, present=mask)
    ref = L.forward(x)
    assert rel_err(ya, ref["y"]).max() <= Y_TOL


def test_shared_gate_vector():
    cfg = SHRUNK["qwen3.6-35b-a3b"]
    data = gen.make_layer(cfg, with_sh_gate_vec=True)
    check_layer(cfg, data=data, sh_gate_vec=data.sh_gate_vec)


@pytest.mark.parametrize("name", ["deepseek-v4-flash", "gpt-oss-full", "qwen-q2k"])
def test_determinism(name):
    """Two runs give identical bytes: the grouped path (5-token chunk), the
    MXFP4 realigned kernels at full width, the Q2_K GEMV kernels."""
    cfg = (gen.CONFIGS["gpt-oss-20b"] if name == "gpt-oss-full" else
           SHRUNK["qwen3.6-35b-a3b"].with_(fmt_gu=gen.Q2_K, fmt_d=gen.Q2_K) if name == "qwen-q2k"
           else SHRUNK[name])
    data = gen.make_layer(cfg)
    x, xb = gen.make_x(cfg, T=cfg.T)
    dl = DeviceLayer(data, path=M.MOE_PATH_GROUPED if name == "deepseek-v4-flash" else 0)
    xt, dt = x_to_device(data, x, xb)
    a = run_layer(dl, xt, dt, cfg.T)
    b = run_layer(dl, xt, dt, cfg.T)
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_zero_input_and_k_equals_E():
    cfg = gen.CONFIGS["tiny"].with_(k=8)
    data = gen.make_layer(cfg)
    x = np.zeros((2, cfg.H), np.float32)
    x[1], _ = gen.make_x(cfg, T=1)
    dl = DeviceLayer(data)
    y, ids, w = run_layer(dl, torch.from_numpy(x).cuda(), M.MOE_DTYPE_F32, 2)
    assert list(ids[0]) == list(range(8))
    assert not y[0].any()
    ref = oracle.Layer(data).forward(x)
    assert np.array_equal(ids, ref["ids"])
    assert rel_err(y[1], ref["y"][1]) <= Y_TOL


def test_zero_tokens_on_device():
    cfg = gen.CONFIGS["tiny"]
    data = gen.make_layer(cfg)
    dl = DeviceLayer(data)
    y = torch.full((1, cfg.H), 3.0, device="cuda")
    ws = dl.workspace(0)
    M.moe_layer_forward(dl.desc, torch.zeros((1, cfg.H), device="cuda"), 0, 0, y, None, None,
                        ws, ws.numel())
    torch.cuda.synchronize()
    assert (y == 3.0).all()


def test_layer_copies_identical():
    cfg = SHRUNK["qwen3.6-35b-a3b"]
    data = gen.make_layer(cfg)
    x, _ = gen.make_x(cfg, T=2)
    dl = DeviceLayer(data, copies=2)
    xt = torch.from_numpy(x).cuda()
    a = run_layer(dl, xt, 0, 2, copy=0)
    b = run_layer(dl, xt, 0, 2, copy=1)
    assert np.array_equal(a[0], b[0])


@pytest.mark.parametrize("name,T", [("qwen3.6-35b-a3b", 1), ("tiny", 1), ("qwen3.6-35b-a3b", 3),
                                    ("gpt-oss-20b", 1), ("gpt-oss-full", 2)])
def test_expert_ffn_given_routing_decode(name, T):
    """Caller-given routing on the decode path (the fused expert kernel at one
    token): repeated and out-of-range ids, an absent expert, shared expert; the
    MXFP4 cases (q8 in 32-value blocks, bf16 x, biases) run the realigned
    kernels, at full width for gpt-oss-full."""
    cfg = (gen.CONFIGS[name] if name == "tiny" else
           gen.CONFIGS["gpt-oss-20b"] if name == "gpt-oss-full" else SHRUNK[name])
    mx = cfg.fmt_gu == gen.MXFP4
    data = gen.make_layer(cfg)
    x, xb = gen.make_x(cfg, T=T, x_index=11)
    rng = np.random.default_rng(5)
    ids = np.stack([rng.choice(cfg.E, cfg.k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[0, -1] = cfg.E  # out of range: contributes nothing
    w = rng.random((T, cfg.k)).astype(np.float32)
    present = np.ones(cfg.E, bool)
    present[ids[0, 0]] = False  # an absent expert
    dl = DeviceLayer(data, present=present)
    B = 32 if mx else 256
    afmt = M.MOE_AFMT_Q8_32 if mx else M.MOE_AFMT_Q8_K
    qs = torch.empty((T, cfg.H), dtype=torch.int8, device="cuda")
    d = torch.empty((T, cfg.H // B), dtype=torch.float32, device="cuda")
    bs = None if mx else torch.empty((T, cfg.H // 16), dtype=torch.int16, device="cuda")
    q = M.qact(qs, d, bs, afmt, T, cfg.H)
    xt, dt = x_to_device(data, x, xb)
    M.moe_quantize_act_q8k(xt, dt, T, cfg.H, afmt, q)
    y = torch.empty((T, cfg.H), dtype=torch.float32, device="cuda")
    ws = dl.workspace(T)
    for _ in range(2):  # twice: the done flags are cleared per call
        M.moe_expert_ffn(dl.desc, q, xt, dt, T, torch.from_numpy(ids).cuda(),
                         torch.from_numpy(w).cuda(), y, ws, ws.numel())
        torch.cuda.synchronize()
        L = oracle.Layer(data, present=present)
        for t in range(T):
            ref = L.expert_part(x[t], ids[t], w[t])
            assert rel_err(y[t].cpu().numpy(), ref) <= Y_TOL
