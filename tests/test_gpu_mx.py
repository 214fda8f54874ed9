"""MXFP8-activation layers (MXFP4 experts on the block-scaled MFMA path)
against the oracle's MXFP8 mode: the quantizer bit for bit, integer-exact
pre-activations bitwise, whole layers within the layer tolerance."""
import zlib

import numpy as np
import pytest
import torch

import gen
import oracle
import quantized_moe_expert_route_amd as M
from gen.device import DeviceLayer, x_to_device
from tests.gpu_common import check_layer, run_layer, say, x_cases
from tests.shrunk import SHRUNK

pytestmark = pytest.mark.gpu


def deinterleave(q: np.ndarray) -> np.ndarray:
    """Natural element order of pair-interleaved MXFP8 blocks (byte 2j = element
    j, byte 2j + 1 = element j + 16)."""
    b = q.reshape(-1, 16, 2)
    return np.concatenate([b[:, :, 0], b[:, :, 1]], axis=1).reshape(q.shape)


def mx8_cfg(base, **kw):
    return base.with_(name=f"{base.name}-mx8", fmt_gu=gen.MXFP4, fmt_d=gen.MXFP4, act_quant=1,
                      **kw)


@pytest.mark.parametrize("T,H", [(1, 32), (3, 2880), (5, 2048), (2, 7168)])
@pytest.mark.parametrize("bf16", [False, True])
def test_quantize_mx8_bitexact(T, H, bf16):
    say(f"quantize mx8 T={T} H={H} bf16={bf16}")
    x = x_cases(T, H, 11)
    if T > 2:
        x[2, 64:96] = np.float32(2.0 ** -20) * np.arange(32)  # deep subnormal E4M3 range
        x[2, 96:128] = np.linspace(-3, 3, 32).astype(np.float32) * 1e30
    if bf16:
        x = (torch.from_numpy(x).to(torch.bfloat16).float()).numpy()
        xt = torch.from_numpy(x).to(torch.bfloat16).cuda()
        dt = M.MOE_DTYPE_BF16
    else:
        xt = torch.from_numpy(x).cuda()
        dt = M.MOE_DTYPE_F32
    pitch = M.mx8_scale_pitch(H)
    q = torch.zeros((T, H), dtype=torch.uint8, device="cuda")
    e = torch.full((T, pitch), 0xAB, dtype=torch.uint8, device="cuda")
    xq = M.qact(q, None, None, M.MOE_AFMT_MXFP8, T, H, scales=e)
    M.moe_quantize_act_q8k(xt, dt, T, H, M.MOE_AFMT_MXFP8, xq)
    torch.cuda.synchronize()
    gq, ge = q.cpu().numpy(), e.cpu().numpy()
    for t in range(T):
        rq, re = oracle.quantize_mx8(x[t])
        assert np.array_equal(deinterleave(gq[t]), rq), t
        assert np.array_equal(ge[t, :H // 32], re), t
        assert np.all(ge[t, H // 32:] == 0xAB)  # padding untouched


# (name, overrides, T)
LAYERS = [
    ("gpt-oss-20b", dict(), 1), ("gpt-oss-20b", dict(), 3), ("gpt-oss-20b", dict(), 16),
    ("qwen3.6-35b-a3b", dict(), 3), ("qwen3.6-35b-a3b", dict(), 12),
    ("kimi-k2", dict(), 7), ("deepseek-v4-flash", dict(), 5),
    ("gpt-oss-20b", dict(H=2880, F=2880, E=32), 16),
    ("qwen3.6-35b-a3b", dict(H=1056, F=96, E=8, k=3), 9),
]


@pytest.mark.parametrize("name,over,T", LAYERS)
def test_layer_mx8(name, over, T):
    """Shrunk workload shapes with MXFP4 experts and MXFP8 activations (gpt-oss:
    biases, clamped SwiGLU, bf16 x, widths of 10 and 9 blocks; Qwen3.6 and
    Kimi: shared expert; DeepSeek: sigmoid router with selection bias), the
    full gpt-oss width at 16 tokens, and a ragged 33-block width."""
    cfg = mx8_cfg(SHRUNK[name], **over).with_(T=T)
    check_layer(cfg, x_index=T)


def test_layer_mx8_full_gptoss_sampled():
    """The full gpt-oss-20b layer (E 32, k 4, H = F = 2880) on a 64-token chunk;
    the oracle checks 16 sampled tokens and every token's routing."""
    cfg = mx8_cfg(gen.CONFIGS["gpt-oss-20b"]).with_(T=64)
    rng = np.random.default_rng(4)
    tokens = sorted(rng.choice(64, 16, replace=False))
    y, ids, w, _ = check_layer(cfg, x_index=5, tokens=tokens)
    data = gen.make_layer(cfg)
    x, _ = gen.make_x(cfg, T=64, x_index=5)
    L = oracle.Layer(data)
    for t in range(64):
        lg = oracle.router_logits(data.w_router, x[t])
        assert np.array_equal(ids[t], oracle.topk(lg, cfg.k, data.sel_bias)), t


def test_mx8_determinism_and_forced_path():
    cfg = mx8_cfg(SHRUNK["gpt-oss-20b"]).with_(T=16)
    data = gen.make_layer(cfg)
    x, xb = gen.make_x(cfg, T=16, x_index=1)
    dl = DeviceLayer(data)
    xt, dt = x_to_device(data, x, xb)
    y0, i0, w0 = run_layer(dl, xt, dt, 16)
    for _ in range(3):
        y1, i1, w1 = run_layer(dl, xt, dt, 16)
        assert np.array_equal(y0, y1) and np.array_equal(i0, i1)
    assert M.moe_layer_stage_count(dl.desc, 1) == 7
    d = dl.desc
    d.path = M.MOE_PATH_GEMV
    assert M.moe_workspace_size(d, 1) == 0
    d.path = M.MOE_PATH_AUTO


def test_mx8_expert_ffn_given_routing():
    """moe_expert_ffn on caller-quantized MXFP8 x with given ids and weights
    (an id outside [0, E) and an absent expert contribute nothing)."""
    cfg = mx8_cfg(SHRUNK["qwen3.6-35b-a3b"]).with_(T=5)
    data = gen.make_layer(cfg)
    present = np.ones(cfg.E, bool)
    present[3] = False
    x, _ = gen.make_x(cfg, T=5, x_index=3)
    rng = np.random.default_rng(8)
    ids = np.stack([rng.choice(cfg.E, cfg.k, replace=False) for _ in range(5)]).astype(np.int32)
    ids[0, 0] = 3
    ids[1, 1] = cfg.E + 7
    w = rng.uniform(0.1, 1.0, ids.shape).astype(np.float32)
    dl = DeviceLayer(data, present=present)
    H = cfg.H
    pitch = M.mx8_scale_pitch(H)
    q = torch.zeros((5, H), dtype=torch.uint8, device="cuda")
    e = torch.zeros((5, pitch), dtype=torch.uint8, device="cuda")
    xq = M.qact(q, None, None, M.MOE_AFMT_MXFP8, 5, H, scales=e)
    xt = torch.from_numpy(x).cuda()
    M.moe_quantize_act_q8k(xt, M.MOE_DTYPE_F32, 5, H, M.MOE_AFMT_MXFP8, xq)
    y = torch.empty((5, H), dtype=torch.float32, device="cuda")
    ws = dl.workspace(5)
    M.moe_expert_ffn(dl.desc, xq, xt, M.MOE_DTYPE_F32, 5, torch.from_numpy(ids).cuda(),
                     torch.from_numpy(w).cuda(), y, ws, ws.numel())
    torch.cuda.synchronize()
    L = oracle.Layer(data, present=present)
    got = y.cpu().numpy()
    for t in range(5):
        ref = L.expert_part(x[t], ids[t], w[t])
        assert np.abs(got[t] - ref).max() <= 2e-3 * np.linalg.norm(ref), t


def e4m3_int_x(T, H, rng):
    """Activations whose MXFP8 codes are exact with scale 2^0: small integers
    (exact in E4M3) and one +-256 per block of 32 (block max in [256, 512))."""
    x = rng.integers(-16, 17, (T, H)).astype(np.float32)
    for t in range(T):
        for b0 in range(0, H, 32):
            x[t, b0 + rng.integers(32)] = 256.0 if rng.random() < 0.5 else -256.0
    return x


def test_mx8_preact_exact():
    """Integer-exact case of the block-scaled MFMA: MXFP4 blocks with scale 2^0
    and activations exact in E4M3 with scale 2^0: every gate/up pre-activation
    is a multiple of 0.5 below 2^22, so the MFMA's sums are exact and equal the
    oracle's exact MXFP4 x MXFP8 row dots bitwise."""
    cfg = gen.LayerConfig("exact-mx8", H=1024, F=256, E=8, k=2, T=9, seed=31, shared=True,
                          fmt_gu=gen.MXFP4, fmt_d=gen.MXFP4, act_quant=1)
    rng = np.random.default_rng(zlib.crc32(b"mx8-exact"))
    pool = np.zeros((cfg.n_pool, cfg.expert_bytes), np.uint8)
    nb, rb, gb = cfg.H // 32, gen.row_bytes(gen.MXFP4, cfg.H), cfg.gate_bytes
    for e in range(cfg.n_pool):
        for m in range(2):
            mat = pool[e, m * gb:(m + 1) * gb].reshape(cfg.F, cfg.stride_gu)
            blk = rng.integers(0, 256, (cfg.F * nb, 17), dtype=np.uint8)
            blk[:, 0] = 127
            mat[:, :rb] = blk.reshape(cfg.F, rb)
    w_router = gen.normal(cfg.seed, gen.T_ROUTER, 0, cfg.E, cfg.H, 0.02)
    data = gen.LayerData(cfg, w_router, None, pool, None, None, None,
                         np.zeros((cfg.T, cfg.H), np.float32), None)
    dl = DeviceLayer(data, path=M.MOE_PATH_GROUPED)
    T = cfg.T
    x = e4m3_int_x(T, cfg.H, rng)
    pitch = M.mx8_scale_pitch(cfg.H)
    q = torch.zeros((T, cfg.H), dtype=torch.uint8, device="cuda")
    esc = torch.zeros((T, pitch), dtype=torch.uint8, device="cuda")
    xq = M.qact(q, None, None, M.MOE_AFMT_MXFP8, T, cfg.H, scales=esc)
    M.moe_quantize_act_q8k(torch.from_numpy(x).cuda(), M.MOE_DTYPE_F32, T, cfg.H,
                           M.MOE_AFMT_MXFP8, xq)
    torch.cuda.synchronize()
    assert np.all(esc.cpu().numpy()[:, :nb] == 127)
    ids = np.stack([rng.choice(cfg.E, cfg.k, replace=False) for _ in range(T)]).astype(np.int32)
    P = T * cfg.k + T
    ws = dl.workspace(T)
    for which in (0, 1):
        out = torch.full((P, cfg.F), float("nan"), dtype=torch.float32, device="cuda")
        M.moe_test_preact(dl.desc, xq, T, torch.from_numpy(ids).cuda(), which, out, ws,
                          ws.numel())
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        for p in range(P):
            t, e = (p // cfg.k, int(ids[p // cfg.k, p % cfg.k])) if p < T * cfg.k \
                else (p - T * cfg.k, cfg.E)
            rq, re = oracle.quantize_mx8(x[t])
            mat = (data.gate(e) if which == 0 else data.up(e)).reshape(cfg.F, cfg.stride_gu)
            for r in range(cfg.F):
                want = oracle.row_dot_mx8(mat[r], cfg.H, rq, re)
                assert abs(want) < 2 ** 22 and want * 2 == int(want * 2)
                assert got[p, r] == np.float32(want), (which, p, r, got[p, r], want)
