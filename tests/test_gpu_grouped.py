"""GPU parity of the expert-grouped (multi-token, int8 MFMA) path against the
oracle, the path forced with the descriptor's path field (the automatic rule
picks it only past ~160 MB of per-pair expert bytes, which these shrunk shapes
never reach): ids exact, outputs within 2e-3 of ||y||_2 per token. Covers experts
with several 16-token tiles, ragged tiles, the dense k = E case, bf16 input,
Q6_K down rows, the shared-expert gate vector, NULL experts, invalid ids,
agreement with the per-pair decode path, expert matrices stored in 64-row
tiles (the same bytes as row order, and the repack itself byte-exact), and
the full Kimi-K2-shaped 256-token chunk (routing on every token, outputs on
40) in both block orders."""
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
GP = M.MOE_PATH_GROUPED
TILE = M.MOE_LAYOUT_TILE64


@pytest.mark.parametrize("name,T", [("tiny", 5), ("tiny", 37), ("deepseek-v4-flash", 33),
                                    ("kimi-k2", 20), ("qwen3.6-35b-a3b", 18)])
def test_grouped_shrunk(name, T):
    """Ragged tiles and experts with more than 16 routed tokens."""
    check_layer(SHRUNK[name], T=T, x_index=T, path=GP)


def tile64_reference(rows: np.ndarray, n_rows: int, nb: int, BB: int) -> np.ndarray:
    """TILE64 order written out from its definition: block b of row r at
    ((r // 64) nb + b) 64 BB + (r % 64) BB."""
    out = np.zeros(n_rows * nb * BB, np.uint8)
    for r in range(n_rows):
        for b in range(nb):
            o = ((r // 64) * nb + b) * 64 * BB + (r % 64) * BB
            out[o:o + BB] = rows[r, b * BB:(b + 1) * BB]
    return out


@pytest.mark.parametrize("fmt,BB,n_rows,K,stride", [(M.MOE_WFMT_Q4_K, 144, 128, 512, 304),
                                                     (M.MOE_WFMT_Q6_K, 210, 192, 768, 640),
                                                     (M.MOE_WFMT_Q4_K, 144, 64, 256, 144)])
def test_repack_tile64_bytes(fmt, BB, n_rows, K, stride):
    """The repack moves whole blocks to where the definition puts them; row
    padding is dropped."""
    rng = np.random.default_rng(n_rows + K)
    rows = rng.integers(0, 256, (n_rows, stride), dtype=np.uint8)
    src = torch.from_numpy(rows.reshape(-1)).cuda()
    nbytes = M.tile64_bytes(fmt, n_rows, K)
    dst = torch.full((nbytes + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    M.moe_repack_tile64(fmt, src, stride, n_rows, K, dst)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    assert np.array_equal(got[:nbytes], tile64_reference(rows, n_rows, K // 256, BB))
    assert (got[nbytes:] == 0xA5).all()  # nothing written past the matrix


@pytest.mark.parametrize("name,T", [("tiny", 37), ("deepseek-v4-flash", 33), ("kimi-k2", 20),
                                    ("qwen3.6-35b-a3b", 18), ("deepseek-v4-flash", 1)])
def test_grouped_tile64(name, T):
    """Expert matrices in 64-row tiles: oracle parity, and the same bytes as the
    grouped path over row-order matrices (the kernels do the same arithmetic;
    only the addresses of a stage's blocks differ)."""
    cfg = SHRUNK[name]
    data = gen.make_layer(cfg)
    y, ids, w, _ = check_layer(cfg, data=data, T=T, x_index=T + 1, layout=TILE)
    x, xb = gen.make_x(cfg, T=T, x_index=T + 1)
    dr = DeviceLayer(data, path=GP, layout=M.MOE_LAYOUT_ROWS)
    xt, dt = x_to_device(data, x, xb)
    yr, idr, wr = run_layer(dr, xt, dt, T)
    assert np.array_equal(ids, idr) and np.array_equal(w, wr)
    assert np.array_equal(y.view(np.uint32), yr.view(np.uint32))


def test_grouped_tile64_null_experts_and_given_routing():
    """64-row tiles with NULL experts and caller-given routing (moe_expert_ffn)."""
    cfg = SHRUNK["deepseek-v4-flash"]
    mask = np.random.default_rng(5).random(cfg.E) < 0.6
    check_layer(cfg, T=14, x_index=3, present=mask, layout=TILE)
    data = gen.make_layer(cfg)
    T = 9
    x, _ = gen.make_x(cfg, T=T, x_index=4)
    rng = np.random.default_rng(8)
    ids = np.stack([rng.choice(cfg.E, cfg.k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, cfg.k)).astype(np.float32)
    dl = DeviceLayer(data, layout=TILE)
    xt = torch.from_numpy(x).cuda()
    qs = torch.empty((T, cfg.H), dtype=torch.int8, device="cuda")
    d = torch.empty((T, cfg.H // 256), dtype=torch.float32, device="cuda")
    bs = torch.empty((T, cfg.H // 16), dtype=torch.int16, device="cuda")
    q = M.qact(qs, d, bs, M.MOE_AFMT_Q8_K, T, cfg.H)
    M.moe_quantize_act_q8k(xt, M.MOE_DTYPE_F32, T, cfg.H, M.MOE_AFMT_Q8_K, q)
    y = torch.empty((T, cfg.H), dtype=torch.float32, device="cuda")
    ws = dl.workspace(T)
    M.moe_expert_ffn(dl.desc, q, xt, M.MOE_DTYPE_F32, T, torch.from_numpy(ids).cuda(),
                     torch.from_numpy(w).cuda(), y, ws, ws.numel())
    torch.cuda.synchronize()
    L = oracle.Layer(data)
    for t in range(T):
        assert rel_err(y[t].cpu().numpy(), L.expert_part(x[t], ids[t], w[t])) <= Y_TOL, t


def test_grouped_dense_k_equals_E():
    """Every token routed to every expert: each expert gets 40 pairs (3 tiles)."""
    cfg = gen.CONFIGS["tiny"].with_(k=8)
    check_layer(cfg, T=40, x_index=1, path=GP)


def test_grouped_biases():
    """Q4_K experts with gate/up/down biases (the register-staged tile kernels)
    and Q6_K gate/up rows."""
    check_layer(SHRUNK["kimi-k2"].with_(biases=True), T=11, x_index=5, path=GP)
    check_layer(SHRUNK["deepseek-v4-flash"].with_(fmt_gu=gen.Q6_K), T=9, x_index=5, path=GP)


def test_grouped_bf16_input():
    cfg = SHRUNK["kimi-k2"].with_(x_bf16=True)
    check_layer(cfg, T=9, x_index=4, path=GP)


def test_grouped_shared_gate_vector():
    cfg = SHRUNK["kimi-k2"]
    data = gen.make_layer(cfg, with_sh_gate_vec=True)
    check_layer(cfg, data=data, T=21, sh_gate_vec=data.sh_gate_vec, path=GP)


def test_grouped_null_experts_and_partition():
    cfg = SHRUNK["deepseek-v4-flash"].with_(shared=False)
    data = gen.make_layer(cfg)
    T = 24
    x, xb = gen.make_x(cfg, T=T, x_index=6)
    mask = np.random.default_rng(11).random(cfg.E) < 0.5
    outs = []
    for present in (None, mask, ~mask):
        dl = DeviceLayer(data, present=present, path=GP)
        xt, dt = x_to_device(data, x, xb)
        outs.append(run_layer(dl, xt, dt, T))
    (yf, idf, wf), (ya, ida, _), (yb, idb, _) = outs
    assert np.array_equal(idf, ida) and np.array_equal(idf, idb)
    assert rel_err(ya + yb, yf).max() <= 1e-5
    ref = oracle.Layer(data, present=mask).forward(x, threads=8)
    assert rel_err(ya, ref["y"]).max() <= Y_TOL


def test_grouped_all_absent():
    """No present expert and no shared expert: y = 0; only the shared expert: y = shared FFN."""
    cfg = SHRUNK["kimi-k2"]
    data = gen.make_layer(cfg)
    T = 8
    x, xb = gen.make_x(cfg, T=T, x_index=2)
    none = np.zeros(cfg.E, bool)
    dl = DeviceLayer(data, present=none, path=GP)
    xt, dt = x_to_device(data, x, xb)
    y, ids, _ = run_layer(dl, xt, dt, T)
    ref = oracle.Layer(data, present=none).forward(x, threads=8)
    assert np.array_equal(ids, ref["ids"])
    assert rel_err(y, ref["y"]).max() <= Y_TOL
    cfg2 = cfg.with_(shared=False)
    data2 = gen.make_layer(cfg2)
    dl2 = DeviceLayer(data2, present=none, path=GP)
    y2, _, _ = run_layer(dl2, xt, dt, T)
    assert not y2.any()


def test_grouped_matches_decode_path():
    """The same tokens through the grouped path (one chunk) and the per-pair path
    (chunks of <= 4 tokens): identical routing, outputs within tolerance."""
    cfg = SHRUNK["deepseek-v4-flash"]
    data = gen.make_layer(cfg)
    T = 12
    x, xb = gen.make_x(cfg, T=T, x_index=9)
    dl = DeviceLayer(data, path=GP)
    dlp = DeviceLayer(data, path=M.MOE_PATH_GEMV)
    xt, dt = x_to_device(data, x, xb)
    yg, idg, wg = run_layer(dl, xt, dt, T)
    parts = [run_layer(dlp, xt[i:i + 4].contiguous(), dt, 4) for i in range(0, T, 4)]
    yd = np.concatenate([p[0] for p in parts])
    idd = np.concatenate([p[1] for p in parts])
    wd = np.concatenate([p[2] for p in parts])
    assert np.array_equal(idg, idd)
    assert np.abs(wg - wd).max() <= 1e-6
    assert rel_err(yg, yd).max() <= Y_TOL


def test_grouped_expert_ffn_invalid_ids():
    """Caller-given routing with out-of-range ids: those slots contribute nothing."""
    cfg = SHRUNK["kimi-k2"].with_(shared=False)
    data = gen.make_layer(cfg)
    T = 10
    x, _ = gen.make_x(cfg, T=T, x_index=8)
    rng = np.random.default_rng(3)
    ids = np.stack([rng.choice(cfg.E, cfg.k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, cfg.k)).astype(np.float32)
    bad = ids.copy()
    bad[:, 0] = -1
    bad[2, 1] = cfg.E
    dl = DeviceLayer(data, path=GP)
    xt = torch.from_numpy(x).cuda()
    qs = torch.empty((T, cfg.H), dtype=torch.int8, device="cuda")
    d = torch.empty((T, cfg.H // 256), dtype=torch.float32, device="cuda")
    bs = torch.empty((T, cfg.H // 16), dtype=torch.int16, device="cuda")
    q = M.qact(qs, d, bs, M.MOE_AFMT_Q8_K, T, cfg.H)
    M.moe_quantize_act_q8k(xt, M.MOE_DTYPE_F32, T, cfg.H, M.MOE_AFMT_Q8_K, q)
    y = torch.empty((T, cfg.H), dtype=torch.float32, device="cuda")
    ws = dl.workspace(T)
    M.moe_expert_ffn(dl.desc, q, xt, M.MOE_DTYPE_F32, T, torch.from_numpy(bad).cuda(),
                     torch.from_numpy(w).cuda(), y, ws, ws.numel())
    torch.cuda.synchronize()
    yg = y.cpu().numpy()
    L = oracle.Layer(data)
    for t in range(T):
        ref = L.expert_part(x[t], bad[t], w[t])
        keep = (bad[t] >= 0) & (bad[t] < cfg.E)
        ref_valid = L.expert_part(x[t], np.where(keep, bad[t], ids[t]), np.where(keep, w[t], 0))
        assert np.array_equal(ref, ref_valid)  # the oracle drops those slots too
        assert rel_err(yg[t], ref) <= Y_TOL, t


def test_grouped_full_kimi_k2():
    """Kimi-K2-shaped layer at full size (384 experts, H 7168, F 2048, 9.5 GB of
    Q4_K experts), one 256-token chunk as the benchmark runs it (experts in
    64-row tiles), and the same chunk over row-order experts (identical bytes
    out). Routing (ids exact, weights within 1e-6) is checked on all 256
    tokens against the oracle's router and top-k; the layer output on 40
    tokens (first, last and a spread in between)."""
    cfg = gen.CONFIGS["kimi-k2"]
    say("kimi-k2 full: generating the layer")
    data = gen.make_layer(cfg)
    T = cfg.T
    x, xb = gen.make_x(cfg, T=T, x_index=0)
    dl = DeviceLayer(data, layout=TILE)
    xt, dt = x_to_device(data, x, xb)
    y, ids, w = run_layer(dl, xt, dt, T)
    del dl
    say("kimi-k2 full: row-order experts")
    dr = DeviceLayer(data, layout=M.MOE_LAYOUT_ROWS)
    yr, idr, wr = run_layer(dr, xt, dt, T)
    del dr
    assert np.array_equal(ids, idr) and np.array_equal(w, wr)
    assert np.array_equal(y.view(np.uint32), yr.view(np.uint32))
    say("kimi-k2 full: oracle routing of all 256 tokens")
    for t in range(T):
        lg = oracle.router_logits(data.w_router, x[t])
        ref_ids = oracle.topk(lg, cfg.k, data.sel_bias)
        ref_w = oracle.route_weights(lg, ref_ids, cfg.router, cfg.norm_topk, cfg.route_scale)
        assert np.array_equal(ids[t], ref_ids), t
        assert np.abs(w[t] - ref_w).max() <= 1e-6, t
    tokens = sorted(set([0, 1, 2, 127, 128, 200, 254, 255] + list(range(3, 256, 8))))
    assert len(tokens) >= 32
    say(f"kimi-k2 full: oracle layer output on {len(tokens)} tokens")
    ref = oracle.Layer(data).forward(x, tokens=tokens, threads=16)
    assert np.array_equal(ids[tokens], ref["ids"])
    err = rel_err(y[tokens], ref["y"])
    say(f"  max rel err {err.max():.3e} over {len(tokens)} tokens")
    assert err.max() <= Y_TOL, err
