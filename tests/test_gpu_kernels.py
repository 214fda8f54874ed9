"""GPU parity of the individual steps: q8 activations (bit-exact), integer block
partials (exact), router ids (exact) and weights."""
import numpy as np
import pytest
import torch

import gen
import oracle
import quantized_moe_expert_route_amd as M
from gen.device import DeviceLayer, x_to_device
from tests.gpu_common import random_blocks, upload_q8, x_cases, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("afmt,B", [(M.MOE_AFMT_Q8_K, 256), (M.MOE_AFMT_Q8_32, 32)])
@pytest.mark.parametrize("T,H", [(1, 512), (5, 2048), (3, 7168), (2, 2880)])
@pytest.mark.parametrize("bf16", [False, True])
def test_quantize_bitexact(afmt, B, T, H, bf16):
    if H % B:
        pytest.skip("width not a multiple of the block")
    say(f"quant afmt={afmt} T={T} H={H} bf16={bf16}")
    x = x_cases(T, H, 3)
    if bf16:
        xb = gen.round_bf16(x)
        x = gen.bf16_to_f32(xb)
        xt = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
        dt = M.MOE_DTYPE_BF16
    else:
        xt = torch.from_numpy(x).cuda()
        dt = M.MOE_DTYPE_F32
    qs = torch.empty((T, H), dtype=torch.int8, device="cuda")
    d = torch.empty((T, H // B), dtype=torch.float32, device="cuda")
    bs = torch.empty((T, H // 16), dtype=torch.int16, device="cuda") if B == 256 else None
    q = M.qact(qs, d, bs, afmt, T, H)
    M.moe_quantize_act_q8k(xt, dt, T, H, afmt, q)
    torch.cuda.synchronize()
    for t in range(T):
        rq, rd, rb = oracle.quantize_q8(x[t], B)
        assert np.array_equal(qs[t].cpu().numpy(), rq), t
        assert np.array_equal(d[t].cpu().numpy().view(np.uint32), rd.view(np.uint32)), t
        if B == 256:
            assert np.array_equal(bs[t].cpu().numpy(), rb), t


# MXFP4 widths cover every plan of the realigning routine (pieces per lane and
# blocks per lane: 96 -> 1/1, 1024 -> 2/1, 2048 -> 3/1, 2880 -> 3/2 with the
# tail blocks folded onto spare lanes, 4096 -> 5/2, 8192 -> 9/4) and a width
# past them (8224: the per-block routine).
@pytest.mark.parametrize("fmt,K", [(gen.Q4_K, 512), (gen.Q4_K, 7168), (gen.Q6_K, 768),
                                   (gen.Q6_K, 2048), (gen.MXFP4, 2880), (gen.MXFP4, 96),
                                   (gen.MXFP4, 1024), (gen.MXFP4, 2048), (gen.MXFP4, 4096),
                                   (gen.MXFP4, 8192), (gen.MXFP4, 8224),
                                   (gen.Q5_K, 256), (gen.Q5_K, 2048), (gen.Q2_K, 256),
                                   (gen.Q2_K, 2048), (gen.Q3_K, 256), (gen.Q3_K, 2048),
                                   (gen.Q3_K, 7168), (gen.Q4_0, 32), (gen.Q4_0, 96),
                                   (gen.Q4_0, 2880), (gen.Q5_1, 64), (gen.Q5_1, 2880),
                                   (gen.Q5_1, 4096)])
@pytest.mark.parametrize("kind", ["generated", "random_fields"])
def test_block_dots_exact(fmt, K, kind):
    say(f"block_dots fmt={fmt} K={K} {kind}")
    B = gen.BLOCK_ELEMS[fmt]  # q8 block of the activations these rows consume
    n_rows = 37
    rng = np.random.default_rng(fmt * 100 + K)
    if kind == "generated":
        w = gen.normal(5, gen.T_DOWN, fmt, n_rows, K, 0.02)
        w[0] = 0
        mat = gen.encode_matrix(fmt, w)
    else:
        raw = random_blocks(fmt, n_rows, K, rng)
        stride = gen.row_stride(fmt, K)
        mat = np.zeros((n_rows, stride), np.uint8)
        mat[:, :raw.shape[1]] = raw
    x = x_cases(3, K, 9)
    host, q, keep = upload_q8(x, B)
    rows = torch.from_numpy(mat).cuda()
    nb = K // gen.BLOCK_ELEMS[fmt]
    for token in range(3):
        out = torch.full((n_rows, nb, 2), -7, dtype=torch.int32, device="cuda")
        M.moe_test_block_dots(fmt, rows, n_rows, K, mat.shape[1], q, token, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        for r in range(n_rows):
            ref = oracle.block_partials(fmt, mat[r], K, host[0][token],
                                        host[2][token] if B == 256 else None)
            assert np.array_equal(got[r], ref), (token, r)


def _route(dl, xt, dt, T, logits=True):
    cfg = dl.cfg
    ids = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
    lg = torch.empty((T, cfg.E), dtype=torch.float32, device="cuda") if logits else None
    ws = dl.workspace(T)
    M.moe_route_topk(dl.desc, xt, dt, T, ids, w, lg, ws, ws.numel())
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy(), None if lg is None else lg.cpu().numpy()


ROUTER_CASES = [("tiny", 5), ("qwen3.6-35b-a3b", 9), ("gpt-oss-20b", 3),
                ("deepseek-v4-flash", 16), ("kimi-k2", 40)]


@pytest.mark.parametrize("name,T", ROUTER_CASES)
def test_route_topk(name, T):
    cfg = gen.CONFIGS[name]
    say(f"route {name} T={T}")
    data = gen.make_layer(cfg, experts=[])
    x, xb = gen.make_x(cfg, T=T, x_index=5)
    dl = DeviceLayer(data)
    xt, dt = x_to_device(data, x, xb)
    ids, w, lg = _route(dl, xt, dt, T)
    L = oracle.Layer(data)
    for t in range(T):
        ref_l = oracle.router_logits(data.w_router, x[t])
        ulp = np.spacing(np.abs(ref_l))
        assert np.all(np.abs(lg[t].astype(np.float64) - ref_l) <= ulp)
        ref_ids = oracle.topk(ref_l, cfg.k, data.sel_bias)
        ref_w = oracle.route_weights(ref_l, ref_ids, cfg.router, cfg.norm_topk, cfg.route_scale)
        assert np.array_equal(ids[t], ref_ids), t
        assert np.abs(w[t] - ref_w).max() <= 1e-6
    _ = L


def test_route_ties_and_zero_input():
    cfg = gen.CONFIGS["qwen3.6-35b-a3b"].with_(E=64, k=8)
    data = gen.make_layer(cfg, experts=[])
    # duplicate router rows create exact logit ties
    W = data.w_router
    W[10] = W[3]
    W[40] = W[3]
    W[7] = W[20]
    data.w_router = np.ascontiguousarray(W)
    x, _ = gen.make_x(cfg, T=6)
    x[0] = 0.0
    x[1] = W[3] / np.linalg.norm(W[3]) * 10  # makes experts 3, 10, 40 the top three
    dl = DeviceLayer(data)
    ids, w, lg = _route(dl, torch.from_numpy(x).cuda(), M.MOE_DTYPE_F32, 6)
    assert list(ids[0]) == list(range(8))
    assert np.allclose(w[0], 1 / 8, atol=1e-7)
    assert list(ids[1][:3]) == [3, 10, 40]
    for t in range(6):
        ref_l = oracle.router_logits(data.w_router, x[t])
        assert np.array_equal(ids[t], oracle.topk(ref_l, cfg.k)), t
    # sigmoid router, unnormalized, with route scale
    cfg2 = cfg.with_(router=gen.SIGMOID, norm_topk=0, route_scale=2.5)
    data2 = gen.make_layer(cfg2, experts=[])
    dl2 = DeviceLayer(data2)
    ids2, w2, _ = _route(dl2, torch.from_numpy(x).cuda(), M.MOE_DTYPE_F32, 6, logits=False)
    for t in range(6):
        ref_l = oracle.router_logits(data2.w_router, x[t])
        rid = oracle.topk(ref_l, cfg.k)
        assert np.array_equal(ids2[t], rid)
        assert np.abs(w2[t] - oracle.route_weights(ref_l, rid, gen.SIGMOID, 0, 2.5)).max() <= 2e-6
    # softmax over all experts (norm_topk = 0)
    cfg3 = cfg.with_(norm_topk=0)
    data3 = gen.make_layer(cfg3, experts=[])
    dl3 = DeviceLayer(data3)
    ids3, w3, _ = _route(dl3, torch.from_numpy(x).cuda(), M.MOE_DTYPE_F32, 6, logits=False)
    for t in range(6):
        ref_l = oracle.router_logits(data3.w_router, x[t])
        rid = oracle.topk(ref_l, cfg.k)
        assert np.array_equal(ids3[t], rid)
        assert np.abs(w3[t] - oracle.route_weights(ref_l, rid, gen.SOFTMAX, 0)).max() <= 1e-6


@pytest.mark.parametrize("E,router", [(256, gen.SOFTMAX), (384, gen.SIGMOID), (1024, gen.SOFTMAX)])
def test_route_ties_across_registers(E, router):
    """Exact logit ties between experts held in different registers and lanes of
    the top-k wave (expert e sits in lane e % 64, register e // 64): the lowest
    index must win. Checked through the routing entry point, the decode layer
    (top-k inside the gate/up kernel) and the multi-token layer."""
    cfg = gen.CONFIGS["qwen3.6-35b-a3b"].with_(name="ties", E=E, k=8, H=512, F=256,
                                               router=router, norm_topk=1)
    data = gen.make_layer(cfg, experts=[])
    W = data.w_router
    top = [5, 69, 133, 197]            # one lane, four registers
    for e in top[1:]:
        W[e] = W[top[0]]
    W[70] = W[6]                       # lane 6, registers 1 and 0
    W[E - 1] = W[2]                    # last expert ties with an early one
    data.w_router = np.ascontiguousarray(W)
    T = 6
    x, _ = gen.make_x(cfg, T=T)
    x[0] = 0.0                                         # every logit equal
    x[1] = W[5] / np.linalg.norm(W[5]) * 10            # the four tied rows on top
    x[2] = W[6] / np.linalg.norm(W[6]) * 10
    x[3] = W[2] / np.linalg.norm(W[2]) * 10
    xt = torch.from_numpy(x).cuda()
    refs = [oracle.topk(oracle.router_logits(data.w_router, x[t]), cfg.k) for t in range(T)]
    assert list(refs[0]) == list(range(8))
    assert list(refs[1][:4]) == top
    assert list(refs[2][:2]) == [6, 70]
    assert list(refs[3][:2]) == [2, E - 1]
    dl = DeviceLayer(data)
    ids, _, _ = _route(dl, xt, M.MOE_DTYPE_F32, T, logits=False)
    say(f"ties E={E}: route entry point")
    for t in range(T):
        assert np.array_equal(ids[t], refs[t]), ("route", t, ids[t], refs[t])
    for Tl in (1, T):                  # decode path per token, then the grouped path
        y = torch.empty((Tl, cfg.H), dtype=torch.float32, device="cuda")
        idl = torch.empty((Tl, cfg.k), dtype=torch.int32, device="cuda")
        wl = torch.empty((Tl, cfg.k), dtype=torch.float32, device="cuda")
        ws = dl.workspace(Tl)
        for t0 in range(0, T, Tl):
            M.moe_layer_forward(dl.desc, xt[t0:t0 + Tl].contiguous(), M.MOE_DTYPE_F32, Tl, y,
                                idl, wl, ws, ws.numel())
            torch.cuda.synchronize()
            got = idl.cpu().numpy()
            for i in range(Tl):
                assert np.array_equal(got[i], refs[t0 + i]), ("layer", Tl, t0 + i, got[i])


@pytest.mark.parametrize("E,router", [(256, gen.SOFTMAX), (384, gen.SIGMOID)])
def test_decode_ties_outputs(E, router):
    """Decode outputs under exact logit ties: every gate/up workgroup other than
    the first of a pair selects its own slot's expert (the rank-n selection,
    whose exact rounds run only after a tie), so a wrong choice among tied
    experts changes y. The tied experts get distinct weights; y is checked
    against the oracle token by token."""
    from tests.gpu_common import Y_TOL, rel_err
    cfg = gen.CONFIGS["qwen3.6-35b-a3b"].with_(name="ties-y", E=E, k=8, H=512, F=256,
                                               router=router, norm_topk=1)
    base = gen.make_layer(cfg, experts=[])
    W = base.w_router
    for e in (69, 133, 197):
        W[e] = W[5]
    W[70] = W[6]
    W[E - 1] = W[2]
    x, _ = gen.make_x(cfg, T=4)
    x[0] = 0.0
    x[1] = W[5] / np.linalg.norm(W[5]) * 10
    x[2] = W[6] / np.linalg.norm(W[6]) * 10
    x[3] = W[2] / np.linalg.norm(W[2]) * 10
    used = set()
    for t in range(4):
        used |= {int(e) for e in oracle.topk(oracle.router_logits(W, x[t]), cfg.k)}
    if cfg.shared:
        used.add(cfg.E)
    data = gen.make_layer(cfg, experts=sorted(used))
    data.w_router = np.ascontiguousarray(W)
    dl = DeviceLayer(data)
    L = oracle.Layer(data)
    y = torch.empty((1, cfg.H), dtype=torch.float32, device="cuda")
    idl = torch.empty((1, cfg.k), dtype=torch.int32, device="cuda")
    wl = torch.empty((1, cfg.k), dtype=torch.float32, device="cuda")
    ws = dl.workspace(1)
    for t in range(4):
        say(f"decode ties E={E} token {t}")
        M.moe_layer_forward(dl.desc, torch.from_numpy(x[t:t + 1]).cuda(), M.MOE_DTYPE_F32, 1, y,
                            idl, wl, ws, ws.numel())
        torch.cuda.synchronize()
        ref = L.forward(x[t:t + 1])
        assert np.array_equal(idl.cpu().numpy()[0], ref["ids"][0]), t
        assert rel_err(y.cpu().numpy()[0], ref["y"][0]) <= Y_TOL, t


def _tie_rows(W, rng, E, n_tied, base, per_group):
    """Rows of n_tied experts made identical to row `base`; with per_group, at
    least one of them in each group of 8 top-k lanes (expert e sits in lane
    e % 64), so that every group maximum is the tied key."""
    pool = [e for e in range(E) if e != base]
    tied = set()
    if per_group:
        for g in range(8):
            lanes = [e for e in pool if (e % 64) // 8 == g]
            tied.add(int(rng.choice(lanes)))
    rest = [e for e in pool if e not in tied]
    tied |= {int(e) for e in rng.choice(rest, n_tied - 1 - len(tied), replace=False)}
    for e in tied:
        W[e] = W[base]
    return sorted(tied | {base})


@pytest.mark.parametrize("case", ["tied60", "tied70", "boundary", "spread"])
def test_topk_candidate_threshold(case):
    """The one-pass top-k ranks the keys that reach the smallest of 8 lane-group
    maxima when there are at most 64 of them, and falls back to rounds
    otherwise. Equal top keys just under and over 64 (every group holding one),
    equal keys straddling rank k, and a tie group without a member in some
    lane groups: ids through the routing entry point and the decode layer, and
    the decode output against the oracle."""
    from tests.gpu_common import Y_TOL, rel_err
    E = 256
    cfg = gen.CONFIGS["qwen3.6-35b-a3b"].with_(name="cand-" + case, E=E, k=8, H=512, F=256,
                                               router=gen.SOFTMAX, norm_topk=1)
    base = gen.make_layer(cfg, experts=[])
    W = base.w_router
    rng = np.random.default_rng(11)
    b = 37
    if case == "tied60":
        tied = _tie_rows(W, rng, E, 60, b, True)
    elif case == "tied70":
        tied = _tie_rows(W, rng, E, 70, b, True)
    elif case == "boundary":
        tied = _tie_rows(W, rng, E, 12, b, False)
        tops = [e for e in range(E) if e not in tied][::51][:5]
        for i, e in enumerate(tops):          # five distinct keys above the tied ones
            W[e] = W[b] * np.float32(1.5 + 0.1 * i)
    else:                                    # tie group absent from some lane groups
        tied = [b, 37 + 64, 37 + 128, 37 + 192, 40, 41]
        for e in tied:
            W[e] = W[b]
    x = np.zeros((2, cfg.H), np.float32)
    x[0] = W[b] / np.linalg.norm(W[b]) * 10
    x[1] = W[b] / np.linalg.norm(W[b]) * 10 + rng.standard_normal(cfg.H).astype(np.float32) * 0.5
    refs = [oracle.topk(oracle.router_logits(W, x[t]), cfg.k) for t in range(2)]
    if case in ("tied60", "tied70"):
        assert list(refs[0]) == tied[:8]
    used = {int(e) for r in refs for e in r} | {cfg.E}
    data = gen.make_layer(cfg, experts=sorted(used))
    data.w_router = np.ascontiguousarray(W)
    dl = DeviceLayer(data)
    xt = torch.from_numpy(x).cuda()
    ids, _, _ = _route(dl, xt, M.MOE_DTYPE_F32, 2, logits=False)
    for t in range(2):
        assert np.array_equal(ids[t], refs[t]), (case, "route", t, ids[t], refs[t])
    L = oracle.Layer(data)
    y = torch.empty((1, cfg.H), dtype=torch.float32, device="cuda")
    idl = torch.empty((1, cfg.k), dtype=torch.int32, device="cuda")
    wl = torch.empty((1, cfg.k), dtype=torch.float32, device="cuda")
    ws = dl.workspace(1)
    for t in range(2):
        say(f"candidate top-k {case} token {t}")
        M.moe_layer_forward(dl.desc, xt[t:t + 1].contiguous(), M.MOE_DTYPE_F32, 1, y, idl, wl,
                            ws, ws.numel())
        torch.cuda.synchronize()
        ref = L.forward(x[t:t + 1])
        assert np.array_equal(idl.cpu().numpy()[0], ref["ids"][0]), (case, t)
        assert rel_err(y.cpu().numpy()[0], ref["y"][0]) <= Y_TOL, (case, t)
