"""Oracle pins for the whole layer: brute force and closed forms (CPU)."""
import numpy as np
import pytest

import gen
import oracle
from tests.brute import brute_layer, dense_experts
from tests.shrunk import SHRUNK


def _rel(a, b):
    return np.abs(a - b).max() / max(np.linalg.norm(b), 1e-300)


@pytest.mark.parametrize("name", list(SHRUNK))
def test_layer_matches_dense_brute_force(orc, genlib, name):
    cfg = SHRUNK[name]
    data = gen.make_layer(cfg)
    x, _ = gen.make_x(cfg, T=cfg.T)
    L = oracle.Layer(data)
    out = L.forward(x)
    yb, idb, wb = brute_layer(data, x)
    assert np.array_equal(out["ids"], idb)
    assert np.allclose(out["w"], wb, rtol=1e-12, atol=0)
    for t in range(x.shape[0]):
        assert _rel(out["y"][t], yb[t]) <= 1e-9, (name, t)


@pytest.mark.parametrize("fmt_gu,fmt_d", [(gen.Q3_K, gen.Q3_K), (gen.Q4_0, gen.Q4_0),
                                          (gen.Q5_1, gen.Q5_1), (gen.Q4_0, gen.Q3_K),
                                          (gen.Q3_K, gen.Q5_1), (gen.Q4_K, gen.Q4_0)])
def test_layer_formats_match_dense_brute_force(orc, genlib, fmt_gu, fmt_d):
    """Layers with Q3_K, Q4_0 and Q5_1 matrices (and mixes): the oracle equals a
    brute-force fp64 FFN on the dequantized matrices, with q8 blocks of 32 for
    the 32-weight formats."""
    cfg = SHRUNK["qwen3.6-35b-a3b"].with_(fmt_gu=fmt_gu, fmt_d=fmt_d)
    data = gen.make_layer(cfg)
    x, _ = gen.make_x(cfg, T=cfg.T, x_index=1)
    ref = oracle.Layer(data).forward(x)
    yb, idb, wb = brute_layer(data, x)
    assert np.array_equal(ref["ids"], idb)
    for t in range(cfg.T):
        assert np.abs(ref["y"][t] - yb[t]).max() <= 1e-9 * np.linalg.norm(yb[t])


def test_shared_gate_vector_brute_force(orc, genlib):
    cfg = SHRUNK["qwen3.6-35b-a3b"]
    data = gen.make_layer(cfg, with_sh_gate_vec=True)
    x, _ = gen.make_x(cfg, T=2)
    L = oracle.Layer(data, sh_gate_vec=data.sh_gate_vec)
    out = L.forward(x)
    yb, _, _ = brute_layer(data, x, sh_gate_vec=data.sh_gate_vec)
    for t in range(2):
        assert _rel(out["y"][t], yb[t]) <= 1e-9
    # the gate changes the result compared with weight 1
    y1 = oracle.Layer(data).forward(x)["y"]
    assert _rel(out["y"][0], y1[0]) > 1e-3


def test_k_equals_E_is_dense_softmax_mixture(orc, genlib):
    cfg = gen.CONFIGS["tiny"].with_(k=8)
    data = gen.make_layer(cfg)
    x, _ = gen.make_x(cfg, T=2)
    out = oracle.Layer(data).forward(x)
    dense = dense_experts(data, range(cfg.E))
    for t in range(2):
        assert sorted(out["ids"][t]) == list(range(8))
        logits = (data.w_router.astype(np.float64) @ x[t].astype(np.float64)).astype(np.float32)
        p = np.exp(logits.astype(np.float64) - logits.max())
        p /= p.sum()
        # each expert's FFN via the oracle with one expert present at weight 1
        y = np.zeros(cfg.H)
        for e in range(cfg.E):
            mask = np.zeros(cfg.E, bool)
            mask[e] = True
            ye = oracle.Layer(data, present=mask).expert_part(
                x[t], np.array([e] + [0] * 7, np.int32), np.array([1.0] + [0.0] * 7, np.float32))
            y += p[e] * ye
        assert _rel(out["y"][t], y) <= 1e-12


def test_zero_input(orc, genlib):
    for name in ("tiny", "qwen3.6-35b-a3b", "kimi-k2"):
        cfg = SHRUNK[name]
        data = gen.make_layer(cfg)
        L = oracle.Layer(data, sel_bias=None)
        r = L.token(np.zeros(cfg.H, np.float32))
        assert list(r["ids"]) == list(range(cfg.k))
        assert np.allclose(r["w"], 1.0 / cfg.k, rtol=1e-15)
        assert not r["y"].any()
    # with biases only the biases reach the output
    cfg = SHRUNK["gpt-oss-20b"]
    data = gen.make_layer(cfg)
    r = oracle.Layer(data).token(np.zeros(cfg.H, np.float32))
    assert list(r["ids"]) == list(range(cfg.k))
    yb, _, _ = brute_layer(data, np.zeros((1, cfg.H), np.float32))
    assert _rel(r["y"], yb[0]) <= 1e-9 and np.linalg.norm(r["y"]) > 0


def test_identical_experts_ignore_routing(orc, genlib):
    cfg = SHRUNK["qwen3.6-35b-a3b"].with_(shared=False)
    data = gen.make_layer(cfg)
    data.pool[:] = data.pool[0]
    x, _ = gen.make_x(cfg, T=3)
    out = oracle.Layer(data).forward(x)
    for t in range(3):
        ref = oracle.Layer(data).expert_part(x[t], np.array([5] + [0] * 7, np.int32),
                                             np.array([1.0] + [0.0] * 7, np.float32))
        assert _rel(out["y"][t], ref) <= 1e-13


def test_expert_permutation(orc, genlib):
    cfg = SHRUNK["deepseek-v4-flash"]
    data = gen.make_layer(cfg)
    x, _ = gen.make_x(cfg, T=3)
    out = oracle.Layer(data).forward(x)
    perm = np.random.default_rng(0).permutation(cfg.E)  # new expert i = old expert perm[i]
    inv = np.argsort(perm)
    d2 = gen.make_layer(cfg.with_(E=cfg.E), experts=[])
    d2.w_router = np.ascontiguousarray(data.w_router[perm])
    d2.sel_bias = np.ascontiguousarray(data.sel_bias[perm])
    d2.pool[: cfg.E] = data.pool[perm]
    d2.pool[cfg.E] = data.pool[cfg.E]
    out2 = oracle.Layer(d2).forward(x)
    assert np.array_equal(out2["ids"], inv[out["ids"]])
    assert np.array_equal(out2["y"], out["y"])


def test_route_scale_linear(orc, genlib):
    cfg = SHRUNK["kimi-k2"].with_(shared=False)
    data = gen.make_layer(cfg)
    x, _ = gen.make_x(cfg, T=2)
    y1 = oracle.Layer(data).forward(x)["y"]
    y2 = oracle.Layer(data, route_scale=2.0).forward(x)["y"]
    assert np.array_equal(y2, 2.0 * y1)
    y3 = oracle.Layer(data, route_scale=2.5).forward(x)["y"]
    assert np.allclose(y3, 2.5 * y1, rtol=1e-14, atol=1e-16)


@pytest.mark.parametrize("name", ["qwen3.6-35b-a3b", "gpt-oss-20b", "deepseek-v4-flash"])
def test_null_mask_partition(orc, genlib, name):
    cfg = SHRUNK[name]
    data = gen.make_layer(cfg)
    x, _ = gen.make_x(cfg, T=3)
    mask = np.random.default_rng(1).random(cfg.E) < 0.5
    full = oracle.Layer(data, use_shared=False).forward(x)
    a = oracle.Layer(data, present=mask, use_shared=False).forward(x)
    b = oracle.Layer(data, present=~mask, use_shared=False).forward(x)
    assert np.array_equal(a["ids"], full["ids"]) and np.array_equal(a["w"], full["w"])
    for t in range(3):
        assert _rel(a["y"][t] + b["y"][t], full["y"][t]) <= 1e-13
    # brute force agrees with the masked oracle (weights are not renormalized)
    ya, _, _ = brute_layer(data, x, present=mask)
    if cfg.shared:
        ysh, _, _ = brute_layer(data, x, present=np.zeros(cfg.E, bool))
        ya = ya - ysh
    for t in range(3):
        assert _rel(a["y"][t], ya[t]) <= 1e-9


def test_expert_part_matches_layer(orc, genlib):
    cfg = SHRUNK["kimi-k2"]
    data = gen.make_layer(cfg)
    x, _ = gen.make_x(cfg, T=2)
    L = oracle.Layer(data)
    out = L.forward(x)
    for t in range(2):
        y = L.expert_part(x[t], out["ids"][t], out["w"][t].astype(np.float32))
        assert _rel(y, out["y"][t]) <= 1e-7  # fp32-rounded weights


def test_full_size_decode_token(orc, genlib):
    """One full-size token on the Qwen3.6-shaped decode layer against brute force
    restricted to the selected experts."""
    cfg = gen.CONFIGS["qwen3.6-35b-a3b"]
    data = gen.make_layer(cfg)
    L = oracle.Layer(data)
    r = L.token(data.x[0])
    sel = sorted(set(r["ids"].tolist())) + [cfg.E]
    dense = dense_experts(data, sel)
    yb, idb, _ = brute_layer(data, data.x[:1], dense=dense)
    assert np.array_equal(idb[0], r["ids"])
    assert _rel(r["y"], yb[0]) <= 1e-9


def test_out_of_range_ids_contribute_nothing(orc, genlib):
    """Given routing may carry ids outside [0, E) (a slot that is "not mine"):
    such a slot adds nothing, exactly as a slot of weight 0 does, and equals the
    brute-force sum over the remaining slots."""
    cfg = SHRUNK["kimi-k2"].with_(shared=False)
    data = gen.make_layer(cfg)
    x, _ = gen.make_x(cfg, T=1)
    L = oracle.Layer(data)
    ids = np.arange(cfg.k, dtype=np.int32) * 2
    w = np.linspace(0.5, 1.0, cfg.k).astype(np.float32)
    for bad in (-1, cfg.E, 1 << 30):
        ib = ids.copy()
        ib[3] = bad
        y_bad = L.expert_part(x[0], ib, w)
        wz = w.copy()
        wz[3] = 0.0
        assert np.array_equal(y_bad, L.expert_part(x[0], ids, wz))
    with pytest.raises(ValueError):
        L.expert_part(x[0], ids[:3], w[:3])
