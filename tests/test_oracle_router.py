"""Oracle pins: router logits, top-k, routing weights, activations (CPU)."""
import numpy as np
import pytest
import torch

import gen
import oracle


def test_router_logits_vs_fp64_matmul(orc, genlib):
    W = gen.normal(1, gen.T_ROUTER, 0, 256, 2048, 0.02)
    x = gen.normal(1, gen.T_X, 0, 8, 2048, 1.0)
    for t in range(x.shape[0]):
        got = orc.router_logits(W, x[t])
        ref64 = W.astype(np.float64) @ x[t].astype(np.float64)
        ref = ref64.astype(np.float32)
        # fp64 sums in different orders agree far below fp32 resolution: equal after rounding
        # except (vanishingly rarely) at an fp32 rounding boundary
        ulp = np.spacing(np.abs(ref))
        assert np.all(np.abs(got.astype(np.float64) - ref) <= ulp)
        assert (got == ref).mean() > 0.99


def _full_sort_topk(key, k):
    key = key.astype(np.float32)
    key = np.where(key == 0, np.float32(0), key)
    order = np.lexsort((np.arange(key.size), -key.astype(np.float64)))
    return order[:k]


@pytest.mark.parametrize("E,k", [(8, 2), (256, 8), (32, 4), (384, 8), (256, 6), (5, 5), (1, 1)])
def test_topk_equals_full_sort(orc, genlib, E, k):
    rng = np.random.default_rng(E * 31 + k)
    for trial in range(100):
        logits = rng.standard_normal(E).astype(np.float32)
        if trial % 3 == 0:  # engineered ties
            logits = np.round(logits * 2) / 2
        if trial % 5 == 0:
            logits[rng.integers(0, E, max(1, E // 4))] = logits.max()
        bias = rng.standard_normal(E).astype(np.float32) if trial % 2 else None
        ids = orc.topk(logits, k, bias)
        key = logits if bias is None else (logits + bias).astype(np.float32)
        assert np.array_equal(ids, _full_sort_topk(key, k))


def test_topk_zero_input_and_signed_zero(orc):
    ids = orc.topk(np.zeros(16, np.float32), 4)
    assert list(ids) == [0, 1, 2, 3]
    l = np.zeros(8, np.float32)
    l[[0, 1, 2]] = -0.0
    l[5] = -1
    assert list(orc.topk(l, 7)) == [0, 1, 2, 3, 4, 6, 7]


def test_selection_bias_only_selects(orc):
    l = np.array([3.0, 2.0, 1.0, 0.0], np.float32)
    b = np.array([0.0, 0.0, 0.0, 10.0], np.float32)
    ids = orc.topk(l, 2, b)
    assert list(ids) == [3, 0]
    w = orc.route_weights(l, ids, oracle.SOFTMAX)
    e = np.exp(np.array([0.0, 3.0]))
    assert np.allclose(w, e / e.sum(), rtol=1e-15)


def test_softmax_weights(orc):
    rng = np.random.default_rng(3)
    for trial in range(50):
        E, k = 64, 8
        l = (rng.standard_normal(E) * 3).astype(np.float32)
        ids = orc.topk(l, k)
        w = orc.route_weights(l, ids, oracle.SOFTMAX)
        assert abs(w.sum() - 1) < 1e-12
        ref = torch.softmax(torch.from_numpy(l[ids].astype(np.float64)), 0).numpy()
        assert np.allclose(w, ref, rtol=1e-13, atol=0)
        # equals the full softmax renormalized over the top-k
        full = torch.softmax(torch.from_numpy(l.astype(np.float64)), 0).numpy()
        assert np.allclose(w, full[ids] / full[ids].sum(), rtol=1e-12)
        wf = orc.route_weights(l, ids, oracle.SOFTMAX, norm_topk=0)
        assert np.allclose(wf, full[ids], rtol=1e-12)
        ws = orc.route_weights(l, ids, oracle.SOFTMAX, route_scale=2.5)
        assert np.allclose(ws, 2.5 * w, rtol=1e-15)


def test_sigmoid_weights(orc):
    rng = np.random.default_rng(4)
    for trial in range(50):
        E, k = 256, 6
        l = (rng.standard_normal(E) * 2).astype(np.float32)
        ids = orc.topk(l, k)
        s = torch.sigmoid(torch.from_numpy(l[ids].astype(np.float64))).numpy()
        w = orc.route_weights(l, ids, oracle.SIGMOID, norm_topk=1)
        assert abs(w.sum() - 1) < 1e-12
        assert np.allclose(w, s / s.sum(), rtol=1e-13)
        wu = orc.route_weights(l, ids, oracle.SIGMOID, norm_topk=0)
        assert np.all((wu > 0) & (wu < 1)) and np.allclose(wu, s, rtol=1e-13)
        w3 = orc.route_weights(l, ids, oracle.SIGMOID, norm_topk=1, route_scale=2.5)
        assert abs(w3.sum() - 2.5) < 1e-12


def test_swiglu_vs_torch_silu(orc):
    rng = np.random.default_rng(6)
    g = rng.standard_normal(200) * 4
    u = rng.standard_normal(200) * 4
    ref = (torch.nn.functional.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    got = np.array([orc.act(oracle.SWIGLU, a, b) for a, b in zip(g, u)])
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-300)


def test_clamped_swiglu_properties(orc):
    A, L = 1.702, 7.0
    f = lambda g, u: orc.act(oracle.SWIGLU_OAI, g, u, A, L)
    # zero gate gives zero; gate is clamped from above only; up is clamped both ways
    assert f(0.0, 3.0) == 0.0
    assert f(8.0, 1.0) == f(100.0, 1.0) == f(7.0, 1.0)
    assert f(-9.0, 1.0) != f(-8.0, 1.0)
    assert f(2.0, 9.0) == f(2.0, 7.0) and f(2.0, -9.0) == f(2.0, -7.0)
    assert f(2.0, -7.0) < 0 < f(2.0, 7.0)
    # the (up + 1) term: u = -1 zeroes the output
    assert f(1.3, -1.0) == 0.0
    # inside the clamp it is g * sigmoid(alpha g) * (u + 1); sigmoid from torch
    g, u = 1.25, 0.5
    s = torch.sigmoid(torch.tensor(A * g, dtype=torch.float64)).item()
    assert abs(f(g, u) - g * s * (u + 1)) < 1e-15
