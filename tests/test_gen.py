"""Properties of the seeded input generator (CPU)."""
import numpy as np
import pytest
import torch

import gen


def test_streams_deterministic_and_thread_independent(genlib):
    a = gen.normal(7, gen.T_X, 3, 37, 515, 1.0, threads=1)
    b = gen.normal(7, gen.T_X, 3, 37, 515, 1.0, threads=5)
    assert np.array_equal(a, b)
    c = gen.normal(7, gen.T_X, 4, 37, 515, 1.0, threads=1)
    assert not np.array_equal(a, c)
    # a row only depends on its own stream
    r = gen.normal(7, gen.T_X, 3, 1, 515, 1.0)
    assert np.array_equal(r[0], a[0])


def test_normal_moments(genlib):
    x = gen.normal(1, gen.T_ROUTER, 0, 400, 2500, 0.02).astype(np.float64).ravel()
    n = x.size
    assert abs(x.mean()) < 5 * 0.02 / np.sqrt(n)
    assert abs(x.std() / 0.02 - 1) < 5 / np.sqrt(2 * n)
    kurt = ((x - x.mean()) ** 4).mean() / x.var() ** 2
    assert abs(kurt - 3.0) < 0.05
    # tail mass beyond 3 sigma ~ 0.0027
    assert abs((np.abs(x) > 0.06).mean() - 0.0027) < 0.0005


def test_bf16_rounding_matches_torch(genlib):
    x = gen.normal(3, gen.T_X, 0, 64, 1024, 1.0).ravel()
    x = np.concatenate([x, np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0],
                                    np.float32)])
    ours = gen.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_fp16_ceil(genlib):
    vals = np.concatenate([np.abs(gen.normal(5, 1, 0, 1, 4000, 1e-3)[0]).astype(np.float64),
                           [1e-9, 2 ** -24, 2 ** -14, 1.0, 1.0 + 2 ** -11, 65504.0, 3e-8]])
    for v in vals:
        bits = gen.fp16_ceil_bits(v)
        h = np.array([bits], np.uint16).view(np.float16)[0]
        assert float(h) >= v
        # the next smaller fp16 must be below v
        if bits > 0:
            lower = np.array([bits - 1], np.uint16).view(np.float16)[0]
            assert float(lower) < v


def test_zipf_bias(genlib):
    E, s = 256, 1.1
    b = gen.zipf_bias(3, E, s).astype(np.float64)
    p = np.exp(b)
    assert abs(p.sum() - 1) < 1e-5
    ps = np.sort(p)[::-1]
    ranks = np.arange(1, E + 1)
    expect = ranks ** -s / (ranks ** -s).sum()
    assert np.allclose(ps, expect, rtol=1e-5)
    # it is a permutation: every rank used once
    assert len(np.unique(np.round(np.log(ps) * 1e6))) == E


def test_config_shapes(genlib):
    c = gen.CONFIGS
    assert c["tiny"].expert_algo_bytes == 221184
    assert c["qwen3.6-35b-a3b"].expert_algo_bytes == 1769472
    assert c["gpt-oss-20b"].expert_algo_bytes == 2 * 2880 * 1530 + 2880 * 1530
    assert c["gpt-oss-20b"].stride_gu == 1536
    assert c["deepseek-v4-flash"].expert_algo_bytes == 16318464
    assert c["kimi-k2"].expert_algo_bytes == 24772608
    for cfg in c.values():
        assert cfg.stride_gu % 16 == 0 and cfg.stride_d % 16 == 0


def test_pool_layout_and_subset(genlib):
    cfg = gen.CONFIGS["tiny"]
    d = gen.make_layer(cfg)
    d2 = gen.make_layer(cfg, experts=[3])
    assert np.array_equal(d.pool[3], d2.pool[3])
    assert not d2.pool[2].any()
    # gate rows of expert 3 equal a directly generated matrix
    g = gen.weight_matrix(cfg.seed, gen.T_GATE, 3, cfg.fmt_gu, cfg.F, cfg.H, cfg.stride_gu,
                          cfg.w_std)
    assert np.array_equal(d.gate(3).reshape(cfg.F, -1), g)


@pytest.mark.parametrize("fmt,K", [(gen.Q4_K, 512), (gen.Q6_K, 256), (gen.MXFP4, 96),
                                   (gen.Q5_K, 512), (gen.Q2_K, 512), (gen.Q3_K, 512),
                                   (gen.Q4_0, 96), (gen.Q5_1, 96)])
def test_encode_matrix_padding(genlib, fmt, K):
    x = gen.normal(0, 1, 0, 3, K, 0.02)
    stride = gen.row_stride(fmt, K) + 32
    m = gen.encode_matrix(fmt, x, stride=stride)
    rb = gen.row_bytes(fmt, K)
    assert not m[:, rb:].any()
    for r in range(3):
        for b in range(K // gen.BLOCK_ELEMS[fmt]):
            blk = gen.encode_block(fmt, x[r, b * gen.BLOCK_ELEMS[fmt]:(b + 1) * gen.BLOCK_ELEMS[fmt]])
            assert np.array_equal(m[r, b * gen.BLOCK_BYTES[fmt]:(b + 1) * gen.BLOCK_BYTES[fmt]], blk)
