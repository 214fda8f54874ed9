"""Oracle pins: activation quantization and integer block dots (CPU)."""
import numpy as np
import pytest

import gen
import oracle


@pytest.mark.parametrize("B", [256, 32])
def test_q8_properties(orc, genlib, B):
    x = gen.normal(4, gen.T_X, 0, 64, 1024, 1.0)
    x[0] = 0
    x[1, :B] = 0
    x[2, 5] = 1e30
    x[3] *= 1e-30
    for r in range(x.shape[0]):
        qs, d, bs = orc.quantize_q8(x[r], B)
        for b in range(1024 // B):
            xb = x[r, b * B:(b + 1) * B].astype(np.float64)
            q = qs[b * B:(b + 1) * B].astype(np.int64)
            amax = np.abs(xb).max()
            if amax == 0:
                assert d[b] == 0 and not q.any()
                continue
            assert np.abs(q).max() == 127
            i = int(np.argmax(np.abs(xb)))
            assert q[i] == 127 * np.sign(xb[i])
            assert np.all(np.abs(q) <= 127)
            assert abs(float(d[b]) - amax / 127) <= amax / 127 * 2 ** -23
            err = np.abs(xb - float(d[b]) * q)
            assert err.max() <= float(d[b]) * (0.5 + 2 ** -15)
        if B == 256:
            assert np.array_equal(bs, qs.astype(np.int64).reshape(-1, 16).sum(1))
        else:
            assert bs is None


def test_q8_rounding_ties_to_even(orc):
    # amax = 127 gives iscale = 1 exactly, so q = rne(x)
    x = np.zeros(256, np.float32)
    x[0] = 127
    x[1:9] = [2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5, 126.5]
    qs, d, _ = orc.quantize_q8(x, 256)
    assert d[0] == np.float32(1.0)
    assert list(qs[:9]) == [127, 2, 4, -2, -4, 0, 0, 2, 126]


def test_q8_fp32_product_rounding(orc):
    """The rounding decision uses the fp32 product x*iscale (the stated recipe), which
    differs from rounding the exact product for a few inputs."""
    amax = np.float32(7.0)
    iscale = np.float32(127) / amax
    c = (np.random.default_rng(0).standard_normal(2_000_000) * 7 / 3).astype(np.float32)
    c = c[np.abs(c) <= amax]
    p32 = c * iscale
    exact = c.astype(np.float64) * np.float64(iscale)
    hit = c[np.rint(p32) != np.rint(exact)]
    assert 0 < hit.size <= 31
    x = np.zeros(32, np.float32)
    x[0] = amax
    x[1:1 + hit.size] = hit
    qs, d, _ = orc.quantize_q8(x, 32)
    got = qs[1:1 + hit.size].astype(np.int64)
    assert np.array_equal(got, np.rint(hit * iscale).astype(np.int64))
    assert not np.array_equal(got, np.rint(hit.astype(np.float64) * np.float64(iscale)))


def _rand_act(K, seed):
    x = gen.normal(seed, gen.T_X, 9, 1, K, 1.0)[0]
    return x


@pytest.mark.parametrize("fmt,K", [(gen.Q4_K, 1024), (gen.Q6_K, 1024), (gen.MXFP4, 1024),
                                   (gen.Q5_K, 1024), (gen.Q2_K, 1024), (gen.Q3_K, 1024),
                                   (gen.Q4_0, 1024), (gen.Q5_1, 1024)])
def test_block_dot_identity(orc, genlib, fmt, K):
    """Integer factorization == fp64 dot of fully dequantized weights and activations."""
    B = 32 if gen.BLOCK_ELEMS[fmt] == 32 else 256
    w = gen.normal(3, gen.T_GATE, fmt, 40, K, 0.02)
    w[0] = 0
    w[1] = np.abs(w[1])
    m = gen.encode_matrix(fmt, w)
    for seed in range(3):
        x = _rand_act(K, seed)
        qs, d, bs = orc.quantize_q8(x, B)
        a = qs.astype(np.float64) * np.repeat(d.astype(np.float64), B)
        for r in range(m.shape[0]):
            dense_terms = orc.dequant_row(fmt, m[r], K) * a
            got = orc.row_dot(fmt, m[r], K, qs, d, bs)
            assert abs(got - dense_terms.sum()) <= 1e-12 * (np.abs(dense_terms).sum() + 1e-300)


def test_q4k_integer_exact_case(orc, genlib):
    """d = 1, dmin = 0, integer x with amax 127: d8 = 1, q8(x) = x, S1 is the exact dot."""
    rng = np.random.default_rng(5)
    one = 0x3C00
    for trial in range(20):
        sc = rng.integers(0, 64, 8).astype(np.uint8)
        m = rng.integers(0, 64, 8).astype(np.uint8)
        q = rng.integers(0, 16, 256).astype(np.uint8)
        blk = gen.pack_q4k(one, 0, sc, m, q)
        x = rng.integers(-127, 128, 256).astype(np.float32)
        x[7] = 127
        qs, d, bs = orc.quantize_q8(x, 256)
        assert d[0] == 1 and np.array_equal(qs, x.astype(np.int8))
        p = orc.block_partials(oracle.Q4_K, blk, 256, qs, bs)
        s1 = sum(int(sc[j]) * int(np.dot(q[32 * j:32 * j + 32].astype(np.int64),
                                          x[32 * j:32 * j + 32].astype(np.int64)))
                 for j in range(8))
        s2 = sum(int(m[j]) * int(x[32 * j:32 * j + 32].astype(np.int64).sum()) for j in range(8))
        assert p[0, 0] == s1 and p[0, 1] == s2
        assert orc.row_dot(oracle.Q4_K, blk, 256, qs, d, bs) == float(s1)


def test_partial_ranges_fit_int32(orc, genlib):
    """Worst-case blocks: all quants at their max against amax activations."""
    x = np.full(256, 127, np.float32)
    qs, d, bs = orc.quantize_q8(x, 256)
    b4 = gen.pack_q4k(0x3C00, 0x3C00, np.full(8, 63), np.full(8, 63), np.full(256, 15))
    p = orc.block_partials(oracle.Q4_K, b4, 256, qs, bs)
    assert p[0, 0] == 63 * 15 * 127 * 256 and p[0, 1] == 63 * 127 * 256
    b6 = gen.pack_q6k(0x3C00, np.full(16, -128, np.int8), np.zeros(256, np.uint8))
    p = orc.block_partials(oracle.Q6_K, b6, 256, qs, bs)
    assert p[0, 0] == -128 * -32 * 127 * 256
    x32 = np.full(32, 127, np.float32)
    qs32, d32, _ = orc.quantize_q8(x32, 32)
    bm = gen.pack_mxfp4(127, np.full(32, 7))
    p = orc.block_partials(oracle.MXFP4, bm, 32, qs32, None)
    assert p[0, 0] == 12 * 127 * 32
    b3 = gen.pack_q3k(0x3C00, np.zeros(16, np.uint8), np.full(256, -4, np.int8))
    p = orc.block_partials(oracle.Q3_K, b3, 256, qs, bs)
    assert p[0, 0] == -32 * -4 * 127 * 256
    p = orc.block_partials(oracle.Q4_0, gen.pack_q40(0x3C00, np.zeros(32)), 32, qs32, None)
    assert p[0, 0] == -8 * 127 * 32
    p = orc.block_partials(oracle.Q5_1, gen.pack_q51(0x3C00, 0x3C00, np.full(32, 31)), 32, qs32,
                           None)
    assert p[0, 0] == 31 * 127 * 32 and p[0, 1] == 127 * 32
