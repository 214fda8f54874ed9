"""Pins of the oracle's MXFP8 activation mode (OCP MX v1.0 elements and shared
scale) against the spec's constants, closed forms, exhaustive properties and
a brute-force dense layer."""
import math
import os

import numpy as np
import pytest

import gen
import oracle
from tests.brute import brute_layer
from tests.shrunk import SHRUNK

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_values.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            code, val = line.split()
            rows.append((int(code, 16), float(val)))
    return rows


def test_e4m3_spec_values(orc):
    for code, want in _golden():
        got = oracle.e4m3(code)
        if math.isnan(want):
            assert math.isnan(got), hex(code)
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), hex(code)


def test_e4m3_structure(orc):
    """Strictly increasing over the finite positive codes; subnormals are equally
    spaced multiples of the smallest one; each later binade doubles the previous
    one; the sign bit negates."""
    v = [oracle.e4m3(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(v, v[1:]))
    for c in range(1, 9):
        assert v[c] == c * v[1]
    for c in range(8, 0x7F - 8):
        assert v[c + 8] == 2 * v[c]
    for c in range(0x7F):
        assert oracle.e4m3(c | 0x80) == -v[c]


def test_e4m3_round_trip_ties_and_saturation(orc):
    v = [oracle.e4m3(c) for c in range(0x7F)]
    for c in range(0x7F):
        assert oracle.e4m3_round(v[c]) == c
        assert oracle.e4m3_round(-v[c]) == (c | 0x80 if c else 0)
    for c in range(0x7E):
        mid = (v[c] + v[c + 1]) / 2  # exact in fp64
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_round(mid) == even, hex(c)
        assert oracle.e4m3_round(np.nextafter(mid, np.inf)) == c + 1
        assert oracle.e4m3_round(np.nextafter(mid, -np.inf)) == c
    # beyond the largest normal: saturation (464 would be the midpoint to 480)
    for big in (448.0001, 464.0, 480.0, 1e6, np.finfo(np.float64).max):
        assert oracle.e4m3_round(big) == 0x7E and oracle.e4m3_round(-big) == 0xFE
    # half the smallest subnormal ties to zero (even), and the result is +0
    assert oracle.e4m3_round(2.0 ** -10) == 0 and oracle.e4m3_round(-(2.0 ** -10)) == 0
    assert oracle.e4m3_round(2.0 ** -10 * 1.001) == 0x01


def test_quantize_mx8_worked_blocks(orc):
    """Scale = 2^(floor(log2 amax) - 8): amax 1.0 -> byte 119 and 1.0 -> 256 =
    code 0x78, 0.5 -> 128 = 0x70, 0.3 -> 76.8 -> 80 = 0x6A; amax 500 -> byte
    127 and 500 saturates at 448; amax 0 -> byte 0 and zero codes; a block
    whose max is a power of two times 1.75 lands on 448 exactly."""
    x = np.zeros(128, np.float32)
    x[0], x[1], x[2], x[3] = 1.0, 0.5, 0.3, -0.3
    x[32], x[33] = 500.0, -1.0
    x[96], x[97] = 1.75 * 2.0 ** -20, -(2.0 ** -30)
    q, e = oracle.quantize_mx8(x)
    assert list(e) == [119, 127, 0, 127 - 20 - 8]
    assert list(q[:4]) == [0x78, 0x70, 0x6A, 0xEA]
    assert q[32] == 0x7E and q[33] == oracle.e4m3_round(-1.0)
    assert np.all(q[64:96] == 0)
    assert q[96] == 0x7E
    assert oracle.e4m3(int(q[97])) == -(2.0 ** -30) / 2.0 ** (int(e[3]) - 127)


def test_quantize_mx8_scale_shift_and_error_bound(orc):
    """Scaling a block by 2^k shifts its scale byte by k and keeps the codes; an
    element in the normal range is within 2^-4 relative of its value, one in the
    subnormal range within 2^-10 of the scale; only values above 448 X clip."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(32 * 64) * np.exp(rng.uniform(-8, 8, 32 * 64))).astype(np.float32)
    q, e = oracle.quantize_mx8(x)
    for k in (-20, -3, 1, 17):
        q2, e2 = oracle.quantize_mx8((x * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(q2, q) and np.array_equal(e2.astype(int), e.astype(int) + k)
    vals = np.array([oracle.e4m3(int(c)) for c in q])
    X = np.repeat(np.ldexp(1.0, e.astype(np.int64) - 127), 32)
    y = x.astype(np.float64) / X
    err = np.abs(vals - y)
    normal = (np.abs(y) >= 2.0 ** -6) & (np.abs(y) <= 448)
    assert np.all(err[normal] <= np.abs(y[normal]) * 2.0 ** -4)
    assert np.all(err[np.abs(y) < 2.0 ** -6] <= 2.0 ** -10)
    assert np.all(np.abs(vals[np.abs(y) > 448]) == 448)
    # the block maximum sits in [256, 512) X
    amax = np.abs(y).reshape(-1, 32).max(axis=1)
    assert np.all((amax >= 256) & (amax < 512))


def test_row_dot_mx8_is_dense_dot(orc, genlib):
    """The exact MXFP4 x MXFP8 row dot equals the fp64 dot of the dequantized
    row (the separately pinned MXFP4 decode) with the dequantized activations."""
    rng = np.random.default_rng(5)
    K = 2880
    w = gen.normal(9, gen.T_DOWN, gen.MXFP4, 6, K, 0.02)
    mat = gen.encode_matrix(gen.MXFP4, w)
    x = (rng.standard_normal(K) * 2).astype(np.float32)
    q, e = oracle.quantize_mx8(x)
    a = np.array([oracle.e4m3(int(c)) for c in q]) * np.repeat(
        np.ldexp(1.0, e.astype(np.int64) - 127), 32)
    for r in range(mat.shape[0]):
        dense = oracle.dequant_row(gen.MXFP4, mat[r], K)
        got = oracle.row_dot_mx8(mat[r], K, q, e)
        want = float(np.dot(dense, a))
        assert abs(got - want) <= 1e-12 * max(1.0, np.abs(dense * a).sum())


@pytest.mark.parametrize("name", ["gpt-oss-20b", "qwen3.6-35b-a3b"])
def test_layer_mx8_matches_dense_brute_force(orc, genlib, name):
    """The MXFP8 activation mode of the layer (x and h quantized to MXFP8, MXFP4
    experts, with gpt-oss's biases and clamped SwiGLU) equals a brute-force fp64
    FFN on the dequantized matrices; it differs from the q8 mode."""
    base = SHRUNK[name]
    cfg = base.with_(fmt_gu=gen.MXFP4, fmt_d=gen.MXFP4, act_quant=1)
    data = gen.make_layer(cfg)
    x, _ = gen.make_x(cfg, T=cfg.T, x_index=2)
    ref = oracle.Layer(data).forward(x)
    yb, idb, _ = brute_layer(data, x)
    assert np.array_equal(ref["ids"], idb)
    for t in range(cfg.T):
        assert np.abs(ref["y"][t] - yb[t]).max() <= 1e-9 * np.linalg.norm(yb[t])
    q8 = oracle.Layer(gen.make_layer(cfg.with_(act_quant=0))).forward(x)["y"]
    assert np.abs(q8 - ref["y"]).max() > 1e-6 * np.abs(ref["y"]).max()
