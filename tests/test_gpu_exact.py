"""Exact integer parity of the production kernel bodies against the oracle.

Two exports, both running the code the layer runs:
  * moe_test_tile_dots: the int32 super-block sums of the multi-token path's
    int8-MFMA tile kernels (LDS ring + MFMA tiles), per (token, row, super-block),
    against the oracle's integer block partials, bit for bit.
  * moe_test_preact: the gate/up pre-activations of the layer's own gate/up
    stage on the integer-exact case (block scale d = 1, dmin = 0, small sub-block
    scales, integer activations with block maximum 127 so that q8(x) = x and
    d8 = 1): every pre-activation is then an integer (MXFP4: a multiple of 0.5)
    below 2^24, so the kernels' fp32 block rescale and sums are exact and must
    equal the oracle's summed integer partials bitwise. Covers the per-pair GEMV
    kernels (Q4_K, Q6_K, Q5_K, Q2_K, Q3_K, Q4_0, Q5_1, MXFP4 realigned and
    per-block) and the
    grouped MFMA kernels (LDS ring, and register-staged with biases).
"""
import zlib

import numpy as np
import pytest
import torch

import gen
import oracle
import quantized_moe_expert_route_amd as M
from gen.device import DeviceLayer
from tests.gpu_common import random_blocks, say, upload_q8, x_cases

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------- tile kernels
@pytest.mark.parametrize("mode,n_rows,K,n_tok", [
    (0, 128, 2048, 16), (0, 64, 7168, 5), (0, 128, 512, 1),
    (1, 256, 512, 16), (1, 128, 2048, 7),
    (2, 128, 1024, 16), (2, 64, 2048, 3)])
@pytest.mark.parametrize("kind", ["generated", "random_fields"])
def test_tile_dots_exact(mode, n_rows, K, n_tok, kind):
    fmt = gen.Q6_K if mode == 2 else gen.Q4_K
    say(f"tile_dots mode={mode} rows={n_rows} K={K} tokens={n_tok} {kind}")
    rng = np.random.default_rng(1000 * mode + K + n_tok)
    stride = gen.row_stride(fmt, K)
    if kind == "generated":
        w = gen.normal(7, gen.T_DOWN, 10 * mode + fmt, n_rows, K, 0.02)
        mat = gen.encode_matrix(fmt, w)
    else:
        raw = random_blocks(fmt, n_rows, K, rng)
        mat = np.zeros((n_rows, stride), np.uint8)
        mat[:, :raw.shape[1]] = raw
    x = x_cases(n_tok, K, 11 + mode)
    host, q, keep = upload_q8(x, 256)
    rows = torch.from_numpy(mat).cuda()
    nb = K // 256
    n_m = 2 if mode == 0 else 1
    out = torch.full((n_m, n_tok, n_rows, nb), -7, dtype=torch.int32, device="cuda")
    wsb = M.moe_test_tile_dots_ws(mode, n_rows, K, n_tok)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    M.moe_test_tile_dots(mode, rows, n_rows, K, stride, q, n_tok, out, ws, wsb)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for t in range(n_tok):
        for r in range(n_rows):
            ref = oracle.block_partials(fmt, mat[r], K, host[0][t], host[2][t])[:, 0]
            for m in range(n_m):
                assert np.array_equal(got[m, t, r], ref), (m, t, r)


# ------------------------------------------------- integer-exact pre-activations
def exact_blocks(fmt: int, n: int, rng) -> np.ndarray:
    """n blocks with block scale 1 (and dmin 0), sub-block scales small enough
    that a 1024-wide row's summed integer partials stay below 2^24, and
    arbitrary quant bytes."""
    if fmt == gen.Q4_K or fmt == gen.Q5_K:
        nbytes = 144 if fmt == gen.Q4_K else 176
        b = rng.integers(0, 256, (n, nbytes), dtype=np.uint8)
        b[:, 0:2] = [0x00, 0x3C]                  # d = 1
        b[:, 2:4] = 0                             # dmin = 0
        top = 3 if fmt == gen.Q4_K else 1         # sub-block scales sc_j <= top
        b[:, 4:8] = rng.integers(0, top + 1, (n, 4))                   # sc_0..3, no high bits
        b[:, 12:16] = (b[:, 12:16] & 0xF0) | rng.integers(0, top + 1, (n, 4))  # sc_4..7 low bits
        # bytes 8..11 (m_0..3 and the high bits of m_4..7) stay arbitrary
        return b
    if fmt == gen.Q6_K:
        b = rng.integers(0, 256, (n, 210), dtype=np.uint8)
        b[:, 192:208] = rng.integers(-2, 3, (n, 16)).astype(np.int8).view(np.uint8)
        b[:, 208:210] = [0x00, 0x3C]              # d = 1
        return b
    if fmt == gen.Q2_K:
        b = rng.integers(0, 256, (n, 84), dtype=np.uint8)
        b[:, 80:82] = [0x00, 0x3C]                # d = 1
        b[:, 82:84] = 0                           # dmin = 0
        return b
    if fmt == gen.Q3_K:
        b = rng.integers(0, 256, (n, 110), dtype=np.uint8)
        # stored scales 30..33 (used as -2..1): low nibbles 14, 15, 0, 1 with
        # top bits 1, 1, 2, 2
        sc = rng.integers(30, 34, (n, 16))
        for s in range(16):
            lo, hi = sc[:, s] & 15, sc[:, s] >> 4
            j = 96 + s % 8
            b[:, j] = (b[:, j] & 0xF0) | lo if s < 8 else (b[:, j] & 0x0F) | (lo << 4)
            k, sh = 104 + s % 4, 2 * (s // 4)
            b[:, k] = (b[:, k] & (0xFF ^ (3 << sh))) | (hi << sh)
        b[:, 108:110] = [0x00, 0x3C]              # d = 1
        return b
    if fmt == gen.Q4_0:
        b = rng.integers(0, 256, (n, 18), dtype=np.uint8)
        b[:, 0:2] = [0x00, 0x3C]                  # d = 1
        return b
    if fmt == gen.Q5_1:
        b = rng.integers(0, 256, (n, 24), dtype=np.uint8)
        b[:, 0:2] = [0x00, 0x3C]                  # d = 1
        b[:, 2:4] = 0                             # m = 0
        return b
    b = rng.integers(0, 256, (n, 17), dtype=np.uint8)
    b[:, 0] = 127                                 # E8M0 scale 2^0
    return b


def exact_layer(cfg, rng):
    """LayerData whose gate/up matrices hold exact_blocks rows (down rows are
    zero blocks: the pre-activation export does not read them)."""
    pool = np.zeros((cfg.n_pool, cfg.expert_bytes), np.uint8)
    be = gen.BLOCK_ELEMS[cfg.fmt_gu]
    nb = cfg.H // be
    rb = gen.row_bytes(cfg.fmt_gu, cfg.H)
    gb = cfg.gate_bytes
    for e in range(cfg.n_pool):
        for m in range(2):
            mat = pool[e, m * gb:(m + 1) * gb].reshape(cfg.F, cfg.stride_gu)
            mat[:, :rb] = exact_blocks(cfg.fmt_gu, cfg.F * nb, rng).reshape(cfg.F, rb)
    w_router = gen.normal(cfg.seed, gen.T_ROUTER, 0, cfg.E, cfg.H, 0.02)
    b = None
    if cfg.biases:
        b = (np.zeros((cfg.E, cfg.F), np.float32), np.zeros((cfg.E, cfg.F), np.float32),
             np.zeros((cfg.E, cfg.H), np.float32))
    x = np.zeros((cfg.T, cfg.H), np.float32)
    return gen.LayerData(cfg, w_router, None, pool, *(b or (None, None, None)), x, None)


def integer_x(T, H, B, rng) -> np.ndarray:
    """Integer activations with block maximum |x| = 127: q8(x) = x and d8 = 1."""
    x = rng.integers(-127, 128, (T, H)).astype(np.float32)
    for t in range(T):
        for b0 in range(0, H, B):
            x[t, b0 + rng.integers(B)] = 127.0 if rng.random() < 0.5 else -127.0
    return x


EXACT_CASES = [
    # name, layer overrides, T ("grouped" in the name: the expert-grouped path)
    ("q4k-gemv", dict(), 1),
    ("q4k-gemv-3tok", dict(), 3),
    ("q4k-grouped-ring", dict(), 7),
    ("q4k-grouped-ring-many", dict(), 37),
    ("q4k-grouped-bias", dict(biases=True), 9),
    ("q4k-gemv-bias", dict(biases=True), 2),
    ("q6k-gemv", dict(fmt_gu=gen.Q6_K, fmt_d=gen.Q6_K), 1),
    ("q6k-grouped", dict(fmt_gu=gen.Q6_K, fmt_d=gen.Q6_K), 9),
    ("q5k-gemv", dict(fmt_gu=gen.Q5_K, fmt_d=gen.Q5_K), 2),
    ("q2k-gemv", dict(fmt_gu=gen.Q2_K, fmt_d=gen.Q2_K), 2),
    ("mxfp4-realigned", dict(fmt_gu=gen.MXFP4, fmt_d=gen.MXFP4), 2),
    ("mxfp4-realigned-8tok", dict(fmt_gu=gen.MXFP4, fmt_d=gen.MXFP4), 8),
    ("mxfp4-per-block", dict(fmt_gu=gen.MXFP4, fmt_d=gen.MXFP4, H=8224, F=64, E=4), 2),
    ("q3k-gemv", dict(fmt_gu=gen.Q3_K, fmt_d=gen.Q3_K), 2),
    ("q40-gemv", dict(fmt_gu=gen.Q4_0, fmt_d=gen.Q4_0), 3),
    ("q40-gemv-ragged", dict(fmt_gu=gen.Q4_0, fmt_d=gen.Q4_0, H=1056, F=96), 2),
    ("q51-gemv", dict(fmt_gu=gen.Q5_1, fmt_d=gen.Q5_1), 2),
]


@pytest.mark.parametrize("name,over,T", EXACT_CASES)
def test_preact_integer_exact(name, over, T):
    base = gen.LayerConfig("exact", H=1024, F=256, E=8, k=2, T=T, seed=21, shared=True)
    cfg = base.with_(**over)
    say(f"preact exact {name} T={T} H={cfg.H} F={cfg.F}")
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    data = exact_layer(cfg, rng)
    present = np.ones(cfg.E, bool)
    present[cfg.E - 1] = False  # one expert not present: its rows stay untouched
    path = M.MOE_PATH_GROUPED if "grouped" in name else M.MOE_PATH_GEMV
    dl = DeviceLayer(data, present=present, path=path)
    B = gen.BLOCK_ELEMS[cfg.fmt_gu]  # q8 block of the gate/up activations
    x = integer_x(T, cfg.H, B, rng)
    host, q, keep = upload_q8(x, B)
    assert np.all(host[1] == 1.0) and np.array_equal(host[0], x.astype(np.int8))
    ids = np.stack([rng.choice(cfg.E, cfg.k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[0, 0] = cfg.E - 1
    P = T * cfg.k + T
    ws = dl.workspace(T)
    idt = torch.from_numpy(ids).cuda()
    for which in (0, 1):
        out = torch.full((P, cfg.F), float("nan"), dtype=torch.float32, device="cuda")
        M.moe_test_preact(dl.desc, q, T, idt, which, out, ws, ws.numel())
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        for p in range(P):
            if p < T * cfg.k:
                t, e = p // cfg.k, int(ids[p // cfg.k, p % cfg.k])
                if not present[e]:
                    assert np.all(np.isnan(got[p])), p
                    continue
            else:
                t, e = p - T * cfg.k, cfg.E
            mat = (data.gate(e) if which == 0 else data.up(e)).reshape(cfg.F, cfg.stride_gu)
            for r in range(cfg.F):
                part = oracle.block_partials(cfg.fmt_gu, mat[r], cfg.H, host[0][t],
                                             host[2][t] if B == 256 else None)
                s = int(part[:, 0].astype(np.int64).sum())
                want = s / 2 if cfg.fmt_gu == gen.MXFP4 else s
                assert abs(want) < 2 ** 23
                assert got[p, r] == np.float32(want), (which, p, r, got[p, r], want)
        if which == 0:
            # the oracle's fp64 row dot (block values rescaled by d8, d, dmin)
            # of the shared expert's first gate row equals the integer sum
            row = data.gate(cfg.E).reshape(cfg.F, cfg.stride_gu)[0]
            rd = oracle.row_dot(cfg.fmt_gu, row, cfg.H, host[0][T - 1], host[1][T - 1],
                                host[2][T - 1] if B == 256 else None)
            assert rd == float(got[T * cfg.k + T - 1, 0])
