"""Oracle pins: scalar decoders, block layouts, round-trip bounds (CPU).

The pages name the block formats only; the byte layouts follow the ggml/GGUF
conventions. These tests pin the oracle's decoders to library routines
(numpy fp16), to the OCP MX v1.0 value table, to field-level formulas on
hand-packed blocks (packed by the generator's independent packer), and to the
closed-form round-trip bounds of the covering encoders.
"""
import os

import numpy as np
import pytest

import gen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_fp16_all_finite_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    fin = np.isfinite(ref)
    got = np.array([orc.fp16(int(b)) for b in bits[fin]])
    assert np.array_equal(got, ref[fin])
    assert np.array_equal(np.signbit(got), np.signbit(ref[fin]))


def test_e8m0(orc):
    for e in range(255):
        assert orc.e8m0(e) == np.ldexp(1.0, e - 127)


def test_e2m1_against_ocp_table(orc):
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_values.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) == 16
    for code, val in rows:
        got = orc.e2m1(int(code))
        assert got == float(val)
        assert np.signbit(got) == val.startswith("-")


def _q4k_fields(rng):
    sc = rng.integers(0, 64, 8).astype(np.uint8)
    m = rng.integers(0, 64, 8).astype(np.uint8)
    q = rng.integers(0, 16, 256).astype(np.uint8)
    return sc, m, q


def test_q4k_hand_packed_fields(orc, genlib):
    rng = np.random.default_rng(0)
    for trial in range(50):
        sc, m, q = _q4k_fields(rng)
        d_bits = int(rng.integers(0x1000, 0x3000))
        dmin_bits = int(rng.integers(0x1000, 0x3000))
        blk = gen.pack_q4k(d_bits, dmin_bits, sc, m, q)
        d = float(np.array([d_bits], np.uint16).view(np.float16)[0])
        dmin = float(np.array([dmin_bits], np.uint16).view(np.float16)[0])
        assert np.array_equal(orc.block_quants(oracle.Q4_K, blk), q)
        want = np.array([d * sc[n // 32] * q[n] - dmin * m[n // 32] for n in range(256)])
        assert np.array_equal(orc.dequant_row(oracle.Q4_K, blk, 256), want)


def test_q4k_byte_layout(orc):
    """A Q4_K block written byte by byte from the layout (no packer): d fp16 at
    byte 0, dmin at 2, twelve scale bytes at 4, nibbles at 16. Scale bytes 0..3
    hold sc_0..3 in bits 0..5 and bits 4..5 of sc_4..7 in bits 6..7; bytes 4..7
    the same for m; bytes 8..11 bits 0..3 of sc_4..7 (low nibble) and of m_4..7
    (high nibble). Chunk c = bytes 16 + 32c ..: byte i low nibble = weight
    64c + i, high nibble = weight 64c + 32 + i."""
    # sc = [1, 2, 3, 63, 17, 33, 48, 5], m = [0, 1, 62, 3, 20, 0, 35, 63]
    scales = [0x41, 0x82, 0xC3, 0x3F,     # sc_0..3 | high bits of sc_4..7 (1, 2, 3, 0)
              0x40, 0x01, 0xBE, 0xC3,     # m_0..3 | high bits of m_4..7 (1, 0, 2, 3)
              0x41, 0x01, 0x30, 0xF5]     # low bits: sc_4..7 (1, 1, 0, 5), m_4..7 (4, 0, 3, 15)
    blk = np.zeros(144, np.uint8)
    blk[0:2] = [0x00, 0x3C]               # d = 1.0
    blk[2:4] = [0x00, 0x38]               # dmin = 0.5
    blk[4:16] = scales
    blk[16 + 0] = 0x21                    # weight 0: 1, weight 32: 2
    blk[16 + 64 + 7] = 0xE9               # weight 135: 9, weight 167: 14
    blk[16 + 96 + 31] = 0xF0              # weight 223: 0, weight 255: 15
    q = np.zeros(256, np.int64)
    q[[0, 32, 135, 167, 255]] = [1, 2, 9, 14, 15]
    assert np.array_equal(orc.block_quants(oracle.Q4_K, blk), q)
    sc = [1, 2, 3, 63, 17, 33, 48, 5]
    m = [0, 1, 62, 3, 20, 0, 35, 63]
    want = np.array([sc[n // 32] * q[n] - 0.5 * m[n // 32] for n in range(256)])
    assert want[0] == 1.0 and want[32] == 3.5 and want[135] == 143.0
    assert want[167] == 462.0 and want[223] == -17.5 and want[255] == 43.5
    assert np.array_equal(orc.dequant_row(oracle.Q4_K, blk, 256), want)


def test_q6k_byte_layout(orc):
    """A Q6_K block written byte by byte: ql[128] at 0, qh[64] at 128, int8
    scales[16] at 192, fp16 d at 208. In half h, for i < 32 with g = qh[32h + i]:
    weight 128h + i = low nibble of ql[64h + i] | (g & 3) << 4, weight
    128h + 32 + i = low nibble of ql[64h + 32 + i] | (g >> 2 & 3) << 4, weight
    128h + 64 + i = high nibble of ql[64h + i] | (g >> 4 & 3) << 4, weight
    128h + 96 + i = high nibble of ql[64h + 32 + i] | (g >> 6 & 3) << 4;
    w = d * scales[n / 16] * (q - 32)."""
    blk = np.zeros(210, np.uint8)
    blk[128:192] = 0xAA                   # every high-bit pair = 2: q = 32 + nibble
    blk[192:208] = 1                      # scales 1 ...
    blk[192 + 0] = 0xFE                   # ... scales[0] = -2
    blk[192 + 9] = 0x7F                   # scales[9] = 127
    blk[192 + 15] = 0x03                  # scales[15] = 3
    blk[208:210] = [0x00, 0x38]           # d = 0.5
    blk[0] = 0x53                         # weight 0: nibble 3; weight 64: nibble 5
    blk[32 + 5] = 0x01                    # weight 37: nibble 1 ...
    blk[128 + 5] = 0xA2                   # ... with high bits 0 (g >> 2 & 3 = 0)
    blk[64 + 16] = 0x0F                   # weight 144 (h 1, i 16): nibble 15
    blk[64 + 32 + 31] = 0x70              # weight 255 (h 1, i 31): high nibble 7 ...
    blk[128 + 32 + 31] = 0x6A             # ... with high bits 1 (g >> 6 = 1)
    q = np.full(256, 32, np.int64)
    q[[0, 64, 37, 144, 255]] = [35, 37, 1, 47, 23]
    assert np.array_equal(orc.block_quants(oracle.Q6_K, blk), q)
    sc = np.ones(16)
    sc[0], sc[9], sc[15] = -2, 127, 3
    want = np.array([0.5 * sc[n // 16] * (q[n] - 32) for n in range(256)])
    assert want[0] == -3.0 and want[64] == 2.5 and want[37] == -15.5
    assert want[144] == 952.5 and want[255] == -13.5 and want[191] == 0.0
    assert np.array_equal(orc.dequant_row(oracle.Q6_K, blk, 256), want)


def test_mxfp4_byte_layout(orc):
    """An MXFP4 block written byte by byte: E8M0 scale at byte 0, then 16
    bytes: byte 1 + i low nibble = element i, high nibble = element i + 16;
    nibble bit 3 = sign, bits 0..2 index {0, 0.5, 1, 1.5, 2, 3, 4, 6}."""
    blk = np.zeros(17, np.uint8)
    blk[0] = 128                          # scale 2
    blk[1 + 0] = 0x9F                     # element 0: -6; element 16: -0.5
    blk[1 + 15] = 0x25                    # element 15: 3; element 31: 1
    blk[1 + 7] = 0x80                     # element 7: +0; element 23: -0 (equal to 0)
    blk[1 + 3] = 0x4A                     # element 3: -1; element 19: 2
    want = np.zeros(32)
    want[[0, 16, 15, 31, 3, 19]] = [-12.0, -1.0, 6.0, 2.0, -2.0, 4.0]
    got = orc.dequant_row(oracle.MXFP4, blk, 32)
    assert np.array_equal(got, want)
    # the raw quants are 2 * e2m1, which at scale 2 equal the values themselves
    assert np.array_equal(orc.block_quants(oracle.MXFP4, blk), want.astype(np.int64))


def test_q3k_byte_layout(orc):
    """A Q3_K block written byte by byte: hmask[32] at 0, qs[64] at 32, twelve
    scale bytes at 96, fp16 d at 108. Weight 128h + 32j + l (l < 32) has its low
    2 bits in bits 2j..2j+1 of qs[32h + l] and its high bit in bit 4h + j of
    hmask[l]; q = low + 4 * high - 4. Sub-block s has a 6-bit scale whose low 4
    bits are the low (s < 8) or high (s >= 8) nibble of scale byte s mod 8 and
    whose top 2 bits are bits 2 (s / 4).. of scale byte 8 + s mod 4;
    w = d * (scale - 32) * q."""
    blk = np.zeros(110, np.uint8)
    blk[0:32] = 0xFF                      # every high bit set: q = low bits
    blk[108:110] = [0x00, 0x38]           # d = 0.5
    blk[96 + 0] = 0x01                    # scale 0 low bits 1 (scale 8 low bits 0)
    blk[96 + 1] = 0x80                    # scale 9 low bits 8 (high nibble)
    blk[96 + 7] = 0xF0                    # scale 15 low bits 15 (high nibble)
    blk[104:108] = [0xAA, 0xAA, 0xAA, 0xEA]  # top bits 2 for all, 3 for scale 15
    blk[32 + 0] = 0x03                    # weight 0 (h 0, j 0, l 0): low bits 3
    blk[32 + 32 + 22] = 0x01              # weight 150 (h 1, j 0, l 22): low bits 1 ...
    blk[22] = 0xEF                        # ... high bit (bit 4) cleared: q = 1 - 4
    blk[32 + 32 + 31] = 0x80              # weight 255 (h 1, j 3, l 31): low bits 2
    q = np.zeros(256, np.int64)
    q[[0, 150, 255]] = [3, -3, 2]
    assert np.array_equal(orc.block_quants(oracle.Q3_K, blk), q)
    sc = np.full(16, 32)
    sc[0], sc[9], sc[15] = 33, 40, 63
    want = np.array([0.5 * (sc[n // 16] - 32) * q[n] for n in range(256)])
    assert want[0] == 1.5 and want[150] == -12.0 and want[255] == 31.0
    assert np.array_equal(orc.dequant_row(oracle.Q3_K, blk, 256), want)


def test_q40_byte_layout(orc):
    """A Q4_0 block written byte by byte: fp16 d at 0, 16 nibble bytes at 2;
    byte j holds element j (low nibble) and element j + 16 (high nibble);
    w = d * (q - 8)."""
    blk = np.full(18, 0x88, np.uint8)     # every q = 8: w = 0
    blk[0:2] = [0x00, 0x34]               # d = 0.25
    blk[2 + 0] = 0x8F                     # element 0: 15; element 16: 8
    blk[2 + 15] = 0x08                    # element 15: 8; element 31: 0
    blk[2 + 5] = 0x38                     # element 5: 8; element 21: 3
    q = np.full(32, 8, np.int64)
    q[[0, 31, 21]] = [15, 0, 3]
    assert np.array_equal(orc.block_quants(oracle.Q4_0, blk), q)
    want = 0.25 * (q - 8).astype(np.float64)
    assert want[0] == 1.75 and want[31] == -2.0 and want[21] == -1.25
    assert np.array_equal(orc.dequant_row(oracle.Q4_0, blk, 32), want)


def test_q51_byte_layout(orc):
    """A Q5_1 block written byte by byte: fp16 d at 0, fp16 m at 2, 32-bit qh
    (little-endian) at 4, 16 nibble bytes at 8; bit j of qh is the fifth bit of
    element j; byte j holds the low 4 bits of element j (low nibble) and of
    element j + 16 (high nibble); w = d * q + m."""
    blk = np.zeros(24, np.uint8)
    blk[0:2] = [0x00, 0x38]               # d = 0.5
    blk[2:4] = [0x00, 0xBC]               # m = -1.0
    blk[4:8] = [0x01, 0x02, 0x00, 0x80]   # fifth bits of elements 0, 9 and 31
    blk[8 + 0] = 0x25                     # element 0: 5 (+16); element 16: 2
    blk[8 + 15] = 0xF0                    # element 15: 0; element 31: 15 (+16)
    q = np.zeros(32, np.int64)
    q[[0, 16, 31, 9]] = [21, 2, 31, 16]
    assert np.array_equal(orc.block_quants(oracle.Q5_1, blk), q)
    want = 0.5 * q.astype(np.float64) - 1.0
    assert want[0] == 9.5 and want[16] == 0.0 and want[31] == 14.5 and want[9] == 7.0
    assert np.array_equal(orc.dequant_row(oracle.Q5_1, blk, 32), want)


def test_q3k_hand_packed_fields(orc, genlib):
    rng = np.random.default_rng(6)
    for trial in range(50):
        sc = rng.integers(0, 64, 16).astype(np.uint8)
        q = rng.integers(-4, 4, 256).astype(np.int8)
        d_bits = int(rng.integers(0x0400, 0x3C00))
        blk = gen.pack_q3k(d_bits, sc, q)
        d = float(np.array([d_bits], np.uint16).view(np.float16)[0])
        assert np.array_equal(orc.block_quants(oracle.Q3_K, blk), q)
        want = np.array([d * (int(sc[n // 16]) - 32) * int(q[n]) for n in range(256)])
        assert np.array_equal(orc.dequant_row(oracle.Q3_K, blk, 256), want)


def test_q40_q51_hand_packed_fields(orc, genlib):
    rng = np.random.default_rng(7)
    for trial in range(50):
        d_bits = int(rng.integers(0x0400, 0x3C00))
        m_bits = int(rng.integers(0x0400, 0x3C00)) | (0x8000 if trial % 2 else 0)
        d = float(np.array([d_bits], np.uint16).view(np.float16)[0])
        m = float(np.array([m_bits], np.uint16).view(np.float16)[0])
        q4 = rng.integers(0, 16, 32).astype(np.uint8)
        b4 = gen.pack_q40(d_bits, q4)
        assert np.array_equal(orc.block_quants(oracle.Q4_0, b4), q4)
        assert np.array_equal(orc.dequant_row(oracle.Q4_0, b4, 32), d * (q4.astype(np.float64) - 8))
        q5 = rng.integers(0, 32, 32).astype(np.uint8)
        b5 = gen.pack_q51(d_bits, m_bits, q5)
        assert np.array_equal(orc.block_quants(oracle.Q5_1, b5), q5)
        assert np.array_equal(orc.dequant_row(oracle.Q5_1, b5, 32), d * q5.astype(np.float64) + m)


def test_q5k_hand_packed_fields(orc, genlib):
    rng = np.random.default_rng(3)
    for trial in range(50):
        sc, m, _ = _q4k_fields(rng)
        q = rng.integers(0, 32, 256).astype(np.uint8)
        d_bits = int(rng.integers(0x1000, 0x3000))
        dmin_bits = int(rng.integers(0x1000, 0x3000))
        blk = gen.pack_q5k(d_bits, dmin_bits, sc, m, q)
        d = float(np.array([d_bits], np.uint16).view(np.float16)[0])
        dmin = float(np.array([dmin_bits], np.uint16).view(np.float16)[0])
        assert np.array_equal(orc.block_quants(oracle.Q5_K, blk), q)
        want = np.array([d * sc[n // 32] * q[n] - dmin * m[n // 32] for n in range(256)])
        assert np.array_equal(orc.dequant_row(oracle.Q5_K, blk, 256), want)


def test_q5k_byte_layout(orc):
    """A Q5_K block written byte by byte: d = 1, dmin = 0, scales 1. The fifth
    bit of weight 64c + l sits in bit 2c of qh[l] (byte 16 + l), that of weight
    64c + 32 + l in bit 2c + 1; nibbles at byte 48 as in Q4_K."""
    blk = np.zeros(176, np.uint8)
    blk[0:2] = [0x00, 0x3C]          # d = 1.0 (fp16)
    blk[4:8] = 1                     # sc_0..3 = 1 (low 6 bits), m = 0
    blk[12:16] = 0x01                # sc_4..7 low bits = 1, m high nibble 0
    blk[48 + 0] = 0x21               # weight 0: nibble 1; weight 32: nibble 2
    blk[48 + 32 * 3 + 5] = 0xF7      # weight 197: 7; weight 229: 15
    blk[16 + 0] = 0b00000011         # weight 0 and weight 32: + 16
    blk[16 + 5] = 0b10000000         # weight 64*3 + 32 + 5 = 229: + 16
    want = np.zeros(256, np.int64)
    want[0], want[32], want[197], want[229] = 17, 18, 7, 31
    assert np.array_equal(orc.block_quants(oracle.Q5_K, blk), want)
    assert np.array_equal(orc.dequant_row(oracle.Q5_K, blk, 256), want.astype(np.float64))


def test_q2k_hand_packed_fields(orc, genlib):
    rng = np.random.default_rng(4)
    for trial in range(50):
        sc = rng.integers(0, 16, 16).astype(np.uint8)
        m = rng.integers(0, 16, 16).astype(np.uint8)
        q = rng.integers(0, 4, 256).astype(np.uint8)
        d_bits = int(rng.integers(0x1000, 0x3000))
        dmin_bits = int(rng.integers(0x1000, 0x3000))
        blk = gen.pack_q2k(d_bits, dmin_bits, sc, m, q)
        d = float(np.array([d_bits], np.uint16).view(np.float16)[0])
        dmin = float(np.array([dmin_bits], np.uint16).view(np.float16)[0])
        assert np.array_equal(orc.block_quants(oracle.Q2_K, blk), q)
        want = np.array([d * sc[n // 16] * q[n] - dmin * m[n // 16] for n in range(256)])
        assert np.array_equal(orc.dequant_row(oracle.Q2_K, blk, 256), want)


def test_q2k_byte_layout(orc):
    """A Q2_K block written byte by byte: scales[s] = scale | min << 4 for the
    16 weights of sub-block s; weight 128h + 32j + l is bits 2j..2j+1 of
    qs[32h + l] (byte 16 + 32h + l); d at byte 80, dmin at 82."""
    blk = np.zeros(84, np.uint8)
    blk[80:82] = [0x00, 0x3C]          # d = 1.0
    blk[82:84] = [0x00, 0x38]          # dmin = 0.5
    blk[0] = 0x21                      # sub-block 0: scale 1, min 2
    blk[15] = 0x03                     # sub-block 15: scale 3, min 0
    blk[16 + 0] = 0b11100100           # weights 0, 32, 64, 96: 0, 1, 2, 3
    blk[16 + 32 + 31] = 0b10000000     # weight 128 + 96 + 31 = 255: 2
    want_q = np.zeros(256, np.int64)
    want_q[[0, 32, 64, 96, 255]] = [0, 1, 2, 3, 2]
    assert np.array_equal(orc.block_quants(oracle.Q2_K, blk), want_q)
    want = np.zeros(256)
    want[:16] = -1.0                   # sub-block 0: 1 * q - 0.5 * 2 with q = 0
    want[255] = 3.0 * 2
    want[32], want[64], want[96] = 0.0, 0.0, 0.0  # their sub-blocks have scale 0, min 0
    assert np.array_equal(orc.dequant_row(oracle.Q2_K, blk, 256), want)


def test_q6k_hand_packed_fields(orc, genlib):
    rng = np.random.default_rng(1)
    for trial in range(50):
        sc = rng.integers(-128, 128, 16).astype(np.int8)
        q = rng.integers(0, 64, 256).astype(np.uint8)
        d_bits = int(rng.integers(0x0400, 0x3000))
        blk = gen.pack_q6k(d_bits, sc, q)
        d = float(np.array([d_bits], np.uint16).view(np.float16)[0])
        assert np.array_equal(orc.block_quants(oracle.Q6_K, blk), q)
        want = np.array([d * int(sc[n // 16]) * (int(q[n]) - 32) for n in range(256)])
        assert np.array_equal(orc.dequant_row(oracle.Q6_K, blk, 256), want)


def test_mxfp4_hand_packed_fields(orc, genlib):
    rng = np.random.default_rng(2)
    table = {int(c): float(v) for c, v in
             (l.split() for l in open(os.path.join(GOLDEN, "e2m1_values.txt"))
              if l.strip() and not l.startswith("#"))}
    for trial in range(50):
        e = int(rng.integers(0, 255))
        codes = rng.integers(0, 16, 32).astype(np.uint8)
        blk = gen.pack_mxfp4(e, codes)
        want = np.array([table[int(c)] * np.ldexp(1.0, e - 127) for c in codes])
        assert np.array_equal(orc.dequant_row(oracle.MXFP4, blk, 32), want)
        assert np.array_equal(orc.block_quants(oracle.MXFP4, blk),
                              np.array([int(2 * table[int(c)]) for c in codes]))


def _blocks(fmt, n, std, seed):
    be = gen.BLOCK_ELEMS[fmt]
    x = gen.normal(seed, 1, fmt, n, be, std)
    # edge blocks: all zero, all positive, all negative, a single spike, constant
    x[0] = 0
    x[1] = np.abs(x[1])
    x[2] = -np.abs(x[2])
    x[3] = 0
    x[3, be // 2] = 5 * std
    x[4] = std
    return x


@pytest.mark.parametrize("std", [0.02, 1.0, 1e-4])
def test_q4k_round_trip_bound(orc, genlib, std):
    x = _blocks(gen.Q4_K, 300, std, 11)
    for r in range(x.shape[0]):
        blk = gen.encode_block(gen.Q4_K, x[r])
        xh = orc.dequant_row(oracle.Q4_K, blk, 256)
        d = orc.fp16(int(blk[0]) | int(blk[1]) << 8)
        q = orc.block_quants(oracle.Q4_K, blk)
        # decoded per-sub-block step: d * sc_j, recovered from two elements with different q
        err = np.abs(x[r].astype(np.float64) - xh)
        for j in range(8):
            xs = x[r, 32 * j:32 * j + 32].astype(np.float64)
            rng_j = max(xs.max(), 0) - min(xs.min(), 0)
            # data-only bound: the covering step is at most range/15 plus one unit of d and dmin
            loose = (rng_j / 15 + d + 2 * abs(orc.fp16(int(blk[2]) | int(blk[3]) << 8))) / 2
            assert err[32 * j:32 * j + 32].max() <= loose * (1 + 1e-9) + 1e-300, (r, j)
        assert q.min() >= 0 and q.max() <= 15


@pytest.mark.parametrize("std", [0.02, 1.0, 1e-4])
def test_q5k_round_trip_bound(orc, genlib, std):
    x = _blocks(gen.Q5_K, 300, std, 14)
    for r in range(x.shape[0]):
        blk = gen.encode_block(gen.Q5_K, x[r])
        xh = orc.dequant_row(oracle.Q5_K, blk, 256)
        d = orc.fp16(int(blk[0]) | int(blk[1]) << 8)
        q = orc.block_quants(oracle.Q5_K, blk)
        err = np.abs(x[r].astype(np.float64) - xh)
        for j in range(8):
            xs = x[r, 32 * j:32 * j + 32].astype(np.float64)
            rng_j = max(xs.max(), 0) - min(xs.min(), 0)
            # as for Q4_K with 31 steps over the sub-block's range
            loose = (rng_j / 31 + d + 2 * abs(orc.fp16(int(blk[2]) | int(blk[3]) << 8))) / 2
            assert err[32 * j:32 * j + 32].max() <= loose * (1 + 1e-9) + 1e-300, (r, j)
        assert q.min() >= 0 and q.max() <= 31


@pytest.mark.parametrize("std", [0.02, 1.0, 1e-4])
def test_q2k_round_trip_bound(orc, genlib, std):
    x = _blocks(gen.Q2_K, 300, std, 15)
    for r in range(x.shape[0]):
        blk = gen.encode_block(gen.Q2_K, x[r])
        xh = orc.dequant_row(oracle.Q2_K, blk, 256)
        d = orc.fp16(int(blk[80]) | int(blk[81]) << 8)
        dmin = orc.fp16(int(blk[82]) | int(blk[83]) << 8)
        q = orc.block_quants(oracle.Q2_K, blk)
        err = np.abs(x[r].astype(np.float64) - xh)
        for s in range(16):
            xs = x[r, 16 * s:16 * s + 16].astype(np.float64)
            rng_s = max(xs.max(), 0) - min(xs.min(), 0)
            # covering step at most range/3 plus one unit of d and dmin, error half a step
            loose = (rng_s / 3 + d + 2 * dmin) / 2
            assert err[16 * s:16 * s + 16].max() <= loose * (1 + 1e-9) + 1e-300, (r, s)
        assert q.min() >= 0 and q.max() <= 3


@pytest.mark.parametrize("std", [0.02, 1.0, 1e-4])
def test_q6k_round_trip_bound(orc, genlib, std):
    x = _blocks(gen.Q6_K, 300, std, 12)
    for r in range(x.shape[0]):
        blk = gen.encode_block(gen.Q6_K, x[r])
        xh = orc.dequant_row(oracle.Q6_K, blk, 256)
        d = orc.fp16(int(blk[208]) | int(blk[209]) << 8)
        sc = blk[192:208].view(np.int8).astype(np.float64)
        err = np.abs(x[r].astype(np.float64) - xh)
        for s in range(16):
            step = d * sc[s]
            assert err[16 * s:16 * s + 16].max() <= step / 2 * (1 + 1e-12) + 1e-300
            xs = x[r, 16 * s:16 * s + 16].astype(np.float64)
            need = max(xs.max() / 31, -xs.min() / 32, 0)
            assert step <= need + d * (1 + 1e-12)  # covering step is the smallest that fits


@pytest.mark.parametrize("std", [0.02, 1.0, 1e-4])
def test_q3k_round_trip_bound(orc, genlib, std):
    x = _blocks(gen.Q3_K, 300, std, 16)
    for r in range(x.shape[0]):
        blk = gen.encode_block(gen.Q3_K, x[r])
        xh = orc.dequant_row(oracle.Q3_K, blk, 256)
        d = orc.fp16(int(blk[108]) | int(blk[109]) << 8)
        q = orc.block_quants(oracle.Q3_K, blk)
        err = np.abs(x[r].astype(np.float64) - xh)
        for s2 in range(16):
            xs = x[r, 16 * s2:16 * s2 + 16].astype(np.float64)
            need = max(xs.max() / 3, -xs.min() / 4, 0)
            # the covering step lies in [need, need + d] and the error is half a step
            assert err[16 * s2:16 * s2 + 16].max() <= (need + d) / 2 * (1 + 1e-9) + 1e-300
        assert q.min() >= -4 and q.max() <= 3


@pytest.mark.parametrize("fmt", [gen.Q4_0, gen.Q5_1])
@pytest.mark.parametrize("std", [0.02, 1.0, 1e-4])
def test_q40_q51_round_trip_bound(orc, genlib, fmt, std):
    x = _blocks(fmt, 600, std, 17 + fmt)
    for r in range(x.shape[0]):
        blk = gen.encode_block(fmt, x[r])
        xh = orc.dequant_row(fmt, blk, 32)
        d = orc.fp16(int(blk[0]) | int(blk[1]) << 8)
        err = np.abs(x[r].astype(np.float64) - xh)
        assert err.max() <= d / 2 * (1 + 1e-12) + 1e-300, r
        xs = x[r].astype(np.float64)
        if fmt == gen.Q4_0:
            need = max(xs.max() / 7, -xs.min() / 8, 0)
        else:
            m = orc.fp16(int(blk[2]) | int(blk[3]) << 8)
            assert m <= min(xs.min(), 0)
            need = (max(xs.max(), 0) - m) / 31
        assert d <= need * (1 + 2 ** -10) + 2 ** -24  # the smallest fp16 step that covers


@pytest.mark.parametrize("std", [0.02, 1.0, 1e-4])
def test_mxfp4_round_trip_bound(orc, genlib, std):
    x = _blocks(gen.MXFP4, 600, std, 13)
    for r in range(x.shape[0]):
        blk = gen.encode_block(gen.MXFP4, x[r])
        xh = orc.dequant_row(oracle.MXFP4, blk, 32)
        amax = np.abs(x[r]).max()
        if amax == 0:
            assert not xh.any() and blk[0] == 0
            continue
        E = int(np.floor(np.log2(float(amax)))) - 2
        assert int(blk[0]) == E + 127
        xs = x[r].astype(np.float64)
        err = np.abs(xs - xh)
        inside = np.abs(xs) <= 6 * 2.0 ** E
        assert err[inside].max(initial=0) <= 2.0 ** E
        assert err.max() < 2 * 2.0 ** E
        # magnitude 0 never gets the negative-zero code
        codes = np.concatenate([blk[1:17] & 15, blk[1:17] >> 4])
        assert not (codes == 8).any()


def test_relative_rms_informational(orc, genlib):
    for fmt, K, lim in ((gen.Q4_K, 256, 0.12), (gen.Q6_K, 256, 0.03), (gen.MXFP4, 32, 0.16)):
        x = gen.normal(9, 1, 0, 200, K, 0.02)
        m = gen.encode_matrix(fmt, x)
        xh = np.stack([orc.dequant_row(fmt, m[r], K) for r in range(200)])
        rel = np.sqrt(((xh - x) ** 2).mean()) / np.sqrt((x.astype(np.float64) ** 2).mean())
        assert rel < lim, (fmt, rel)
