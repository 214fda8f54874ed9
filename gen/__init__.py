"""Seeded synthetic inputs for the routed-expert FFN layer.

Thin ctypes wrapper over ``gen/moegen.c`` plus the five workload presets.
This module holds no arithmetic of the layer itself; it only draws random
tensors and encodes weight matrices into the stored block formats, so that the
oracle and the HIP library can be fed the same bytes.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoegen.so")
_lib = None

Q4_K, Q6_K, MXFP4, Q5_K, Q2_K, Q3_K, Q4_0, Q5_1 = 0, 1, 2, 3, 4, 5, 6, 7
FMT_NAMES = {Q4_K: "Q4_K", Q6_K: "Q6_K", MXFP4: "MXFP4", Q5_K: "Q5_K", Q2_K: "Q2_K",
             Q3_K: "Q3_K", Q4_0: "Q4_0", Q5_1: "Q5_1"}
BLOCK_BYTES = {Q4_K: 144, Q6_K: 210, MXFP4: 17, Q5_K: 176, Q2_K: 84, Q3_K: 110, Q4_0: 18,
               Q5_1: 24}
BLOCK_ELEMS = {Q4_K: 256, Q6_K: 256, MXFP4: 32, Q5_K: 256, Q2_K: 256, Q3_K: 256, Q4_0: 32,
               Q5_1: 32}

T_ROUTER, T_X, T_GATE, T_UP, T_DOWN, T_BGATE, T_BUP, T_BDOWN, T_ZIPF, T_SHVEC = range(1, 11)

SOFTMAX, SIGMOID = 0, 1
SWIGLU, SWIGLU_OAI = 0, 1


def build(verbose: bool = False) -> str:
    """Compile libmoegen.so with gcc (no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-o", _LIB_PATH, os.path.join(_HERE, "moegen.c"), "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = C.CDLL(_LIB_PATH)
        u64, u32, i32, f64, vp, sz = C.c_uint64, C.c_uint32, C.c_int, C.c_double, C.c_void_p, C.c_size_t
        L.mg_stream.argtypes = [u64, u32, u32, u32]
        L.mg_stream.restype = u64
        L.mg_u64.argtypes = [u64, u64]
        L.mg_u64.restype = u64
        L.mg_normal_row.argtypes = [u64, u32, u32, u32, i32, f64, vp]
        L.mg_normal_matrix.argtypes = [u64, u32, u32, i32, i32, f64, vp, i32]
        L.mg_round_bf16.argtypes = [vp, vp, sz]
        L.mg_fp16_ceil_bits.argtypes = [f64]
        L.mg_fp16_ceil_bits.restype = C.c_uint16
        for n in ("mg_encode_q4k", "mg_encode_q6k", "mg_encode_mxfp4", "mg_encode_q5k",
                  "mg_encode_q2k", "mg_encode_q3k", "mg_encode_q40", "mg_encode_q51"):
            getattr(L, n).argtypes = [vp, vp]
        L.mg_encode_matrix.argtypes = [i32, vp, i32, i32, sz, vp, i32]
        L.mg_pack_q4k.argtypes = [C.c_uint16, C.c_uint16, vp, vp, vp, vp]
        L.mg_pack_q6k.argtypes = [C.c_uint16, vp, vp, vp]
        L.mg_pack_q5k.argtypes = [C.c_uint16, C.c_uint16, vp, vp, vp, vp]
        L.mg_pack_q2k.argtypes = [C.c_uint16, C.c_uint16, vp, vp, vp, vp]
        L.mg_pack_mxfp4.argtypes = [C.c_uint8, vp, vp]
        L.mg_pack_q3k.argtypes = [C.c_uint16, vp, vp, vp]
        L.mg_pack_q40.argtypes = [C.c_uint16, vp, vp]
        L.mg_pack_q51.argtypes = [C.c_uint16, C.c_uint16, vp, vp]
        L.mg_weight_matrix.argtypes = [u64, u32, u32, i32, i32, i32, sz, f64, vp, i32]
        L.mg_zipf_bias.argtypes = [u64, i32, f64, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ---------------------------------------------------------------- raw helpers
def normal(seed: int, tensor: int, expert: int, rows: int, cols: int, std: float,
           threads: int | None = None) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.float32)
    lib().mg_normal_matrix(seed, tensor, expert, rows, cols, std, _ptr(out),
                           threads or default_threads())
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().mg_round_bf16(_ptr(x), _ptr(out), x.size)
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def fp16_ceil_bits(v: float) -> int:
    return int(lib().mg_fp16_ceil_bits(float(v)))


def encode_block(fmt: int, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.size == BLOCK_ELEMS[fmt]
    out = np.zeros(BLOCK_BYTES[fmt], dtype=np.uint8)
    fn = {Q4_K: "mg_encode_q4k", Q6_K: "mg_encode_q6k", MXFP4: "mg_encode_mxfp4",
          Q5_K: "mg_encode_q5k", Q2_K: "mg_encode_q2k", Q3_K: "mg_encode_q3k",
          Q4_0: "mg_encode_q40", Q5_1: "mg_encode_q51"}[fmt]
    getattr(lib(), fn)(_ptr(x), _ptr(out))
    return out


def row_bytes(fmt: int, K: int) -> int:
    assert K % BLOCK_ELEMS[fmt] == 0
    return K // BLOCK_ELEMS[fmt] * BLOCK_BYTES[fmt]


def row_stride(fmt: int, K: int) -> int:
    """Row stride in bytes: row bytes rounded up to a multiple of 16."""
    return (row_bytes(fmt, K) + 15) // 16 * 16


def encode_matrix(fmt: int, x: np.ndarray, stride: int | None = None,
                  threads: int | None = None) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, K = x.shape
    stride = stride or row_stride(fmt, K)
    out = np.empty((rows, stride), dtype=np.uint8)
    lib().mg_encode_matrix(fmt, _ptr(x), rows, K, stride, _ptr(out), threads or default_threads())
    return out


def pack_q4k(d_bits: int, dmin_bits: int, sc, m, q) -> np.ndarray:
    sc = np.ascontiguousarray(sc, dtype=np.uint8); m = np.ascontiguousarray(m, dtype=np.uint8)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    assert sc.size == 8 and m.size == 8 and q.size == 256
    out = np.zeros(144, dtype=np.uint8)
    lib().mg_pack_q4k(d_bits, dmin_bits, _ptr(sc), _ptr(m), _ptr(q), _ptr(out))
    return out


def pack_q5k(d_bits: int, dmin_bits: int, sc, m, q) -> np.ndarray:
    sc = np.ascontiguousarray(sc, dtype=np.uint8); m = np.ascontiguousarray(m, dtype=np.uint8)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    assert sc.size == 8 and m.size == 8 and q.size == 256
    out = np.zeros(176, dtype=np.uint8)
    lib().mg_pack_q5k(d_bits, dmin_bits, _ptr(sc), _ptr(m), _ptr(q), _ptr(out))
    return out


def pack_q2k(d_bits: int, dmin_bits: int, sc, m, q) -> np.ndarray:
    sc = np.ascontiguousarray(sc, dtype=np.uint8); m = np.ascontiguousarray(m, dtype=np.uint8)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    assert sc.size == 16 and m.size == 16 and q.size == 256
    out = np.zeros(84, dtype=np.uint8)
    lib().mg_pack_q2k(d_bits, dmin_bits, _ptr(sc), _ptr(m), _ptr(q), _ptr(out))
    return out


def pack_q6k(d_bits: int, sc, q) -> np.ndarray:
    sc = np.ascontiguousarray(sc, dtype=np.int8); q = np.ascontiguousarray(q, dtype=np.uint8)
    assert sc.size == 16 and q.size == 256
    out = np.zeros(210, dtype=np.uint8)
    lib().mg_pack_q6k(d_bits, _ptr(sc), _ptr(q), _ptr(out))
    return out


def pack_q3k(d_bits: int, sc, q) -> np.ndarray:
    """sc: 16 stored 6-bit scales (0..63, used as sc - 32); q: 256 values in -4..3."""
    sc = np.ascontiguousarray(sc, dtype=np.uint8); q = np.ascontiguousarray(q, dtype=np.int8)
    assert sc.size == 16 and q.size == 256
    out = np.zeros(110, dtype=np.uint8)
    lib().mg_pack_q3k(d_bits, _ptr(sc), _ptr(q), _ptr(out))
    return out


def pack_q40(d_bits: int, q) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    assert q.size == 32
    out = np.zeros(18, dtype=np.uint8)
    lib().mg_pack_q40(d_bits, _ptr(q), _ptr(out))
    return out


def pack_q51(d_bits: int, m_bits: int, q) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    assert q.size == 32
    out = np.zeros(24, dtype=np.uint8)
    lib().mg_pack_q51(d_bits, m_bits, _ptr(q), _ptr(out))
    return out


def pack_mxfp4(e: int, codes) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    assert codes.size == 32
    out = np.zeros(17, dtype=np.uint8)
    lib().mg_pack_mxfp4(e, _ptr(codes), _ptr(out))
    return out


def weight_matrix(seed: int, tensor: int, expert: int, fmt: int, rows: int, K: int,
                  stride: int, std: float, out: np.ndarray | None = None,
                  threads: int | None = None) -> np.ndarray:
    if out is None:
        out = np.empty((rows, stride), dtype=np.uint8)
    assert out.nbytes == rows * stride and out.flags["C_CONTIGUOUS"]
    lib().mg_weight_matrix(seed, tensor, expert, fmt, rows, K, stride, std, _ptr(out),
                           threads or default_threads())
    return out


def zipf_bias(seed: int, E: int, s: float) -> np.ndarray:
    out = np.empty(E, dtype=np.float32)
    lib().mg_zipf_bias(seed, E, s, _ptr(out))
    return out


# ---------------------------------------------------------------- workloads
@dataclass(frozen=True)
class LayerConfig:
    """Shape and data recipe of one synthetic MoE layer workload."""
    name: str
    H: int
    F: int
    E: int
    k: int
    T: int
    seed: int
    router: int = SOFTMAX
    norm_topk: int = 1
    route_scale: float = 1.0
    fmt_gu: int = Q4_K
    fmt_d: int = Q4_K
    shared: bool = False
    act: int = SWIGLU
    act_alpha: float = 1.702
    act_limit: float = 7.0
    biases: bool = False
    x_bf16: bool = False
    zipf_s: float = 0.0
    w_std: float = 0.02
    router_std: float = 0.02
    bias_std: float = 0.01
    x_std: float = 1.0
    act_quant: int = 0  # activation numerics: 0 q8, 1 MXFP8 (MXFP4 layers, block-scaled MMA)
    # order of the expert matrices' blocks on the device: 0 rows (GGUF order),
    # 1 64-row tiles (moe_layout TILE64; layers on the grouped path at every T),
    # 2 MX16 (MXFP4 rows with aligned nibble fields; the per-pair path)
    layout: int = 0
    description: str = ""

    @property
    def stride_gu(self) -> int:
        return row_stride(self.fmt_gu, self.H)

    @property
    def stride_d(self) -> int:
        return row_stride(self.fmt_d, self.F)

    @property
    def gate_bytes(self) -> int:
        return self.F * self.stride_gu

    @property
    def down_bytes(self) -> int:
        return self.H * self.stride_d

    @property
    def expert_bytes(self) -> int:
        """Bytes one expert occupies in the pool (gate, up, down; padded rows)."""
        return 2 * self.gate_bytes + self.down_bytes

    @property
    def expert_algo_bytes(self) -> int:
        """Block bytes of one expert (gate + up + down), padding excluded."""
        return 2 * self.F * row_bytes(self.fmt_gu, self.H) + self.H * row_bytes(self.fmt_d, self.F)

    @property
    def n_pool(self) -> int:
        return self.E + (1 if self.shared else 0)

    def with_(self, **kw) -> "LayerConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return LayerConfig(**d)


CONFIGS = {
    "tiny": LayerConfig(
        "tiny", H=512, F=256, E=8, k=2, T=1, seed=0,
        description="tiny MoE layer, 1 token: H 512, 8 experts top-2 softmax, F 256, Q4_K"),
    "qwen3.6-35b-a3b": LayerConfig(
        "qwen3.6-35b-a3b", H=2048, F=512, E=256, k=8, T=1, seed=1, shared=True,
        description="Qwen3.6-35B-A3B-shaped decode layer: H 2048, 256 experts top-8 softmax "
                    "+ shared, F 512, Q4_K"),
    "gpt-oss-20b": LayerConfig(
        "gpt-oss-20b", H=2880, F=2880, E=32, k=4, T=1, seed=2, fmt_gu=MXFP4, fmt_d=MXFP4,
        act=SWIGLU_OAI, biases=True, x_bf16=True,
        description="gpt-oss-20B-shaped decode layer: H 2880, 32 experts top-4 softmax, "
                    "F 2880, MXFP4 + fp32 biases, clamped SwiGLU, bf16 x"),
    "deepseek-v4-flash": LayerConfig(
        "deepseek-v4-flash", H=4096, F=2048, E=256, k=6, T=16, seed=3, router=SIGMOID,
        fmt_gu=Q4_K, fmt_d=Q6_K, shared=True, zipf_s=1.1,
        description="DeepSeek-V4-Flash-shaped 16-token verify chunk: H 4096, 256 experts "
                    "top-6 sigmoid (normalized) + shared, F 2048, Q4_K gate/up, Q6_K down, "
                    "Zipf(1.1) routing skew"),
    "kimi-k2": LayerConfig(
        "kimi-k2", H=7168, F=2048, E=384, k=8, T=256, seed=4, router=SIGMOID, shared=True,
        description="Kimi-K2-shaped 256-token prefill chunk: H 7168, 384 experts top-8 sigmoid "
                    "+ shared, F 2048, Q4_K"),
    # a format extension measured on the Qwen3.6 decode shape (not one of the five workloads)
    "qwen3.6-35b-a3b-q5k": LayerConfig(
        "qwen3.6-35b-a3b-q5k", H=2048, F=512, E=256, k=8, T=1, seed=5, shared=True,
        fmt_gu=Q5_K, fmt_d=Q5_K,
        description="Qwen3.6-35B-A3B-shaped decode layer with Q5_K experts: H 2048, 256 experts "
                    "top-8 softmax + shared, F 512, Q5_K"),
    "qwen3.6-35b-a3b-q2k": LayerConfig(
        "qwen3.6-35b-a3b-q2k", H=2048, F=512, E=256, k=8, T=1, seed=6, shared=True,
        fmt_gu=Q2_K, fmt_d=Q2_K,
        description="Qwen3.6-35B-A3B-shaped decode layer with Q2_K experts: H 2048, 256 experts "
                    "top-8 softmax + shared, F 512, Q2_K"),
    # the gpt-oss shape as a 16-token verify chunk: the q8 per-pair path and the
    # MXFP8-activation block-scaled MFMA path (not one of the five workloads)
    "gpt-oss-20b-t16": LayerConfig(
        "gpt-oss-20b-t16", H=2880, F=2880, E=32, k=4, T=16, seed=2, fmt_gu=MXFP4, fmt_d=MXFP4,
        act=SWIGLU_OAI, biases=True, x_bf16=True,
        description="gpt-oss-20B-shaped 16-token chunk: H 2880, 32 experts top-4 softmax, "
                    "F 2880, MXFP4 + fp32 biases, clamped SwiGLU, bf16 x, q8 activations"),
    "gpt-oss-20b-mx8": LayerConfig(
        "gpt-oss-20b-mx8", H=2880, F=2880, E=32, k=4, T=16, seed=2, fmt_gu=MXFP4, fmt_d=MXFP4,
        act=SWIGLU_OAI, biases=True, x_bf16=True, act_quant=1,
        description="gpt-oss-20B-shaped 16-token chunk: H 2880, 32 experts top-4 softmax, "
                    "F 2880, MXFP4 + fp32 biases, clamped SwiGLU, bf16 x, MXFP8 activations "
                    "on the block-scaled MFMA"),
}
CONFIG_ORDER = ["tiny", "qwen3.6-35b-a3b", "gpt-oss-20b", "deepseek-v4-flash", "kimi-k2"]


@dataclass
class LayerData:
    """Host-side tensors of one synthetic layer (numpy)."""
    cfg: LayerConfig
    w_router: np.ndarray            # [E, H] fp32
    sel_bias: np.ndarray | None     # [E] fp32
    pool: np.ndarray                # [n_pool, expert_bytes] uint8
    b_gate: np.ndarray | None       # [E, F] fp32
    b_up: np.ndarray | None         # [E, F] fp32
    b_down: np.ndarray | None       # [E, H] fp32
    x: np.ndarray                   # [T, H] fp32 values the layer sees
    x_bf16: np.ndarray | None       # [T, H] uint16 bf16 bits when x arrives as bf16
    sh_gate_vec: np.ndarray | None = None
    extra: dict = field(default_factory=dict)

    def gate(self, e: int) -> np.ndarray:
        return self.pool[e, : self.cfg.gate_bytes]

    def up(self, e: int) -> np.ndarray:
        c = self.cfg
        return self.pool[e, c.gate_bytes: 2 * c.gate_bytes]

    def down(self, e: int) -> np.ndarray:
        c = self.cfg
        return self.pool[e, 2 * c.gate_bytes: 2 * c.gate_bytes + c.down_bytes]


def make_x(cfg: LayerConfig, T: int | None = None, x_index: int = 0):
    """x for one forward: N(0, 1) rows; index selects a member of the x pool."""
    T = cfg.T if T is None else T
    x = normal(cfg.seed, T_X, x_index, T, cfg.H, cfg.x_std)
    if cfg.x_bf16:
        xb = round_bf16(x)
        return bf16_to_f32(xb), xb
    return x, None


def make_layer(cfg: LayerConfig, threads: int | None = None, with_sh_gate_vec: bool = False,
               experts: list[int] | None = None) -> LayerData:
    """Generate a whole layer. `experts` restricts weight generation to a subset
    (the others stay zero) when only some experts are needed."""
    th = threads or default_threads()
    s = cfg.seed
    w_router = normal(s, T_ROUTER, 0, cfg.E, cfg.H, cfg.router_std, th)
    sel_bias = zipf_bias(s, cfg.E, cfg.zipf_s) if cfg.zipf_s > 0 else None
    pool = np.zeros((cfg.n_pool, cfg.expert_bytes), dtype=np.uint8)
    which = range(cfg.n_pool) if experts is None else experts
    for e in which:
        gb, db = cfg.gate_bytes, cfg.down_bytes
        row = pool[e]
        weight_matrix(s, T_GATE, e, cfg.fmt_gu, cfg.F, cfg.H, cfg.stride_gu, cfg.w_std,
                      out=row[:gb].reshape(cfg.F, cfg.stride_gu), threads=th)
        weight_matrix(s, T_UP, e, cfg.fmt_gu, cfg.F, cfg.H, cfg.stride_gu, cfg.w_std,
                      out=row[gb:2 * gb].reshape(cfg.F, cfg.stride_gu), threads=th)
        weight_matrix(s, T_DOWN, e, cfg.fmt_d, cfg.H, cfg.F, cfg.stride_d, cfg.w_std,
                      out=row[2 * gb:2 * gb + db].reshape(cfg.H, cfg.stride_d), threads=th)
    b_gate = b_up = b_down = None
    if cfg.biases:
        b_gate = normal(s, T_BGATE, 0, cfg.E, cfg.F, cfg.bias_std, th)
        b_up = normal(s, T_BUP, 0, cfg.E, cfg.F, cfg.bias_std, th)
        b_down = normal(s, T_BDOWN, 0, cfg.E, cfg.H, cfg.bias_std, th)
    x, xb = make_x(cfg)
    shv = normal(s, T_SHVEC, 0, 1, cfg.H, cfg.router_std, th)[0] if with_sh_gate_vec else None
    return LayerData(cfg, w_router, sel_bias, pool, b_gate, b_up, b_down, x, xb, shv)
