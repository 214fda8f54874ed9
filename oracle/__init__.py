"""Python access to the fp64 CPU oracle (``oracle/moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``. The product library never imports
or loads it.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

Q4_K, Q6_K, MXFP4, Q5_K, Q2_K, Q3_K, Q4_0, Q5_1 = 0, 1, 2, 3, 4, 5, 6, 7
SOFTMAX, SIGMOID = 0, 1
SWIGLU, SWIGLU_OAI = 0, 1
ACTQ_Q8, ACTQ_MXFP8 = 0, 1
BLOCK_ELEMS = {Q4_K: 256, Q6_K: 256, MXFP4: 32, Q5_K: 256, Q2_K: 256, Q3_K: 256, Q4_0: 32,
               Q5_1: 32}
BLOCK_BYTES = {Q4_K: 144, Q6_K: 210, MXFP4: 17, Q5_K: 176, Q2_K: 84, Q3_K: 110, Q4_0: 18,
               Q5_1: 24}


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-o", _LIB_PATH, os.path.join(_HERE, "moe_oracle.c"), "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _LIB_PATH


class OrLayer(C.Structure):
    _fields_ = [
        ("H", C.c_int), ("F", C.c_int), ("E", C.c_int), ("k", C.c_int),
        ("router", C.c_int), ("norm_topk", C.c_int), ("route_scale", C.c_double),
        ("w_router", C.c_void_p), ("sel_bias", C.c_void_p),
        ("fmt_gate", C.c_int), ("fmt_up", C.c_int), ("fmt_down", C.c_int),
        ("stride_gate", C.c_size_t), ("stride_up", C.c_size_t), ("stride_down", C.c_size_t),
        ("gate", C.c_void_p), ("up", C.c_void_p), ("down", C.c_void_p),
        ("b_gate", C.c_void_p), ("b_up", C.c_void_p), ("b_down", C.c_void_p),
        ("act", C.c_int), ("act_alpha", C.c_double), ("act_limit", C.c_double),
        ("sh_gate", C.c_void_p), ("sh_up", C.c_void_p), ("sh_down", C.c_void_p),
        ("sh_gate_vec", C.c_void_p), ("act_quant", C.c_int),
    ]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = C.CDLL(_LIB_PATH)
        i32, f64, vp, u16, u8 = C.c_int, C.c_double, C.c_void_p, C.c_uint16, C.c_uint8
        L.or_fp16.argtypes = [u16]; L.or_fp16.restype = f64
        L.or_e8m0.argtypes = [u8]; L.or_e8m0.restype = f64
        L.or_e2m1.argtypes = [u8]; L.or_e2m1.restype = f64
        L.or_e4m3.argtypes = [u8]; L.or_e4m3.restype = f64
        L.or_e4m3_round.argtypes = [f64]; L.or_e4m3_round.restype = u8
        L.or_quantize_mx8.argtypes = [vp, i32, vp, vp]
        L.or_row_dot_mx8.argtypes = [vp, i32, vp, vp]; L.or_row_dot_mx8.restype = f64
        L.or_block_quants.argtypes = [i32, vp, vp]
        L.or_dequant_block.argtypes = [i32, vp, vp]
        L.or_dequant_row.argtypes = [i32, vp, i32, vp]
        L.or_quantize_q8.argtypes = [vp, i32, i32, vp, vp, vp]
        L.or_block_partials.argtypes = [i32, vp, i32, vp, vp, vp]
        L.or_block_value.argtypes = [i32, vp, vp, C.c_float]; L.or_block_value.restype = f64
        L.or_row_dot.argtypes = [i32, vp, i32, vp, vp, vp]; L.or_row_dot.restype = f64
        L.or_router_logits.argtypes = [vp, vp, i32, i32, vp]
        L.or_topk.argtypes = [vp, vp, i32, i32, vp]
        L.or_route_weights.argtypes = [vp, vp, i32, i32, i32, i32, f64, vp]
        L.or_act.argtypes = [i32, f64, f64, f64, f64]; L.or_act.restype = f64
        L.or_expert_ffn.argtypes = [C.POINTER(OrLayer), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                    vp]
        L.or_layer_token.argtypes = [C.POINTER(OrLayer), vp, vp, vp, vp, vp, vp]
        L.or_expert_part_token.argtypes = [C.POINTER(OrLayer), vp, vp, vp, vp]
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


# ------------------------------------------------------------- scalar helpers
def fp16(bits: int) -> float:
    return lib().or_fp16(bits)


def e8m0(e: int) -> float:
    return lib().or_e8m0(e)


def e2m1(code: int) -> float:
    return lib().or_e2m1(code)


def e4m3(code: int) -> float:
    return lib().or_e4m3(code)


def e4m3_round(v: float) -> int:
    """Nearest finite E4M3 code (ties to even, saturating at +-448, zero -> +0)."""
    return int(lib().or_e4m3_round(float(v)))


def quantize_mx8(x: np.ndarray):
    """MXFP8 of a 1-D fp32 vector: (E4M3 codes uint8 [n], E8M0 scale bytes uint8 [n/32])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    n = x.size
    q = np.empty(n, dtype=np.uint8)
    e = np.empty(n // 32, dtype=np.uint8)
    lib().or_quantize_mx8(_p(x), n, _p(q), _p(e))
    return q, e


def row_dot_mx8(row: np.ndarray, K: int, q, e) -> float:
    """Exact fp64 dot of one MXFP4 row with MXFP8 activations."""
    row = np.ascontiguousarray(row, dtype=np.uint8)
    return lib().or_row_dot_mx8(_p(row), K, _p(np.ascontiguousarray(q, np.uint8)),
                                _p(np.ascontiguousarray(e, np.uint8)))


def block_quants(fmt: int, blk: np.ndarray) -> np.ndarray:
    blk = np.ascontiguousarray(blk, dtype=np.uint8)
    q = np.zeros(BLOCK_ELEMS[fmt], dtype=np.int32)
    lib().or_block_quants(fmt, _p(blk), _p(q))
    return q


def dequant_row(fmt: int, row: np.ndarray, K: int) -> np.ndarray:
    row = np.ascontiguousarray(row, dtype=np.uint8)
    out = np.empty(K, dtype=np.float64)
    lib().or_dequant_row(fmt, _p(row), K, _p(out))
    return out


def dequant_matrix(fmt: int, mat: np.ndarray, K: int) -> np.ndarray:
    mat = np.ascontiguousarray(mat, dtype=np.uint8)
    return np.stack([dequant_row(fmt, mat[r], K) for r in range(mat.shape[0])])


def quantize_q8(x: np.ndarray, B: int):
    """q8 of a 1-D fp32 vector: (qs int8 [n], d fp32 [n/B], bsums int16 [n/16] or None)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    n = x.size
    qs = np.empty(n, dtype=np.int8)
    d = np.empty(n // B, dtype=np.float32)
    bs = np.empty(n // 16, dtype=np.int16) if B == 256 else None
    lib().or_quantize_q8(_p(x), n, B, _p(qs), _p(d), _p(bs))
    return qs, d, bs


def block_partials(fmt: int, row: np.ndarray, K: int, qs, bsums) -> np.ndarray:
    row = np.ascontiguousarray(row, dtype=np.uint8)
    nb = K // BLOCK_ELEMS[fmt]
    out = np.zeros((nb, 2), dtype=np.int32)
    if bsums is None:
        bsums = np.zeros(K // 16, dtype=np.int16)
    lib().or_block_partials(fmt, _p(row), K, _p(np.ascontiguousarray(qs, np.int8)),
                            _p(np.ascontiguousarray(bsums, np.int16)), _p(out))
    return out


def row_dot(fmt: int, row: np.ndarray, K: int, qs, d, bsums) -> float:
    row = np.ascontiguousarray(row, dtype=np.uint8)
    if bsums is None:
        bsums = np.zeros(K // 16, dtype=np.int16)
    return lib().or_row_dot(fmt, _p(row), K, _p(np.ascontiguousarray(qs, np.int8)),
                            _p(np.ascontiguousarray(d, np.float32)),
                            _p(np.ascontiguousarray(bsums, np.int16)))


def router_logits(w_router: np.ndarray, x: np.ndarray) -> np.ndarray:
    E, H = w_router.shape
    out = np.empty(E, dtype=np.float32)
    lib().or_router_logits(_p(np.ascontiguousarray(w_router, np.float32)),
                           _p(np.ascontiguousarray(x, np.float32)), E, H, _p(out))
    return out


def topk(logits: np.ndarray, k: int, sel_bias: np.ndarray | None = None) -> np.ndarray:
    logits = np.ascontiguousarray(logits, np.float32)
    ids = np.empty(k, dtype=np.int32)
    sb = None if sel_bias is None else np.ascontiguousarray(sel_bias, np.float32)
    lib().or_topk(_p(logits), _p(sb), logits.size, k, _p(ids))
    return ids


def route_weights(logits, ids, router: int, norm_topk: int = 1, route_scale: float = 1.0):
    logits = np.ascontiguousarray(logits, np.float32)
    ids = np.ascontiguousarray(ids, np.int32)
    w = np.empty(ids.size, dtype=np.float64)
    lib().or_route_weights(_p(logits), _p(ids), logits.size, ids.size, router, norm_topk,
                           route_scale, _p(w))
    return w


def act(kind: int, g: float, u: float, alpha: float = 1.702, limit: float = 7.0) -> float:
    return lib().or_act(kind, alpha, limit, g, u)


# ------------------------------------------------------------------- layer
class Layer:
    """Oracle view of a generated layer (host numpy buffers, kept alive here).

    `present` optionally masks experts (False = NULL pointer, "not mine")."""

    def __init__(self, data, present=None, route_scale=None, norm_topk=None, use_shared=True,
                 sh_gate_vec=None, sel_bias="data"):
        cfg = data.cfg
        self.data = data
        self.cfg = cfg
        self._keep = []
        E = cfg.E
        if present is None:
            present = np.ones(E, dtype=bool)
        self.present = np.asarray(present, dtype=bool)
        pool_base = data.pool.ctypes.data
        es = data.pool.strides[0]

        def ptrs(off):
            arr = (C.c_void_p * E)()
            for e in range(E):
                arr[e] = pool_base + e * es + off if self.present[e] else None
            self._keep.append(arr)
            return C.cast(arr, C.c_void_p)

        def bias_ptrs(b):
            if b is None:
                return None
            arr = (C.c_void_p * E)()
            for e in range(E):
                arr[e] = b.ctypes.data + e * b.strides[0]
            self._keep.append(arr)
            return C.cast(arr, C.c_void_p)

        L = OrLayer()
        L.H, L.F, L.E, L.k = cfg.H, cfg.F, cfg.E, cfg.k
        L.router = cfg.router
        L.norm_topk = cfg.norm_topk if norm_topk is None else norm_topk
        L.route_scale = cfg.route_scale if route_scale is None else route_scale
        L.w_router = _p(data.w_router)
        sb = data.sel_bias if isinstance(sel_bias, str) else sel_bias
        self.sel_bias = sb
        L.sel_bias = _p(sb)
        L.fmt_gate = L.fmt_up = cfg.fmt_gu
        L.fmt_down = cfg.fmt_d
        L.stride_gate = L.stride_up = cfg.stride_gu
        L.stride_down = cfg.stride_d
        L.gate = ptrs(0)
        L.up = ptrs(cfg.gate_bytes)
        L.down = ptrs(2 * cfg.gate_bytes)
        L.b_gate = bias_ptrs(data.b_gate)
        L.b_up = bias_ptrs(data.b_up)
        L.b_down = bias_ptrs(data.b_down)
        L.act = cfg.act
        L.act_alpha, L.act_limit = cfg.act_alpha, cfg.act_limit
        if cfg.shared and use_shared:
            base = pool_base + E * es
            L.sh_gate, L.sh_up, L.sh_down = base, base + cfg.gate_bytes, base + 2 * cfg.gate_bytes
        shv = sh_gate_vec if sh_gate_vec is not None else None
        if shv is not None:
            shv = np.ascontiguousarray(shv, np.float32)
            self._keep.append(shv)
        L.sh_gate_vec = _p(shv)
        L.act_quant = getattr(cfg, "act_quant", ACTQ_Q8)
        self.L = L

    def token(self, x_row: np.ndarray, want_h: bool = False):
        """One token: returns dict(y fp64 [H], ids, w fp64, logits fp32, h32)."""
        cfg = self.cfg
        x_row = np.ascontiguousarray(x_row, np.float32)
        y = np.empty(cfg.H, np.float64)
        ids = np.empty(cfg.k, np.int32)
        w = np.empty(cfg.k, np.float64)
        logits = np.empty(cfg.E, np.float32)
        h32 = np.zeros((cfg.k + 1, cfg.F), np.float32) if want_h else None
        lib().or_layer_token(C.byref(self.L), _p(x_row), _p(y), _p(ids), _p(w), _p(logits),
                             _p(h32))
        return dict(y=y, ids=ids, w=w, logits=logits, h32=h32)

    def forward(self, x: np.ndarray, tokens=None, threads: int = 1, want_h: bool = False):
        """Tokens in parallel host threads (the C code itself is single-threaded)."""
        tokens = list(range(x.shape[0])) if tokens is None else list(tokens)
        if threads <= 1:
            res = [self.token(x[t], want_h) for t in tokens]
        else:
            with ThreadPoolExecutor(threads) as ex:
                res = list(ex.map(lambda t: self.token(x[t], want_h), tokens))
        out = {k: np.stack([r[k] for r in res]) for k in ("y", "ids", "w", "logits")}
        if want_h:
            out["h32"] = np.stack([r["h32"] for r in res])
        return out

    def expert_part(self, x_row: np.ndarray, ids: np.ndarray, w: np.ndarray) -> np.ndarray:
        """Expert part of one token for given routing (k ids and weights; an id
        outside [0, E) contributes nothing), plus the shared expert."""
        cfg = self.cfg
        if len(ids) != cfg.k or len(w) != cfg.k:
            raise ValueError(f"expert_part needs exactly k = {cfg.k} ids and weights")
        y = np.empty(cfg.H, np.float64)
        lib().or_expert_part_token(C.byref(self.L), _p(np.ascontiguousarray(x_row, np.float32)),
                                   _p(np.ascontiguousarray(ids, np.int32)),
                                   _p(np.ascontiguousarray(w, np.float32)), _p(y))
        return y
