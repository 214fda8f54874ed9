"""Python binding of the MI355X routed-expert MoE FFN library (libmoe_route.so).

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI declared in ``include/moe.h``. Functions keep the C names and
argument order. Tensor arguments may be torch tensors (their device pointer is
passed), raw integer addresses, or None (NULL). ``stream`` may be a
``torch.cuda.Stream``, a raw ``hipStream_t`` integer, or None (torch's current
stream). A non-OK status raises ``MoeError``.

The library is built in-tree by ``quantized_moe_expert_route_amd._build.build()``;
importing this module does not build it, and using it without the built library
raises immediately (there is no fallback implementation).
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_route.so")

# enums (include/moe.h)
MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_ENOWORKSPACE, MOE_EHIP = range(5)
(MOE_WFMT_Q4_K, MOE_WFMT_Q6_K, MOE_WFMT_MXFP4, MOE_WFMT_Q5_K, MOE_WFMT_Q2_K, MOE_WFMT_Q3_K,
 MOE_WFMT_Q4_0, MOE_WFMT_Q5_1) = range(8)
MOE_AFMT_Q8_K, MOE_AFMT_Q8_32, MOE_AFMT_MXFP8 = range(3)
MOE_ACTQ_Q8, MOE_ACTQ_MXFP8 = range(2)
MOE_DTYPE_F32, MOE_DTYPE_BF16 = range(2)
MOE_ROUTER_SOFTMAX, MOE_ROUTER_SIGMOID = range(2)
MOE_ACT_SWIGLU, MOE_ACT_SWIGLU_OAI = range(2)
MOE_PATH_AUTO, MOE_PATH_GEMV, MOE_PATH_GROUPED = range(3)
MOE_LAYOUT_ROWS, MOE_LAYOUT_TILE64, MOE_LAYOUT_MX16 = range(3)
MOE_MAX_EXPERTS = 1024
MOE_MAX_TOPK = 16

ABI_FUNCTIONS = (
    "moe_abi_version", "moe_status_str", "moe_workspace_size", "moe_quantize_act_q8k",
    "moe_route_topk", "moe_expert_ffn", "moe_layer_forward", "moe_layer_forward_timed",
    "moe_layer_stage_count", "moe_layer_stage_name", "moe_test_block_dots",
    "moe_test_tile_dots", "moe_test_tile_dots_ws", "moe_test_preact",
    "moe_layer_forward_noalloc", "moe_probe_read_wall", "moe_probe_mfma_i8",
    "moe_probe_empty_chain", "moe_repack_tile64", "moe_repack_mx16", "moe_test_block_dots_mx16",
    # expert pool (include/moe_pool.h)
    "moe_pool_create", "moe_pool_destroy", "moe_pool_host_slab", "moe_pool_layer_tables",
    "moe_pool_resolve", "moe_pool_prefetch", "moe_pool_get_stats", "moe_pool_policy_trace",
    "moe_pool_layer_step", "moe_pool_step_workspace",
)
MOE_NOALLOC_SCRATCH_BYTES = 32 << 20


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {moe_status_str(status)} (status {status})")


class MoeQact(C.Structure):
    _fields_ = [("qs", C.c_void_p), ("d", C.c_void_p), ("bsums", C.c_void_p),
                ("fmt", C.c_int32), ("T", C.c_int32), ("H", C.c_int32),
                ("scales", C.c_void_p)]


class MoePoolConfig(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("n_experts", C.c_int32), ("slab_bytes", C.c_size_t),
                ("up_offset", C.c_size_t), ("down_offset", C.c_size_t),
                ("n_slots", C.c_int32), ("n_transient", C.c_int32)]


POOL_STAT_FIELDS = ("epochs", "requests", "hits_resident", "hits_transient", "admitted",
                    "transient_loads", "promotions", "evictions", "prefetch_loads",
                    "prefetch_hits", "bytes_h2d")


class MoePoolStats(C.Structure):
    _fields_ = [(n, C.c_int64) for n in POOL_STAT_FIELDS]


class MoeLayerDesc(C.Structure):
    _fields_ = [
        ("hidden", C.c_int32), ("ffn", C.c_int32), ("n_expert", C.c_int32), ("top_k", C.c_int32),
        ("router", C.c_int32), ("norm_topk", C.c_int32), ("route_scale", C.c_float),
        ("w_router", C.c_void_p), ("sel_bias", C.c_void_p),
        ("fmt_gate", C.c_int32), ("fmt_up", C.c_int32), ("fmt_down", C.c_int32),
        ("stride_gate", C.c_size_t), ("stride_up", C.c_size_t), ("stride_down", C.c_size_t),
        ("gate", C.c_void_p), ("up", C.c_void_p), ("down", C.c_void_p),
        ("b_gate", C.c_void_p), ("b_up", C.c_void_p), ("b_down", C.c_void_p),
        ("act", C.c_int32), ("act_alpha", C.c_float), ("act_limit", C.c_float),
        ("sh_gate", C.c_void_p), ("sh_up", C.c_void_p), ("sh_down", C.c_void_p),
        ("sh_gate_vec", C.c_void_p), ("path", C.c_int32), ("act_quant", C.c_int32),
        ("layout", C.c_int32),
    ]


_lib = None


def lib():
    """Load libmoe_route.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "quantized_moe_expert_route_amd._build.build() (no fallback)")
        L = C.CDLL(LIB_PATH)
        vp, i32, sz = C.c_void_p, C.c_int, C.c_size_t
        D = C.POINTER(MoeLayerDesc)
        Q = C.POINTER(MoeQact)
        L.moe_abi_version.argtypes = []
        L.moe_abi_version.restype = i32
        L.moe_status_str.argtypes = [i32]
        L.moe_status_str.restype = C.c_char_p
        L.moe_workspace_size.argtypes = [D, i32]
        L.moe_workspace_size.restype = sz
        L.moe_quantize_act_q8k.argtypes = [vp, i32, i32, i32, i32, Q, vp]
        L.moe_route_topk.argtypes = [D, vp, i32, i32, vp, vp, vp, vp, sz, vp]
        L.moe_expert_ffn.argtypes = [D, Q, vp, i32, i32, vp, vp, vp, vp, sz, vp]
        L.moe_layer_forward.argtypes = [D, vp, i32, i32, vp, vp, vp, vp, sz, vp]
        L.moe_layer_forward_noalloc.argtypes = [D, vp, i32, i32, vp, vp, vp, vp]
        L.moe_probe_read_wall.argtypes = [vp, sz, i32, vp, vp]
        L.moe_probe_mfma_i8.argtypes = [i32, i32, i32, vp, vp]
        L.moe_probe_empty_chain.argtypes = [i32, vp]
        L.moe_layer_forward_timed.argtypes = [D, vp, i32, i32, vp, vp, vp, vp, sz, vp,
                                              C.POINTER(vp), i32]
        L.moe_layer_stage_count.argtypes = [D, i32]
        L.moe_layer_stage_count.restype = i32
        L.moe_layer_stage_name.argtypes = [D, i32, i32]
        L.moe_layer_stage_name.restype = C.c_char_p
        L.moe_test_block_dots.argtypes = [i32, vp, i32, i32, sz, Q, i32, vp, vp]
        L.moe_repack_tile64.argtypes = [i32, vp, sz, i32, i32, vp, vp]
        L.moe_repack_mx16.argtypes = [vp, sz, i32, i32, vp, sz, vp]
        L.moe_test_block_dots_mx16.argtypes = [vp, i32, i32, sz, Q, i32, vp, vp]
        L.moe_test_tile_dots.argtypes = [i32, vp, i32, i32, sz, Q, i32, vp, vp, sz, vp]
        L.moe_test_tile_dots_ws.argtypes = [i32, i32, i32, i32]
        L.moe_test_tile_dots_ws.restype = sz
        L.moe_test_preact.argtypes = [D, Q, i32, vp, i32, vp, vp, sz, vp]
        PC = C.POINTER(MoePoolConfig)
        L.moe_pool_create.argtypes = [PC, C.POINTER(vp)]
        L.moe_pool_destroy.argtypes = [vp]
        L.moe_pool_destroy.restype = None
        L.moe_pool_host_slab.argtypes = [vp, i32, i32]
        L.moe_pool_host_slab.restype = vp
        L.moe_pool_layer_tables.argtypes = [vp, i32, C.POINTER(vp), C.POINTER(vp), C.POINTER(vp)]
        L.moe_pool_resolve.argtypes = [vp, i32, vp, i32, vp]
        L.moe_pool_prefetch.argtypes = [vp, i32, vp, i32, vp]
        L.moe_pool_get_stats.argtypes = [vp, C.POINTER(MoePoolStats)]
        L.moe_pool_policy_trace.argtypes = [PC, i32, vp, vp, vp, vp, vp, vp, vp]
        L.moe_pool_layer_step.argtypes = [vp, i32, D, D, vp, i32, i32, vp, vp, vp, vp, sz, vp]
        L.moe_pool_step_workspace.argtypes = [D, i32]
        L.moe_pool_step_workspace.restype = sz
        for n in ("moe_quantize_act_q8k", "moe_route_topk", "moe_expert_ffn", "moe_layer_forward",
                  "moe_layer_forward_timed", "moe_test_block_dots", "moe_test_tile_dots",
                  "moe_test_preact", "moe_layer_forward_noalloc", "moe_probe_read_wall",
                  "moe_probe_mfma_i8", "moe_probe_empty_chain", "moe_pool_create", "moe_pool_layer_tables",
                  "moe_pool_resolve", "moe_pool_prefetch", "moe_pool_get_stats",
                  "moe_pool_policy_trace", "moe_pool_layer_step"):
            getattr(L, n).restype = i32
        _lib = L
    return _lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    raise TypeError(f"cannot pass {type(t)} as a device pointer")


def _stream(s) -> int | None:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(fn: str, st: int):
    if st != MOE_OK:
        raise MoeError(fn, st)


def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_status_str(s: int) -> str:
    return lib().moe_status_str(s).decode()


def moe_workspace_size(desc: MoeLayerDesc, T: int) -> int:
    return lib().moe_workspace_size(C.byref(desc), T)


def moe_quantize_act_q8k(x, dtype: int, T: int, H: int, fmt: int, out: MoeQact, stream=None):
    _check("moe_quantize_act_q8k",
           lib().moe_quantize_act_q8k(_ptr(x), dtype, T, H, fmt, C.byref(out), _stream(stream)))


def moe_route_topk(desc, x, dtype, T, ids, w, logits, ws, ws_bytes, stream=None):
    _check("moe_route_topk",
           lib().moe_route_topk(C.byref(desc), _ptr(x), dtype, T, _ptr(ids), _ptr(w),
                                _ptr(logits), _ptr(ws), ws_bytes, _stream(stream)))


def moe_expert_ffn(desc, xq: MoeQact, x, dtype, T, ids, w, y, ws, ws_bytes, stream=None):
    _check("moe_expert_ffn",
           lib().moe_expert_ffn(C.byref(desc), C.byref(xq), _ptr(x), dtype, T, _ptr(ids),
                                _ptr(w), _ptr(y), _ptr(ws), ws_bytes, _stream(stream)))


def moe_layer_forward(desc, x, dtype, T, y, ids_out, w_out, ws, ws_bytes, stream=None):
    _check("moe_layer_forward",
           lib().moe_layer_forward(C.byref(desc), _ptr(x), dtype, T, _ptr(y), _ptr(ids_out),
                                   _ptr(w_out), _ptr(ws), ws_bytes, _stream(stream)))


def moe_layer_forward_noalloc(desc, x, dtype, T, y, ids_out, w_out, stream=None):
    _check("moe_layer_forward_noalloc",
           lib().moe_layer_forward_noalloc(C.byref(desc), _ptr(x), dtype, T, _ptr(y),
                                           _ptr(ids_out), _ptr(w_out), _stream(stream)))


def moe_probe_read_wall(buf, nbytes, nwg, sink, stream=None):
    _check("moe_probe_read_wall",
           lib().moe_probe_read_wall(_ptr(buf), nbytes, nwg, _ptr(sink), _stream(stream)))


def moe_probe_empty_chain(n: int, stream=None):
    _check("moe_probe_empty_chain", lib().moe_probe_empty_chain(n, _stream(stream)))


def moe_probe_mfma_i8(k64, iters, nwg, sink, stream=None):
    _check("moe_probe_mfma_i8",
           lib().moe_probe_mfma_i8(k64, iters, nwg, _ptr(sink), _stream(stream)))


def moe_layer_forward_timed(desc, x, dtype, T, y, ids_out, w_out, ws, ws_bytes, stream,
                            events: list[int]):
    arr = (C.c_void_p * len(events))(*events)
    _check("moe_layer_forward_timed",
           lib().moe_layer_forward_timed(C.byref(desc), _ptr(x), dtype, T, _ptr(y),
                                         _ptr(ids_out), _ptr(w_out), _ptr(ws), ws_bytes,
                                         _stream(stream), arr, len(events)))


def moe_layer_stage_count(desc, T: int) -> int:
    return lib().moe_layer_stage_count(C.byref(desc), T)


def moe_layer_stage_name(desc, T: int, stage: int) -> str | None:
    r = lib().moe_layer_stage_name(C.byref(desc), T, stage)
    return None if r is None else r.decode()


def moe_repack_tile64(fmt, src, src_stride, n_rows, K, dst, stream=None):
    """One expert matrix from row order into 64-row tiles (moe_layout TILE64)."""
    _check("moe_repack_tile64",
           lib().moe_repack_tile64(fmt, _ptr(src), src_stride, n_rows, K, _ptr(dst),
                                   _stream(stream)))


def tile64_bytes(fmt, n_rows, K) -> int:
    """Bytes of one matrix in TILE64 order (no row padding)."""
    return n_rows * (K // 256) * {MOE_WFMT_Q4_K: 144, MOE_WFMT_Q6_K: 210}[fmt]


def moe_test_block_dots(fmt, rows, n_rows, K, stride, xq: MoeQact, token, out, stream=None):
    _check("moe_test_block_dots",
           lib().moe_test_block_dots(fmt, _ptr(rows), n_rows, K, stride, C.byref(xq), token,
                                     _ptr(out), _stream(stream)))


def moe_test_block_dots_mx16(rows, n_rows, K, stride, xq: MoeQact, token, out, stream=None):
    _check("moe_test_block_dots_mx16",
           lib().moe_test_block_dots_mx16(_ptr(rows), n_rows, K, stride, C.byref(xq), token,
                                          _ptr(out), _stream(stream)))


def moe_repack_mx16(src, src_stride, n_rows, K, dst, dst_stride, stream=None):
    """One MXFP4 matrix from row order into the MX16 order (moe_layout MX16)."""
    _check("moe_repack_mx16",
           lib().moe_repack_mx16(_ptr(src), src_stride, n_rows, K, _ptr(dst), dst_stride,
                                 _stream(stream)))


def moe_test_tile_dots(mode, rows, n_rows, K, stride, xq: MoeQact, n_tok, out, ws, ws_bytes,
                       stream=None):
    _check("moe_test_tile_dots",
           lib().moe_test_tile_dots(mode, _ptr(rows), n_rows, K, stride, C.byref(xq), n_tok,
                                    _ptr(out), _ptr(ws), ws_bytes, _stream(stream)))


def moe_test_tile_dots_ws(mode: int, n_rows: int, K: int, n_tok: int) -> int:
    return lib().moe_test_tile_dots_ws(mode, n_rows, K, n_tok)


def moe_test_preact(desc, xq: MoeQact, T, ids, which, out, ws, ws_bytes, stream=None):
    _check("moe_test_preact",
           lib().moe_test_preact(C.byref(desc), C.byref(xq), T, _ptr(ids), which, _ptr(out),
                                 _ptr(ws), ws_bytes, _stream(stream)))


def qact(qs, d, bsums, fmt: int, T: int, H: int, scales=None) -> MoeQact:
    """A moe_qact over caller buffers (scales: MXFP8 E8M0 rows)."""
    return MoeQact(_ptr(qs), _ptr(d), _ptr(bsums), fmt, T, H, _ptr(scales))


def mx8_scale_pitch(H: int) -> int:
    """Bytes per row of MXFP8 scales (H / 32 rounded up to a multiple of 16)."""
    return (H // 32 + 15) // 16 * 16


# ------------------------------------------------------------------ HIP events
_hip = None


def hip():
    """libamdhip64 for events on the library's stream (timing only)."""
    global _hip
    if _hip is None:
        h = C.CDLL("libamdhip64.so")
        h.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        h.hipEventDestroy.argtypes = [C.c_void_p]
        h.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        h.hipEventSynchronize.argtypes = [C.c_void_p]
        h.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        _hip = h
    return _hip


class HipEvent:
    def __init__(self):
        self.h = C.c_void_p()
        r = hip().hipEventCreate(C.byref(self.h))
        if r != 0:
            raise RuntimeError(f"hipEventCreate failed ({r})")

    @property
    def handle(self) -> int:
        return self.h.value

    def record(self, stream=None):
        r = hip().hipEventRecord(self.h, _stream(stream))
        if r != 0:
            raise RuntimeError(f"hipEventRecord failed ({r})")

    def synchronize(self):
        hip().hipEventSynchronize(self.h)

    def elapsed_ms(self, end: "HipEvent") -> float:
        out = C.c_float()
        r = hip().hipEventElapsedTime(C.byref(out), self.h, end.h)
        if r != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({r})")
        return out.value

    def __del__(self):
        try:
            if self.h:
                hip().hipEventDestroy(self.h)
        except Exception:
            pass


# ------------------------------------------------------------------ expert pool
def _np_ptr(a):
    return None if a is None else a.ctypes.data


class Pool:
    """moe_pool: pinned host tier + device slot arena (include/moe_pool.h)."""

    def __init__(self, n_layers, n_experts, slab_bytes, up_offset, down_offset, n_slots,
                 n_transient):
        self.cfg = MoePoolConfig(n_layers, n_experts, slab_bytes, up_offset, down_offset,
                                 n_slots, n_transient)
        h = C.c_void_p()
        _check("moe_pool_create", lib().moe_pool_create(C.byref(self.cfg), C.byref(h)))
        self.h = h

    def host_slab(self, layer, expert):
        """numpy uint8 view of one expert's pinned host slab."""
        import numpy as np
        p = lib().moe_pool_host_slab(self.h, layer, expert)
        if not p:
            raise IndexError((layer, expert))
        return np.ctypeslib.as_array((C.c_uint8 * self.cfg.slab_bytes).from_address(p))

    def tables(self, layer):
        g, u, d = C.c_void_p(), C.c_void_p(), C.c_void_p()
        _check("moe_pool_layer_tables",
               lib().moe_pool_layer_tables(self.h, layer, C.byref(g), C.byref(u), C.byref(d)))
        return g.value, u.value, d.value

    def resolve(self, layer, ids_host, stream=None):
        import numpy as np
        ids = np.ascontiguousarray(ids_host, np.int32).ravel()
        _check("moe_pool_resolve", lib().moe_pool_resolve(self.h, layer, _np_ptr(ids), ids.size,
                                                          _stream(stream)))

    def prefetch(self, layer, ids_host, stream=None):
        import numpy as np
        ids = np.ascontiguousarray(ids_host, np.int32).ravel()
        _check("moe_pool_prefetch", lib().moe_pool_prefetch(self.h, layer, _np_ptr(ids), ids.size,
                                                            _stream(stream)))

    def layer_step(self, layer, desc, next_desc, x, dtype, T, ids, w, y, ws, ws_bytes,
                   stream=None):
        """moe_pool_layer_step: route, resolve (+ prefetch of layer + 1 when
        next_desc is given), quantize and expert FFN of one layer."""
        _check("moe_pool_layer_step",
               lib().moe_pool_layer_step(self.h, layer, C.byref(desc),
                                         C.byref(next_desc) if next_desc is not None else None,
                                         _ptr(x), dtype, T, _ptr(ids), _ptr(w), _ptr(y), _ptr(ws),
                                         ws_bytes, _stream(stream)))

    def stats(self) -> dict:
        s = MoePoolStats()
        _check("moe_pool_get_stats", lib().moe_pool_get_stats(self.h, C.byref(s)))
        return {n: getattr(s, n) for n in POOL_STAT_FIELDS}

    def close(self):
        if self.h:
            lib().moe_pool_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def moe_pool_step_workspace(desc, T: int) -> int:
    return lib().moe_pool_step_workspace(C.byref(desc), T)


def moe_pool_policy_trace(cfg: MoePoolConfig, ops):
    """Run the slot policy alone over ops = [(kind 0 resolve / 1 prefetch, layer,
    ids)]; returns (per-op list of (key, slot, copy) or None for a failed
    resolve, stats dict without bytes_h2d)."""
    import numpy as np
    kind = np.array([o[0] for o in ops], np.int32)
    layer = np.array([o[1] for o in ops], np.int32)
    lens = [len(o[2]) for o in ops]
    off = np.zeros(len(ops) + 1, np.int32)
    off[1:] = np.cumsum(lens)
    ids = np.concatenate([np.asarray(o[2], np.int32) for o in ops]) if ops else np.zeros(0, np.int32)
    out = np.zeros(3 * max(1, int(off[-1])), np.int32)
    n_out = np.zeros(len(ops), np.int32)
    stats = np.zeros(10, np.int64)
    _check("moe_pool_policy_trace",
           lib().moe_pool_policy_trace(C.byref(cfg), len(ops), _np_ptr(kind), _np_ptr(layer),
                                       _np_ptr(off), _np_ptr(ids), _np_ptr(out), _np_ptr(n_out),
                                       _np_ptr(stats)))
    res, w = [], 0
    for n in n_out:
        if n < 0:
            res.append(None)
            continue
        res.append([tuple(int(v) for v in out[3 * (w + i):3 * (w + i) + 3]) for i in range(n)])
        w += n
    return res, dict(zip(POOL_STAT_FIELDS[:10], (int(v) for v in stats)))
