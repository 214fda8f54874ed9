"""Upload a generated layer to the GPU and describe it to the library.

Input plumbing for the tests and the benchmark: device tensors (torch), the
per-expert device pointer tables and a filled ``MoeLayerDesc``. Layer copies
are device-to-device clones at distinct addresses, so a rotation over copies
reads HBM instead of caches.
"""
from __future__ import annotations

import numpy as np
import torch

import quantized_moe_expert_route_amd as M


def _dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def x_to_device(data, x_np: np.ndarray | None = None, xb_np: np.ndarray | None = None,
                device="cuda"):
    """x as the layer receives it: fp32 [T, H], or bf16 when the workload says so.
    Returns (tensor, dtype enum)."""
    cfg = data.cfg
    if cfg.x_bf16:
        xb = data.x_bf16 if xb_np is None else xb_np
        t = _dev(xb.view(np.int16), device).view(torch.bfloat16)
        return t, M.MOE_DTYPE_BF16
    x = data.x if x_np is None else x_np
    return _dev(x.astype(np.float32), device), M.MOE_DTYPE_F32


def interleave_gate_up(data) -> np.ndarray:
    """The pool with each expert's gate and up matrices stored as one fused
    tensor of alternating rows (gate row r at 2r, up row r at 2r + 1), as
    checkpoints that keep a fused gate_up projection do; the stacked form
    (all gate rows, then all up rows) is the default pool layout."""
    cfg = data.cfg
    pool = data.pool.copy()
    n, s = cfg.F, cfg.stride_gu
    for e in range(pool.shape[0]):
        g = data.pool[e, :n * s].reshape(n, s)
        u = data.pool[e, n * s:2 * n * s].reshape(n, s)
        fused = pool[e, :2 * n * s].reshape(n, 2, s)
        fused[:, 0], fused[:, 1] = g, u
    return pool


def tile_pool(cfg, pool_rows: torch.Tensor) -> torch.Tensor:
    """The pool with every expert matrix (the shared expert's too) reordered
    by the library into 64-row tiles (moe_layout TILE64), each at the offset
    its row-order matrix had."""
    out = torch.zeros_like(pool_rows)
    es = cfg.expert_bytes
    s = torch.cuda.current_stream().cuda_stream
    for e in range(cfg.n_pool):
        base = e * es
        for off, fmt, n, K, st in ((0, cfg.fmt_gu, cfg.F, cfg.H, cfg.stride_gu),
                                   (cfg.gate_bytes, cfg.fmt_gu, cfg.F, cfg.H, cfg.stride_gu),
                                   (2 * cfg.gate_bytes, cfg.fmt_d, cfg.H, cfg.F, cfg.stride_d)):
            M.moe_repack_tile64(fmt, pool_rows.data_ptr() + base + off, st, n, K,
                                out.data_ptr() + base + off, stream=s)
    torch.cuda.synchronize()
    return out


def mx16_pool(cfg, pool_rows: torch.Tensor) -> torch.Tensor:
    """The pool with every MXFP4 row (the shared expert's too) reordered by the
    library into the MX16 order (moe_layout MX16): per row, the 16 nibble bytes
    of every block, then the scale bytes; same row strides. Rows are repacked
    one by one, so stacked and interleaved gate/up tensors alike."""
    out = torch.zeros_like(pool_rows)
    es = cfg.expert_bytes
    s = torch.cuda.current_stream().cuda_stream
    for e in range(cfg.n_pool):
        base = e * es
        for off, n, K, st in ((0, 2 * cfg.F, cfg.H, cfg.stride_gu),
                              (2 * cfg.gate_bytes, cfg.H, cfg.F, cfg.stride_d)):
            M.moe_repack_mx16(pool_rows.data_ptr() + base + off, st, n, K,
                              out.data_ptr() + base + off, st, stream=s)
    torch.cuda.synchronize()
    return out


class DeviceLayer:
    def __init__(self, data, copies: int = 1, present=None, route_scale=None, norm_topk=None,
                 use_shared: bool = True, sh_gate_vec=None, sel_bias="data", device="cuda",
                 path: int = 0, interleaved: bool = False, layout: int | None = None):
        cfg = data.cfg
        self.cfg = cfg
        self.device = device
        E = cfg.E
        present = np.ones(E, bool) if present is None else np.asarray(present, bool)
        self.present = present
        self.layout = cfg.layout if layout is None else layout
        if self.layout == M.MOE_LAYOUT_TILE64 and interleaved:
            raise ValueError("64-row tiles have their own order: no interleaved gate/up")
        # gate/up row r of an expert: interleaved at (2r, 2r + 1) of one fused
        # tensor, else stacked (gate matrix, then up matrix)
        up_off = cfg.stride_gu if interleaved else cfg.gate_bytes
        gu_stride = 2 * cfg.stride_gu if interleaved else cfg.stride_gu
        pool0 = _dev(interleave_gate_up(data) if interleaved else data.pool, device)
        if self.layout == M.MOE_LAYOUT_TILE64:
            pool0 = tile_pool(cfg, pool0)
        elif self.layout == M.MOE_LAYOUT_MX16:
            pool0 = mx16_pool(cfg, pool0)
        self.pools = [pool0] + [pool0.clone() for _ in range(1, copies)]
        self.w_router = _dev(data.w_router, device)
        sb = data.sel_bias if isinstance(sel_bias, str) else sel_bias
        self.sel_bias = None if sb is None else _dev(sb.astype(np.float32), device)
        self.b_gate = self.b_up = self.b_down = None
        if data.b_gate is not None:
            self.b_gate = _dev(data.b_gate, device)
            self.b_up = _dev(data.b_up, device)
            self.b_down = _dev(data.b_down, device)
        self.sh_gate_vec = None if sh_gate_vec is None else _dev(
            np.asarray(sh_gate_vec, np.float32), device)
        es = cfg.expert_bytes
        self._tables = []
        self.descs = []
        for pool in self.pools:
            base = pool.data_ptr()
            g = [base + e * es if present[e] else 0 for e in range(E)]
            u = [base + e * es + up_off if present[e] else 0 for e in range(E)]
            dn = [base + e * es + 2 * cfg.gate_bytes if present[e] else 0 for e in range(E)]
            tg = torch.tensor(g, dtype=torch.int64, device=device)
            tu = torch.tensor(u, dtype=torch.int64, device=device)
            td = torch.tensor(dn, dtype=torch.int64, device=device)
            keep = [tg, tu, td]
            d = M.MoeLayerDesc()
            d.hidden, d.ffn, d.n_expert, d.top_k = cfg.H, cfg.F, E, cfg.k
            d.router = cfg.router
            d.norm_topk = cfg.norm_topk if norm_topk is None else norm_topk
            d.route_scale = cfg.route_scale if route_scale is None else route_scale
            d.w_router = self.w_router.data_ptr()
            d.sel_bias = None if self.sel_bias is None else self.sel_bias.data_ptr()
            d.fmt_gate = d.fmt_up = cfg.fmt_gu
            d.fmt_down = cfg.fmt_d
            d.stride_gate = d.stride_up = gu_stride
            d.stride_down = cfg.stride_d
            d.gate, d.up, d.down = tg.data_ptr(), tu.data_ptr(), td.data_ptr()
            if self.b_gate is not None:
                bt = []
                for b, n in ((self.b_gate, cfg.F), (self.b_up, cfg.F), (self.b_down, cfg.H)):
                    t = torch.tensor([b.data_ptr() + e * n * 4 for e in range(E)],
                                     dtype=torch.int64, device=device)
                    bt.append(t)
                keep += bt
                d.b_gate, d.b_up, d.b_down = (t.data_ptr() for t in bt)
            d.act = cfg.act
            d.act_alpha, d.act_limit = cfg.act_alpha, cfg.act_limit
            if cfg.shared and use_shared:
                sh = base + E * es
                d.sh_gate, d.sh_up, d.sh_down = sh, sh + up_off, sh + 2 * cfg.gate_bytes
            d.sh_gate_vec = None if self.sh_gate_vec is None else self.sh_gate_vec.data_ptr()
            d.path = path  # moe_path: 0 auto, 1 per-pair GEMV, 2 expert-grouped
            d.act_quant = getattr(cfg, "act_quant", 0)  # moe_actq: 0 q8, 1 MXFP8
            d.layout = self.layout  # moe_layout: 0 rows, 1 64-row tiles, 2 MX16 rows
            self._tables.append(keep)
            self.descs.append(d)

    @property
    def desc(self) -> M.MoeLayerDesc:
        return self.descs[0]

    def workspace(self, T: int) -> torch.Tensor:
        n = M.moe_workspace_size(self.desc, T)
        if n == 0:
            raise ValueError("invalid descriptor or token count")
        return torch.empty(n, dtype=torch.uint8, device=self.device)
