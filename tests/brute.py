"""Brute-force dense fp64 evaluation of the layer for the oracle pins (numpy/torch).

Weights are fully dequantized into dense fp64 matrices and multiplied with
numpy; routing uses numpy's lexsort and torch's softmax/sigmoid. Only separately
pinned oracle primitives are reused: block dequantization and the q8 and
MXFP8 activation recipes."""
import numpy as np

import gen
import torch

import oracle


def dense_experts(data, experts):
    cfg = data.cfg
    out = {}
    for e in experts:
        out[e] = (oracle.dequant_matrix(cfg.fmt_gu, data.gate(e).reshape(cfg.F, -1), cfg.H),
                  oracle.dequant_matrix(cfg.fmt_gu, data.up(e).reshape(cfg.F, -1), cfg.H),
                  oracle.dequant_matrix(cfg.fmt_d, data.down(e).reshape(cfg.H, -1), cfg.F))
    return out


def act(cfg, g, u):
    g = torch.from_numpy(g)
    u = torch.from_numpy(u)
    if cfg.act == 0:
        return (torch.nn.functional.silu(g) * u).numpy()
    gc = torch.clamp(g, max=cfg.act_limit)
    uc = torch.clamp(u, min=-cfg.act_limit, max=cfg.act_limit)
    return (gc * torch.sigmoid(cfg.act_alpha * gc) * (uc + 1)).numpy()


def qdeq(v, B):
    qs, d, _ = oracle.quantize_q8(v.astype(np.float32), B)
    return qs.astype(np.float64) * np.repeat(d.astype(np.float64), B)


def brute_layer(data, x, present=None, route_scale=None, sh_gate_vec=None, dense=None,
                sel_bias="data"):
    cfg = data.cfg
    E, k = cfg.E, cfg.k
    present = np.ones(E, bool) if present is None else present
    rs = cfg.route_scale if route_scale is None else route_scale
    sb = data.sel_bias if isinstance(sel_bias, str) else sel_bias
    Bx = 32 if gen.BLOCK_ELEMS[cfg.fmt_gu] == 32 else 256
    Bh = 32 if gen.BLOCK_ELEMS[cfg.fmt_d] == 32 else 256
    if dense is None:
        dense = dense_experts(data, range(cfg.n_pool))
    ys, idss, ws = [], [], []
    for t in range(x.shape[0]):
        xt = x[t].astype(np.float32)
        logits = (data.w_router.astype(np.float64) @ xt.astype(np.float64)).astype(np.float32)
        key = logits if sb is None else (logits + sb).astype(np.float32)
        ids = np.lexsort((np.arange(E), -key.astype(np.float64)))[:k]
        lt = torch.from_numpy(logits.astype(np.float64))
        if cfg.router == 0:
            w = torch.softmax(lt[ids], 0).numpy() if cfg.norm_topk else \
                torch.softmax(lt, 0).numpy()[ids]
        else:
            s = torch.sigmoid(lt[ids]).numpy()
            w = s / s.sum() if cfg.norm_topk else s
        w = w * rs
        mx8 = getattr(cfg, "act_quant", 0) == 1
        a = mx8deq(xt) if mx8 else qdeq(xt, Bx)
        y = np.zeros(cfg.H)

        def ffn(e, bias_idx):
            Wg, Wu, Wd = dense[e]
            g = Wg @ a
            u = Wu @ a
            if bias_idx is not None and data.b_gate is not None:
                g = g + data.b_gate[bias_idx]
                u = u + data.b_up[bias_idx]
            h32 = act(cfg, g, u).astype(np.float32)
            o = Wd @ (mx8deq(h32) if mx8 else qdeq(h32, Bh))
            if bias_idx is not None and data.b_down is not None:
                o = o + data.b_down[bias_idx]
            return o

        for j, e in enumerate(ids):
            if present[e]:
                y += w[j] * ffn(e, e)
        if cfg.shared:
            wsh = 1.0
            if sh_gate_vec is not None:
                wsh = torch.sigmoid(torch.tensor(float(
                    sh_gate_vec.astype(np.float64) @ xt.astype(np.float64)), dtype=torch.float64)).item()
            y += wsh * ffn(E, None)
        ys.append(y)
        idss.append(ids)
        ws.append(w)
    return np.stack(ys), np.stack(idss), np.stack(ws)


def mx8deq(v):
    """MXFP8 (OCP MX v1.0) round trip of a vector through the oracle's
    separately pinned quantizer and element decode."""
    q, e = oracle.quantize_mx8(v.astype(np.float32))
    vals = np.array([oracle.e4m3(int(c)) for c in range(256)])
    return vals[q] * np.repeat(np.ldexp(1.0, e.astype(np.int64) - 127), 32)
