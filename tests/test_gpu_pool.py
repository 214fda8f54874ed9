"""Expert pool on the GPU: a stack of layers whose routed experts live only in
the pinned host tier, resolved into a small device arena each step (with and
without next-layer prefetch), gives bitwise the outputs of the same stack with
every expert resident, and the oracle's within the layer tolerance."""
import ctypes as C

import numpy as np
import pytest
import torch

import gen
import oracle
import quantized_moe_expert_route_amd as M
from gen.device import DeviceLayer, x_to_device
from tests.gpu_common import Y_TOL, rel_err, say
from tests.shrunk import SHRUNK

pytestmark = pytest.mark.gpu


def make_stack(base, L):
    return [gen.make_layer(base.with_(seed=base.seed + 101 * l)) for l in range(L)]


def pool_desc(dl: DeviceLayer, pool: M.Pool, layer: int):
    """The layer's descriptor with the routed experts' tables taken from the
    pool (the shared expert stays in the resident upload)."""
    d = M.MoeLayerDesc()
    C.pointer(d)[0] = dl.desc
    d.gate, d.up, d.down = pool.tables(layer)
    return d


def run_stack(descs, cfg, x0, pool=None, prefetch=False, route_descs=None):
    """Residual stack x_{l+1} = x_l + y_l; returns per-layer (y, ids)."""
    T, H = x0.shape
    afmt = M.MOE_AFMT_Q8_K if gen.BLOCK_ELEMS[cfg.fmt_gu] == 256 else M.MOE_AFMT_Q8_32
    B = gen.BLOCK_ELEMS[cfg.fmt_gu]
    xq_t = (torch.empty((T, H), dtype=torch.int8, device="cuda"),
            torch.empty((T, H // B), dtype=torch.float32, device="cuda"),
            torch.empty((T, H // 16), dtype=torch.int16, device="cuda"))
    xq = M.qact(xq_t[0], xq_t[1], xq_t[2] if B == 256 else None, afmt, T, H)
    ids = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
    nids = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
    nw = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
    ws_n = max(M.moe_workspace_size(d, T) for d in descs)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    x = torch.from_numpy(x0).cuda()
    out = []
    for l, d in enumerate(descs):
        M.moe_route_topk(d, x, M.MOE_DTYPE_F32, T, ids, w, None, ws, ws_n)
        ids_h = ids.cpu().numpy()
        if pool is not None:
            pool.resolve(l, ids_h)
            if prefetch and l + 1 < len(descs):
                # next layer's router on this layer's input
                M.moe_route_topk(descs[l + 1], x, M.MOE_DTYPE_F32, T, nids, nw, None, ws, ws_n)
                pool.prefetch(l + 1, nids.cpu().numpy())
        M.moe_quantize_act_q8k(x, M.MOE_DTYPE_F32, T, H, afmt, xq)
        y = torch.empty((T, H), dtype=torch.float32, device="cuda")
        M.moe_expert_ffn(d, xq, x, M.MOE_DTYPE_F32, T, ids, w, y, ws, ws_n)
        torch.cuda.synchronize()
        out.append((y.cpu().numpy(), ids_h, x.cpu().numpy(), w.cpu().numpy()))
        x = x + y
    return out


@pytest.mark.parametrize("name,T,slots,trans,prefetch,layout", [
    ("qwen3.6-35b-a3b", 2, 24, 16, False, 0), ("qwen3.6-35b-a3b", 2, 24, 16, True, 0),
    ("qwen3.6-35b-a3b", 1, 12, 8, True, 0), ("gpt-oss-20b", 3, 14, 12, True, 0),
    ("deepseek-v4-flash", 2, 20, 12, False, 0),
    ("gpt-oss-20b", 2, 14, 12, False, M.MOE_LAYOUT_MX16)])
def test_pool_stack_matches_resident(name, T, slots, trans, prefetch, layout):
    L, steps = 4, 6
    base = SHRUNK[name].with_(T=T)
    stack = make_stack(base, L)
    dls = [DeviceLayer(data, layout=layout) for data in stack]
    cfg = base
    pool = M.Pool(L, cfg.E, cfg.expert_bytes, cfg.gate_bytes, 2 * cfg.gate_bytes, slots, trans)
    for l, (data, dl) in enumerate(zip(stack, dls)):
        # the host tier holds the experts in the layer's own byte order (MX16:
        # the device repack of the row-order bytes)
        src = data.pool if layout == 0 else dl.pools[0].cpu().numpy().reshape(data.pool.shape[0], -1)
        for e in range(cfg.E):
            pool.host_slab(l, e)[:] = src[e]
    pdescs = [pool_desc(dl, pool, l) for l, dl in enumerate(dls)]
    rdescs = [dl.desc for dl in dls]
    say(f"pool {name} T={T} slots={slots}/{trans} prefetch={prefetch}")
    for step in range(steps):
        x0, _ = gen.make_x(base, T=T, x_index=step)
        x0 = x0.astype(np.float32)
        got = run_stack(pdescs, cfg, x0, pool=pool, prefetch=prefetch)
        want = run_stack(rdescs, cfg, x0)
        for l in range(L):
            assert np.array_equal(got[l][1], want[l][1]), (step, l)
            assert np.array_equal(got[l][0], want[l][0]), (step, l)
    st = pool.stats()
    say(f"  stats {st}")
    assert st["epochs"] == L * steps
    assert st["evictions"] > 0 and st["hits_resident"] > 0
    assert st["bytes_h2d"] == (st["admitted"] + st["transient_loads"]) * cfg.expert_bytes
    if prefetch:
        assert st["prefetch_loads"] > 0 and st["prefetch_hits"] > 0
    # the last step's last layer against the oracle
    y, ids, x, w = got[L - 1]
    Lo = oracle.Layer(stack[L - 1])
    for t in range(T):
        ref = Lo.expert_part(x[t], ids[t], w[t])
        assert rel_err(y[t][None], ref[None]).max() <= Y_TOL
    pool.close()


def test_pool_resolve_too_many_unique_experts():
    base = SHRUNK["qwen3.6-35b-a3b"]
    pool = M.Pool(1, base.E, base.expert_bytes, base.gate_bytes, 2 * base.gate_bytes, 6, 4)
    with pytest.raises(M.MoeError) as ei:
        pool.resolve(0, np.arange(7, dtype=np.int32))
    assert ei.value.status == M.MOE_ENOWORKSPACE
    pool.resolve(0, np.arange(6, dtype=np.int32))
    torch.cuda.synchronize()
    g, u, d = pool.tables(0)
    tab = torch.empty(3 * base.E, dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    hip = M.hip()
    hip.hipMemcpy.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_int]
    host = np.zeros(3 * base.E, np.int64)
    assert hip.hipMemcpy(host.ctypes.data, g, host.nbytes, 2) == 0  # device to host
    assert np.all(host[:6] != 0) and np.all(host[6:base.E] == 0)
    assert np.all(host[base.E + 6:2 * base.E] == 0)
    pool.close()


@pytest.mark.parametrize("name,T,prefetch", [("qwen3.6-35b-a3b", 2, True),
                                             ("gpt-oss-20b", 3, False)])
def test_pool_layer_step_matches_resident(name, T, prefetch):
    """moe_pool_layer_step (route, host round trip, resolve, prefetch, quantize,
    FFN in one native call) over a residual stack: bitwise the resident run."""
    L, steps = 3, 4
    base = SHRUNK[name].with_(T=T)
    stack = make_stack(base, L)
    dls = [DeviceLayer(data) for data in stack]
    cfg = base
    # transient slots >= the unique experts of one step (T k, at most E)
    n_tr = min(cfg.E, T * cfg.k)
    pool = M.Pool(L, cfg.E, cfg.expert_bytes, cfg.gate_bytes, 2 * cfg.gate_bytes, n_tr + 8, n_tr)
    for l, data in enumerate(stack):
        for e in range(cfg.E):
            pool.host_slab(l, e)[:] = data.pool[e]
    pdescs = [pool_desc(dl, pool, l) for l, dl in enumerate(dls)]
    rdescs = [dl.desc for dl in dls]
    ws_n = max(M.moe_pool_step_workspace(d, T) for d in pdescs)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    ids = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
    for step in range(steps):
        x0, _ = gen.make_x(base, T=T, x_index=step)
        x = torch.from_numpy(x0.astype(np.float32)).cuda()
        want = run_stack(rdescs, cfg, x0.astype(np.float32))
        for l in range(L):
            y = torch.empty((T, cfg.H), dtype=torch.float32, device="cuda")
            nd = pdescs[l + 1] if prefetch and l + 1 < L else None
            pool.layer_step(l, pdescs[l], nd, x, M.MOE_DTYPE_F32, T, ids, w, y, ws, ws_n)
            torch.cuda.synchronize()
            assert np.array_equal(ids.cpu().numpy(), want[l][1]), (step, l)
            assert np.array_equal(y.cpu().numpy(), want[l][0]), (step, l)
            x = x + y
    st = pool.stats()
    assert st["evictions"] > 0
    if prefetch:
        assert st["prefetch_loads"] > 0
    pool.close()
