"""moe_layer_forward_noalloc (workspace from the library's static device
scratch) against moe_layer_forward with a caller workspace: the same kernels
on the same inputs give the same bytes (ids, weights and y bitwise equal; y
also within the layer tolerance of the oracle). Calls run back to back on the
one scratch, the second with a smaller input, then a layer of another format.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
import quantized_moe_expert_route_amd as M
from gen.device import DeviceLayer, x_to_device
from tests.gpu_common import Y_TOL, rel_err, run_layer, say
from tests.shrunk import SHRUNK

pytestmark = pytest.mark.gpu


def _noalloc(dl, xt, dt, T):
    cfg = dl.cfg
    y = torch.full((T, cfg.H), float("nan"), dtype=torch.float32, device="cuda")
    ids = torch.full((T, cfg.k), -5, dtype=torch.int32, device="cuda")
    w = torch.full((T, cfg.k), float("nan"), dtype=torch.float32, device="cuda")
    M.moe_layer_forward_noalloc(dl.desc, xt, dt, T, y, ids, w)
    torch.cuda.synchronize()
    return y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("seq", [
    # (workload, T) in call order: grouped path, then a smaller GEMV call; and
    # the reverse order on the Qwen3.6 decode shape at full size
    [("kimi-k2", 20), ("kimi-k2", 3), ("gpt-oss-20b", 2)],
    [("qwen3.6-35b-a3b-full", 1), ("qwen3.6-35b-a3b-full", 9), ("deepseek-v4-flash", 1)],
    # MXFP4 rows in the MX16 order: h quantized once per pair in the scratch
    [("gpt-oss-20b-mx16", 3), ("gpt-oss-20b-mx16", 1)],
])
def test_noalloc_matches_forward(seq):
    for name, T in seq:
        cfg = (gen.CONFIGS["qwen3.6-35b-a3b"] if name.endswith("-full")
               else SHRUNK[name.replace("-mx16", "")])
        say(f"noalloc {cfg.name} T={T}")
        data = gen.make_layer(cfg)
        x, xb = gen.make_x(cfg, T=T, x_index=T + 3)
        # the shrunk Kimi-K2 chunk on the expert-grouped path, the rest as the
        # automatic rule picks
        dl = DeviceLayer(data, path=M.MOE_PATH_GROUPED if (name, T) == ("kimi-k2", 20) else 0,
                         layout=M.MOE_LAYOUT_MX16 if name.endswith("-mx16") else None)
        xt, dt = x_to_device(data, x, xb)
        assert M.moe_workspace_size(dl.desc, T) <= M.MOE_NOALLOC_SCRATCH_BYTES
        y0, ids0, w0 = run_layer(dl, xt, dt, T)
        y1, ids1, w1 = _noalloc(dl, xt, dt, T)
        assert np.array_equal(ids0, ids1)
        assert np.array_equal(w0.view(np.uint32), w1.view(np.uint32))
        assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))
        ref = oracle.Layer(data).forward(x, tokens=[0, T - 1], threads=2)
        assert np.array_equal(ids1[[0, T - 1]], ref["ids"])
        assert rel_err(y1[[0, T - 1]], ref["y"]).max() <= Y_TOL
