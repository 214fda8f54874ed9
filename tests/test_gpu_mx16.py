"""MXFP4 rows in the MX16 order (moe_layout MX16): the device repack against
the order written out from its definition, the integer block partials of the
MX16 GEMV routine against the oracle (exact), and whole layers against the
oracle and bitwise against the same layer in row order."""
import numpy as np
import pytest
import torch

import gen
import oracle
import quantized_moe_expert_route_amd as M
from gen.device import DeviceLayer, x_to_device
from tests.gpu_common import check_layer, random_blocks, run_layer, say, upload_q8, x_cases

pytestmark = pytest.mark.gpu


def mx16_reference(mat: np.ndarray, K: int, dst_stride: int, fill: int) -> np.ndarray:
    """Rows of 17-byte blocks (scale byte, then 16 nibble bytes) in the MX16
    order: the nibble bytes of block b at 16 b, the scale byte of block b at
    16 nb + b, zeros up to the next multiple of 4, the rest of the row as it
    was (fill)."""
    nb = K // 32
    out = np.full((mat.shape[0], dst_stride), fill, np.uint8)
    for r in range(mat.shape[0]):
        for b in range(nb):
            blk = mat[r, 17 * b:17 * b + 17]
            out[r, 16 * b:16 * b + 16] = blk[1:]
            out[r, 16 * nb + b] = blk[0]
        end = 16 * nb + (nb + 3) // 4 * 4
        out[r, 17 * nb:end] = 0
    return out


@pytest.mark.parametrize("K,n_rows", [(32, 3), (96, 5), (2880, 7), (8192, 2)])
def test_repack_mx16_bytes(K, n_rows):
    rng = np.random.default_rng(K)
    nb = K // 32
    stride = gen.row_stride(gen.MXFP4, K) + 16
    mat = rng.integers(0, 256, (n_rows, stride), dtype=np.uint8)
    dst_stride = stride + 32
    dst = torch.full((n_rows * dst_stride,), 0xAB, dtype=torch.uint8, device="cuda")
    src = torch.from_numpy(mat.reshape(-1).copy()).cuda()
    M.moe_repack_mx16(src, stride, n_rows, K, dst, dst_stride)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().reshape(n_rows, dst_stride)
    assert np.array_equal(got, mx16_reference(mat, K, dst_stride, 0xAB)), (K, nb)


@pytest.mark.parametrize("K", [32, 96, 2048, 2880, 3072, 4096, 8192])
@pytest.mark.parametrize("kind", ["generated", "random_fields"])
def test_block_dots_mx16_exact(K, kind):
    """Every MX16 slot pattern: 1 block, 3 (one lane group), 64, 90 and 96
    (folded tails), 128, 256 blocks per row."""
    say(f"block_dots mx16 K={K} {kind}")
    n_rows = 37
    rng = np.random.default_rng(K + 7)
    stride = gen.row_stride(gen.MXFP4, K)
    if kind == "generated":
        w = gen.normal(5, gen.T_DOWN, gen.MXFP4, n_rows, K, 0.02)
        w[0] = 0
        mat = gen.encode_matrix(gen.MXFP4, w)
    else:
        raw = random_blocks(gen.MXFP4, n_rows, K, rng)
        mat = np.zeros((n_rows, stride), np.uint8)
        mat[:, :raw.shape[1]] = raw
    x = x_cases(3, K, 9)
    host, q, keep = upload_q8(x, 32)
    src = torch.from_numpy(mat).cuda()
    rows = torch.zeros_like(src)
    M.moe_repack_mx16(src, mat.shape[1], n_rows, K, rows, mat.shape[1])
    nb = K // 32
    for token in range(3):
        out = torch.full((n_rows, nb, 2), -7, dtype=torch.int32, device="cuda")
        M.moe_test_block_dots_mx16(rows, n_rows, K, mat.shape[1], q, token, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        for r in range(n_rows):
            ref = oracle.block_partials(gen.MXFP4, mat[r], K, host[0][token], None)
            assert np.array_equal(got[r], ref), (token, r)


def _mx_cfg(H, F, E=8, k=2, name="mx16"):
    return gen.CONFIGS["gpt-oss-20b"].with_(name=name, H=H, F=F, E=E, k=k)


@pytest.mark.parametrize("H,F,T", [(2880, 2880, 1), (2880, 2880, 3), (1024, 512, 2),
                                   (3072, 4096, 1), (96, 2880, 2), (8192, 1024, 1)])
def test_layer_mx16_matches_rows(H, F, T):
    """The layer in the MX16 order against the oracle, and bitwise equal to the
    same layer in row order (same block dots, same summation order)."""
    cfg = _mx_cfg(H, F) if (H, F) != (2880, 2880) else gen.CONFIGS["gpt-oss-20b"]
    data = gen.make_layer(cfg)
    y16, ids16, w16, _ = check_layer(cfg, data=data, T=T, layout=M.MOE_LAYOUT_MX16)
    x, xb = gen.make_x(cfg, T=T, x_index=0)
    dl = DeviceLayer(data, layout=M.MOE_LAYOUT_ROWS)
    xt, dt = x_to_device(data, x, xb)
    y, ids, w = run_layer(dl, xt, dt, T)
    assert np.array_equal(ids, ids16) and np.array_equal(w, w16)
    assert np.array_equal(y.view(np.uint32), y16.view(np.uint32)), "MX16 and row order differ"


def test_layer_mx16_shared_and_absent():
    """Shared expert with a gate vector, sigmoid router, NULL experts and an
    interleaved (fused) gate_up tensor, in the MX16 order."""
    cfg = _mx_cfg(2880, 1440, E=16, k=4, name="mx16-shared").with_(shared=True,
                                                                     router=gen.SIGMOID)
    data = gen.make_layer(cfg)
    present = np.ones(cfg.E, bool)
    present[[1, 5, 9]] = False
    rng = np.random.default_rng(3)
    vec = rng.standard_normal(cfg.H).astype(np.float32) * 0.05
    say("mx16 shared/absent")
    check_layer(cfg, data=data, T=3, present=present, sh_gate_vec=vec,
                layout=M.MOE_LAYOUT_MX16)
    check_layer(cfg, data=data, T=2, interleaved=True, layout=M.MOE_LAYOUT_MX16)
