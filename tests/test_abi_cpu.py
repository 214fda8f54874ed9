"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and host-side validation rejects bad arguments before any
work is enqueued. Every call here fails validation (or is a T = 0 no-op), so
nothing reaches a kernel launch."""
import ctypes as C
import os
import re

import pytest

import gen
import quantized_moe_expert_route_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # 256-aligned address that is never dereferenced


def header_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for h in sorted(os.listdir(inc)):
        if h.endswith(".h"):
            src = re.sub(r"/\*.*?\*/", "", open(os.path.join(inc, h)).read(), flags=re.S)
            names |= set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_library_exports_header_symbols():
    L = M.lib()
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(M.ABI_FUNCTIONS)


def test_version_and_status_strings():
    assert M.moe_abi_version() == 5
    for s in range(5):
        assert M.moe_status_str(s)
    assert M.moe_status_str(99) == "unknown status"


def good_desc(cfg=None):
    cfg = cfg or gen.CONFIGS["qwen3.6-35b-a3b"]
    d = M.MoeLayerDesc()
    d.hidden, d.ffn, d.n_expert, d.top_k = cfg.H, cfg.F, cfg.E, cfg.k
    d.router = cfg.router
    d.norm_topk = 1
    d.route_scale = 1.0
    d.w_router = FAKE
    d.fmt_gate = d.fmt_up = cfg.fmt_gu
    d.fmt_down = cfg.fmt_d
    d.stride_gate = d.stride_up = cfg.stride_gu
    d.stride_down = cfg.stride_d
    d.gate, d.up, d.down = FAKE, FAKE + 4096, FAKE + 8192
    d.act = cfg.act
    d.act_alpha, d.act_limit = 1.702, 7.0
    return d


def test_workspace_size_valid_and_invalid():
    d = good_desc()
    n1 = M.moe_workspace_size(d, 1)
    n16 = M.moe_workspace_size(d, 16)
    assert n1 > 0 and n16 > n1 and n1 % 256 == 0
    assert M.moe_workspace_size(d, 0) > 0
    assert M.moe_workspace_size(d, -1) == 0
    bad = good_desc()
    bad.top_k = 0
    assert M.moe_workspace_size(bad, 1) == 0


MUTATIONS = [
    ("hidden", 0), ("hidden", 2048 + 32), ("ffn", 100), ("n_expert", 0), ("n_expert", 1025),
    ("top_k", 0), ("top_k", 257), ("top_k", 17), ("router", 2), ("norm_topk", 2), ("act", 5),
    ("fmt_gate", 3), ("fmt_gate", 8), ("fmt_down", -1), ("fmt_down", 8), ("stride_gate", 1024),
    ("stride_gate", 1152 + 8),
    ("stride_down", 280), ("w_router", 0), ("w_router", FAKE + 4), ("gate", 0), ("down", 0),
    ("up", FAKE + 2), ("sh_gate", FAKE),
]


@pytest.mark.parametrize("field,value", MUTATIONS)
def test_desc_validation(field, value):
    d = good_desc()
    setattr(d, field, value)
    assert M.moe_workspace_size(d, 1) == 0
    with pytest.raises(M.MoeError) as ei:
        M.moe_layer_forward(d, FAKE, M.MOE_DTYPE_F32, 1, FAKE, None, None, FAKE, 1 << 40, stream=0)
    assert ei.value.status in (M.MOE_EINVAL, M.MOE_EUNSUPPORTED)


def test_gate_up_format_mismatch_unsupported():
    d = good_desc()
    d.fmt_up = M.MOE_WFMT_Q6_K
    with pytest.raises(M.MoeError) as ei:
        M.moe_layer_forward(d, FAKE, 0, 1, FAKE, None, None, FAKE, 1 << 40, stream=0)
    assert ei.value.status == M.MOE_EUNSUPPORTED


def test_call_validation():
    d = good_desc()
    ws = M.moe_workspace_size(d, 4)
    cases = [
        lambda: M.moe_layer_forward(d, 0, 0, 4, FAKE, None, None, FAKE, ws, stream=0),
        lambda: M.moe_layer_forward(d, FAKE + 8, 0, 4, FAKE, None, None, FAKE, ws, stream=0),
        lambda: M.moe_layer_forward(d, FAKE, 7, 4, FAKE, None, None, FAKE, ws, stream=0),
        lambda: M.moe_layer_forward(d, FAKE, 0, 4, 0, None, None, FAKE, ws, stream=0),
        lambda: M.moe_layer_forward(d, FAKE, 0, 4, FAKE, None, None, 0, ws, stream=0),
        lambda: M.moe_layer_forward(d, FAKE, 0, 4, FAKE, None, None, FAKE + 16, ws, stream=0),
        lambda: M.moe_layer_forward(d, FAKE, 0, -1, FAKE, None, None, FAKE, ws, stream=0),
        lambda: M.moe_layer_forward(d, FAKE, 0, 100000, FAKE, None, None, FAKE, 1 << 40,
                                    stream=0),
        lambda: M.moe_route_topk(d, FAKE, 0, 4, 0, FAKE, None, FAKE, ws, stream=0),
        lambda: M.moe_route_topk(d, FAKE, 0, 4, FAKE, FAKE, None, None, ws, stream=0),
    ]
    for i, c in enumerate(cases):
        with pytest.raises(M.MoeError) as ei:
            c()
        assert ei.value.status == M.MOE_EINVAL, i


def test_short_workspace():
    d = good_desc()
    ws = M.moe_workspace_size(d, 4)
    with pytest.raises(M.MoeError) as ei:
        M.moe_layer_forward(d, FAKE, 0, 4, FAKE, None, None, FAKE, ws - 1, stream=0)
    assert ei.value.status == M.MOE_ENOWORKSPACE
    with pytest.raises(M.MoeError) as ei:
        M.moe_route_topk(d, FAKE, 0, 4, FAKE, FAKE, None, FAKE, ws - 256, stream=0)
    assert ei.value.status == M.MOE_ENOWORKSPACE


def test_zero_tokens_is_a_noop():
    d = good_desc()
    ws = M.moe_workspace_size(d, 0)
    M.moe_layer_forward(d, FAKE, 0, 0, FAKE, None, None, FAKE, ws, stream=0)
    M.moe_route_topk(d, FAKE, 0, 0, FAKE, FAKE, None, FAKE, ws, stream=0)


def test_quantize_and_expert_ffn_validation():
    q = M.qact(FAKE, FAKE, FAKE, M.MOE_AFMT_Q8_K, 4, 2048)
    for args in [(0, 0, 4, 2048, 0), (FAKE, 0, 4, 2000, 0), (FAKE, 0, 4, 2048, 2),
                 (FAKE, 0, 4, 96, M.MOE_AFMT_Q8_K), (FAKE, 3, 4, 2048, 0)]:
        with pytest.raises(M.MoeError):
            M.moe_quantize_act_q8k(*args, q, stream=0)
    qn = M.qact(FAKE, FAKE, None, M.MOE_AFMT_Q8_K, 4, 2048)
    with pytest.raises(M.MoeError):
        M.moe_quantize_act_q8k(FAKE, 0, 4, 2048, M.MOE_AFMT_Q8_K, qn, stream=0)
    d = good_desc()
    ws = M.moe_workspace_size(d, 4)
    wrong_fmt = M.qact(FAKE, FAKE, FAKE, M.MOE_AFMT_Q8_32, 4, 2048)
    short_T = M.qact(FAKE, FAKE, FAKE, M.MOE_AFMT_Q8_K, 3, 2048)
    for xq in (wrong_fmt, short_T):
        with pytest.raises(M.MoeError) as ei:
            M.moe_expert_ffn(d, xq, None, 0, 4, FAKE, FAKE, FAKE, FAKE, ws, stream=0)
        assert ei.value.status == M.MOE_EINVAL


def test_block_dots_validation():
    q = M.qact(FAKE, FAKE, FAKE, M.MOE_AFMT_Q8_K, 1, 512)
    bad = [
        (M.MOE_WFMT_Q4_K, 0, 1, 512, 288, q, 0),
        (M.MOE_WFMT_Q4_K, FAKE, 1, 500, 288, q, 0),
        (M.MOE_WFMT_Q4_K, FAKE, 1, 512, 280, q, 0),
        (M.MOE_WFMT_Q4_K, FAKE, 1, 512, 288, q, 1),
        (M.MOE_WFMT_MXFP4, FAKE, 1, 512, 288, q, 0),
        (8, FAKE, 1, 512, 288, q, 0),
        (-1, FAKE, 1, 512, 288, q, 0),
        (M.MOE_WFMT_Q4_0, FAKE, 1, 512, 288, q, 0),   # Q4_0 rows take q8_32 activations
        (M.MOE_WFMT_Q5_1, FAKE, 1, 512, 288, q, 0),
        (M.MOE_WFMT_Q3_K, FAKE, 1, 512, 208, q, 0),   # row of 2 Q3_K blocks is 220 bytes
    ]
    for a in bad:
        with pytest.raises(M.MoeError):
            M.moe_test_block_dots(*a, FAKE, stream=0)


def test_tile64_layout_rules():
    """TILE64 (64-row tiles, super-block-major inside a tile) is read by the
    grouped Q4_K / Q6_K ring kernels only: such a layer takes the grouped path
    at every T, and other formats, biases, MXFP8 activations or a forced GEMV
    path are refused before anything is enqueued."""
    for name in ("deepseek-v4-flash", "qwen3.6-35b-a3b", "kimi-k2"):
        d = good_desc(gen.CONFIGS[name])
        d.layout = M.MOE_LAYOUT_TILE64
        for T in (1, 2, 16, 256):
            assert M.moe_layer_stage_count(d, T) == 7, (name, T)
        assert M.moe_workspace_size(d, 1) > 0
    bad = []
    for field, value in (("layout", 3), ("layout", -1), ("path", M.MOE_PATH_GEMV),
                         ("fmt_gate", M.MOE_WFMT_Q6_K), ("fmt_down", M.MOE_WFMT_Q5_K),
                         ("b_gate", FAKE), ("b_down", FAKE)):
        d = good_desc(gen.CONFIGS["deepseek-v4-flash"])
        d.layout = M.MOE_LAYOUT_TILE64
        setattr(d, field, value)
        if field == "fmt_gate":  # Q6_K rows: 210 bytes per 256 weights
            d.fmt_up = value
            d.stride_gate = d.stride_up = (d.hidden // 256 * 210 + 15) // 16 * 16
        if field == "b_gate":
            d.b_up = FAKE
        bad.append((field, d))
    mx = good_desc(gen.CONFIGS["gpt-oss-20b"])
    mx.layout = M.MOE_LAYOUT_TILE64
    bad.append(("mxfp4", mx))
    for field, d in bad:
        assert M.moe_workspace_size(d, 1) == 0, field
        with pytest.raises(M.MoeError) as ei:
            M.moe_layer_forward(d, FAKE, 0, 1, FAKE, None, None, FAKE, 1 << 40, stream=0)
        want = M.MOE_EINVAL if field == "layout" else M.MOE_EUNSUPPORTED
        assert ei.value.status == want, field


def test_mx16_layout_rules():
    """MX16 (MXFP4 rows with the nibble fields first, then the scale bytes) is
    read by the per-pair MXFP4 kernels only: such a layer takes the GEMV path at
    every T, with h quantized once per pair by a kernel of its own; other
    formats, MXFP8 activations, a forced grouped path and widths past those
    kernels' plans (256 blocks per row) are refused before anything is
    enqueued."""
    d = good_desc(gen.CONFIGS["gpt-oss-20b"])
    d.layout = M.MOE_LAYOUT_MX16
    for T in (1, 2, 16, 256):
        assert M.moe_layer_stage_count(d, T) == 4, T
        assert [M.moe_layer_stage_name(d, T, i) for i in range(4)] == [
            "router", "gateup", "hquant", "down"]
    assert M.moe_workspace_size(d, 1) > 0
    bad = []
    for field, value in (("path", M.MOE_PATH_GROUPED), ("act_quant", M.MOE_ACTQ_MXFP8)):
        d = good_desc(gen.CONFIGS["gpt-oss-20b"])
        d.layout = M.MOE_LAYOUT_MX16
        setattr(d, field, value)
        bad.append((field, d))
    for name in ("qwen3.6-35b-a3b", "deepseek-v4-flash"):
        d = good_desc(gen.CONFIGS[name])
        d.layout = M.MOE_LAYOUT_MX16
        bad.append((name, d))
    wide = good_desc(gen.CONFIGS["gpt-oss-20b"].with_(H=32 * 257))
    wide.layout = M.MOE_LAYOUT_MX16
    bad.append(("257 blocks", wide))
    for field, d in bad:
        assert M.moe_workspace_size(d, 1) == 0, field
        with pytest.raises(M.MoeError) as ei:
            M.moe_layer_forward(d, FAKE, 0, 1, FAKE, None, None, FAKE, 1 << 40, stream=0)
        assert ei.value.status == M.MOE_EUNSUPPORTED, field
    ok = good_desc(gen.CONFIGS["gpt-oss-20b"].with_(H=32 * 256))
    ok.layout = M.MOE_LAYOUT_MX16
    assert M.moe_workspace_size(ok, 1) > 0


def test_repack_mx16_validation():
    """moe_repack_mx16 and moe_test_block_dots_mx16 arguments are checked on the
    host (nothing enqueued)."""
    big = 1 << 30
    bad = [
        (0, 1536, 4, 2880, FAKE + big, 1536),
        (FAKE, 1536, 4, 2880, 0, 1536),
        (FAKE + 8, 1536, 4, 2880, FAKE + big, 1536),
        (FAKE, 1536, 4, 2880, FAKE + big + 8, 1536),
        (FAKE, 1536, 0, 2880, FAKE + big, 1536),       # no rows
        (FAKE, 1536, 4, 2870, FAKE + big, 1536),       # K not a multiple of 32
        (FAKE, 1529, 4, 2880, FAKE + big, 1536),       # source row shorter than 90 blocks
        (FAKE, 1536, 4, 2880, FAKE + big, 1520),       # destination row below 1440 + 92
        (FAKE, 1536, 4, 2880, FAKE + big, 1544),       # destination stride not 16-aligned
        (FAKE, 1536, 4, 2880, FAKE + 4096, 1536),      # destination overlaps the source
        (FAKE + 4096, 1536, 4, 2880, FAKE, 1536),
    ]
    for i, a in enumerate(bad):
        with pytest.raises(M.MoeError) as ei:
            M.moe_repack_mx16(*a, stream=0)
        assert ei.value.status == M.MOE_EINVAL, i
    q = M.qact(FAKE, FAKE, None, M.MOE_AFMT_Q8_32, 1, 2880)
    for i, (stride, K, tok) in enumerate(((1520, 2880, 0), (1536, 2870, 0), (1536, 2880, 1),
                                         (1544, 2880, 0))):
        with pytest.raises(M.MoeError) as ei:
            M.moe_test_block_dots_mx16(FAKE, 4, K, stride, q, tok, FAKE, stream=0)
        assert ei.value.status == M.MOE_EINVAL, i
    qw = M.qact(FAKE, FAKE, None, M.MOE_AFMT_Q8_32, 1, 32 * 257)
    with pytest.raises(M.MoeError) as ei:
        M.moe_test_block_dots_mx16(FAKE, 4, 32 * 257, 4384, qw, 0, FAKE,
                                   stream=0)
    assert ei.value.status == M.MOE_EUNSUPPORTED


def test_repack_tile64_validation():
    """moe_repack_tile64 arguments are checked on the host (nothing enqueued)."""
    Q4, Q6 = M.MOE_WFMT_Q4_K, M.MOE_WFMT_Q6_K
    big = 1 << 30
    bad = [
        (M.MOE_WFMT_MXFP4, FAKE, 288, 64, 512, FAKE + big),
        (M.MOE_WFMT_Q5_K, FAKE, 352, 64, 512, FAKE + big),
        (Q4, 0, 288, 64, 512, FAKE + big),
        (Q4, FAKE, 288, 64, 512, 0),
        (Q4, FAKE + 8, 288, 64, 512, FAKE + big),
        (Q4, FAKE, 288, 64, 512, FAKE + big + 2),
        (Q4, FAKE, 288, 32, 512, FAKE + big),        # rows not a multiple of 64
        (Q4, FAKE, 288, 0, 512, FAKE + big),
        (Q4, FAKE, 288, 64, 500, FAKE + big),        # K not a multiple of 256
        (Q4, FAKE, 280, 64, 512, FAKE + big),        # stride below the row's 288 bytes
        (Q6, FAKE, 421, 64, 512, FAKE + big),        # odd stride
        (Q4, FAKE, 288, 64, 512, FAKE + 4096),       # destination overlaps the source
        (Q4, FAKE + 4096, 288, 64, 512, FAKE),
    ]
    for i, a in enumerate(bad):
        with pytest.raises(M.MoeError) as ei:
            M.moe_repack_tile64(*a, stream=0)
        assert ei.value.status == M.MOE_EINVAL, i


def test_stage_names_and_path_rule():
    """Dispatch rule (moe_path AUTO): any layer with a matrix in a format other
    than Q4_K and Q6_K takes the per-pair GEMV path (3 kernels, or 4 when an MXFP4 down is
    too large for the kernel that quantizes h itself: h then gets a kernel of
    its own); other layers take the grouped path (7 kernels) when an expert has
    8 MB of blocks or more, or once T (k + shared) times the expert's block
    bytes reaches 160 MB. GEMV / GROUPED force a path where the formats allow it."""
    d = good_desc()  # Qwen3.6 shape without the shared expert: 8 x 1.77 MB per token
    for T in (1, 4, 5, 11):
        assert M.moe_layer_stage_count(d, T) == 3, T
        assert [M.moe_layer_stage_name(d, T, i) for i in range(3)] == ["router", "gateup", "down"]
    for T in (12, 16, 256, 2048):
        assert M.moe_layer_stage_count(d, T) == 7, T
    assert [M.moe_layer_stage_name(d, 16, i) for i in range(7)] == [
        "router", "topk", "bucket", "gateup", "hquant", "down", "combine"]
    assert M.moe_layer_stage_name(d, 1, 9) is None
    assert M.moe_layer_stage_count(d, 0) == 0
    d.sh_gate, d.sh_up, d.sh_down = FAKE, FAKE + 256, FAKE + 512  # + shared: 9 slots
    assert M.moe_layer_stage_count(d, 10) == 3 and M.moe_layer_stage_count(d, 11) == 7
    d.path = M.MOE_PATH_GEMV
    assert M.moe_layer_stage_count(d, 256) == 3
    d.path = M.MOE_PATH_GROUPED
    assert M.moe_layer_stage_count(d, 1) == 7 and M.moe_layer_stage_count(d, 2) == 7
    d.path = 3
    assert M.moe_layer_stage_count(d, 1) == 0 and M.moe_workspace_size(d, 1) == 0
    # 16.3 MB DeepSeek-V4-Flash-shaped experts: grouped at every T (>= 8 MB)
    q6 = good_desc(gen.CONFIGS["deepseek-v4-flash"])
    for T in (1, 2, 16):
        assert M.moe_layer_stage_count(q6, T) == 7
    q6.path = M.MOE_PATH_GEMV
    assert M.moe_layer_stage_count(q6, 1) == 3
    mx = good_desc(gen.CONFIGS["gpt-oss-20b"])
    for T in (1, 16, 256):
        assert M.moe_layer_stage_count(mx, T) == 3
        assert [M.moe_layer_stage_name(mx, T, i) for i in range(3)] == [
            "router", "gateup", "down"]
    mx.path = M.MOE_PATH_GROUPED  # no MXFP4 tile kernels: the GEMV path regardless
    assert M.moe_layer_stage_count(mx, 16) == 3
    # nine slots of 2048-value h: their LDS images exceed the fused kernel's budget
    mx9 = good_desc(gen.CONFIGS["gpt-oss-20b"].with_(E=16, F=2048, k=9))
    assert M.moe_layer_stage_count(mx9, 1) == 4
    assert [M.moe_layer_stage_name(mx9, 1, i) for i in range(4)] == [
        "router", "gateup", "hquant", "down"]
    # Q5_K, Q2_K, Q3_K, Q4_0 and Q5_1 layers (gate/up or down) take the GEMV path at every T
    for fg, fd in ((gen.Q5_K, gen.Q5_K), (gen.Q4_K, gen.Q5_K), (gen.Q5_K, gen.Q6_K),
                   (gen.Q2_K, gen.Q2_K), (gen.Q4_K, gen.Q2_K), (gen.Q3_K, gen.Q3_K),
                   (gen.Q4_K, gen.Q3_K), (gen.Q4_0, gen.Q4_0), (gen.Q5_1, gen.Q6_K),
                   (gen.Q4_K, gen.Q5_1)):
        q5 = good_desc(gen.CONFIGS["deepseek-v4-flash"].with_(fmt_gu=fg, fmt_d=fd))
        assert M.moe_layer_stage_count(q5, 16) == 3
    # the grouped workspace holds the per-pair rows: it grows with T * k * H
    d = good_desc()
    assert M.moe_workspace_size(d, 12) > M.moe_workspace_size(d, 11) + 12 * 8 * 2048 * 4


def test_tile_dots_validation():
    q = M.qact(FAKE, FAKE, FAKE, M.MOE_AFMT_Q8_K, 16, 2048)
    assert M.moe_test_tile_dots_ws(0, 128, 2048, 16) >= 1024 + 4 * 16 * 128
    assert M.moe_test_tile_dots_ws(3, 128, 2048, 16) == 0
    assert M.moe_test_tile_dots_ws(0, 128, 2048, 17) == 0
    ws = M.moe_test_tile_dots_ws(1, 256, 2048, 16)
    bad = [
        (3, FAKE, 128, 2048, 1152, q, 16),        # unknown mode
        (0, FAKE, 100, 2048, 1152, q, 16),        # gate/up rows not a multiple of 64
        (1, FAKE, 192, 2048, 1152, q, 16),        # down rows not a multiple of 128
        (0, FAKE, 128, 2048, 1152, q, 17),        # more than 16 tokens
        (0, FAKE, 128, 2048, 1152, q, 0),
        (0, FAKE, 128, 2000, 1152, q, 16),        # width not a multiple of 256
        (0, FAKE, 128, 2048, 1140, q, 16),        # stride below the row bytes
        (2, FAKE, 128, 2048, 1672, q, 16),        # Q6_K stride not a multiple of 16
        (0, FAKE + 8, 128, 2048, 1152, q, 16),    # misaligned rows
        (0, FAKE, 128, 1024, 576, q, 16),         # activations of another width
    ]
    for a in bad:
        with pytest.raises(M.MoeError) as ei:
            M.moe_test_tile_dots(*a, FAKE, FAKE, ws, stream=0)
        assert ei.value.status == M.MOE_EINVAL, a
    with pytest.raises(M.MoeError) as ei:
        M.moe_test_tile_dots(1, FAKE, 256, 2048, 1152, q, 16, FAKE, FAKE, ws - 1, stream=0)
    assert ei.value.status == M.MOE_ENOWORKSPACE


def test_preact_validation():
    d = good_desc()
    ws = M.moe_workspace_size(d, 4)
    q = M.qact(FAKE, FAKE, FAKE, M.MOE_AFMT_Q8_K, 4, 2048)
    for which, xq, ids in ((2, q, FAKE), (0, M.qact(FAKE, FAKE, FAKE, M.MOE_AFMT_Q8_32, 4, 2048),
                                          FAKE), (0, q, 0)):
        with pytest.raises(M.MoeError) as ei:
            M.moe_test_preact(d, xq, 4, ids, which, FAKE, FAKE, ws, stream=0)
        assert ei.value.status == M.MOE_EINVAL
    with pytest.raises(M.MoeError) as ei:
        M.moe_test_preact(d, q, 4, FAKE, 0, FAKE, FAKE, ws - 1, stream=0)
    assert ei.value.status == M.MOE_ENOWORKSPACE


def test_gemv_plan_rejects_rows_past_the_task_cap():
    """The per-pair GEMV kernels take at most 8 block tasks per 8-lane group: a
    Q4_K gate/up row of 129 super-blocks (H = 33024) would need more, so the
    layer call refuses it on the host (nothing is launched) instead of leaving
    blocks uncomputed."""
    cfg = gen.CONFIGS["tiny"].with_(H=33024, F=256, E=8, k=2)
    d = good_desc(cfg)
    d.path = M.MOE_PATH_GEMV  # (the automatic rule sends 14 MB experts to the tiles)
    ws = M.moe_workspace_size(d, 1)
    assert ws > 0
    with pytest.raises(M.MoeError) as ei:
        M.moe_layer_forward(d, FAKE, 0, 1, FAKE, None, None, FAKE, ws, stream=0)
    assert ei.value.status == M.MOE_EUNSUPPORTED
    # and the down projection of a 129-super-block F row as well
    cfg = gen.CONFIGS["tiny"].with_(H=512, F=33024, E=8, k=2, fmt_d=gen.Q6_K)
    d = good_desc(cfg)
    d.path = M.MOE_PATH_GEMV
    ws = M.moe_workspace_size(d, 1)
    with pytest.raises(M.MoeError) as ei:
        M.moe_layer_forward(d, FAKE, 0, 1, FAKE, None, None, FAKE, ws, stream=0)
    assert ei.value.status == M.MOE_EUNSUPPORTED


def test_noalloc_refuses_chunks_past_the_scratch():
    """moe_layer_forward_noalloc works out of a 32 MiB static device array: the
    Kimi-K2-shaped 256-token chunk needs ~95 MB of workspace, so the call is
    refused on the host before anything is enqueued (no device is touched)."""
    cfg = gen.CONFIGS["kimi-k2"]
    d = good_desc(cfg)
    d.sh_gate, d.sh_up, d.sh_down = FAKE, FAKE + 256, FAKE + 512
    assert M.moe_workspace_size(d, 256) > M.MOE_NOALLOC_SCRATCH_BYTES
    assert M.moe_workspace_size(d, 64) <= M.MOE_NOALLOC_SCRATCH_BYTES
    with pytest.raises(M.MoeError) as ei:
        M.moe_layer_forward_noalloc(d, FAKE, 0, 256, FAKE, None, None, stream=0)
    assert ei.value.status == M.MOE_ENOWORKSPACE
    with pytest.raises(M.MoeError) as ei:  # argument checks come first
        M.moe_layer_forward_noalloc(d, FAKE + 8, 0, 256, FAKE, None, None, stream=0)
    assert ei.value.status == M.MOE_EINVAL
    M.moe_layer_forward_noalloc(d, FAKE, 0, 0, FAKE, None, None, stream=0)  # T = 0: no-op


def test_probe_validation():
    """The measurement probes reject bad arguments before any launch."""
    for n in (0, -1, 4097):
        with pytest.raises(M.MoeError) as ei:
            M.moe_probe_empty_chain(n, stream=0)
        assert ei.value.status == M.MOE_EINVAL
    with pytest.raises(M.MoeError):
        M.moe_probe_read_wall(FAKE + 8, 1 << 20, 64, FAKE, stream=0)
    with pytest.raises(M.MoeError):
        M.moe_probe_read_wall(FAKE, (1 << 20) + 4, 64, FAKE, stream=0)
    with pytest.raises(M.MoeError):
        M.moe_probe_mfma_i8(2, 10, 64, FAKE, stream=0)
    with pytest.raises(M.MoeError):
        M.moe_probe_mfma_i8(0, 10, 0, FAKE, stream=0)
