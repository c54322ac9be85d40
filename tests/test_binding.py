"""The Python binding checks every tensor argument before the library is
called (dtype, shape or byte size, contiguity, device), and the host-only
queries (workspace layout, dispatch scratch size) agree with the workspace
size.  All of this runs without a GPU: every rejection happens before the
library or a device is touched."""

import pytest
import torch

import expert_gemms_amd as moe
from expert_gemms_amd import _lib

T, H, I, K, EL = 4, 256, 256, 2, 4


def good_forward_args(fmt="bf16"):
    """Well-formed CPU tensors for a tiny layer (CPU, so the device check is
    the first to fail when nothing else does)."""
    f = _lib._fmt(fmt)
    b13, s13 = _lib._weight_bytes(f, EL, 2 * I, H)
    b2, s2 = _lib._weight_bytes(f, EL, H, I)
    wdt = torch.bfloat16 if f == 0 else torch.uint8
    div = 2 if f == 0 else 1
    a = dict(
        x=torch.zeros((T, H), dtype=torch.bfloat16),
        topk_ids=torch.zeros((T, K), dtype=torch.int32),
        topk_weights=torch.zeros((T, K), dtype=torch.float32),
        w13_k=torch.zeros(b13 // div, dtype=wdt), w2_k=torch.zeros(b2 // div, dtype=wdt),
        w13_sf_k=torch.zeros(s13, dtype=torch.uint8) if s13 else None,
        w2_sf_k=torch.zeros(s2, dtype=torch.uint8) if s2 else None,
        w13_gscale=torch.ones(EL, dtype=torch.float32) if f == 3 else None,
        w2_gscale=torch.ones(EL, dtype=torch.float32) if f == 3 else None,
        out=torch.zeros((T, H), dtype=torch.bfloat16),
        workspace=torch.zeros(1 << 20, dtype=torch.uint8),
    )
    return a


def call_forward(fmt="bf16", **over):
    a = good_forward_args(fmt)
    a.update(over)
    return _lib.moe_forward(fmt, T, H, I, K, 0, EL, 0, 0, None, a["x"], a["topk_ids"], a["topk_weights"],
                            a["w13_k"], a["w13_sf_k"], a["w2_k"], a["w2_sf_k"], a["w13_gscale"], a["w2_gscale"],
                            1.0, a["out"], a["workspace"])


def test_well_formed_cpu_tensors_fail_only_on_the_device_check():
    for fmt in ("bf16", "mxfp8", "mxfp4", "nvfp4"):
        with pytest.raises(ValueError, match="must be on a GPU"):
            call_forward(fmt)


@pytest.mark.parametrize("name,bad,exc,msg", [
    ("x", torch.zeros((T, H), dtype=torch.float32), TypeError, "dtype"),
    ("x", torch.zeros((T, H + 128), dtype=torch.bfloat16), ValueError, "shape"),
    ("x", torch.zeros((H, T), dtype=torch.bfloat16).t(), ValueError, "contiguous"),
    ("x", None, ValueError, "required"),
    ("x", [[0.0] * H] * T, TypeError, "torch tensor"),
    ("topk_ids", torch.zeros((T, K), dtype=torch.int64), TypeError, "dtype"),
    ("topk_ids", torch.zeros((T, K + 1), dtype=torch.int32), ValueError, "shape"),
    ("topk_weights", torch.zeros((T, K), dtype=torch.bfloat16), TypeError, "dtype"),
    ("topk_weights", torch.zeros((K, T), dtype=torch.float32).t(), ValueError, "contiguous"),
    ("out", torch.zeros((T, H), dtype=torch.float16), TypeError, "dtype"),
    ("out", torch.zeros((T - 1, H), dtype=torch.bfloat16), ValueError, "shape"),
    ("w13_k", torch.zeros(10, dtype=torch.bfloat16), ValueError, "bytes"),
    ("w2_k", torch.zeros(EL * H * I, dtype=torch.float32), TypeError, "dtype"),
])
def test_forward_rejects_bad_tensors(name, bad, exc, msg):
    with pytest.raises(exc, match=msg):
        call_forward("bf16", **{name: bad})


def test_forward_rejects_bad_block_scaled_arguments():
    with pytest.raises(ValueError, match="w13_sf_k is required"):
        call_forward("mxfp8", w13_sf_k=None)
    with pytest.raises(ValueError, match="bytes"):
        call_forward("mxfp4", w2_sf_k=torch.zeros(7, dtype=torch.uint8))
    with pytest.raises(ValueError, match="w2_gscale is required"):
        call_forward("nvfp4", w2_gscale=None)
    with pytest.raises(ValueError, match="shape"):
        call_forward("nvfp4", w13_gscale=torch.ones(EL + 1, dtype=torch.float32))
    with pytest.raises(TypeError, match="dtype"):
        call_forward("nvfp4", w13_gscale=torch.ones(EL, dtype=torch.float64))


def test_forward_rejects_a_short_workspace():
    with pytest.raises(ValueError, match="at least"):
        _lib.moe_forward("bf16", T, H, I, K, 0, EL, 0, 0, None, *[good_forward_args()[n] for n in (
            "x", "topk_ids", "topk_weights", "w13_k", "w13_sf_k", "w2_k", "w2_sf_k", "w13_gscale", "w2_gscale")],
            1.0, good_forward_args()["out"], torch.zeros(64, dtype=torch.uint8), workspace_bytes=1 << 20)


def test_layer_holder_rejects_too_many_tokens():
    layer = moe.FusedMoE.__new__(moe.FusedMoE)
    layer.max_tokens, layer.hidden = 2, H
    layer.norm_gamma, layer.norm_eps = None, 0.0
    with pytest.raises(ValueError, match="sized for 2"):
        moe.FusedMoE.forward(layer, torch.zeros((3, H), dtype=torch.bfloat16), None, None)


def test_other_wrappers_check_their_tensors():
    z8 = torch.zeros(64, dtype=torch.uint8)
    with pytest.raises(TypeError, match="dtype"):
        moe.moe_quantize_x("mxfp8", T, H, torch.zeros((T, H)), z8, z8)
    with pytest.raises(ValueError, match="bytes"):
        moe.moe_quantize_x("mxfp8", T, H, torch.zeros((T, H), dtype=torch.bfloat16), z8, z8)
    with pytest.raises(ValueError, match="token_scale is required"):
        moe.moe_quantize_x("nvfp4", T, H, torch.zeros((T, H), dtype=torch.bfloat16),
                           torch.zeros(T * H // 2, dtype=torch.uint8), torch.zeros(T * H // 16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="not quantised"):
        moe.moe_quantize_x("bf16", T, H, torch.zeros((T, H), dtype=torch.bfloat16), z8, z8)
    with pytest.raises(TypeError, match="dtype"):
        moe.moe_quantize_weights("mxfp8", 1, 32, 64, torch.zeros((32, 64), dtype=torch.float64), z8, z8)
    with pytest.raises(ValueError, match="shape"):
        i32 = lambda n: torch.zeros(n, dtype=torch.int32)
        moe.moe_dispatch(T, K, 0, 0, EL, 32, torch.zeros((T, K + 1), dtype=torch.int32), i32(8), i32(8),
                         i32(1024), i32(64), i32(64))
    with pytest.raises(ValueError, match="at least"):
        moe.moe_dispatch(T, K, 0, 0, EL, 32, torch.zeros((T, K), dtype=torch.int32), i32(8), i32(8),
                         i32(4), i32(64), i32(64))
    with pytest.raises(ValueError, match="scoring"):
        moe.moe_route(T, 8, 2, torch.zeros((T, 8)), None, None, scoring="relu")
    with pytest.raises(ValueError, match="shape"):
        moe.moe_route(T, 8, 2, torch.zeros((T, 9)), torch.zeros((T, 2), dtype=torch.int32),
                      torch.zeros((T, 2)))
    with pytest.raises(ValueError, match="bytes"):
        moe.moe_transform_weights("bf16", EL, H, I, torch.zeros(3, dtype=torch.bfloat16), None,
                                  torch.zeros(3, dtype=torch.bfloat16), None, None, None, None, None)


def test_dispatch_scratch_size_comes_from_the_library():
    assert _lib.dispatch_scratch_ints(8192, 8, 1, 256) == (8192 * 9 + 2047) // 2048 * 257
    assert _lib.dispatch_scratch_ints(0, 8, 0, 4) == 0
    with pytest.raises(moe.MoEError):
        _lib.dispatch_scratch_ints(4, 0, 0, 4)


@pytest.mark.parametrize("fmt,T_,H_,I_,E_,sh,k,bm", [
    ("bf16", 4096, 4096, 14336, 8, 0, 2, 0),
    ("mxfp8", 8192, 7168, 2048, 256, 1, 8, 0),
    ("mxfp4", 1, 4096, 1536, 128, 0, 8, 0),
    ("mxfp4", 256, 4096, 1536, 128, 0, 8, 64),
    ("nvfp4", 16384, 2048, 768, 64, 0, 6, 0),
])
def test_workspace_layout_fits_the_workspace(fmt, T_, H_, I_, E_, sh, k, bm):
    nbytes = moe.moe_workspace_bytes(fmt, T_, H_, I_, E_, sh, k, bm)
    lay = _lib.moe_workspace_layout(fmt, T_, H_, I_, k, E_, sh, bm, nbytes)
    assert lay["bytes"] <= nbytes
    assert lay["block_m"] == (bm or moe.moe_get_block_m(T_, E_, sh, k, fmt))
    E, S = E_ + sh, T_ * (k + sh)
    M = S + E * (lay["block_m"] - 1)
    sizes = {"counts": 4 * E, "offsets": 4 * (E + 1), "sorted_slot": 4 * M, "slot_row": 4 * S,
             "tile_expert": 4 * (M // lay["block_m"]), "o": S * H_ * (2 if lay["l2_rows_bf16"] else 4)}
    for name, n in sizes.items():
        assert 0 <= lay[name] and lay[name] + n <= lay["bytes"], name
    if fmt == "bf16":
        assert lay["xq"] == lay["xq_sf"] == lay["a2_sf"] == lay["x_tok"] == -1
        assert lay["a2_ld"] == 2 * I_
    else:
        assert lay["xq"] >= 0 and lay["a2_sf"] >= 0 and lay["sf_plane"] >= M + 256
        assert (lay["x_tok"] >= 0) == (fmt == "nvfp4")
        assert lay["a2_ld"] == (I_ // 2 if fmt == "nvfp4" else I_)
    assert lay["l2_rows_bf16"] == int(fmt != "bf16" and lay["l2_ksplit"] == 1)


def test_workspace_layout_drops_k_splits_that_do_not_fit():
    args = ("mxfp4", 1, 4096, 1536, 8, 128, 0, 0)
    full = _lib.moe_workspace_layout(*args, 1 << 40)
    assert full["l1_ksplit"] > 1
    tight = _lib.moe_workspace_layout(*args, full["bytes"] - 1)
    assert tight["l1_ksplit"] == 1 and tight["bytes"] < full["bytes"]
    with pytest.raises(moe.MoEError):
        _lib.moe_workspace_layout(*args, 4096)
    with pytest.raises(moe.MoEError):
        _lib.moe_workspace_layout("mxfp4", 1, 4000, 1536, 8, 128, 0, 0, 1 << 40)
