"""The C-ABI library loads and exports every symbol include/moe.h declares;
host-only entry points and argument validation work without a GPU (every
validation failure returns before anything touches a device)."""

import ctypes
import os
import re

import pytest

import expert_gemms_amd as moe
from expert_gemms_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    assert os.path.exists(_lib.LIB_PATH), "build the library first (python -m expert_gemms_amd.build)"
    lib = ctypes.CDLL(_lib.LIB_PATH)
    names = header_functions()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = moe.lib_handle()
    for s in (0, -1, -2, -3, -4, 7):
        assert isinstance(lib.moe_status_string(s), bytes)
    assert lib.moe_status_string(-3) == b"workspace too small"


def test_block_m_rule():
    assert moe.moe_get_block_m(4096, 8, 0, 2, "bf16") == 256      # 1024 rows per expert
    assert moe.moe_get_block_m(1, 128, 0, 8, "mxfp4") == 32
    assert moe.moe_get_block_m(256, 128, 0, 8, "mxfp4") == 32      # 16 rows per expert
    assert moe.moe_get_block_m(1000, 64, 0, 6, "nvfp4") == 64      # 93.75; NVFP4 prefers 64-row tiles
    assert moe.moe_get_block_m(0, 8, 0, 2, "bf16") == 32
    # 256 expected rows per routed expert: half the groups spill past 256
    assert moe.moe_get_block_m(8192, 256, 1, 8, "mxfp8") == 128
    assert moe.moe_get_block_m(16384, 64, 0, 6, "nvfp4") == 64
    assert moe.moe_get_block_m(16384, 64, 0, 6, "mxfp4") == 128     # block-scaled formats stop at 128
    assert moe.moe_get_block_m(16384, 64, 0, 6, "mxfp8") == 128
    assert moe.moe_get_block_m(16384, 64, 0, 6, "bf16") == 256
    with pytest.raises(moe.MoEError):
        moe.moe_get_block_m(-1, 8, 0, 2, "bf16")
    with pytest.raises(moe.MoEError):
        moe.moe_get_block_m(8, 0, 0, 2, "bf16")


def test_workspace_bytes():
    b256 = moe.moe_workspace_bytes("bf16", 4096, 4096, 14336, 8, 0, 2, 256)
    b32 = moe.moe_workspace_bytes("bf16", 4096, 4096, 14336, 8, 0, 2, 32)
    assert b256 == moe.moe_workspace_bytes("bf16", 4096, 4096, 14336, 8, 0, 2, 0)
    assert b256 > b32 > 8192 * 4096 * 4          # at least the float32 L2 rows
    assert moe.moe_workspace_bytes("bf16", 4096, 4000, 14336, 8, 0, 2, 0) == 0   # H % 128
    assert moe.moe_workspace_bytes("bf16", 4096, 4096, 14336, 8, 0, 2, 48) == 0  # bad block_m
    assert moe.moe_workspace_bytes("mxfp8", 10, 7168, 2048, 256, 1, 8, 0) > 0


class _Fake:
    """Stands in for a tensor: an aligned, never-dereferenced address."""
    def __init__(self, addr=0x10000, n=1 << 20):
        self.addr, self.n = addr, n

    def data_ptr(self):
        return self.addr

    def numel(self):
        return self.n

    def element_size(self):
        return 1


def _fwd(**kw):
    lib = moe.lib_handle()
    a = dict(fmt=0, T=4, H=256, I=256, k=2, start=0, nloc=4, nsh=0, bm=0, act=None, opts=None,
             x=_Fake(), ids=_Fake(), wts=_Fake(), w13=_Fake(), w13sf=None, w2=_Fake(), w2sf=None,
             g13=None, g2=None, l2=1.0, out=_Fake(), ws=_Fake(), wsb=1 << 40)
    a.update(kw)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    act = ctypes.byref(a["act"]) if a["act"] is not None else None
    opts = ctypes.byref(a["opts"]) if a["opts"] is not None else None
    return lib.moe_forward(a["fmt"], a["T"], a["H"], a["I"], a["k"], a["start"], a["nloc"], a["nsh"], a["bm"],
                           act, opts, p(a["x"]), p(a["ids"]), p(a["wts"]), p(a["w13"]), p(a["w13sf"]), p(a["w2"]),
                           p(a["w2sf"]), p(a["g13"]), p(a["g2"]), a["l2"], p(a["out"]), p(a["ws"]),
                           a["wsb"], None)


@pytest.mark.parametrize("kw", [
    dict(H=200), dict(I=100), dict(k=0), dict(nloc=0), dict(nsh=-1), dict(bm=48), dict(fmt=9),
    dict(T=-1), dict(x=None), dict(out=None), dict(ws=None), dict(x=_Fake(0x10004)),
    dict(fmt=1),                                 # MX without scale pointers
    dict(fmt=3, w13sf=_Fake(), w2sf=_Fake()),    # NVFP4 without global scales
    dict(fmt=3, w13sf=_Fake(), w2sf=_Fake(), g13=_Fake(), g2=_Fake(), l2=0.0),
    dict(act=_lib.Activation(0, 0, 0.0, float("inf"), 0.0)),
    dict(act=_lib.Activation(0, 1, -1.0, 1.0, 0.0)),
    dict(nloc=999, nsh=2),                       # more than 1000 local experts
    dict(opts=_lib.Options(0x10000, -1.0, 0)),   # negative norm eps
    dict(opts=_lib.Options(0x10004, 1e-6, 0)),   # unaligned gamma
    dict(opts=_lib.Options(0x10000, 1e-6, 0), H=16640),   # norm row does not fit LDS
    dict(opts=_lib.Options(None, 0.0, 1)),       # weight on input with top_k = 2
    dict(opts=_lib.Options(None, 0.0, 1), k=1, nsh=1),     # ... or with a shared expert
    dict(H=16384, I=65536),                      # one expert's w13 reaches 4 GiB (32-bit copy offsets)
    dict(fmt=1, w13sf=_Fake(), w2sf=_Fake(), T=1 << 19, H=8192),   # x's MX codes reach 4 GiB
])
def test_forward_rejects_invalid_arguments(kw):
    assert _fwd(**kw) == _lib.E_INVALID


def test_forward_other_statuses_without_gpu():
    assert _fwd(T=0) == _lib.OK                                  # nothing to do, nothing enqueued
    assert _fwd(act=_lib.Activation(1, 0, 0.0, 1.0, 0.0)) == _lib.E_UNSUPPORTED
    assert _fwd(wsb=16) == _lib.E_WORKSPACE
    # all arguments valid: the device check fails cleanly on a GPU-less host
    import torch
    if not torch.cuda.is_available():
        assert _fwd() == _lib.E_UNSUPPORTED


def test_other_entry_points_validate():
    lib = moe.lib_handle()
    P = ctypes.c_void_p
    f = P(0x10000)
    assert lib.moe_dispatch(4, 2, 0, 0, 4, 48, f, f, f, f, f, f, None, None) == _lib.E_INVALID
    assert lib.moe_dispatch(4, 0, 0, 0, 4, 32, f, f, f, f, f, f, None, None) == _lib.E_INVALID
    assert lib.moe_quantize_x(0, 4, 256, f, f, f, None, None) == _lib.E_INVALID       # BF16 has no quantiser
    assert lib.moe_quantize_x(1, 4, 100, f, f, f, None, None) == _lib.E_INVALID
    assert lib.moe_quantize_x(3, 4, 256, f, f, f, None, None) == _lib.E_INVALID       # NVFP4 needs token scales
    assert lib.moe_quantize_weights(1, 2, 64, 48, f, f, f, None, None) == _lib.E_INVALID
    assert lib.moe_transform_weights(0, 2, 200, 256, f, None, f, None, f, None, f, None, None) == _lib.E_INVALID
    assert lib.moe_transform_weights(1, 2, 256, 256, f, None, f, None, f, None, f, None, None) == _lib.E_INVALID


def test_route_validates():
    lib = moe.lib_handle()
    P = ctypes.c_void_p
    f = P(0x10000)
    bad = [
        (4, 0, 1, 0, 1, 1),       # no experts
        (4, 8, 9, 0, 1, 1),       # top_k > E
        (4, 2000, 8, 0, 1, 1),    # E > 1024
        (4, 64, 8, 2, 1, 1),      # unknown scoring
        (4, 64, 8, 1, 5, 1),      # groups do not divide E
        (4, 64, 8, 1, 8, 9),      # topk_groups > num_groups
        (4, 64, 8, 1, 16, 1),     # one kept group of 4 experts < top_k
    ]
    for T, E, k, sc, G, TG in bad:
        assert lib.moe_route(T, E, k, f, None, sc, G, TG, 1, 1.0, None, f, f, None) == _lib.E_INVALID
    assert lib.moe_route(4, 64, 8, f, None, 0, 1, 1, 1, float("inf"), None, f, f, None) == _lib.E_INVALID
    assert lib.moe_route(4, 64, 8, None, None, 0, 1, 1, 1, 1.0, None, f, f, None) == _lib.E_INVALID
    assert lib.moe_route(0, 64, 8, None, None, 0, 1, 1, 1, 1.0, None, None, None, None) == _lib.OK


def test_l1_split_only_for_few_tiles():
    """The float32 L1 parts of a K-split L1 GEMM are sized into the workspace
    only when the split rule picks it: never for a prefill-sized launch (the
    Mixtral-shaped layer's workspace stays well under the 3.7 GB that four
    parts of 8192 x 28672 floats would add), always for a single decode
    token (the parts of 8 slots add 8 * 3072 * 4 bytes per part)."""
    big = moe.moe_workspace_bytes("bf16", 4096, 4096, 14336, 8, 0, 2, 0)
    assert 0 < big < 1_000_000_000
    one = moe.moe_workspace_bytes("mxfp4", 1, 4096, 1536, 128, 0, 8, 0)
    two = moe.moe_workspace_bytes("mxfp4", 2, 4096, 1536, 128, 0, 8, 0)
    assert one > 0 and two > one


def _noalloc(**kw):
    lib = moe.lib_handle()
    a = dict(fmt=0, T=4, H=256, I=256, k=2, nloc=4, nsh=0, bm=0, x=_Fake(), ids=_Fake(), wts=_Fake(),
             w13=_Fake(), w2=_Fake(), out=_Fake())
    a.update(kw)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    return lib.moe_forward_noalloc(a["fmt"], a["T"], a["H"], a["I"], a["k"], 0, a["nloc"], a["nsh"], a["bm"],
                                   None, None, p(a["x"]), p(a["ids"]), p(a["wts"]), p(a["w13"]), None, p(a["w2"]),
                                   None, None, None, 1.0, p(a["out"]), None)


def test_noalloc_checks_before_touching_a_device():
    """Invalid arguments, and layers whose intermediate buffers exceed the
    fixed 64 MiB scratch, are rejected on the host."""
    assert _lib.NOALLOC_SCRATCH_BYTES == 64 << 20
    assert _noalloc(H=200) == _lib.E_INVALID
    assert _noalloc(x=None) == _lib.E_INVALID
    assert _noalloc(out=_Fake(0x10008)) == _lib.E_INVALID
    assert _noalloc(T=0) == _lib.OK
    # 20000 tokens of a hidden-4096 top-2 BF16 layer: far beyond 64 MiB
    assert _noalloc(T=20000, H=4096, I=1024) == _lib.E_TOO_LARGE
    assert b"no-allocation" in moe.lib_handle().moe_status_string(_lib.E_TOO_LARGE)
    # the decode-sized MXFP4 layer at 256 tokens fits (default BLOCK_M)
    need = moe.moe_workspace_bytes("mxfp4", 256, 4096, 1536, 128, 0, 8,
                                   moe.moe_get_block_m(256, 128, 0, 8, "mxfp4"))
    assert need <= _lib.NOALLOC_SCRATCH_BYTES
