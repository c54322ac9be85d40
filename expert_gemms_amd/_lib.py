"""ctypes binding of ``libmoe_gfx950.so`` (the C ABI in ``include/moe.h``).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Tensors are torch tensors on the current HIP device; PyTorch
provides the device memory and the stream.  A missing library raises; there
is no fallback path.
"""

import ctypes
import os
import threading

import torch

# MOE_LIBRARY names another build of the same library (the tests' host-
# sanitizer build); unset, the in-tree library is loaded
LIB_PATH = os.environ.get("MOE_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                         "libmoe_gfx950.so")

FMT = {"bf16": 0, "mxfp8": 1, "mxfp4": 2, "nvfp4": 3}
OK, E_INVALID, E_UNSUPPORTED, E_WORKSPACE, E_HIP, E_TOO_LARGE = 0, -1, -2, -3, -4, -5
NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTS = (
    "moe_status_string", "moe_get_block_m", "moe_workspace_bytes", "moe_transform_weights",
    "moe_quantize_weights", "moe_quantize_x", "moe_dispatch", "moe_forward", "moe_forward_profiled",
    "moe_route", "moe_dispatch_scratch_ints", "moe_workspace_layout", "moe_forward_noalloc",
)
SCORING = {"softmax": 0, "sigmoid": 1}
STEPS = ("quant_x", "dispatch", "l1", "l2", "combine")


class MoEError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status} ({_lib().moe_status_string(status).decode()})")


class Options(ctypes.Structure):
    """``moe_options_t``: post-expert RMSNorm (gamma pointer, eps) and the
    routing weight applied on the input."""
    _fields_ = [("post_expert_norm_gamma", ctypes.c_void_p), ("post_expert_norm_eps", ctypes.c_float),
                ("apply_router_weight_on_input", ctypes.c_int)]


class Activation(ctypes.Structure):
    """``moe_activation_t``: swiglu with optional clamp, alpha, beta."""
    _fields_ = [("kind", ctypes.c_int), ("has_clamp", ctypes.c_int), ("clamp", ctypes.c_float),
                ("alpha", ctypes.c_float), ("beta", ctypes.c_float)]


class WorkspaceLayout(ctypes.Structure):
    """``moe_workspace_layout_t``: byte offsets of moe_forward's intermediate
    buffers inside its workspace (-1: not used by the format)."""
    _fields_ = [("block_m", ctypes.c_int), ("l1_ksplit", ctypes.c_int), ("l2_ksplit", ctypes.c_int),
                ("l2_rows_bf16", ctypes.c_int)] + \
               [(n, ctypes.c_int64) for n in ("sf_plane", "a2_ld", "counts", "offsets", "sorted_slot", "slot_row",
                                              "tile_expert", "xq", "xq_sf", "x_tok", "a1_sf", "a2", "a2_sf", "o",
                                              "bytes")]


_LIB = None
_P = ctypes.c_void_p
_I = ctypes.c_int


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m expert_gemms_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.moe_status_string.argtypes = [_I]
        lib.moe_status_string.restype = ctypes.c_char_p
        lib.moe_get_block_m.argtypes = [_I, _I, _I, _I, _I]
        lib.moe_get_block_m.restype = _I
        lib.moe_workspace_bytes.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I]
        lib.moe_workspace_bytes.restype = ctypes.c_size_t
        lib.moe_transform_weights.argtypes = [_I, _I, _I, _I] + [_P] * 9
        lib.moe_transform_weights.restype = _I
        lib.moe_quantize_weights.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P]
        lib.moe_quantize_weights.restype = _I
        lib.moe_quantize_x.argtypes = [_I, _I, _I, _P, _P, _P, _P, _P]
        lib.moe_quantize_x.restype = _I
        lib.moe_dispatch.argtypes = [_I] * 6 + [_P] * 8
        lib.moe_dispatch.restype = _I
        lib.moe_forward.argtypes = ([_I] * 9 + [ctypes.POINTER(Activation), ctypes.POINTER(Options)] + [_P] * 9
                                    + [ctypes.c_float, _P, _P, ctypes.c_size_t, _P])
        lib.moe_forward.restype = _I
        lib.moe_forward_profiled.argtypes = lib.moe_forward.argtypes + [_P]
        lib.moe_forward_profiled.restype = _I
        lib.moe_forward_noalloc.argtypes = ([_I] * 9 + [ctypes.POINTER(Activation), ctypes.POINTER(Options)]
                                            + [_P] * 9 + [ctypes.c_float, _P, _P])
        lib.moe_forward_noalloc.restype = _I
        lib.moe_route.argtypes = [_I, _I, _I, _P, _P, _I, _I, _I, _I, ctypes.c_float, _P, _P, _P, _P]
        lib.moe_route.restype = _I
        lib.moe_dispatch_scratch_ints.argtypes = [_I, _I, _I, _I]
        lib.moe_dispatch_scratch_ints.restype = ctypes.c_int64
        lib.moe_workspace_layout.argtypes = [_I] * 8 + [ctypes.c_size_t, ctypes.POINTER(WorkspaceLayout)]
        lib.moe_workspace_layout.restype = _I
        _LIB = lib
    return _LIB


def lib_handle():
    """The loaded ctypes library (loads it on first use)."""
    return _lib()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _nbytes(t):
    return t.numel() * t.element_size()


def _tensor(t, name, *, dtype=None, shape=None, nbytes=None, min_bytes=None, optional=False):
    """Checks one tensor argument before it is handed to the library: a
    torch tensor, of the given dtype (one or a tuple), shape or byte size,
    contiguous, on the current GPU.  Raises TypeError / ValueError; returns
    the tensor (None for an allowed missing optional argument)."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if dtype is not None:
        ok = dtype if isinstance(dtype, tuple) else (dtype,)
        if t.dtype not in ok:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {' or '.join(str(d) for d in ok)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if nbytes is not None and _nbytes(t) != nbytes:
        raise ValueError(f"{name} holds {_nbytes(t)} bytes, expected {nbytes}")
    if min_bytes is not None and _nbytes(t) < min_bytes:
        raise ValueError(f"{name} holds {_nbytes(t)} bytes, at least {min_bytes} needed")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    _PENDING.append((name, t))
    return t


class _Pending(threading.local):
    """Tensors whose form has been checked and whose device is checked next
    (all forms first, then all devices, so each wrong form is reported as
    such); one list per host thread."""
    def __init__(self):
        self.items = []

    def append(self, item):
        self.items.append(item)

    def clear(self):
        self.items = []


_PENDING = _Pending()


def _on_gpu():
    """The device check of every tensor checked since the last call."""
    pending = _PENDING.items
    _PENDING.clear()
    for name, t in pending:
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU, not {t.device}")
        if t.device.index != torch.cuda.current_device():
            raise ValueError(f"{name} is on {t.device}, but the current device is "
                             f"cuda:{torch.cuda.current_device()}")


def _weight_bytes(fmt, n_experts, rows, cols):
    """(element bytes, block-scale bytes) of canonical / kernel-layout weights."""
    f = _fmt(fmt)
    if f == 0:
        return n_experts * rows * cols * 2, 0
    vpe = 2 if f in (2, 3) else 1
    grp = 16 if f == 3 else 32
    return n_experts * rows * cols // vpe, n_experts * rows * cols // grp


U8 = torch.uint8
# BF16 weights may be held as bfloat16 or as their 16-bit patterns
BF16_BITS = (torch.bfloat16, torch.int16, torch.uint16, torch.uint8)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status, what):
    if status != OK:
        raise MoEError(status, what)


def _fmt(fmt):
    return FMT[fmt] if isinstance(fmt, str) else int(fmt)


# ---------------------------------------------------------------- API

def moe_get_block_m(num_tokens, num_local_experts, num_shared, top_k, fmt):
    r = _lib().moe_get_block_m(num_tokens, num_local_experts, num_shared, top_k, _fmt(fmt))
    if r < 0:
        raise MoEError(r, "moe_get_block_m")
    return r


def moe_workspace_bytes(fmt, max_tokens, hidden, inter, num_local_experts, num_shared, top_k, block_m=0):
    return int(_lib().moe_workspace_bytes(_fmt(fmt), max_tokens, hidden, inter, num_local_experts,
                                          num_shared, top_k, block_m))


def moe_transform_weights(fmt, num_experts, hidden, inter, w13, w13_sf, w2, w2_sf,
                          w13_k, w13_sf_k, w2_k, w2_sf_k, stream=None):
    _PENDING.clear()
    b13, s13 = _weight_bytes(fmt, num_experts, 2 * inter, hidden)
    b2, s2 = _weight_bytes(fmt, num_experts, hidden, inter)
    wdt = BF16_BITS if _fmt(fmt) == 0 else U8
    scaled = _fmt(fmt) != 0
    for t, n, b in ((w13, "w13", b13), (w13_k, "w13_k", b13), (w2, "w2", b2), (w2_k, "w2_k", b2)):
        _tensor(t, n, dtype=wdt, nbytes=b)
    for t, n, b in ((w13_sf, "w13_sf", s13), (w13_sf_k, "w13_sf_k", s13), (w2_sf, "w2_sf", s2),
                    (w2_sf_k, "w2_sf_k", s2)):
        _tensor(t, n, dtype=U8, nbytes=b, optional=not scaled)
    _on_gpu()
    _check(_lib().moe_transform_weights(_fmt(fmt), num_experts, hidden, inter, _ptr(w13), _ptr(w13_sf),
                                        _ptr(w2), _ptr(w2_sf), _ptr(w13_k), _ptr(w13_sf_k), _ptr(w2_k),
                                        _ptr(w2_sf_k), _stream(stream)), "moe_transform_weights")


def moe_quantize_weights(fmt, num_experts, rows, cols, src, codes, scales, gscale=None, stream=None):
    _PENDING.clear()
    if _fmt(fmt) == 0:
        raise ValueError("BF16 weights are not quantised")
    b, sb = _weight_bytes(fmt, num_experts, rows, cols)
    _tensor(src, "src", dtype=torch.float32, nbytes=num_experts * rows * cols * 4)
    _tensor(codes, "codes", dtype=U8, nbytes=b)
    _tensor(scales, "scales", dtype=U8, nbytes=sb)
    _tensor(gscale, "gscale", dtype=torch.float32, shape=(num_experts,), optional=_fmt(fmt) != 3)
    _on_gpu()
    _check(_lib().moe_quantize_weights(_fmt(fmt), num_experts, rows, cols, _ptr(src), _ptr(codes),
                                       _ptr(scales), _ptr(gscale), _stream(stream)), "moe_quantize_weights")


def moe_quantize_x(fmt, num_tokens, hidden, x, codes, scales, token_scale=None, stream=None):
    _PENDING.clear()
    if _fmt(fmt) == 0:
        raise ValueError("BF16 activations are not quantised")
    nv = _fmt(fmt) == 3
    _tensor(x, "x", dtype=torch.bfloat16, shape=(num_tokens, hidden))
    _tensor(codes, "codes", dtype=U8, nbytes=num_tokens * hidden // (2 if nv else 1))
    _tensor(scales, "scales", dtype=U8, nbytes=num_tokens * hidden // (16 if nv else 32))
    _tensor(token_scale, "token_scale", dtype=torch.float32, shape=(num_tokens,), optional=not nv)
    _on_gpu()
    _check(_lib().moe_quantize_x(_fmt(fmt), num_tokens, hidden, _ptr(x), _ptr(codes), _ptr(scales),
                                 _ptr(token_scale), _stream(stream)), "moe_quantize_x")


def moe_dispatch(num_tokens, top_k, num_shared, expert_start, num_local_experts, block_m, topk_ids,
                 counts, offsets, sorted_slot, slot_row, tile_expert, block_counts=None, stream=None):
    """``block_counts``: optional int32 scratch of ``dispatch_scratch_ints``
    values (many-workgroup dispatch from 16384 slots on)."""
    _PENDING.clear()
    E = num_local_experts + num_shared
    S = num_tokens * (top_k + num_shared)
    M = S + E * (block_m - 1)
    i32 = torch.int32
    _tensor(topk_ids, "topk_ids", dtype=i32, shape=(num_tokens, top_k))
    _tensor(counts, "counts", dtype=i32, min_bytes=4 * E)
    _tensor(offsets, "offsets", dtype=i32, min_bytes=4 * (E + 1))
    _tensor(sorted_slot, "sorted_slot", dtype=i32, min_bytes=4 * M)
    _tensor(slot_row, "slot_row", dtype=i32, min_bytes=4 * S)
    _tensor(tile_expert, "tile_expert", dtype=i32, min_bytes=4 * (M // block_m))
    _tensor(block_counts, "block_counts", dtype=i32,
            min_bytes=4 * dispatch_scratch_ints(num_tokens, top_k, num_shared, num_local_experts), optional=True)
    _on_gpu()
    _check(_lib().moe_dispatch(num_tokens, top_k, num_shared, expert_start, num_local_experts, block_m,
                               _ptr(topk_ids), _ptr(counts), _ptr(offsets), _ptr(sorted_slot),
                               _ptr(slot_row), _ptr(tile_expert), _ptr(block_counts), _stream(stream)),
           "moe_dispatch")


def dispatch_scratch_ints(num_tokens, top_k, num_shared, num_local_experts):
    """Size (int32 values) of moe_dispatch's optional block_counts scratch
    (``moe_dispatch_scratch_ints``)."""
    n = _lib().moe_dispatch_scratch_ints(num_tokens, top_k, num_shared, num_local_experts)
    if n < 0:
        raise MoEError(E_INVALID, "moe_dispatch_scratch_ints")
    return int(n)


def moe_workspace_layout(fmt, num_tokens, hidden, inter, top_k, num_local_experts, num_shared, block_m,
                         workspace_bytes):
    """Offsets of moe_forward's intermediate buffers in its workspace, as a
    dict (``moe_workspace_layout``)."""
    lay = WorkspaceLayout()
    _check(_lib().moe_workspace_layout(_fmt(fmt), num_tokens, hidden, inter, top_k, num_local_experts, num_shared,
                                       block_m, workspace_bytes, ctypes.byref(lay)), "moe_workspace_layout")
    return {n: getattr(lay, n) for n, _ in WorkspaceLayout._fields_}


def _check_forward_args(fmt, num_tokens, hidden, inter, top_k, num_local_experts, num_shared, x, topk_ids,
                        topk_weights, w13_k, w13_sf_k, w2_k, w2_sf_k, w13_gscale, w2_gscale, out, workspace,
                        workspace_bytes, norm_gamma, workspace_required=True):
    _PENDING.clear()
    f = _fmt(fmt)
    T, E = num_tokens, num_local_experts + num_shared
    _tensor(x, "x", dtype=torch.bfloat16, shape=(T, hidden))
    _tensor(topk_ids, "topk_ids", dtype=torch.int32, shape=(T, top_k))
    _tensor(topk_weights, "topk_weights", dtype=torch.float32, shape=(T, top_k))
    b13, s13 = _weight_bytes(f, E, 2 * inter, hidden)
    b2, s2 = _weight_bytes(f, E, hidden, inter)
    wdt = BF16_BITS if f == 0 else U8
    _tensor(w13_k, "w13_k", dtype=wdt, nbytes=b13)
    _tensor(w2_k, "w2_k", dtype=wdt, nbytes=b2)
    _tensor(w13_sf_k, "w13_sf_k", dtype=U8, nbytes=s13, optional=f == 0)
    _tensor(w2_sf_k, "w2_sf_k", dtype=U8, nbytes=s2, optional=f == 0)
    _tensor(w13_gscale, "w13_gscale", dtype=torch.float32, shape=(E,), optional=f != 3)
    _tensor(w2_gscale, "w2_gscale", dtype=torch.float32, shape=(E,), optional=f != 3)
    _tensor(out, "out", dtype=torch.bfloat16, shape=(T, hidden))
    _tensor(norm_gamma, "norm_gamma", dtype=torch.float32, shape=(hidden,), optional=True)
    if workspace_required:
        _tensor(workspace, "workspace", min_bytes=workspace_bytes)
    _on_gpu()


def moe_forward(fmt, num_tokens, hidden, inter, top_k, expert_start, num_local_experts, num_shared,
                block_m, act, x, topk_ids, topk_weights, w13_k, w13_sf_k, w2_k, w2_sf_k,
                w13_gscale, w2_gscale, l2_activation_scale, out, workspace, workspace_bytes=None,
                stream=None, step_events=None, norm_gamma=None, norm_eps=0.0, weight_on_input=False):
    """``step_events``: None, or 2 * len(STEPS) recorded torch.cuda.Event
    objects (begin/end per step) -> calls moe_forward_profiled.
    ``norm_gamma``/``norm_eps``: post-expert RMSNorm; ``weight_on_input``:
    the routing weight scales the input (moe_options_t)."""
    a = None
    if act is not None:
        a = ctypes.byref(act if isinstance(act, Activation) else Activation(
            0, int(act.get("clamp") is not None), float(act.get("clamp") or 0.0),
            float(act.get("alpha", 1.0)), float(act.get("beta", 0.0))))
    opts = None
    if norm_gamma is not None or weight_on_input:
        opts = ctypes.byref(Options(None if norm_gamma is None else norm_gamma.data_ptr(), float(norm_eps),
                                    int(bool(weight_on_input))))
    if workspace_bytes is None:
        if not isinstance(workspace, torch.Tensor):
            raise TypeError(f"workspace must be a torch tensor, got {type(workspace).__name__}")
        nbytes = _nbytes(workspace)
    else:
        nbytes = workspace_bytes
    _check_forward_args(fmt, num_tokens, hidden, inter, top_k, num_local_experts, num_shared, x, topk_ids,
                        topk_weights, w13_k, w13_sf_k, w2_k, w2_sf_k, w13_gscale, w2_gscale, out, workspace, nbytes,
                        norm_gamma)
    args = (_fmt(fmt), num_tokens, hidden, inter, top_k, expert_start, num_local_experts,
            num_shared, block_m, a, opts, _ptr(x), _ptr(topk_ids), _ptr(topk_weights),
            _ptr(w13_k), _ptr(w13_sf_k), _ptr(w2_k), _ptr(w2_sf_k), _ptr(w13_gscale),
            _ptr(w2_gscale), float(l2_activation_scale), _ptr(out), _ptr(workspace),
            nbytes, _stream(stream))
    if step_events is None:
        _check(_lib().moe_forward(*args), "moe_forward")
    else:
        arr = (ctypes.c_void_p * len(step_events))(*[ctypes.c_void_p(e.cuda_event) for e in step_events])
        _check(_lib().moe_forward_profiled(*args, arr), "moe_forward_profiled")
    return out


def moe_forward_noalloc(fmt, num_tokens, hidden, inter, top_k, expert_start, num_local_experts, num_shared,
                        block_m, act, x, topk_ids, topk_weights, w13_k, w13_sf_k, w2_k, w2_sf_k,
                        w13_gscale, w2_gscale, l2_activation_scale, out, stream=None):
    """moe_forward without a workspace: the library's fixed per-GPU scratch
    holds the intermediate buffers (MoEError E_TOO_LARGE if they do not fit).
    Calls that may overlap on one GPU race for that scratch."""
    a = None
    if act is not None:
        a = ctypes.byref(act if isinstance(act, Activation) else Activation(
            0, int(act.get("clamp") is not None), float(act.get("clamp") or 0.0),
            float(act.get("alpha", 1.0)), float(act.get("beta", 0.0))))
    _PENDING.clear()
    _check_forward_args(fmt, num_tokens, hidden, inter, top_k, num_local_experts, num_shared, x, topk_ids,
                        topk_weights, w13_k, w13_sf_k, w2_k, w2_sf_k, w13_gscale, w2_gscale, out, None, None, None,
                        workspace_required=False)
    _check(_lib().moe_forward_noalloc(_fmt(fmt), num_tokens, hidden, inter, top_k, expert_start, num_local_experts,
                                      num_shared, block_m, a, None, _ptr(x), _ptr(topk_ids), _ptr(topk_weights),
                                      _ptr(w13_k), _ptr(w13_sf_k), _ptr(w2_k), _ptr(w2_sf_k), _ptr(w13_gscale),
                                      _ptr(w2_gscale), float(l2_activation_scale), _ptr(out), _stream(stream)),
           "moe_forward_noalloc")
    return out


def moe_route(num_tokens, num_experts, top_k, logits, topk_ids, topk_weights, *, bias=None, scoring="softmax",
              num_groups=1, topk_groups=1, renormalize=True, routed_scaling_factor=1.0, is_padding=None,
              stream=None):
    """Router top-k (``moe_route``): float32 logits [T, E] -> int32 ids and
    float32 weights [T, top_k], written into the given tensors."""
    _PENDING.clear()
    if scoring not in SCORING:
        raise ValueError(f"scoring must be one of {sorted(SCORING)}")
    _tensor(logits, "logits", dtype=torch.float32, shape=(num_tokens, num_experts))
    _tensor(topk_ids, "topk_ids", dtype=torch.int32, shape=(num_tokens, top_k))
    _tensor(topk_weights, "topk_weights", dtype=torch.float32, shape=(num_tokens, top_k))
    _tensor(bias, "bias", dtype=torch.float32, shape=(num_experts,), optional=True)
    _tensor(is_padding, "is_padding", dtype=(torch.uint8, torch.bool), shape=(num_tokens,), optional=True)
    _on_gpu()
    _check(_lib().moe_route(num_tokens, num_experts, top_k, _ptr(logits), _ptr(bias), SCORING[scoring],
                            num_groups, topk_groups, int(bool(renormalize)), float(routed_scaling_factor),
                            _ptr(is_padding), _ptr(topk_ids), _ptr(topk_weights), _stream(stream)), "moe_route")
    return topk_ids, topk_weights
