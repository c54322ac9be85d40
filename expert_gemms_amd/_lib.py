"""ctypes binding of ``libmoe_gfx950.so`` (the C ABI in ``include/moe.h``).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Tensors are torch tensors on the current HIP device; PyTorch
provides the device memory and the stream.  A missing library raises; there
is no fallback path.
"""

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_gfx950.so")

FMT = {"bf16": 0, "mxfp8": 1, "mxfp4": 2, "nvfp4": 3}
OK, E_INVALID, E_UNSUPPORTED, E_WORKSPACE, E_HIP = 0, -1, -2, -3, -4

EXPORTS = (
    "moe_status_string", "moe_get_block_m", "moe_workspace_bytes", "moe_transform_weights",
    "moe_quantize_weights", "moe_quantize_x", "moe_dispatch", "moe_forward", "moe_forward_profiled",
    "moe_route",
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
        lib.moe_route.argtypes = [_I, _I, _I, _P, _P, _I, _I, _I, _I, ctypes.c_float, _P, _P, _P, _P]
        lib.moe_route.restype = _I
        _LIB = lib
    return _LIB


def lib_handle():
    """The loaded ctypes library (loads it on first use)."""
    return _lib()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


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
    _check(_lib().moe_transform_weights(_fmt(fmt), num_experts, hidden, inter, _ptr(w13), _ptr(w13_sf),
                                        _ptr(w2), _ptr(w2_sf), _ptr(w13_k), _ptr(w13_sf_k), _ptr(w2_k),
                                        _ptr(w2_sf_k), _stream(stream)), "moe_transform_weights")


def moe_quantize_weights(fmt, num_experts, rows, cols, src, codes, scales, gscale=None, stream=None):
    _check(_lib().moe_quantize_weights(_fmt(fmt), num_experts, rows, cols, _ptr(src), _ptr(codes),
                                       _ptr(scales), _ptr(gscale), _stream(stream)), "moe_quantize_weights")


def moe_quantize_x(fmt, num_tokens, hidden, x, codes, scales, token_scale=None, stream=None):
    _check(_lib().moe_quantize_x(_fmt(fmt), num_tokens, hidden, _ptr(x), _ptr(codes), _ptr(scales),
                                 _ptr(token_scale), _stream(stream)), "moe_quantize_x")


def moe_dispatch(num_tokens, top_k, num_shared, expert_start, num_local_experts, block_m, topk_ids,
                 counts, offsets, sorted_slot, slot_row, tile_expert, block_counts=None, stream=None):
    """``block_counts``: optional int32 scratch of ``dispatch_scratch_ints``
    values (many-workgroup dispatch from 16384 slots on)."""
    _check(_lib().moe_dispatch(num_tokens, top_k, num_shared, expert_start, num_local_experts, block_m,
                               _ptr(topk_ids), _ptr(counts), _ptr(offsets), _ptr(sorted_slot),
                               _ptr(slot_row), _ptr(tile_expert), _ptr(block_counts), _stream(stream)),
           "moe_dispatch")


def dispatch_scratch_ints(num_tokens, top_k, num_shared, num_local_experts):
    """Size (int32 values) of moe_dispatch's optional block_counts scratch."""
    S = num_tokens * (top_k + num_shared)
    return (S + 2047) // 2048 * (num_local_experts + num_shared)


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
    nbytes = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
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


def moe_route(num_tokens, num_experts, top_k, logits, topk_ids, topk_weights, *, bias=None, scoring="softmax",
              num_groups=1, topk_groups=1, renormalize=True, routed_scaling_factor=1.0, is_padding=None,
              stream=None):
    """Router top-k (``moe_route``): float32 logits [T, E] -> int32 ids and
    float32 weights [T, top_k], written into the given tensors."""
    _check(_lib().moe_route(num_tokens, num_experts, top_k, _ptr(logits), _ptr(bias), SCORING[scoring],
                            num_groups, topk_groups, int(bool(renormalize)), float(routed_scaling_factor),
                            _ptr(is_padding), _ptr(topk_ids), _ptr(topk_weights), _stream(stream)), "moe_route")
    return topk_ids, topk_weights
