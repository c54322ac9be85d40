"""Block quantisers of the layer (oracle side).

Sources on the pages:

* "DeepGEMM MegaMoE experts" page, module docstring: MX weights and
  activations carry one UE8M0 scale per 1x32 block; NVFP4 weights carry one
  E4M3 scale per 1x16 block plus a per-expert FP32 global scale; NVFP4
  dispatch scales each token by its own FP32 scale.  ``MegaMoEWeightSpec``:
  FP4 packs two values per byte along K.
* "Qwen4-Exp MegaMoE" page, ``_requantize``: MX scales are power-of-two FP32
  values whose exponent byte is the UE8M0 code.

Readings where the pages stop short (each one is listed in the design doc):

* MX scale choice: the smallest power of two 2^e with ``amax <= fmax * 2^e``
  (no element clips); the code is ``127 + e`` clamped to [1, 254]; an all-zero
  block gets code 0 and zero elements.
* NVFP4: block scale ``bs = E4M3(amax16 / (6 * g))``, elements
  ``E2M1(v * (1 / (bs * g)))``, with every product, quotient and reciprocal
  taken in float32; a block whose scale rounds to zero is all zero.
* Per-token NVFP4 dispatch scale ``g_t = amax_t / (6 * 448)`` (1 if the row is
  zero); a per-expert NVFP4 weight scale is ``amax(|W_e|) / (6 * 448)``.

Every function takes and returns NumPy arrays; the quantised axis is the last
one.
"""

import numpy as np

from . import codecs

MX_GROUP = 32
NV_GROUP = 16
_FMAX = {"e4m3": codecs.E4M3_MAX, "e2m1": codecs.E2M1_MAX}


# --------------------------------------------------------------------------
# MX (UE8M0 scale per 32 along K)
# --------------------------------------------------------------------------

def mx_scale_codes(amax, elem):
    """UE8M0 code per block from the block's float32 amax.

    The smallest e with amax <= fmax * 2**e, written exactly: with
    amax = m * 2**p (1 <= m < 2) and fmax = 1.75 * 2**8 (E4M3) or 1.5 * 2**2
    (E2M1), e = p - 8 + [m > 1.75] or p - 2 + [m > 1.5].
    """
    amax = np.asarray(amax, dtype=np.float64)
    nz = amax > 0
    f, x = np.frexp(np.where(nz, amax, 1.0))
    m, p = 2.0 * f, x.astype(np.int64) - 1
    if elem == "e4m3":
        e = p - 8 + (m > 1.75)
    elif elem == "e2m1":
        e = p - 2 + (m > 1.5)
    else:
        raise ValueError(elem)
    c = np.clip(127 + e, 1, 254)
    return np.where(nz, c, 0).astype(np.uint8)


def mx_quantize(v, elem, codes=None):
    """float32 [..., K] -> (codes uint8 [..., K] (4-bit codes for E2M1,
    unpacked), UE8M0 scales uint8 [..., K/32]).  ``codes``: UE8M0 scales to
    quantise the elements with instead of choosing them (a given decision)."""
    v = np.asarray(v, dtype=np.float32)
    K = v.shape[-1]
    if K % MX_GROUP:
        raise ValueError("K must be a multiple of 32")
    blk = v.reshape(v.shape[:-1] + (K // MX_GROUP, MX_GROUP)).astype(np.float64)
    amax = np.abs(blk).max(axis=-1)
    c = mx_scale_codes(amax, elem) if codes is None else np.broadcast_to(
        np.asarray(codes, dtype=np.uint8), amax.shape)
    # v * 2**(127 - c): exact (a power-of-two scaling) in float64.
    scaled = blk * np.ldexp(1.0, 127 - c.astype(np.int64))[..., None]
    enc = codecs.e4m3_encode if elem == "e4m3" else codecs.e2m1_encode
    q = enc(scaled)
    q = np.where((c == 0)[..., None], np.uint8(0), q).astype(np.uint8)
    return q.reshape(v.shape), c


def mx_dequantize(q, c, elem):
    """(codes [..., K], scales [..., K/32]) -> float64 values."""
    dec = codecs.e4m3_decode if elem == "e4m3" else codecs.e2m1_decode
    vals = dec(q)
    K = vals.shape[-1]
    s = codecs.ue8m0_decode(c)
    blk = vals.reshape(vals.shape[:-1] + (K // MX_GROUP, MX_GROUP)) * s[..., None]
    return blk.reshape(vals.shape)


# --------------------------------------------------------------------------
# NVFP4 (E4M3 scale per 16 along K, FP32 global scale)
# --------------------------------------------------------------------------

def nvfp4_global_scale(amax):
    """FP32 global scale amax / (6 * 448), or 1 where amax is zero."""
    amax = np.asarray(amax, dtype=np.float32)
    g = amax / np.float32(6.0 * 448.0)
    return np.where(amax > 0, g, np.float32(1.0)).astype(np.float32)


def nvfp4_quantize(v, g, bs=None):
    """float32 [..., K] with global scale ``g`` (float32, broadcast over the
    leading axes, shape [...]) -> (E2M1 codes uint8 [..., K] unpacked,
    E4M3 block-scale codes uint8 [..., K/16]).  ``bs``: E4M3 block scales to
    quantise the elements with instead of choosing them (a given decision)."""
    v = np.asarray(v, dtype=np.float32)
    K = v.shape[-1]
    if K % NV_GROUP:
        raise ValueError("K must be a multiple of 16")
    g = np.asarray(g, dtype=np.float32)
    blk = v.reshape(v.shape[:-1] + (K // NV_GROUP, NV_GROUP))
    amax = np.abs(blk).max(axis=-1)                          # float32, exact
    gb = np.broadcast_to(g[..., None], amax.shape).astype(np.float32)
    six_g = (np.float32(6.0) * gb).astype(np.float32)
    t = (amax / six_g).astype(np.float32)
    bs = codecs.e4m3_encode(t) if bs is None else np.broadcast_to(np.asarray(bs, dtype=np.uint8), amax.shape)
    bsv = codecs.e4m3_decode(bs).astype(np.float32)          # exact in float32
    denom = (bsv * gb).astype(np.float32)
    safe = np.where(denom > 0, denom, np.float32(1.0))
    r = (np.float32(1.0) / safe).astype(np.float32)
    prod = (blk * r[..., None]).astype(np.float32)
    q = codecs.e2m1_encode(prod)
    q = np.where((bsv == 0)[..., None], np.uint8(0), q).astype(np.uint8)
    return q.reshape(v.shape), bs


def nvfp4_dequantize(q, bs, g):
    """-> float64 values e2m1(q) * e4m3(bs) * g."""
    vals = codecs.e2m1_decode(q)
    K = vals.shape[-1]
    s = codecs.e4m3_decode(bs)
    g = np.asarray(g, dtype=np.float64)
    blk = vals.reshape(vals.shape[:-1] + (K // NV_GROUP, NV_GROUP)) * s[..., None]
    return blk.reshape(vals.shape) * g[..., None]
