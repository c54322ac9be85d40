"""Element codecs of the layer's number formats (oracle side, NumPy).

Formats, as the "DeepGEMM MegaMoE experts" page names them in its module
docstring and ``MegaMoEWeightSpec`` (BF16 activations, FP8 E4M3 and FP4 E2M1
values, UE8M0 and E4M3 block scales), with the element encodings of the OCP
8-bit floating point and OCP Microscaling (MX) v1.0 specifications:

* BF16: IEEE binary32 with the low 16 bits dropped; held here as ``uint16``
  bit patterns because NumPy has no bfloat16.
* E4M3 (OCP "E4M3FN"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; largest
  finite 448; subnormals are multiples of 2^-9; S.1111.111 is NaN; no inf.
* E2M1 (OCP MX FP4): 1 sign, 2 exponent (bias 1), 1 mantissa bit; magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* UE8M0: an unsigned biased exponent; the "Qwen4-Exp MegaMoE" page
  (``_requantize``) decodes it by shifting the byte into the float32 exponent
  field and encodes a power-of-two float32 scale by shifting its exponent
  field back down.

Rounding everywhere is round-to-nearest, ties to the even code, saturating at
the largest finite magnitude.  The sign of a code is the sign bit of the value
it encodes, so a negative value that rounds to zero encodes as negative zero.
"""

import numpy as np


# --------------------------------------------------------------------------
# generic: round a non-negative float64 magnitude onto a binary float grid
# --------------------------------------------------------------------------

def _floor_log2(a):
    """floor(log2(a)) for a > 0 (exact, via frexp: a = f * 2**x, f in [0.5, 1))."""
    _, x = np.frexp(a)
    return x.astype(np.int64) - 1


def round_to_grid(a, mbits, emin, maxval):
    """Round magnitudes ``a`` (float64, >= 0) to the nearest value of a binary
    format with ``mbits`` mantissa bits and minimum normal exponent ``emin``
    (subnormal step 2**(emin - mbits)), ties to even, saturating at ``maxval``.

    Exact in float64: the quotient by a power of two and ``rint`` (which rounds
    half to even) introduce no error for the magnitudes used here.
    """
    a = np.asarray(a, dtype=np.float64)
    out = np.zeros_like(a)
    nz = a > 0
    e = np.maximum(_floor_log2(np.where(nz, a, 1.0)), emin)
    step = np.ldexp(1.0, e - mbits)
    r = np.rint(a / step) * step
    out = np.where(nz, np.minimum(r, maxval), 0.0)
    return out


# --------------------------------------------------------------------------
# BF16
# --------------------------------------------------------------------------

def bf16_decode(bits):
    """uint16 bit patterns -> float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_encode_f32(v):
    """float32 -> bf16 bits, round to nearest even (finite inputs)."""
    v = np.asarray(v, dtype=np.float32)
    u = v.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_round_f64(v):
    """float64 -> nearest bf16 value (as float64), one rounding, ties to even."""
    v = np.asarray(v, dtype=np.float64)
    mag = round_to_grid(np.abs(v), 7, -126, np.inf)
    return np.copysign(mag, v)


# --------------------------------------------------------------------------
# E4M3 (FP8, OCP E4M3FN)
# --------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_decode(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    M = c & 0x7
    mag = np.where(E == 0, M * 2.0 ** -9, (1.0 + M / 8.0) * np.ldexp(1.0, E - 7))
    mag = np.where((E == 0xF) & (M == 0x7), np.nan, mag)
    return s * mag


def e4m3_encode(v):
    """float (any precision, finite) -> E4M3 code, RNE, saturating to 448."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.int64) << 7
    r = round_to_grid(np.abs(v), 3, -6, E4M3_MAX)
    sub = r < 2.0 ** -6
    code_sub = np.rint(r / 2.0 ** -9).astype(np.int64)
    e = _floor_log2(np.where(sub, 1.0, r))
    m = np.rint((np.where(sub, 1.0, r) / np.ldexp(1.0, e) - 1.0) * 8).astype(np.int64)
    code_norm = ((e + 7) << 3) | m
    return (sign | np.where(sub, code_sub, code_norm)).astype(np.uint8)


# --------------------------------------------------------------------------
# E2M1 (FP4, OCP MX)
# --------------------------------------------------------------------------

E2M1_MAX = 6.0
_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x8, -1.0, 1.0)
    return s * _E2M1_MAG[c & 0x7]


def e2m1_encode(v):
    """float -> 4-bit E2M1 code (in a uint8), RNE, saturating to 6."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.int64) << 3
    r = round_to_grid(np.abs(v), 1, 0, E2M1_MAX)
    # r is one of the eight magnitudes; its index is the magnitude code.
    mag_code = np.searchsorted(_E2M1_MAG, r)
    return (sign | mag_code).astype(np.uint8)


def fp4_pack(codes):
    """[..., K] 4-bit codes -> [..., K/2] bytes; element 2i in the low nibble,
    element 2i+1 in the high nibble ("two values per storage element along K").
    """
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def fp4_unpack(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# --------------------------------------------------------------------------
# UE8M0 (MX block scale)
# --------------------------------------------------------------------------

def ue8m0_decode(codes):
    """Byte -> float32 by placing it in the float32 exponent field (the
    ``_requantize`` decode rule); code 0 therefore decodes to +0.0."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.uint32) << 23
    return c.view(np.float32).astype(np.float64)


def ue8m0_encode_pow2(scale_f32):
    """Power-of-two float32 scale -> its exponent byte (the ``_requantize``
    encode rule: float32 bits shifted right by 23)."""
    s = np.asarray(scale_f32, dtype=np.float32)
    return ((s.view(np.uint32) >> 23) & 0xFF).astype(np.uint8)
