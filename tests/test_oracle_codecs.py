"""Pins of the oracle's element codecs against things other than the oracle:
torch's own float8/bfloat16 conversions, brute-force nearest-value search, and
the bit rules and value tables the golden fixtures cite."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import codecs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- E4M3

def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2                      # S.1111.111 only
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    assert np.nanmax(ours) == 448.0 and codecs.E4M3_MAX == 448.0


def _e4m3_neighbours():
    """All finite non-negative E4M3 values, sorted, as (value, code)."""
    codes = np.arange(127, dtype=np.uint8)            # 0x00..0x7E
    return codecs.e4m3_decode(codes), codes


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(20000) * 50,
        rng.uniform(-2.0 ** -5, 2.0 ** -5, 5000),     # subnormal range
        rng.uniform(-463.0, 463.0, 5000),   # torch turns |v| > 464 into NaN
    ]).astype(np.float32)
    # exact midpoints between neighbouring codes, both signs
    vals, _ = _e4m3_neighbours()
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids, vals.astype(np.float32)])
    ours = codecs.e4m3_encode(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_is_nearest_ties_even_bruteforce():
    vals, codes = _e4m3_neighbours()
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.uniform(0, 448, 3000), (vals[1:] + vals[:-1]) / 2])
    got = codecs.e4m3_encode(v)
    for x, c in zip(v, got):
        d = np.abs(vals - x)
        best = np.nonzero(d == d.min())[0]
        if best.size == 2:                      # tie: the even code wins
            want = codes[best[0]] if codes[best[0]] % 2 == 0 else codes[best[1]]
        else:
            want = codes[best[0]]
        assert c == want, (x, c, want)


def test_e4m3_saturates_and_keeps_sign():
    assert codecs.e4m3_encode(np.array([448.0, 460.0, 464.0, 480.0, 1e6]))[:].tolist() == [0x7E] * 5
    assert codecs.e4m3_encode(np.array([-1e6]))[0] == 0xFE
    # a negative value that rounds to zero is negative zero (torch agrees)
    assert codecs.e4m3_encode(np.array([-1e-9]))[0] == 0x80
    assert torch.tensor([-1e-9]).to(torch.float8_e4m3fn).view(torch.uint8).item() == 0x80


# ---------------------------------------------------------------- E2M1

def test_e2m1_decode_table():
    g = _gold("e2m1_values.json")["code_to_value"]
    ours = codecs.e2m1_decode(np.arange(16, dtype=np.uint8))
    for c, v in g.items():
        assert ours[int(c)] == v and np.signbit(ours[int(c)]) == np.signbit(v)


def test_e2m1_tie_table_and_bruteforce():
    g = _gold("e2m1_values.json")["rne_ties"]["cases"]
    for x, want in g:
        for s in (1.0, -1.0):
            c = codecs.e2m1_encode(np.array([s * x]))[0]
            assert codecs.e2m1_decode(np.array([c]))[0] == s * want
    mags = codecs.e2m1_decode(np.arange(8, dtype=np.uint8))
    rng = np.random.default_rng(3)
    for x in rng.uniform(0, 8, 4000):
        c = codecs.e2m1_encode(np.array([x]))[0]
        d = np.abs(mags - min(x, 6.0))
        best = np.nonzero(d == d.min())[0]
        want = best[0] if best.size == 1 else [b for b in best if b % 2 == 0][0]
        assert c == want


def test_fp4_pack_nibble_order():
    c = np.array([[1, 2, 3, 4, 15, 0]], dtype=np.uint8)
    p = codecs.fp4_pack(c)
    assert p.tolist() == [[0x21, 0x43, 0x0F]]
    assert np.array_equal(codecs.fp4_unpack(p), c)


# ---------------------------------------------------------------- BF16

def test_bf16_encode_matches_torch():
    rng = np.random.default_rng(4)
    v = (rng.standard_normal(50000) * np.exp(rng.uniform(-30, 30, 50000))).astype(np.float32)
    # exact ties: bf16 value plus half an ulp
    base = (v.view(np.uint32) & 0xFFFF0000).view(np.float32)
    ties = (base.view(np.uint32) | 0x8000).view(np.float32)
    v = np.concatenate([v, ties])
    ours = codecs.bf16_encode_f32(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(codecs.bf16_decode(ours),
                          torch.from_numpy(v).to(torch.bfloat16).double().numpy())


def test_bf16_round_f64_single_rounding():
    rng = np.random.default_rng(5)
    v32 = (rng.standard_normal(20000) * 100).astype(np.float32)
    # float32-exact inputs: one rounding equals torch's float32 -> bf16
    ref = torch.from_numpy(v32).to(torch.bfloat16).double().numpy()
    assert np.array_equal(codecs.bf16_round_f64(v32.astype(np.float64)), ref)
    # a float64 just above a bf16 midpoint must round up even though its
    # float32 rounding would land on the midpoint (double rounding)
    one_ulp = 2.0 ** -7
    x = 1.0 + one_ulp / 2 + 2.0 ** -40
    assert codecs.bf16_round_f64(np.array([x]))[0] == 1.0 + one_ulp


# ---------------------------------------------------------------- UE8M0

def test_ue8m0_bit_rules_from_pages():
    g = _gold("ue8m0_bit_rules.json")
    for c, v in g["decode"]:
        assert codecs.ue8m0_decode(np.array([c], dtype=np.uint8))[0] == v
    for v, c in g["encode_pow2"]:
        assert codecs.ue8m0_encode_pow2(np.array([v], dtype=np.float32))[0] == c


def test_ue8m0_decode_matches_torch_e8m0_for_nonzero_codes():
    codes = np.arange(1, 255, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(codecs.ue8m0_decode(codes), ref)
    # round trip of every power of two the format holds
    assert np.array_equal(codecs.ue8m0_encode_pow2(codecs.ue8m0_decode(codes).astype(np.float32)), codes)
