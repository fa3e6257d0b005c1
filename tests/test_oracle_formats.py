"""Pins for the oracle's element decoders and its bf16 rounding.

The decoders are checked against things other than their own formulas: the
OCP value tables stored under tests/golden (cited there), torch's dtype
conversions (bfloat16, float8_e4m3fn) as independent library routines, and
exact-representability facts the configs rely on.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute
from oracle import csa2_ref as ref

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _table(name):
    rows = []
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = line.split()
        rows.append((int(code, 0), float(val)))
    return rows


def _same(a, b):
    if math.isnan(b):
        return math.isnan(a)
    return a == b and math.copysign(1, a) == math.copysign(1, b)


def test_e2m1_matches_ocp_table():
    rows = _table("e2m1_values.txt")
    assert len(rows) == 16
    for code, val in rows:
        assert _same(ref.e2m1(code), val), (code, ref.e2m1(code), val)


def test_e4m3_landmarks():
    for code, val in _table("e4m3_landmarks.txt"):
        assert _same(ref.e4m3(code), val), (hex(code), ref.e4m3(code), val)


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    lib_vals = brute.dec_e4m3(codes)
    for c in range(256):
        assert _same(ref.e4m3(c), float(lib_vals[c])), hex(c)


def test_bf16_decode_matches_torch_all_patterns():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    t = brute.dec_bf16(pats)
    ours = ref.bf16_array(pats)
    nan = np.isnan(t)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], t[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(t[~nan]))


def test_round_bf16_matches_torch_from_float32():
    rng = np.random.default_rng(7)
    # random float32 bit patterns over a wide exponent range, plus subnormals
    vals = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * np.float32(2.0) ** rng.integers(-60, 60, 4000).astype(np.float32),
        (rng.standard_normal(200) * 1e-39).astype(np.float32),
    ])
    exp = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for v, e in zip(vals, exp):
        assert ref.round_bf16(float(v)) == int(e), (float(v), hex(ref.round_bf16(float(v))), hex(int(e)))


@pytest.mark.parametrize("x,bits", [
    (1.0 + 2 ** -8, 0x3F80),          # tie, even neighbour is 1.0
    (1.0 + 3 * 2 ** -8, 0x3F82),      # tie, even neighbour is 1 + 2^-6
    (1.0 + 2 ** -8 + 2 ** -30, 0x3F81),  # just above the tie rounds up
    (-2.5, 0xC020),
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (3.4e38, 0x7F80),                 # overflows to +inf under RNE
])
def test_round_bf16_ties_and_edges(x, bits):
    assert ref.round_bf16(x) == bits


def test_small_integers_exact_in_every_format():
    # index q/k values are integers in [-3, 3]; they must survive bf16,
    # E4M3 and E2M1 exactly (so any storage precision gives the same scores)
    for v in range(-3, 4):
        assert ref.bf16(ref.round_bf16(v)) == v
        code = int(torch.tensor([float(v)]).to(torch.float8_e4m3fn).view(torch.uint8)[0])
        assert ref.e4m3(code) == v
    e2m1_vals = {ref.e2m1(c) for c in range(16)}
    assert {-3, -2, -1, 0, 1, 2, 3} <= e2m1_vals


def test_nvfp4_dequant_matches_brute():
    rng = np.random.default_rng(3)
    packed = rng.integers(0, 256, (5, 256), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (5, 32), dtype=np.uint8)  # finite E4M3 codes
    ours = ref.dequant_nvfp4(packed, scales)
    assert np.array_equal(ours, brute.dec_nvfp4(packed, scales))
    # element 2i is the low nibble of byte i
    p = np.zeros((1, 256), np.uint8)
    p[0, 0] = 0x71  # low nibble code 1 (0.5), high nibble code 7 (6.0)
    s = np.full((1, 32), 0x38, np.uint8)  # scale 1.0
    d = ref.dequant_nvfp4(p, s)
    assert d[0, 0] == 0.5 and d[0, 1] == 6.0 and np.all(d[0, 2:] == 0)


def test_fp8_dequant_row_scale():
    rng = np.random.default_rng(4)
    src = rng.integers(0, 0x7F, (6, 64), dtype=np.uint8)
    sc = rng.random(6).astype(np.float32) + 0.5
    ours = ref.dequant_fp8(src, sc)
    exp = brute.dec_e4m3(src) * sc[:, None].astype(np.float64)
    assert np.array_equal(ours, exp)


# ---- the index query rounded to the key format (NVFP4 article, section 3.3:
# FP4 index queries; E4M3 keys meet an E4M3 query, MXFP4 keys an E2M1 one)
def _all_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    return bits, vals


def test_query_round_e4m3_matches_torch_cast():
    bits, vals = _all_bf16()
    fin = np.isfinite(vals)
    inside = fin & (np.abs(vals) < 464.0)
    want = brute.round_e4m3(vals[inside])
    got = np.array([ref.e4m3(ref.round_e4m3(v)) for v in vals[inside]])
    assert np.array_equal(got, want)
    # beyond torch's saturating range (and infinities) the format's largest
    # finite magnitude, 448, with the input's sign
    outside = ~inside & ~np.isnan(vals)
    got_out = np.array([ref.e4m3(ref.round_e4m3(v)) for v in vals[outside]])
    assert np.array_equal(got_out, np.where(vals[outside] < 0, -448.0, 448.0))
    # ties go to the even code: 2^-10 (half the smallest subnormal) -> 0,
    # 3 * 2^-10 -> 2^-8 (code 2), 1 + 1/16 -> 1, 1 + 3/16 -> 1.25
    for x, code in ((2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (1 + 1 / 16, 0x38),
                    (1 + 3 / 16, 0x3A), (-(1 + 3 / 16), 0xBA)):
        assert ref.round_e4m3(x) == code, (x, ref.round_e4m3(x), code)


def test_query_round_e2m1_matches_exact_nearest():
    from fractions import Fraction

    table = _table("e2m1_values.txt")
    mags = sorted({abs(v) for _, v in table})
    code_of = {abs(v): c for c, v in table if c < 8}
    bits, vals = _all_bf16()
    sel = np.isfinite(vals) & (np.abs(vals) <= 8.0)
    for v in vals[sel][::7].tolist() + [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.75, 6.0, 7.9]:
        a = Fraction(abs(v))
        d = [abs(a - Fraction(m)) for m in mags]
        best = min(d)
        ties = [m for m, dd in zip(mags, d) if dd == best]
        m = ties[0] if len(ties) == 1 else [t for t in ties if code_of[t] % 2 == 0][0]
        want = code_of[m] | (8 if v < 0 else 0)
        assert ref.round_e2m1(v) == want, (v, ref.round_e2m1(v), want)
        assert ref.e2m1(ref.round_e2m1(v)) == brute.round_e2m1(np.array([v]))[0], v
    assert ref.e2m1(ref.round_e2m1(1e30)) == 6.0 and ref.e2m1(ref.round_e2m1(-7.0)) == -6.0
