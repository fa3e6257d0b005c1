"""Pins for the oracle's NVFP4 quantiser and the compressor's decode state.

The NVFP4 article (section 3.2) stores the compressed cache as E2M1 values in
groups of 16 with one E4M3 scale, and keeps the unfinished half of a token
pair in the compressor's state during decode.  The quantiser's reading
(nearest E4M3 scale to amax/6, nearest E2M1 code to x/scale, ties to even,
saturating) is checked here against things other than the oracle's own
search: exact rational arithmetic (fractions.Fraction), torch's float8_e4m3fn
conversion as an independent library routine, the OCP value table under
tests/golden, exact round trips of representable groups, and the error bound
the format allows.  The decode state is checked against the batch
compressor's closed form: latent g pools raw tokens 2g and 2g+1.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import csa2_ref as ref

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _e2m1_table():
    vals = {}
    for line in open(os.path.join(GOLD, "e2m1_values.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            code, val = line.split()
            vals[int(code, 0)] = float(val)
    return vals


E2M1 = _e2m1_table()
MAGS = [Fraction(E2M1[c]) for c in range(8)]


def _e4m3_value(code):
    # torch's decoder: an independent library routine for the FP8 format
    return float(torch.tensor([code], dtype=torch.uint8).view(torch.float8_e4m3fn).float())


E4M3_POS = [Fraction(_e4m3_value(c)) for c in range(0x7F)]  # finite, >= 0


def _nearest(target, values):
    """Exact nearest value's index, ties to the even index (= even code)."""
    best, best_d = None, None
    for i, v in enumerate(values):
        d = abs(v - target)
        if best is None or d < best_d or (d == best_d and i % 2 == 0):
            best, best_d = i, d
    return best


def _bits(x):
    return float(np.float32(x))


# ---------------------------------------------------------------- scale
def test_scale_round_trips_every_e4m3_code():
    # amax = 6 * s for a representable scale s must give s back exactly
    for c in range(0x7F):
        amax = 6.0 * _e4m3_value(c)
        assert np.float32(amax) == amax
        assert ref.quant_scale_e4m3(amax) == c, hex(c)


def test_scale_matches_exact_nearest_and_torch():
    rng = np.random.default_rng(11)
    amaxes = np.concatenate([
        rng.lognormal(0.0, 3.0, 4000),                 # wide spread of group maxima
        [6 * (a + b) / 2 for a, b in zip(map(float, E4M3_POS), map(float, E4M3_POS[1:]))],
        [0.0, 1e-30, 6 * 2.0 ** -10, 6 * 2.0 ** -10 * 1.0001, 6 * 448.0, 6 * 464.0, 1e6],
    ]).astype(np.float32)
    for a in amaxes:
        a = float(a)
        want = _nearest(Fraction(a) / 6, E4M3_POS)
        got = ref.quant_scale_e4m3(a)
        assert got == want, (a, got, want)
        if a / 6 < 448.0:  # torch's conversion is round-to-nearest-even in range
            t = torch.tensor([a / 6], dtype=torch.float64).to(torch.float8_e4m3fn)
            assert int(t.view(torch.uint8)) == got, (a, got)


def test_scale_midpoints_round_to_even():
    # exact midpoints between neighbouring codes go to the even code
    for c in range(0x7E):
        mid = (E4M3_POS[c] + E4M3_POS[c + 1]) / 2
        a = float(mid * 6)
        assert Fraction(a) == mid * 6  # representable, so this is a true tie
        got = ref.quant_scale_e4m3(a)
        assert got == (c if c % 2 == 0 else c + 1), (hex(c), hex(got))


# --------------------------------------------------------------- element
def test_e2m1_ties_and_saturation():
    s_code = 0x38  # 1.0
    # (x, expected code) from the OCP table: ties go to the code whose
    # mantissa bit is 0
    cases = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),
             (6.0, 7), (6.5, 7), (100.0, 7), (0.2499, 0), (0.2501, 1), (-0.75, 10),
             (-5.0001, 15), (-0.1, 8), (0.0, 0),
             # quotients far past 6 (the distances to 4 and 6 equal in double)
             (1e30, 7), (-3e38, 15)]
    for x, want in cases:
        assert ref.quant_e2m1(x, s_code) == want, (x, want)
        if abs(x) <= 6:
            assert abs(E2M1[want]) == abs(E2M1[want & 7])


def test_e2m1_matches_exact_nearest():
    rng = np.random.default_rng(12)
    for _ in range(3000):
        sc = int(rng.integers(1, 0x7F))
        s = E4M3_POS[sc]
        x = _bits(rng.normal() * float(s) * rng.choice([0.3, 1.0, 3.0, 8.0]))
        want = _nearest(abs(Fraction(x)) / s, MAGS) | (8 if x < 0 else 0)
        assert ref.quant_e2m1(x, sc) == want, (x, sc)


def test_zero_scale_gives_zero_codes():
    assert ref.quant_e2m1(1e-6, 0) == 0
    x = np.zeros((2, 32), np.float32)
    x[1, :16] = 1e-5  # amax/6 below half the smallest E4M3 subnormal (2^-10)
    packed, scales = ref.quant_nvfp4(x)
    assert not packed.any() and not scales.any()


# ---------------------------------------------------------------- groups
def _representable_groups(rng, rows):
    """Rows of 16-groups x = e2m1(code) * s with one |code| = 6 per group."""
    cols = 64
    sc = rng.integers(0x08, 0x7F, (rows, cols // 16))           # normal scales
    codes = rng.choice([c for c in range(16) if c != 8], (rows, cols))
    codes[:, ::16] = rng.choice([7, 15], (rows, cols // 16))      # amax = 6 s
    x = np.zeros((rows, cols), np.float64)
    for r in range(rows):
        for c in range(cols):
            x[r, c] = E2M1[int(codes[r, c])] * float(E4M3_POS[int(sc[r, c // 16])])
    assert (x.astype(np.float32) == x).all()
    return x.astype(np.float32), codes, sc


def test_representable_groups_round_trip_exactly():
    rng = np.random.default_rng(13)
    x, codes, sc = _representable_groups(rng, 40)
    packed, scales = ref.quant_nvfp4(x)
    assert (scales == sc).all()
    lo, hi = packed & 15, packed >> 4
    got = np.stack([lo, hi], -1).reshape(x.shape)
    assert (got == codes).all()
    assert (ref.dequant_nvfp4(packed, scales) == x).all()


def test_quant_error_bound():
    # with a normal, unsaturated scale s: |dequant - x| <= s (the largest
    # half-gap of E2M1 is 1, between 4 and 6; a value clipped to 6 is at
    # most amax/s - 6 <= 6/(1 - 2^-4) - 6 < 1 away), and s <= amax/6 * 17/16
    rng = np.random.default_rng(14)
    x = (rng.normal(size=(300, 512)) * rng.lognormal(0, 2, (300, 1))).astype(np.float32)
    packed, scales = ref.quant_nvfp4(x)
    dq = ref.dequant_nvfp4(packed, scales)
    s = np.repeat(np.array([[ref.e4m3(int(c)) for c in row] for row in scales]), 16, axis=1)
    amax = np.repeat(np.abs(x).reshape(300, 32, 16).max(-1), 16, axis=1).astype(np.float64)
    normal = amax / 6 >= 2.0 ** -6  # the scale's target lies in E4M3's normal range
    assert normal.mean() > 0.9
    err = np.abs(dq - x)
    assert (err[normal] <= s[normal]).all()
    assert (s[normal] <= amax[normal] / 6 * 17 / 16).all()
    assert (s[normal] >= amax[normal] / 6 * 15 / 16).all()
    # a subnormal scale is off amax/6 by at most half its quantum 2^-9, so a
    # clipped value is at most 6 * 2^-10 away on top of the code's half-gap
    assert (err[~normal] <= s[~normal] + 6 * 2.0 ** -10).all()
    # and every element took the nearest code under its scale
    for r, c in [(0, 0), (7, 100), (299, 511)] + [tuple(v) for v in rng.integers(0, [300, 512], (200, 2))]:
        sc = int(scales[r, c // 16])
        want = _nearest(abs(Fraction(float(x[r, c]))) / E4M3_POS[sc], MAGS)
        assert abs(dq[r, c]) == float(MAGS[want] * E4M3_POS[sc])


def test_packing_order_low_nibble_first():
    x = np.zeros((1, 16), np.float32)
    x[0, 0], x[0, 1] = 6.0, -1.0   # scale 1.0: codes 7 and 10
    packed, scales = ref.quant_nvfp4(x)
    assert scales[0, 0] == 0x38 and packed[0, 0] == (7 | (10 << 4))


# ------------------------------------------------------ compressor to NVFP4
def test_compress_nvfp4_is_quantised_pooling():
    rng = np.random.default_rng(15)
    B, T = 2, 10
    raw = torch.randn(B, T, 512, generator=torch.Generator().manual_seed(3)).bfloat16()
    gate = torch.randn(B, T, 512, generator=torch.Generator().manual_seed(4)).bfloat16()
    raw, gate = raw.view(torch.uint16).numpy(), gate.view(torch.uint16).numpy()
    packed, scales, y = ref.compress_nvfp4(raw, gate)
    assert packed.shape == (B, T // 2, 256) and scales.shape == (B, T // 2, 32)
    # closed form of the pooling for one channel (softmax over two logits)
    xr = torch.from_numpy(raw.astype(np.int16)).view(torch.bfloat16).double().numpy()
    gr = torch.from_numpy(gate.astype(np.int16)).view(torch.bfloat16).double().numpy()
    b, g, c = 1, 3, 77
    w = 1.0 / (1.0 + math.exp(gr[b, 2 * g + 1, c] - gr[b, 2 * g, c]))
    assert abs(y[b, g, c] - (w * xr[b, 2 * g, c] + (1 - w) * xr[b, 2 * g + 1, c])) < 1e-12
    dq = ref.dequant_nvfp4(packed.reshape(-1, 256), scales.reshape(-1, 32)).reshape(y.shape)
    s = np.repeat(np.vectorize(lambda v: ref.e4m3(int(v)))(scales), 16, axis=-1)
    assert (np.abs(dq - y) <= s * (1 + 1e-6)).all()


# ------------------------------------------------------------ decode state
@pytest.mark.parametrize("fmt", ["bf16", "nvfp4"])
def test_decode_state_matches_batch_compressor(fmt):
    """Streaming one token per step through the carried state fills the cache
    exactly as the batch compressor does over the same tokens: latent g is
    the pooling of raw tokens 2g and 2g+1, whichever step each arrived in."""
    g = torch.Generator().manual_seed(21)
    B, T, n_cache = 3, 14, 6
    raw = torch.randn(B, T, 512, generator=g).bfloat16().view(torch.uint16).numpy()
    gate = torch.randn(B, T, 512, generator=g).bfloat16().view(torch.uint16).numpy()
    start = [0, 3, 5]  # sequence b begins streaming at raw position start[b]
    state = np.zeros((B, 2, 512), np.uint16)
    for b in range(B):
        if start[b] % 2:  # its pending partner was left in state by earlier work
            state[b, 0], state[b, 1] = raw[b, start[b] - 1], gate[b, start[b] - 1]
    if fmt == "bf16":
        cache = np.zeros((B, n_cache, 512), np.uint16)
    else:
        cache = (np.zeros((B, n_cache, 256), np.uint8), np.zeros((B, n_cache, 32), np.uint8))
    for step in range(T):
        pos = np.array([s + step if s + step < T else -1 for s in start])
        kv_tok = np.stack([raw[b, min(p, T - 1)] for b, p in enumerate(pos)])
        gate_tok = np.stack([gate[b, min(p, T - 1)] for b, p in enumerate(pos)])
        ref.compress_decode(state, kv_tok, gate_tok, pos, cache, n_cache, fmt)
    if fmt == "bf16":
        want, _ = ref.compress(raw, gate)
    else:
        want = ref.compress_nvfp4(raw, gate)[:2]
    for b in range(B):
        lo = (start[b] - 1) // 2 if start[b] % 2 else start[b] // 2  # first latent completed
        hi = min(T // 2, n_cache)
        if fmt == "bf16":
            assert (cache[b, lo:hi] == want[b, lo:hi]).all()
            assert not cache[b, :lo].any() and not cache[b, hi:].any()
        else:
            assert (cache[0][b, lo:hi] == want[0][b, lo:hi]).all()
            assert (cache[1][b, lo:hi] == want[1][b, lo:hi]).all()
            assert not cache[1][b, :lo].any()
