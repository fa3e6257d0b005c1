"""Pins for the oracle's MXFP4 index keys (E2M1 codes with one E8M0 scale per
32 dims; the NVFP4 article, section 3.3, quantises the index keys to FP4 and
section 4 describes MXFP4's UE8M0 block scale).

Checked against: the OCP MX E8M0 landmarks under tests/golden, torch's
float8_e8m0fnu decoder for every code, and the oracle's own bf16 key path
(itself pinned elsewhere): MXFP4 keys whose values are bf16 values must give
the same scores as those values stored as bf16, which fails on a wrong
nibble order, a wrong scale block, or a wrong exponent bias."""
import math
import os

import numpy as np
import torch

from oracle import csa2_ref as ref

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_e8m0_landmarks():
    for line in open(os.path.join(GOLD, "e8m0_landmarks.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = line.split()
        got = ref.e8m0(int(code, 0))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val), (code, got, val)


def test_e8m0_all_codes_match_torch():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    for c in range(256):
        got = ref.e8m0(c)
        assert (math.isnan(got) and math.isnan(t[c])) or got == t[c], c


def _mx_keys(rng, B, N, scale_lo=125, scale_hi=129):
    codes = rng.integers(0, 256, (B, N, 64), dtype=np.uint8)
    scales = rng.integers(scale_lo, scale_hi + 1, (B, N, 4), dtype=np.uint8)
    return codes, scales


def _as_bf16(codes, scales):
    """The same keys as exact bf16 values, decoded without the oracle: the
    OCP E2M1 table and powers of two."""
    e2m1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])
    lo, hi = codes & 15, codes >> 4
    nib = np.stack([lo, hi], -1).reshape(*codes.shape[:2], 128)
    v = e2m1[nib] * np.repeat(2.0 ** (scales.astype(np.float64) - 127), 32, axis=-1)
    t = torch.from_numpy(v).float()
    assert torch.equal(t.bfloat16().float(), t)  # every such value is a bf16 value
    return t.bfloat16().view(torch.uint16).numpy()


def test_mxfp4_keys_score_as_their_bf16_values():
    rng = np.random.default_rng(5)
    B, Tq, N = 2, 3, 77
    q = torch.randint(-3, 4, (B, Tq, 32, 128), generator=torch.Generator().manual_seed(1))
    q = q.float().bfloat16().view(torch.uint16).numpy()
    w = (rng.integers(1, 17, (B, Tq, 32)) / 16).astype(np.float32)
    q_pos = np.array([[10, 100, 153], [0, 60, 153]], np.int64)
    codes, scales = _mx_keys(rng, B, N)
    sc_mx, bm_mx = ref.scan(q, w, (codes, scales), q_pos, want_scores=True)
    sc_bf, bm_bf = ref.scan(q, w, _as_bf16(codes, scales), q_pos, want_scores=True)
    assert np.array_equal(sc_mx, sc_bf) and np.array_equal(bm_mx, bm_bf)
    blocks = np.tile(np.array([0, 3, 9], np.int32), (B * Tq, 1))
    c_mx = ref.cand(q, w, (codes, scales), q_pos, blocks)
    c_bf = ref.cand(q, w, _as_bf16(codes, scales), q_pos, blocks)
    assert np.array_equal(c_mx[0], c_bf[0]) and np.array_equal(c_mx[1], c_bf[1])
    # and a planted nibble swap would not pass
    swapped = ((codes & 15) << 4) | (codes >> 4)
    sc_sw, _ = ref.scan(q, w, (swapped.astype(np.uint8), scales), q_pos, want_scores=True)
    assert not np.array_equal(sc_sw, sc_bf)
