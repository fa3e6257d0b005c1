"""Pins for the indexer's query rounding (NVFP4 article, section 3.3: the
index queries are FP4 in the model; reading: a bf16 index query is rounded to
the format of the keys it meets -- E4M3 for FP8 keys, E2M1 for MXFP4 keys --
and used as is against bf16 keys).

The oracle's scan and candidate scores for non-integer queries are checked
against the brute force, which rounds with torch's float8_e4m3fn cast and a
neighbour search in the OCP E2M1 value list and scores with one dense einsum.
A query left unrounded must give different scores (the check has teeth)."""
import numpy as np
import torch

from oracle import brute
from oracle import csa2_ref as ref

B, TQ, N = 2, 3, 83


def _query(seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, TQ, 32, 128), generator=g) * 1.7
    return q.bfloat16().view(torch.int16).numpy().view(np.uint16)


def _common(seed):
    rng = np.random.default_rng(seed)
    w = (rng.integers(1, 17, (B, TQ, 32)) / 16).astype(np.float32)
    q_pos = np.array([[9, 100, 165], [0, 64, 170]], np.int64)
    return rng, w, q_pos


def _brute_rows(q, w, q_pos, score_fn):
    out = np.full((B * TQ, N), -np.inf)
    for r in range(B * TQ):
        b, j = divmod(r, TQ)
        nv = brute.visible(q_pos[b, j], N)
        out[r, :nv] = score_fn(b, j)[:nv]
    return out


def _check(q, w, q_pos, keys, score_fn, unrounded_keys):
    sc, bm = ref.scan(q, w, keys, q_pos, want_scores=True)
    want = _brute_rows(q, w, q_pos, score_fn)
    np.testing.assert_allclose(sc, want, rtol=1e-13, atol=0)
    nb = (N + 7) // 8
    pad = np.full((B * TQ, nb * 8), -np.inf)
    pad[:, :N] = want
    assert np.array_equal(bm, pad.reshape(B * TQ, nb, 8).max(-1))
    blocks = np.tile(np.array([0, 4, 7, nb - 1, -1], np.int32), (B * TQ, 1))
    cs, ci = ref.cand(q, w, keys, q_pos, blocks)
    for r in range(B * TQ):
        for j, bl in enumerate(blocks[r]):
            for i in range(8):
                g = bl * 8 + i
                if bl >= 0 and g < N and np.isfinite(want[r, g]):
                    assert ci[r, 8 * j + i] == g
                    assert abs(cs[r, 8 * j + i] - want[r, g]) <= 1e-13 * abs(want[r, g])
                else:
                    assert ci[r, 8 * j + i] == -1 and cs[r, 8 * j + i] == -np.inf
    # the same key values stored as bf16 meet the unrounded query: different
    sc_u, _ = ref.scan(q, w, unrounded_keys, q_pos, want_scores=True)
    assert not np.array_equal(sc_u, sc)


def test_fp8_keys_meet_an_e4m3_query():
    rng, w, q_pos = _common(3)
    q = _query(4)
    codes = rng.integers(0, 256, (B, N, 128)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38  # no NaN keys
    vals = brute.dec_e4m3(codes)
    as_bf16 = torch.from_numpy(vals).float().bfloat16()  # E4M3 values are bf16 values
    assert torch.equal(as_bf16.double(), torch.from_numpy(vals))
    _check(q, w, q_pos, codes,
           lambda b, j: brute.index_scores(q[b, j], w[b, j], codes[b]),
           as_bf16.view(torch.int16).numpy().view(np.uint16))


def test_mxfp4_keys_meet_an_e2m1_query():
    rng, w, q_pos = _common(5)
    q = _query(6)
    codes = rng.integers(0, 256, (B, N, 64)).astype(np.uint8)
    scales = rng.integers(124, 130, (B, N, 4)).astype(np.uint8)
    nib = np.stack([codes & 15, codes >> 4], -1).reshape(B, N, 128)
    kd = brute.dec_e2m1(nib) * np.repeat(2.0 ** (scales.astype(np.float64) - 127), 32, axis=-1)
    as_bf16 = torch.from_numpy(kd).float().bfloat16()
    assert torch.equal(as_bf16.double(), torch.from_numpy(kd))
    _check(q, w, q_pos, (codes, scales),
           lambda b, j: brute.index_scores(q[b, j], w[b, j], None, kd=kd[b]),
           as_bf16.view(torch.int16).numpy().view(np.uint16))


def test_integer_queries_are_unchanged_by_the_rounding():
    """The configs' index queries (integers in [-3, 3]) are exact in E4M3 and
    E2M1, so every key format scores them as the bf16 query."""
    for v in range(-3, 4):
        assert ref.e4m3(ref.round_e4m3(v)) == v and ref.e2m1(ref.round_e2m1(v)) == v
