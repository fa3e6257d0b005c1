"""Brute-force NumPy formulations used to pin the C oracle on tiny inputs.

TEST INFRASTRUCTURE ONLY.  Each function restates a step of the CSA2 path in
a deliberately different form from ``csa2_ref.c`` so that a slip in either
(dropped term, wrong index, transposed operand) shows up as a mismatch:

* decoding uses torch's dtype conversions (bf16, float8_e4m3fn) and the OCP
  E2M1 value list, not the bit-field formulas; the index query's rounding to
  the key format uses torch's float8_e4m3fn cast and a neighbour search in
  the E2M1 value list, not a scan over codes;
* the compressor uses the two-token closed form y = x1 + sigmoid(l0-l1)(x0-x1);
* indexer scores are one dense einsum over all latents;
* the block stage ranks every block with ``np.lexsort`` and then swaps the
  newest block in for the last pick when it was not chosen;
* attention is dense: every latent and every window slot is scored, then
  everything outside Sel and the window is masked to -inf, and the sink is an
  extra column of the softmax.
"""
from __future__ import annotations

import numpy as np
import torch

D, HQ, HI, DI, BLK = 512, 64, 32, 128, 8

# OCP MX specification, E2M1 element encoding: magnitudes of codes 0..7.
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def dec_bf16(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def dec_e4m3(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def dec_e2m1(nib: np.ndarray) -> np.ndarray:
    nib = np.asarray(nib)
    mag = E2M1_MAG[nib & 7]
    return np.where(nib & 8, -mag, mag)


def dec_nvfp4(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[..., cols/2] bytes + [..., cols/16] E4M3 scales -> [..., cols]."""
    lo = packed & 15
    hi = packed >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)
    sc = np.repeat(dec_e4m3(scales), 16, axis=-1)
    return dec_e2m1(codes) * sc


def dec_keys(k):
    return dec_bf16(k) if k.dtype == np.uint16 else dec_e4m3(k)


def round_e4m3(x: np.ndarray) -> np.ndarray:
    """Values to the nearest E4M3 value by torch's float8_e4m3fn cast (which
    rounds to nearest even and saturates to 448 only below 464: callers keep
    |x| < 464)."""
    x = np.asarray(x, np.float64)
    assert np.all(np.abs(x) < 464.0)
    return torch.from_numpy(x).float().to(torch.float8_e4m3fn).to(torch.float64).numpy()


def round_e2m1(x: np.ndarray) -> np.ndarray:
    """Values to the nearest E2M1 value, ties to the even code, saturating at
    6: the neighbours of |x| in the sorted magnitude list, the closer one, or
    the one with an even code on a tie."""
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    hi = np.clip(np.searchsorted(E2M1_MAG, a, side="left"), 0, 7)
    lo = np.clip(hi - 1, 0, 7)
    dlo, dhi = a - E2M1_MAG[lo], E2M1_MAG[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a >= 6.0, 7, pick)
    mag = E2M1_MAG[pick]
    return np.where(x < 0, -mag, mag)


def compress(raw, gate):
    x = dec_bf16(raw)
    l = dec_bf16(gate)
    x0, x1 = x[:, 0::2], x[:, 1::2]
    l0, l1 = l[:, 0::2], l[:, 1::2]
    sig = 1.0 / (1.0 + np.exp(-(l0 - l1)))
    return x1 + sig * (x0 - x1)


def visible(t, N):
    return min(N, (int(t) + 1) // 2) if t >= 0 else 0


def index_scores(q, w, k, kd=None):
    """q [32][128] bits, w [32], k [N][128] -> dense scores [N].  The query
    meets E4M3 keys rounded to E4M3; ``kd`` (decoded keys) stands for MXFP4
    keys, which meet the query rounded to E2M1."""
    qd = dec_bf16(q)
    if kd is not None:
        qd = round_e2m1(qd)
    else:
        if k.dtype != np.uint16:
            qd = round_e4m3(qd)
        kd = dec_keys(k)
    dots = np.einsum("hd,nd->hn", qd, kd)
    return np.einsum("h,hn->n", w.astype(np.float64), np.maximum(dots, 0.0))


def topk_ids(scores, ids, k):
    """Top-k ids by (score desc, id asc) via a full lexsort."""
    order = np.lexsort((ids, -scores))
    return ids[order[:k]]


def decode_row(inp, r, K_b, K, W, scale):
    """Whole decode path for query row r, brute force.  Returns dict."""
    cfg_B, Tq = inp["q_pos"].shape
    b, tq = divmod(r, Tq)
    t = int(inp["q_pos"][b, tq])
    lat = inp["lat"]
    N = lat.shape[1]
    nv = visible(t, N)
    # candidate-source scores and block maxima
    s_src = index_scores(inp["qs"][b, tq], inp["ws"][b, tq], inp["ks"][b])
    s_src[nv:] = -np.inf
    nb = (nv + BLK - 1) // BLK
    padded = np.full(nb * BLK, -np.inf)
    padded[:nv] = s_src[:nv]
    bmax = padded.reshape(nb, BLK).max(axis=1) if nb else np.zeros(0)
    newest = nb - 1
    if nb <= K_b:
        blocks = np.arange(nb)
    else:
        blocks = topk_ids(bmax, np.arange(nb), K_b)
        if newest not in blocks:
            blocks[-1] = newest
    blocks = np.sort(blocks)
    cand = np.array([g for bl in blocks for g in range(bl * BLK, bl * BLK + BLK) if g < nv], dtype=np.int64)
    s_cur = index_scores(inp["qi"][b, tq], inp["wi"][b, tq], inp["ki"][b])
    sel = np.sort(topk_ids(s_cur[cand], cand, K)) if len(cand) else cand
    # dense attention over every latent and window slot, masked
    if lat.dtype == np.uint16:
        kv_lat = dec_bf16(lat[b])
    else:
        kv_lat = dec_nvfp4(lat[b], inp["lat_scale"][b])
    win = inp["win"]
    W_cap = win.shape[1]
    if win.dtype == np.uint16:
        kv_win = dec_bf16(win[b])
    else:
        kv_win = dec_e4m3(win[b]) * inp["win_scale"][b][:, None].astype(np.float64)
    mask_lat = np.zeros(N, bool)
    mask_lat[sel] = True
    mask_win = np.zeros(W_cap, bool)
    for p in range(max(0, t - W + 1), t + 1):
        mask_win[p % W_cap] = True
    kv = np.concatenate([kv_lat, kv_win], axis=0)
    mask = np.concatenate([mask_lat, mask_win])
    qd = dec_bf16(inp["q"][b, tq])                      # [64][512]
    logits = qd @ kv.T * scale                          # [64][N+W_cap]
    logits[:, ~mask] = -np.inf
    sink = inp["sink"].astype(np.float64)[:, None]
    full = np.concatenate([logits, sink], axis=1)
    m = full.max(axis=1, keepdims=True)
    e = np.exp(full - m)
    z = e.sum(axis=1, keepdims=True)
    p = e[:, :-1] / z
    out = p @ kv
    lse = (m + np.log(z))[:, 0]
    return dict(block_max=bmax, blocks=blocks, cand=cand, sel=sel, out=out, lse=lse,
                n_rows=int(mask.sum()))
