"""ctypes wrapper around the plain CPU oracle ``libcsa2ref.so``.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  Arrays are host
numpy arrays; bf16 data is passed as its uint16 bit pattern, FP8 / NVFP4 data
as uint8 codes.  Results in floating point are float64.

The step functions mirror the hot path (NVFP4 article sections 3-3.4):
compress (2:1 softmax-gated pooling), scan (indexer score of every visible
latent and the per-block maximum), select (top-k by score, ties to the
smaller id, an optional forced id), cand (indexer over the latents of the
chosen blocks), attn (64-head attention over the selected latents plus the
raw window, with a per-head sink).  ``decode`` chains them per the method.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "libcsa2ref.so")

BF16, E4M3, NVFP4, F32, MXFP4 = 1, 2, 3, 4, 5
MXFP4_ROW = 68
D, HQ, HI, DI, BLK = 512, 64, 32, 128, 8
_FMT = {"bf16": BF16, "fp8": E4M3, "nvfp4": NVFP4, "f32": F32}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from oracle import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        P, I, I64, D_ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.csa2ref_threads.restype = I
        L.csa2ref_threads.argtypes = []
        L.csa2ref_set_threads.restype = None
        L.csa2ref_set_threads.argtypes = [I]
        L.csa2ref_bf16.restype = D_
        L.csa2ref_bf16.argtypes = [ctypes.c_uint16]
        L.csa2ref_e4m3.restype = D_
        L.csa2ref_e4m3.argtypes = [ctypes.c_uint8]
        L.csa2ref_e2m1.restype = D_
        L.csa2ref_e2m1.argtypes = [ctypes.c_uint8]
        L.csa2ref_e8m0.restype = D_
        L.csa2ref_e8m0.argtypes = [ctypes.c_uint8]
        L.csa2ref_round_e4m3.restype = ctypes.c_uint8
        L.csa2ref_round_e4m3.argtypes = [D_]
        L.csa2ref_round_e2m1.restype = ctypes.c_uint8
        L.csa2ref_round_e2m1.argtypes = [D_]
        L.csa2ref_round_bf16.restype = ctypes.c_uint16
        L.csa2ref_round_bf16.argtypes = [D_]
        L.csa2ref_n_vis.restype = I64
        L.csa2ref_n_vis.argtypes = [I64, I64]
        L.csa2ref_newest_block.restype = I64
        L.csa2ref_newest_block.argtypes = [I64, I64]
        L.csa2ref_compress.restype = None
        L.csa2ref_compress.argtypes = [I, I, P, I64, P, I64, P, I64, P]
        L.csa2ref_scan.restype = None
        L.csa2ref_scan.argtypes = [I, I, P, P, P, I, I64, I64, P, P, I64, P, I64]
        L.csa2ref_select.restype = None
        L.csa2ref_select.argtypes = [I, I64, P, I64, P, I64, P, I, P, I64]
        L.csa2ref_cand.restype = None
        L.csa2ref_cand.argtypes = [I, I, P, P, P, I, I64, I64, P, P, I, P, P, I64]
        L.csa2ref_attn.restype = None
        L.csa2ref_attn.argtypes = [I, I, P, I64, P, I, P, I64, I64, P, I, I64, P, I, P,
                                   I, I, I64, P, P, D_, P, P]
        L.csa2ref_dequant_fp8.restype = None
        L.csa2ref_dequant_fp8.argtypes = [P, P, I64, I, P]
        L.csa2ref_dequant_nvfp4.restype = None
        L.csa2ref_dequant_nvfp4.argtypes = [P, P, I64, I, P]
        L.csa2ref_quant_scale_e4m3.restype = ctypes.c_uint8
        L.csa2ref_quant_scale_e4m3.argtypes = [ctypes.c_float]
        L.csa2ref_quant_e2m1.restype = ctypes.c_uint8
        L.csa2ref_quant_e2m1.argtypes = [ctypes.c_float, ctypes.c_uint8]
        L.csa2ref_quant_nvfp4.restype = None
        L.csa2ref_quant_nvfp4.argtypes = [P, I64, I, P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    assert a.dtype == np.dtype(dtype), (a.dtype, dtype)
    return a


def _keys(k):
    """Index keys as (array, format, batch stride): uint16 bf16 or uint8 E4M3
    [B][N][128], or an MXFP4 pair (codes uint8 [B][N][64], E8M0 scales uint8
    [B][N][4]) packed into the oracle's 68-byte rows."""
    if isinstance(k, tuple):
        codes, scales = np.ascontiguousarray(k[0], np.uint8), np.ascontiguousarray(k[1], np.uint8)
        B, N = codes.shape[:2]
        assert codes.shape == (B, N, DI // 2) and scales.shape == (B, N, DI // 32)
        packed = np.ascontiguousarray(np.concatenate([codes, scales], axis=2))
        return packed, MXFP4, N * MXFP4_ROW
    k = np.ascontiguousarray(k)
    return k, (BF16 if k.dtype == np.uint16 else E4M3), k.shape[1] * DI


def threads() -> int:
    """OpenMP threads the oracle's next parallel region uses."""
    return lib().csa2ref_threads()


def set_threads(n: int) -> None:
    lib().csa2ref_set_threads(int(n))


# ---------------------------------------------------------------- decoders
def bf16(bits) -> float:
    return lib().csa2ref_bf16(int(bits))


def e4m3(bits) -> float:
    return lib().csa2ref_e4m3(int(bits))


def e8m0(bits) -> float:
    return lib().csa2ref_e8m0(int(bits))


def e2m1(nibble) -> float:
    return lib().csa2ref_e2m1(int(nibble))


def round_bf16(x) -> int:
    return lib().csa2ref_round_bf16(float(x))


def bf16_array(bits: np.ndarray) -> np.ndarray:
    """Decode a uint16 bf16 array to float64 (via the oracle's decoder)."""
    u = np.ascontiguousarray(bits, dtype=np.uint16)
    flat = u.reshape(-1)
    tab = np.array([bf16(i) for i in range(65536)], dtype=np.float64)
    return tab[flat].reshape(u.shape)


def round_e4m3(x) -> int:
    """Nearest E4M3 code to x (ties to even, saturating at 448): the index
    query's rounding for E4M3 keys."""
    return lib().csa2ref_round_e4m3(float(x))


def round_e2m1(x) -> int:
    """Nearest E2M1 nibble to x (ties to even, saturating at 6): the index
    query's rounding for MXFP4 keys."""
    return lib().csa2ref_round_e2m1(float(x))


def n_vis(t, n_cache) -> int:
    return lib().csa2ref_n_vis(int(t), int(n_cache))


def newest_block(t, n_cache) -> int:
    return lib().csa2ref_newest_block(int(t), int(n_cache))


# ------------------------------------------------------------------ steps
def compress(raw: np.ndarray, gate: np.ndarray):
    """raw, gate: uint16 bf16 [B][T][512] -> (bf16 bits [B][T/2][512], float64)."""
    raw, gate = _c(raw, np.uint16), _c(gate, np.uint16)
    B, T, _ = raw.shape
    assert raw.shape == gate.shape and raw.shape[2] == D and T % 2 == 0
    out = np.zeros((B, T // 2, D), np.uint16)
    out64 = np.zeros((B, T // 2, D), np.float64)
    lib().csa2ref_compress(B, T, _p(raw), T * D, _p(gate), T * D, _p(out), (T // 2) * D, _p(out64))
    return out, out64


def scan(q, w, k, q_pos, want_scores=False):
    """Indexer scores of every visible latent and per-block maxima.

    q uint16 [B][Tq][32][128]; w f32 [B][Tq][32]; k [B][N][128] (uint16 bf16 or
    uint8 E4M3) or an MXFP4 (codes, scales) pair; q_pos int64 [B][Tq].  The
    query is rounded to the key format first (E4M3 / E2M1, nearest, ties to
    even, saturating).  Returns (scores [B*Tq][N] or None, block_max
    [B*Tq][ceil(N/8)]), float64 with -inf where invisible."""
    q, w, q_pos = _c(q, np.uint16), _c(w, np.float32), _c(q_pos, np.int64)
    k, k_fmt, k_sb = _keys(k)
    B, Tq = q.shape[:2]
    N = k.shape[1]
    assert q.shape == (B, Tq, HI, DI) and w.shape == (B, Tq, HI) and q_pos.shape == (B, Tq)
    assert k.shape[:2] == (B, N)
    nblk = (N + BLK - 1) // BLK
    sc = np.zeros((B * Tq, N), np.float64) if want_scores else None
    bm = np.zeros((B * Tq, nblk), np.float64)
    lib().csa2ref_scan(B, Tq, _p(q), _p(w), _p(k), k_fmt, k_sb, N, _p(q_pos),
                       _p(sc), N, _p(bm), nblk)
    return sc, bm


def select(scores, k, ids=None, forced=None):
    """Top-k per row by (score desc, id asc); ascending ids padded with -1."""
    scores = _c(scores, np.float64)
    R, n = scores.shape
    ids = _c(ids, np.int32)
    forced = _c(forced, np.int32)
    out = np.zeros((R, k), np.int32)
    lib().csa2ref_select(R, n, _p(scores), n, _p(ids), n, _p(forced), k, _p(out), k)
    return out


def cand(q, w, k, q_pos, blocks):
    """Indexer scores over the latents of the chosen blocks.

    blocks int32 [B*Tq][K_b]; returns (scores float64 [B*Tq][8*K_b],
    ids int32 [B*Tq][8*K_b]) with id -1 / score -inf for absent latents."""
    q, w, q_pos, blocks = _c(q, np.uint16), _c(w, np.float32), _c(q_pos, np.int64), _c(blocks, np.int32)
    k, k_fmt, k_sb = _keys(k)
    B, Tq = q.shape[:2]
    N = k.shape[1]
    K_b = blocks.shape[1]
    assert q.shape == (B, Tq, HI, DI) and w.shape == (B, Tq, HI) and q_pos.shape == (B, Tq)
    assert k.shape[:2] == (B, N) and blocks.shape == (B * Tq, K_b)
    sc = np.zeros((B * Tq, K_b * BLK), np.float64)
    ids = np.zeros((B * Tq, K_b * BLK), np.int32)
    lib().csa2ref_cand(B, Tq, _p(q), _p(w), _p(k), k_fmt, k_sb, N, _p(q_pos),
                       _p(blocks), K_b, _p(sc), _p(ids), K_b * BLK)
    return sc, ids


def attn(q, lat, sel, win, q_pos, sink, W, scale, lat_scale=None, win_scale=None):
    """Sparse attention over Sel + window with sinks.

    q uint16 [B][Tq][64][512]; lat uint16 [B][N][512] (bf16) or uint8
    [B][N][256] (NVFP4, with lat_scale uint8 [B][N][32]); sel int32
    [B*Tq][K]; win uint16 [B][W_cap][512] (bf16) or uint8 (E4M3, with
    win_scale f32 [B][W_cap]); q_pos int64 [B][Tq]; sink f32 [64].
    Returns (out float64 [B*Tq][64][512], lse float64 [B*Tq][64])."""
    q, sel, q_pos, sink = _c(q, np.uint16), _c(sel, np.int32), _c(q_pos, np.int64), _c(sink, np.float32)
    lat, win = np.ascontiguousarray(lat), np.ascontiguousarray(win)
    B, Tq = q.shape[:2]
    assert q.shape == (B, Tq, HQ, D) and sink.shape == (HQ,) and q_pos.shape == (B, Tq)
    assert sel.shape[0] == B * Tq and lat.shape[0] == B and win.shape[0] == B
    assert win.shape[2] == (D if win.dtype == np.uint16 else D)
    if lat.dtype != np.uint16:
        assert lat.shape[2] == D // 2 and lat_scale is not None and lat_scale.shape == (B, lat.shape[1], D // 16)
    else:
        assert lat.shape[2] == D
    if win.dtype != np.uint16:
        assert win_scale is not None and win_scale.shape == (B, win.shape[1])
    N = lat.shape[1]
    W_cap = win.shape[1]
    K = sel.shape[1]
    lat_fmt = BF16 if lat.dtype == np.uint16 else NVFP4
    win_fmt = BF16 if win.dtype == np.uint16 else E4M3
    lat_scale = _c(lat_scale, np.uint8)
    win_scale = _c(win_scale, np.float32)
    out = np.zeros((B * Tq, HQ, D), np.float64)
    lse = np.zeros((B * Tq, HQ), np.float64)
    lib().csa2ref_attn(B, Tq, _p(q), Tq * HQ * D, _p(lat), lat_fmt, _p(lat_scale), N, N,
                       _p(sel), K, K, _p(win), win_fmt, _p(win_scale), W, W_cap, W_cap,
                       _p(q_pos), _p(sink), float(scale), _p(out), _p(lse))
    return out, lse


def dequant_fp8(src, row_scale=None):
    src = _c(src, np.uint8)
    rows, cols = src.shape
    row_scale = _c(row_scale, np.float32)
    dst = np.zeros((rows, cols), np.float64)
    lib().csa2ref_dequant_fp8(_p(src), _p(row_scale), rows, cols, _p(dst))
    return dst


def dequant_nvfp4(packed, scales):
    packed, scales = _c(packed, np.uint8), _c(scales, np.uint8)
    rows = packed.shape[0]
    cols = packed.shape[1] * 2
    dst = np.zeros((rows, cols), np.float64)
    lib().csa2ref_dequant_nvfp4(_p(packed), _p(scales), rows, cols, _p(dst))
    return dst


# ------------------------------------------------- f1: NVFP4 cache writes
def quant_scale_e4m3(amax) -> int:
    return lib().csa2ref_quant_scale_e4m3(float(amax))


def quant_e2m1(x, scale_code) -> int:
    return lib().csa2ref_quant_e2m1(float(x), int(scale_code))


def quant_nvfp4(x):
    """x: float32 [rows][cols] (cols % 16 == 0) -> (packed uint8 [rows][cols/2],
    scales uint8 [rows][cols/16]): nearest E4M3 scale to amax/6 per group of
    16, nearest E2M1 code to x/scale, ties to even (NVFP4 article 3.2)."""
    x = _c(x, np.float32)
    rows, cols = x.shape
    assert cols % 16 == 0
    packed = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 16), np.uint8)
    lib().csa2ref_quant_nvfp4(_p(x), rows, cols, _p(packed), _p(scales))
    return packed, scales


def compress_nvfp4(raw: np.ndarray, gate: np.ndarray):
    """The compressor writing the NVFP4 cache: the pooled value (exact up to
    double rounding) rounded once to fp32, then quantised as quant_nvfp4.
    Returns (packed [B][T/2][256], scales [B][T/2][32], pooled float64)."""
    _, out64 = compress(raw, gate)
    B, G, _ = out64.shape
    packed, scales = quant_nvfp4(out64.astype(np.float32).reshape(B * G, D))
    return packed.reshape(B, G, D // 2), scales.reshape(B, G, D // 16), out64


def compress_decode(state, kv_tok, gate_tok, pos, cache, n_cache, fmt="bf16"):
    """One decode step of the compressor with its carried state (NVFP4
    article 3.2: the unfinished half of a group waits in state; a latent is
    emitted once both tokens of its group are there).

    state : uint16 [B][2][512], the pending (kv, gate) token of each sequence,
            updated in place;  kv_tok, gate_tok : uint16 [B][512], the new
            token at raw position pos[b] (negative = no token).
    An even position only stores the token.  An odd position t pools the
    stored token with the new one into latent t//2 of ``cache``, if that row
    is below n_cache.  cache: fmt "bf16" -> uint16 [B][rows][512];
    fmt "nvfp4" -> (packed uint8 [B][rows][256], scales uint8 [B][rows][32]).
    """
    B = kv_tok.shape[0]
    for b in range(B):
        t = int(pos[b])
        if t < 0:
            continue
        if t % 2 == 0:
            state[b, 0] = kv_tok[b]
            state[b, 1] = gate_tok[b]
            continue
        g = t // 2
        if g >= n_cache:
            continue
        raw = np.stack([state[b, 0], kv_tok[b]])[None]
        gate = np.stack([state[b, 1], gate_tok[b]])[None]
        if fmt == "bf16":
            out, _ = compress(raw, gate)
            cache[b, g] = out[0, 0]
        else:
            packed, scales, _ = compress_nvfp4(raw, gate)
            cache[0][b, g] = packed[0, 0]
            cache[1][b, g] = scales[0, 0]


# --------------------------------------------------------------- pipeline
def decode(inp: dict, K_b: int, K: int, W: int, scale: float, compress_first=False):
    """Run the whole hot path on host arrays, step by step as the method
    states it (NVFP4 article section 3 call tree):
      [compressor] -> candidate-source scan + block max -> block top-K_b with
      the newest block kept -> current indexer over the candidates ->
      position top-K -> attention over Sel + window with sinks.

    ``inp`` holds numpy arrays keyed as the input generator names them
    (q, sink, qs, ws, ks, qi, wi, ki, lat, lat_scale, win, win_scale, q_pos,
    raw, gate) plus ``comp_pos0`` when ``compress_first``, and tok_kv,
    tok_gate, state, step_pos for a compressor decode step, which runs
    first whenever they are present.  Returns a dict of every
    intermediate."""
    res = {}
    lat = inp["lat"]
    if compress_first:
        comp_bits, comp64 = compress(inp["raw"], inp["gate"])
        g0 = inp["comp_pos0"] // 2
        lat = lat.copy()
        lat[:, g0:g0 + comp_bits.shape[1]] = comp_bits
        res["comp"], res["comp64"] = comp_bits, comp64
    lat_scale = inp.get("lat_scale")
    if inp.get("tok_kv") is not None:
        # the compressor's decode step completes a pair and writes its latent
        state = inp["state"].copy()
        lat = lat.copy()
        if lat_scale is not None:
            lat_scale = lat_scale.copy()
            cache, fmt = (lat, lat_scale), "nvfp4"
        else:
            cache, fmt = lat, "bf16"
        compress_decode(state, inp["tok_kv"], inp["tok_gate"], inp["step_pos"], cache,
                        lat.shape[1], fmt)
    res["lat"], res["lat_scale"] = lat, lat_scale
    q_pos = inp["q_pos"]
    B, Tq = q_pos.shape
    N = lat.shape[1]
    ks = (inp["ks"], inp["ks_scale"]) if inp.get("ks_scale") is not None else inp["ks"]
    ki = (inp["ki"], inp["ki_scale"]) if inp.get("ki_scale") is not None else inp["ki"]
    _, bm = scan(inp["qs"], inp["ws"], ks, q_pos)
    forced = np.array([newest_block(t, N) for t in q_pos.reshape(-1)], np.int32)
    blocks = select(bm, K_b, forced=forced)
    csc, cid = cand(inp["qi"], inp["wi"], ki, q_pos, blocks)
    sel = select(csc, K, ids=cid)
    out, lse = attn(inp["q"], lat, sel, inp["win"], q_pos, inp["sink"], W, scale,
                    lat_scale=lat_scale, win_scale=inp.get("win_scale"))
    res.update(block_max=bm, forced=forced, blocks=blocks, cand_scores=csc,
               cand_ids=cid, sel=sel, out=out, lse=lse)
    return res
