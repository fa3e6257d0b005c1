"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
the CPU oracle on the same bytes, and compare.  No method arithmetic here."""
from __future__ import annotations

import sys

import numpy as np
import torch

from compressed_sparse_attention_03_amd import api, gen
from oracle import csa2_ref as ref

BF16_TOL = 2e-2   # max|err| <= tol * max|ref| (bf16 configs)
LOWP_TOL = 5e-2   # NVFP4 / FP8 config


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np_subset(inp: dict, seqs=None, queries=None) -> dict:
    """Host copies of the inputs of some sequences (batch dim) and/or some
    queries (dim 1 of the per-query tensors)."""
    out = {}
    per_query = {"q", "qs", "ws", "qi", "wi", "q_pos"}
    shared = {"sink"}  # per head, not per sequence
    for k, v in inp.items():
        if k == "cfg":
            continue
        if v is None:
            out[k] = None
            continue
        t = v
        if seqs is not None and k not in shared:
            t = t[list(seqs)]
        if queries is not None and k in per_query:
            t = t[:, list(queries)]
        out[k] = gen.to_numpy(t)
    out["comp_pos0"] = inp["cfg"].comp_pos0
    return out


def rows_of(seqs, Tq, queries=None):
    qs = range(Tq) if queries is None else queries
    return [b * Tq + j for b in seqs for j in qs]


def check_close(name, got, ref_vals, tol):
    got = np.asarray(got, np.float64)
    ref_vals = np.asarray(ref_vals, np.float64)
    err = np.abs(got - ref_vals).max() if got.size else 0.0
    scale = np.abs(ref_vals).max() if ref_vals.size else 0.0
    say(f"  {name}: max|err| = {err:.3e}, max|ref| = {scale:.3e}, ratio = {err / max(scale, 1e-30):.3e}")
    assert np.all(np.isfinite(got)), name
    assert err <= tol * scale + 1e-30, (name, err, scale)


def bf16_to_np(t: torch.Tensor):
    return t.detach().float().cpu().numpy().astype(np.float64)


def valid_sorted(a):
    a = np.asarray(a)
    return a[a >= 0]


def run_gpu_path(inp, compress_first=True):
    cfg = inp["cfg"]
    path = api.DecodePath(cfg.B, cfg.Tq, cfg.N, cfg.K_b, cfg.K, cfg.W, one_indexer=cfg.shared_indexer)
    path.run(inp, cfg.scale, compress_first=compress_first)
    torch.cuda.synchronize()
    return path


def oracle_path(inp_np, cfg, compress_first=True):
    return ref.decode(inp_np, cfg.K_b, cfg.K, cfg.W, cfg.scale, compress_first=compress_first)


# ---- NVFP4 cache rows written by the compressor ---------------------------
_E4M3 = None
_E2M1 = None


def _tables():
    global _E4M3, _E2M1
    if _E4M3 is None:
        _E4M3 = np.array([ref.e4m3(c) for c in range(256)])
        _E2M1 = np.array([ref.e2m1(c) for c in range(16)])
    return _E4M3, _E2M1


def unpack_fp4(packed):
    p = np.asarray(packed)
    return np.stack([p & 15, p >> 4], -1).reshape(*p.shape[:-1], p.shape[-1] * 2)


def check_fp4_pooling(name, got_codes, got_scales, raw, gate):
    """NVFP4 rows from the device compressor against the oracle's.

    The device pools in fp32 (error below 1e-6 * (|x0| + |x1|) per channel)
    and the oracle in double, so a group's scale code or an element's code
    may differ only where the exact pooled value lies within that error of a
    rounding midpoint (scale: amax/6 at an E4M3 midpoint; element: |y| at a
    midpoint between E2M1 magnitudes, times the scale).  Every other code is
    bit-exact, and every element meets the format's error bound under the
    device's own scale.  Returns the number of (scale, element) differences."""
    e4, e2 = _tables()
    packed, scales, y64 = ref.compress_nvfp4(raw, gate)
    B, G, _ = y64.shape
    got_codes = np.asarray(got_codes).reshape(B, G, 256)
    got_scales = np.asarray(got_scales).reshape(B, G, 32)
    x = ref.bf16_array(np.asarray(raw)).reshape(B, G, 2, 512)
    eps = 1e-6 * (np.abs(x[:, :, 0]) + np.abs(x[:, :, 1]))
    eps_g = eps.reshape(B, G, 32, 16).max(-1)
    amax = np.abs(y64).reshape(B, G, 32, 16).max(-1)
    mids = (e4[:0x7E] + e4[1:0x7F]) / 2
    ds = got_scales != scales
    for i in zip(*np.nonzero(ds)):
        near = np.abs(amax[i] / 6 - mids).min() * 6
        assert near <= eps_g[i] * (1 + 1e-9), (name, "scale", i, amax[i], near)
    cg, cr = unpack_fp4(got_codes), unpack_fp4(packed)
    s_ref = np.repeat(e4[scales], 16, axis=-1)
    dc = (cg != cr) & ~np.repeat(ds, 16, axis=-1)
    tmid = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for i in zip(*np.nonzero(dc)):
        near = np.abs(np.abs(y64[i]) - tmid * s_ref[i]).min()
        assert near <= eps[i] * (1 + 1e-9), (name, "code", i, y64[i], s_ref[i])
    s_got = np.repeat(e4[got_scales], 16, axis=-1)
    dq = e2[cg] * s_got
    normal = np.repeat(amax / 6 >= 2.0 ** -6, 16, axis=-1)
    bound = s_got + eps + np.where(normal, 0.0, 6 * 2.0 ** -10)
    assert np.all(np.abs(dq - y64) <= bound), name
    say(f"  {name}: {ds.size} groups, {int(ds.sum())} scale and {int(dc.sum())} element codes "
        f"off the oracle's (all at rounding midpoints); error bound met")
    return int(ds.sum()), int(dc.sum())
