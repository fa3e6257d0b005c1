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
    path = api.DecodePath(cfg.B, cfg.Tq, cfg.N, cfg.K_b, cfg.K, cfg.W)
    path.run(inp, cfg.scale, compress_first=compress_first)
    torch.cuda.synchronize()
    return path


def oracle_path(inp_np, cfg, compress_first=True):
    return ref.decode(inp_np, cfg.K_b, cfg.K, cfg.W, cfg.scale, compress_first=compress_first)
