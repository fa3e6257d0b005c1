"""The allocation-free attention entry point (csa2_sparse_attn_noalloc),
called through the C ABI, against the workspace entry point
(csa2_sparse_attn) on the same inputs: two calls in a row, the second with a
smaller input (fewer queries, NVFP4 latents and an FP8 window), each
bit-identical to the workspace call (same kernels, same split of the rows)
and within the parity bar of the oracle."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_03_amd import _lib, api, gen
from oracle import csa2_ref as ref
from tests.gpu_util import BF16_TOL, LOWP_TOL, bf16_to_np, check_close, np_subset, say

pytestmark = pytest.mark.gpu


def _sel(cfg, host, seed):
    rng = np.random.default_rng(seed)
    sel = np.full((cfg.R, cfg.K), -1, np.int32)
    for r in range(cfg.R):
        nv = ref.n_vis(int(host["q_pos"].reshape(-1)[r]), cfg.N)
        m = min(cfg.K, nv) - (r % 3) * 5
        sel[r, :m] = np.sort(rng.choice(nv, m, replace=False))
    return sel


def _one_call(name, kw, tol):
    cfg = gen.shrink(gen.CONFIGS[name], **kw)
    say(f"[noalloc] {cfg.name}: B={cfg.B} Tq={cfg.Tq} N={cfg.N} K={cfg.K} lat={cfg.lat_fmt} "
        f"win={cfg.win_fmt} seed={cfg.seed}")
    inp = gen.make_inputs(cfg, device="cuda")
    host = np_subset(inp)
    sel = _sel(cfg, host, cfg.seed)
    sel_t = torch.from_numpy(sel).cuda()
    R = cfg.R
    need = api.workspace_bytes(_lib.OP_SPARSE_ATTN, R, cfg.K, cfg.W)
    assert 0 < need <= _lib.ATTN_SCRATCH_BYTES
    ws = torch.empty((need // 4 + 4,), dtype=torch.float32, device="cuda")
    out_ws = torch.empty((R, 64, 512), dtype=torch.bfloat16, device="cuda")
    lse_ws = torch.empty((R, 64), dtype=torch.float32, device="cuda")
    api.sparse_attn(inp["q"], inp["lat"], sel_t, inp["win"], inp["q_pos"], inp["sink"], cfg.W,
                    cfg.scale, out_ws, lat_scale=inp["lat_scale"], win_scale=inp["win_scale"],
                    lse=lse_ws, ws=ws)
    out_na = torch.full((R, 64, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse_na = torch.full((R, 64), float("nan"), dtype=torch.float32, device="cuda")
    api.sparse_attn_noalloc(inp["q"], inp["lat"], sel_t, inp["win"], inp["q_pos"], inp["sink"],
                            cfg.W, cfg.scale, out_na, lat_scale=inp["lat_scale"],
                            win_scale=inp["win_scale"], lse=lse_na)
    torch.cuda.synchronize()
    assert torch.equal(out_na, out_ws), "no-alloc output differs from the workspace call's"
    assert torch.equal(lse_na, lse_ws), "no-alloc lse differs from the workspace call's"
    o_ref, lse_ref = ref.attn(host["q"], host["lat"], sel, host["win"], host["q_pos"], host["sink"],
                              cfg.W, cfg.scale, lat_scale=host["lat_scale"],
                              win_scale=host["win_scale"])
    check_close("no-alloc attention out", bf16_to_np(out_na).reshape(o_ref.shape), o_ref, tol)
    assert np.abs(lse_na.cpu().numpy() - lse_ref).max() < 2e-3
    return need


def test_noalloc_matches_workspace_call_twice():
    n1 = _one_call("1m", dict(B=8, N=8192, t_last=16383, K_b=64, win_pos0=16383 - 127, seed=140),
                   BF16_TOL)
    n2 = _one_call("1m_lowp", dict(B=3, N=4096, t_last=8191, K_b=64, K=256, seed=141), LOWP_TOL)
    assert n2 < n1  # the second call is the smaller one
    say(f"  partials: {n1} then {n2} bytes in the shared scratch; outputs bit-identical")


def test_noalloc_refuses_partials_beyond_the_scratch():
    cfg = gen.shrink(gen.CONFIGS["1m_lowp"], B=40, N=1024, t_last=2047, K_b=16, seed=142)
    inp = gen.make_inputs(cfg, device="cuda")
    sel = torch.zeros((cfg.R, cfg.K), dtype=torch.int32, device="cuda")
    out = torch.full((cfg.R, 64, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(_lib.Csa2Error) as e:
        api.sparse_attn_noalloc(inp["q"], inp["lat"], sel, inp["win"], inp["q_pos"], inp["sink"],
                                cfg.W, cfg.scale, out, lat_scale=inp["lat_scale"],
                                win_scale=inp["win_scale"])
    assert e.value.status == _lib.EWORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a refused call wrote its output"
