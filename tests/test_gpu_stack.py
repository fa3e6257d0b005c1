"""Layer stack sharing index results and compressed caches (block stage once,
candidate indexer + position top-K per index source layer, attention per
layer): every published Sel bit-exact and every layer's attention output
within tolerance of the oracle composed the same way."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_03_amd import api, gen
from oracle import csa2_ref as ref
from tests.gpu_util import BF16_TOL, bf16_to_np, check_close, say

pytestmark = pytest.mark.gpu


def _np(t):
    return gen.to_numpy(t)


def test_layer_stack_small():
    cfg = gen.shrink(gen.CONFIGS["1m"], B=2, N=5000, t_last=9999, K_b=64, K=128,
                     win_pos0=9999 - 127, seed=80)
    say(f"[stack] B={cfg.B} N={cfg.N} layers=7")
    inp = gen.make_stack_inputs(cfg, layers=7, window_only=(0, 1), index_sources=(2, 4),
                                kv_sources=(2, 5), device="cuda")
    path = api.LayerStackPath(inp, cfg.K_b, cfg.K, cfg.W)
    path.run(inp, cfg.scale)
    torch.cuda.synchronize()

    q_pos = _np(inp["q_pos"])
    _, bm = ref.scan(_np(inp["qs"]), _np(inp["ws"]), _np(inp["ks"]), q_pos)
    forced = np.array([ref.newest_block(t, cfg.N) for t in q_pos.reshape(-1)], np.int32)
    blocks = ref.select(bm, cfg.K_b, forced=forced)
    assert np.array_equal(path.blocks.cpu().numpy(), blocks), "blocks"
    sel = {}
    for s in inp["index_sources"]:
        cs, ci = ref.cand(_np(inp["qi"][s]), _np(inp["wi"][s]), _np(inp["ki"][s]), q_pos, blocks)
        sel[s] = ref.select(cs, cfg.K, ids=ci)
        assert np.array_equal(path.sel[s].cpu().numpy(), sel[s]), f"Sel of index layer {s}"
    for layer in range(inp["layers"]):
        src = path.source_of(layer)
        if src is None:
            lat, sl = _np(inp["lat"][inp["kv_sources"][0]]), np.zeros((cfg.R, 0), np.int32)
        else:
            lat, sl = _np(inp["lat"][src[1]]), sel[src[0]]
        out, lse = ref.attn(_np(inp["q"][layer]), lat, sl, _np(inp["win"][layer]), q_pos,
                            _np(inp["sink"][layer]), cfg.W, cfg.scale)
        check_close(f"layer {layer} out", bf16_to_np(path.out[layer]), out, BF16_TOL)
        assert np.abs(path.lse[layer].cpu().numpy() - lse).max() < 2e-3
    say("  blocks and every Sel bit-exact; 7 layer outputs within tolerance")
