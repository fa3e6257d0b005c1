"""Layer stack sharing index results and compressed caches (block stage once,
candidate indexer + position top-K per index source layer, attention per
layer): every published Sel bit-exact and every layer's attention output
within tolerance of the oracle's own stack composition (oracle.stack), whose
layer routing is the oracle's reading of the pages, not the product's."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_03_amd import api, gen
from oracle import stack as ostack
from tests.gpu_util import BF16_TOL, bf16_to_np, check_close, say

pytestmark = pytest.mark.gpu


def _host(inp):
    out = {}
    for k, v in inp.items():
        if isinstance(v, torch.Tensor):
            out[k] = gen.to_numpy(v)
        elif isinstance(v, dict):
            out[k] = {s: gen.to_numpy(t) for s, t in v.items()}
        elif isinstance(v, list):
            out[k] = [gen.to_numpy(t) for t in v]
        else:
            out[k] = v
    return out


@pytest.mark.parametrize("layers,window_only,index_sources,kv_sources,seed", [
    (7, (0, 1), (2, 4), (2, 5), 80),
    # an index source after a KV source and a KV source after an index source
    (9, (0,), (1, 3, 7), (1, 5), 81),
])
def test_layer_stack_small(layers, window_only, index_sources, kv_sources, seed):
    cfg = gen.shrink(gen.CONFIGS["1m"], B=2, N=5000, t_last=9999, K_b=64, K=128,
                     win_pos0=9999 - 127, seed=seed)
    say(f"[stack] B={cfg.B} N={cfg.N} layers={layers} index={index_sources} kv={kv_sources}")
    inp = gen.make_stack_inputs(cfg, layers=layers, window_only=window_only,
                                index_sources=index_sources, kv_sources=kv_sources, device="cuda")
    path = api.LayerStackPath(inp, cfg.K_b, cfg.K, cfg.W)
    path.run(inp, cfg.scale)
    torch.cuda.synchronize()

    res = ostack.stack_decode(_host(inp), cfg.K_b, cfg.K, cfg.W, cfg.scale)
    assert np.array_equal(path.blocks.cpu().numpy(), res["blocks"]), "blocks"
    for s in index_sources:
        assert np.array_equal(path.sel[s].cpu().numpy(), res["sel"][s]), f"Sel of index layer {s}"
    for layer in range(layers):
        check_close(f"layer {layer} out", bf16_to_np(path.out[layer]), res["out"][layer], BF16_TOL)
        assert np.abs(path.lse[layer].cpu().numpy() - res["lse"][layer]).max() < 2e-3
    say(f"  blocks and every Sel bit-exact; {layers} layer outputs within tolerance")
