"""The whole pass captured in a HIP graph:
every replay reproduces the eager pass bit for bit, also after other eager
work has overwritten every buffer the pass writes.  No input or expected
value here comes from the oracle: the reference is the eager pass, whose own
parity with the oracle is checked elsewhere."""
import pytest
import torch

from compressed_sparse_attention_03_amd import api, gen
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

BUFFERS = ("block_max", "blocks", "cand_scores", "cand_ids", "sel", "out", "lse")


@pytest.mark.parametrize("name,kw", [
    ("128k", dict(B=4, N=20480, t_last=40959, comp_pos0=40960 - 256, win_pos0=40959 - 127,
                  seed=70)),
    ("1m_lowp", dict(B=3, N=8192, t_last=16383, K_b=128, win_pos0=16383 - 127, seed=71)),
])
def test_graph_replay_matches_eager(name, kw):
    cfg = gen.shrink(gen.CONFIGS[name], **kw)
    say(f"[graph] {name}: B={cfg.B} N={cfg.N} comp_T={cfg.comp_T} seed={cfg.seed}")
    inp = gen.make_inputs(cfg, device="cuda")
    comp = cfg.comp_T > 0
    path = api.DecodePath(cfg.B, cfg.Tq, cfg.N, cfg.K_b, cfg.K, cfg.W)
    path.run(inp, cfg.scale, compress_first=comp)
    torch.cuda.synchronize()
    ref = {k: getattr(path, k).clone() for k in BUFFERS}
    lat_ref = inp["lat"].clone()
    graph = path.capture(inp, cfg.scale, compress_first=comp)
    for rep in range(3):
        # eager work between replays: scribble over everything the pass writes
        for k in BUFFERS:
            getattr(path, k).fill_(-7 - rep)
        if comp:
            g0 = cfg.comp_pos0 // 2
            inp["lat"][:, g0:g0 + cfg.comp_T // 2].fill_(3.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in BUFFERS:
            assert torch.equal(getattr(path, k), ref[k]), f"replay {rep}: {k}"
        assert torch.equal(inp["lat"], lat_ref), f"replay {rep}: latent cache"
    say(f"  3 replays bit-identical to the eager pass")
    del graph, path, inp
    torch.cuda.empty_cache()
