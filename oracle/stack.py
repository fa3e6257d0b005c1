"""Oracle for one decode step through a stack of layers that share index
results and compressed caches.

TEST INFRASTRUCTURE ONLY (imported by the tests, never by the product path).

The NVFP4 article (lpnh.cn/news/2752702) describes the sharing:
  * section 3.3: the block-level stage runs once per token, at the
    candidate-source layer; 8 index source layers run the position-level
    indexer over those candidate blocks and publish their top-512; the other
    layers reuse a published top-512;
  * section 4: 4 KV source layers store the compressed cache; the other
    layers read a source layer's cache through a shared handle;
  * section 3.2: layers 0 and 1 have compression ratio 0, i.e. they attend to
    their sliding window only.
The pages give the layer ids (index sources 2, 8, 14, 20, 24, 28, 32, 36;
KV sources 2, 8, 14, 20; the oQ3e config walkthrough, nxmr.cn/news/161930,
section 2.1/2.2, lists the same), not which source a given layer reads.
Reading taken here: a layer reads the Sel of the most recent index source
layer at or before it, and the cache of the most recent KV source layer at
or before it.  The steps themselves are the oracle's single-layer steps
(csa2_ref.scan / select / cand / attn).
"""
from __future__ import annotations

import numpy as np

from oracle import csa2_ref as ref

# layer ids printed by the pages (see the module docstring)
LAYERS = 40
WINDOW_ONLY = (0, 1)
INDEX_SOURCES = (2, 8, 14, 20, 24, 28, 32, 36)
KV_SOURCES = (2, 8, 14, 20)
CANDIDATE_SOURCE = 20


def latest_at_or_before(layer: int, sources) -> int:
    """The largest source id <= layer, or -1 when there is none."""
    ok = [s for s in sources if s <= layer]
    return max(ok) if ok else -1


def route(layer: int, index_sources=INDEX_SOURCES, kv_sources=KV_SOURCES,
          window_only=WINDOW_ONLY):
    """(index source layer, KV source layer) that ``layer`` reads, or None
    for a window-only layer."""
    if layer in window_only:
        return None
    return latest_at_or_before(layer, index_sources), latest_at_or_before(layer, kv_sources)


def stack_decode(inp: dict, K_b: int, K: int, W: int, scale: float):
    """One token's pass through the stack, on host arrays.

    inp: q_pos int64 [B][Tq]; the candidate-source indexer qs, ws, ks; per
    index source layer s: qi[s], wi[s], ki[s]; per KV source layer s: lat[s]
    (bf16 bits [B][N][512]); per layer l: q[l], win[l], sink[l]; and the
    stack's shape: layers, window_only, index_sources, kv_sources.
    Returns dict(blocks, sel={s: ...}, out=[per layer], lse=[per layer])."""
    q_pos = inp["q_pos"]
    B, Tq = q_pos.shape
    N = next(iter(inp["lat"].values())).shape[1]
    _, bm = ref.scan(inp["qs"], inp["ws"], inp["ks"], q_pos)
    forced = np.array([ref.newest_block(t, N) for t in q_pos.reshape(-1)], np.int32)
    blocks = ref.select(bm, K_b, forced=forced)
    sel = {}
    for s in inp["index_sources"]:
        cs, ci = ref.cand(inp["qi"][s], inp["wi"][s], inp["ki"][s], q_pos, blocks)
        sel[s] = ref.select(cs, K, ids=ci)
    outs, lses = [], []
    for layer in range(inp["layers"]):
        src = route(layer, inp["index_sources"], inp["kv_sources"], inp["window_only"])
        if src is None:
            # no compressed latents: the window (and the sink) only
            lat = np.zeros((B, 1, 512), np.uint16)
            sl = np.zeros((B * Tq, 0), np.int32)
        else:
            lat, sl = inp["lat"][src[1]], sel[src[0]]
        o, l = ref.attn(inp["q"][layer], lat, sl, inp["win"][layer], q_pos, inp["sink"][layer],
                        W, scale)
        outs.append(o)
        lses.append(l)
    return dict(block_max=bm, blocks=blocks, sel=sel, out=outs, lse=lses)
