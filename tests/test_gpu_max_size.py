"""GPU parity at the largest cache the indexer accepts: 2^27 latents of one
sequence (32 GiB of bf16 index keys, 2^24 blocks of 8), the limit that
csa2_index_scores, csa2_select_topk and csa2_gather_select check.  Key byte
offsets pass 2^32 here and key positions reach 2^27 - 1, so every 64-bit
offset computation of the scan, candidate and top-k kernels runs at its
maximum.

One cache serves three passes over it:
- the decode chain for one query (t = 2^28 - 1, everything visible): the
  scan's block maxima, the block top-2048 over the 2^24 maxima with the
  newest block kept, the candidate indexer over the chosen blocks and the
  position top-512;
- the verification scan (5 draft queries) and the prefill scan (64
  consecutive queries whose horizons end inside the last four blocks).

The oracle scores compact copies of the rows it needs: sampled blocks
spread over the whole cache (first, last, around 2^21, 2^23 and 2^24 - 1,
and seeded random ones) plus the cache's last 64 rows, with each query's
horizon mapped into the compact array.  The block top-k is checked on the
full row of block maxima, the candidate scores bit-exactly over all 16,384
candidates.  Inputs are the integer-valued index queries and keys in
[-3, 3] and head weights k/16 of the other configs; skipped when the GPU
has less than 40 GiB free.

FP8 E4M3 and MXFP4 index keys get the same size: the FP8 decode scan (1
and 5 queries) and the prefill scans of both formats (64 queries), checked
at sampled blocks and the last blocks.

The prefill's fused candidate gather + position top-512 reads a score
matrix of 2 rows x 2^27 latents (few rows: one workgroup per row) and of
1100 rows x 2^22 latents (the many-rows kernel, row offsets past 16 GiB),
block ids spread up to the last block and past the cache.

The compressor (bf16 and NVFP4 rows) runs once over 2^23 + 2 raw tokens of
one sequence (8 GiB each of tokens and gate logits, byte offsets past 2^33),
checked at sampled latents and the last one against the oracle's pooling of
the same token pairs.
"""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_03_amd import api, gen
from oracle import csa2_ref as ref
from tests.gpu_util import BF16_TOL, check_close, check_fp4_pooling, say

pytestmark = pytest.mark.gpu

N = 1 << 27          # latents: the indexer's limit (2^24 blocks of 8)
NB = N // 8
HI, DI = 32, 128
K_B, K = 2048, 512
TAIL = 64            # the cache's last rows, copied whole to the oracle
CHUNK_ROWS = 1 << 21


def _keys(g):
    k = torch.empty((1, N, DI), dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, N, CHUNK_ROWS):
        k[0, r0:r0 + CHUNK_ROWS] = torch.randint(-3, 4, (CHUNK_ROWS, DI), generator=g, device="cuda",
                                                 dtype=torch.int32).to(torch.bfloat16)
    return k


def _queries(g, tq):
    q = torch.randint(-3, 4, (1, tq, HI, DI), generator=g, device="cuda",
                      dtype=torch.int32).to(torch.bfloat16)
    w = torch.randint(1, 17, (1, tq, HI), generator=g, device="cuda",
                      dtype=torch.int32).to(torch.float32) / 16.0
    return q, w


def _sample_blocks(rng, count):
    fixed = [0, 1, 2, (1 << 21) - 1, 1 << 21, (1 << 23) + 5, (1 << 24) - 9, NB - TAIL // 8 - 1]
    rnd = rng.choice(NB - TAIL // 8, size=count - len(fixed), replace=False)
    return np.unique(np.concatenate([np.array(fixed, np.int64), rnd.astype(np.int64)]))


def _compact(keys, blocks):
    """Host copies of the rows of `blocks`, then the cache's last TAIL rows
    ([1][8*len(blocks)+TAIL][...]); an MXFP4 (codes, scales) pair gives a pair."""
    if isinstance(keys, tuple):
        return tuple(_compact(k, blocks) for k in keys)
    rows = (torch.from_numpy(blocks).cuda()[:, None] * 8 + torch.arange(8, device="cuda")).reshape(-1)
    inner = keys[0].index_select(0, rows)
    tail = keys[0, N - TAIL:]
    return gen.to_numpy(torch.cat([inner, tail]))[None]


def _check_block_max(name, keys, q, w, q_pos, bm, blocks):
    """Block maxima of sampled blocks and of the last TAIL/8 blocks against
    the oracle on the compact rows; each query's horizon is mapped so that
    the same rows of the tail stay visible."""
    kc = _compact(keys, blocks)
    n_in = 8 * len(blocks)
    n_vis = np.minimum(N, (q_pos.cpu().numpy() + 1) // 2)      # [1][Tq]
    assert np.all(n_vis >= N - TAIL)
    qp_c = 2 * (n_in + TAIL - (N - n_vis)) - 1                   # the same rows visible
    _, bm_ref = ref.scan(gen.to_numpy(q), gen.to_numpy(w), kc, qp_c)
    want = np.concatenate([blocks, np.arange(NB - TAIL // 8, NB)])
    got = bm[:, torch.from_numpy(want).cuda()].cpu().numpy().astype(np.float64)
    assert np.array_equal(got, bm_ref), f"{name}: block maxima"
    say(f"  {name}: block maxima of {len(want)} blocks x {bm.shape[0]} queries bit-exact")


@pytest.fixture(scope="module")
def cache():
    free, _ = torch.cuda.mem_get_info()
    if free < (40 << 30):
        pytest.skip(f"needs 40 GiB of free GPU memory, {free >> 30} GiB free")
    say(f"[gen] max-size cache: 1 sequence x {N} bf16 index keys ({N * DI * 2 >> 30} GiB)")
    g = torch.Generator(device="cuda")
    g.manual_seed(2027)
    keys = _keys(g)
    torch.cuda.synchronize()
    yield g, keys
    del keys
    torch.cuda.empty_cache()


def test_max_cache_decode_chain(cache):
    g, keys = cache
    rng = np.random.default_rng(7)
    q, w = _queries(g, 1)
    t = 2 * N - 1
    q_pos = torch.full((1, 1), t, dtype=torch.int64, device="cuda")
    bm = torch.empty((1, NB), dtype=torch.float32, device="cuda")
    say("[run] scan, block top-2048, candidate indexer, position top-512 at 2^27 latents")
    api.index_scan(q, w, keys, q_pos, block_max=bm)
    blocks = torch.empty((1, K_B), dtype=torch.int32, device="cuda")
    api.select_topk(bm, K_B, blocks, force_last=True)
    csc = torch.empty((1, K_B * 8), dtype=torch.float32, device="cuda")
    cid = torch.empty((1, K_B * 8), dtype=torch.int32, device="cuda")
    api.index_cand(q, w, keys, q_pos, blocks, csc, cid)
    sel = torch.empty((1, K), dtype=torch.int32, device="cuda")
    api.select_topk(csc, K, sel, ids=cid)
    torch.cuda.synchronize()

    _check_block_max("decode scan", keys, q, w, q_pos, bm, _sample_blocks(rng, 512))

    # the block stage over the whole row of 2^24 maxima
    bm_h = bm.cpu().numpy().astype(np.float64)
    blk_ref = ref.select(bm_h, K_B, forced=np.array([ref.newest_block(t, N)], np.int32))
    blk = blocks.cpu().numpy()
    assert np.array_equal(blk, blk_ref), "block selection"
    assert blk[0, -1] == NB - 1
    say(f"  block top-{K_B} of {NB} bit-exact (largest ids {blk[0, -3:].tolist()})")

    # the candidates: the chosen blocks' rows in their order, all visible
    kc = _compact(keys, blk[0].astype(np.int64))[:, :K_B * 8]  # the tail rows dropped
    qp_c = np.array([[2 * K_B * 8 - 1]], np.int64)
    csc_ref, cid_c = ref.cand(gen.to_numpy(q), gen.to_numpy(w), kc, qp_c,
                              np.arange(K_B, dtype=np.int32)[None])
    cid_ref = np.where(cid_c >= 0, blk[0][cid_c // 8].astype(np.int64) * 8 + cid_c % 8, -1)
    assert np.array_equal(cid.cpu().numpy().astype(np.int64), cid_ref), "candidate ids"
    assert np.array_equal(csc.cpu().numpy().astype(np.float64), csc_ref), "candidate scores"

    sel_ref = ref.select(csc.cpu().numpy().astype(np.float64), K, ids=cid.cpu().numpy())
    assert np.array_equal(sel.cpu().numpy(), sel_ref), "position selection"
    say(f"  {K_B * 8} candidate scores and the top-{K} positions bit-exact "
        f"(largest {sel_ref[0, -2:].tolist()})")


@pytest.mark.parametrize("tq", [5, 64])
def test_max_cache_multi_query_scan(cache, tq):
    """tq = 5: the verification scan; tq = 64: the prefill scan (4-wave
    blocks, 8 key ranges of 2^24 keys)."""
    g, keys = cache
    rng = np.random.default_rng(100 + tq)
    q, w = _queries(g, tq)
    # horizons N - 32 + (j + 1) // 2: the last four blocks partly visible
    q_pos = torch.arange(2 * N - 64, 2 * N - 64 + tq, dtype=torch.int64, device="cuda")[None]
    bm = torch.empty((tq, NB), dtype=torch.float32, device="cuda")
    say(f"[run] scan of {tq} queries at 2^27 latents")
    api.index_scan(q, w, keys, q_pos, block_max=bm)
    torch.cuda.synchronize()
    _check_block_max(f"scan, {tq} queries", keys, q, w, q_pos, bm, _sample_blocks(rng, 256))


T_BIG = (1 << 23) + 2   # raw tokens: 2^22 + 1 latents


def _normal_rows(g, rows):
    x = torch.empty((1, rows, 512), dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, rows, CHUNK_ROWS):
        r1 = min(rows, r0 + CHUNK_ROWS)
        x[0, r0:r1] = torch.randn((r1 - r0, 512), generator=g, device="cuda").to(torch.bfloat16)
    return x


def test_large_compress():
    free, _ = torch.cuda.mem_get_info()
    if free < (30 << 30):
        pytest.skip(f"needs 30 GiB of free GPU memory, {free >> 30} GiB free")
    G = T_BIG // 2
    g = torch.Generator(device="cuda")
    g.manual_seed(2029)
    say(f"[gen] compressor input: 1 sequence x {T_BIG} raw tokens (2 x {T_BIG * 1024 >> 30} GiB)")
    raw, gate = _normal_rows(g, T_BIG), _normal_rows(g, T_BIG)
    out = torch.empty((1, G, 512), dtype=torch.bfloat16, device="cuda")
    codes = torch.empty((1, G, 256), dtype=torch.uint8, device="cuda")
    scales = torch.empty((1, G, 32), dtype=torch.uint8, device="cuda")
    say("[run] compress (bf16 rows) and compress_nvfp4 over 2^22 + 1 latents")
    api.compress(raw, gate, out)
    api.compress_nvfp4(raw, gate, codes, scales)
    torch.cuda.synchronize()

    rng = np.random.default_rng(11)
    lat = np.unique(np.concatenate([[0, 1, (1 << 21) + 3, (1 << 22) - 1, G - 1],
                                    rng.choice(G, 507, replace=False)])).astype(np.int64)
    li = torch.from_numpy(lat).cuda()
    pairs = (li[:, None] * 2 + torch.arange(2, device="cuda")).reshape(-1)
    raw_h = gen.to_numpy(raw[0].index_select(0, pairs))[None]
    gate_h = gen.to_numpy(gate[0].index_select(0, pairs))[None]
    del raw, gate
    bits, y64 = ref.compress(raw_h, gate_h)
    got = out[0].index_select(0, li).float().cpu().numpy().astype(np.float64)[None]
    check_close("compress at 2^22 + 1 latents", got, y64, BF16_TOL)
    x = ref.bf16_array(raw_h).reshape(1, len(lat), 2, 512)
    slack = 1e-6 * (np.abs(x[:, :, 0]) + np.abs(x[:, :, 1]))
    assert np.all(np.abs(got - y64) <= np.abs(y64) * 2 ** -8 + slack)
    nd = check_fp4_pooling("compress_nvfp4 at 2^22 + 1 latents",
                           codes[0].index_select(0, li).cpu().numpy()[None],
                           scales[0].index_select(0, li).cpu().numpy()[None], raw_h, gate_h)
    assert sum(nd) <= max(1, len(lat) * 512 // 100000)
    say(f"  {len(lat)} sampled latents (last {int(lat[-1])}) within one bf16 rounding; NVFP4 rows as the oracle's")


def _lowp_keys(g, fmt):
    if fmt == "fp8":
        k = torch.empty((1, N, DI), dtype=torch.uint8, device="cuda")
        for r0 in range(0, N, CHUNK_ROWS):
            x = torch.randint(-3, 4, (CHUNK_ROWS, DI), generator=g, device="cuda", dtype=torch.int32)
            k[0, r0:r0 + CHUNK_ROWS] = x.to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)
        return k, None
    codes = torch.empty((1, N, DI // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((1, N, DI // 32), dtype=torch.uint8, device="cuda")
    for r0 in range(0, N, CHUNK_ROWS):
        codes[0, r0:r0 + CHUNK_ROWS] = torch.randint(0, 256, (CHUNK_ROWS, DI // 2), generator=g,
                                                     device="cuda", dtype=torch.int32).to(torch.uint8)
        scales[0, r0:r0 + CHUNK_ROWS] = torch.randint(126, 128, (CHUNK_ROWS, DI // 32), generator=g,
                                                      device="cuda", dtype=torch.int32).to(torch.uint8)
    return codes, scales


@pytest.mark.parametrize("fmt,tqs", [("fp8", (1, 5, 64)), ("mxfp4", (64,))])
def test_max_cache_lowp_scan(fmt, tqs):
    """FP8 keys (E4M3 codes, the decode scan for 1 and 5 queries and the
    prefill scan) and MXFP4 keys (E2M1 codes with E8M0 scales 2^-1 / 2^0,
    the prefill scan) over 2^27 latents."""
    free, _ = torch.cuda.mem_get_info()
    if free < (24 << 30):
        pytest.skip(f"needs 24 GiB of free GPU memory, {free >> 30} GiB free")
    g = torch.Generator(device="cuda")
    g.manual_seed(2031 if fmt == "fp8" else 2033)
    say(f"[gen] max-size cache: 1 sequence x {N} {fmt} index keys")
    k, k_scale = _lowp_keys(g, fmt)
    keys = k if k_scale is None else (k, k_scale)
    rng = np.random.default_rng(300)
    for tq in tqs:
        q, w = _queries(g, tq)
        q_pos = torch.arange(2 * N - 64, 2 * N - 64 + tq, dtype=torch.int64, device="cuda")[None]
        bm = torch.empty((tq, NB), dtype=torch.float32, device="cuda")
        say(f"[run] {fmt} scan of {tq} queries at 2^27 latents")
        api.index_scan(q, w, k, q_pos, block_max=bm, k_scale=k_scale)
        torch.cuda.synchronize()
        _check_block_max(f"{fmt} scan, {tq} queries", keys, q, w, q_pos, bm, _sample_blocks(rng, 256))
    del k, k_scale, keys
    torch.cuda.empty_cache()


@pytest.mark.parametrize("R,n,seed", [(2, N, 80), (1100, 1 << 22, 81)])
def test_max_gather_select(R, n, seed):
    """The one-pass gather + position top-k over a large score matrix equals
    gather_scores + select_topk and the oracle's selection over the same
    candidates (gathered on the host from the same scores)."""
    free, _ = torch.cuda.mem_get_info()
    if free < R * n * 4 + (4 << 30):
        pytest.skip(f"needs {(R * n * 4 >> 30) + 4} GiB of free GPU memory, {free >> 30} GiB free")
    rng = np.random.default_rng(seed)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    say(f"[gen] score matrix {R} x {n} ({R * n * 4 >> 30} GiB)")
    all_s = torch.empty((R, n), dtype=torch.float32, device="cuda")
    step = max(1, (1 << 26) // n)
    for r0 in range(0, R, step):
        r1 = min(R, r0 + step)
        all_s[r0:r1] = torch.randint(0, 60, (r1 - r0, n), generator=g, device="cuda",
                                     dtype=torch.int32).to(torch.float32) / 16.0
    nblk = n // 8
    kb, k = 2048, 512
    blocks = np.full((R, kb), -1, np.int32)
    for r in range(R):
        m = int(rng.integers(kb // 2, kb + 1)) - 4
        pick = np.unique(np.concatenate([rng.integers(0, nblk, m), [0, nblk - 1]]))
        blocks[r, :len(pick)] = pick
        blocks[r, len(pick):len(pick) + 3] = [1 << 28, 1 << 30, 2**31 - 1]  # past the cache
    # horizons: most rows see everything, some end inside the last blocks
    q_pos = np.where(rng.random(R) < 0.7, 2 * n - 1, 2 * n - 1 - rng.integers(0, 200, R)).astype(np.int64)
    qp = torch.from_numpy(q_pos[None]).cuda()
    b_t = torch.from_numpy(blocks).cuda()
    say(f"[run] gather + top-{k} of {kb} blocks per row over {R} x {n} scores")
    fused = torch.full((R, k), -7, dtype=torch.int32, device="cuda")
    api.gather_select(all_s, qp, b_t, k, fused, n_cache=n)
    sc = torch.empty((R, kb * 8), dtype=torch.float32, device="cuda")
    ids = torch.empty((R, kb * 8), dtype=torch.int32, device="cuda")
    api.gather_scores(all_s, qp, b_t, sc, ids, n_cache=n)
    two = torch.empty((R, k), dtype=torch.int32, device="cuda")
    api.select_topk(sc, k, two, ids=ids)
    torch.cuda.synchronize()
    got = fused.cpu().numpy()
    assert np.array_equal(got, two.cpu().numpy()), "fused != gather + select"
    # oracle: the candidates gathered on the host side of the same scores
    nv = np.minimum((q_pos + 1) // 2, n)
    pos = blocks[:, :, None].astype(np.int64) * 8 + np.arange(8)
    ok = (blocks[:, :, None] >= 0) & (pos < nv[:, None, None])
    vals = torch.gather(all_s, 1, torch.from_numpy(np.clip(pos, 0, n - 1).reshape(R, -1)).cuda())
    cs = np.where(ok.reshape(R, -1), vals.cpu().numpy().astype(np.float64), -np.inf)
    cid = np.where(ok, pos, -1).reshape(R, -1).astype(np.int32)
    assert np.array_equal(got, ref.select(cs, k, ids=cid)), "fused != oracle selection"
    say(f"  gather+select fused at {R} x {n}: bit-exact (largest kept id {int(got.max())})")
    del all_s
    torch.cuda.empty_cache()
