"""Python binding of the CSA2 C ABI: torch tensors in, pointers + sizes out.

Argument marshalling only -- every step runs in the HIP kernels of
``libcsa2.so``; torch only provides device memory and the current stream.
Names follow include/csa2.h.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import BF16, F32, FP8_E4M3, MXFP4, NVFP4, SCORES_CAND, SCORES_SCAN, check, lib

D, HQ, HI, DI, BLK = 512, 64, 32, 128, 8


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _rows_contig(t: torch.Tensor, inner: int, name: str):
    """t is [B, rows, inner] (or [B, rows, ...] flattening to inner) with
    contiguous rows; returns (batch stride, row stride) in elements."""
    if t.stride(-1) != 1:
        raise ValueError(f"{name}: innermost dimension must be contiguous")
    return t.stride(0)


def _key_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    raise TypeError(f"unsupported key dtype {t.dtype}")


def workspace_bytes(op: int, R: int, n: int, k: int) -> int:
    return int(lib().csa2_workspace_bytes(op, R, n, k))


def compress(raw: torch.Tensor, gate: torch.Tensor, out: torch.Tensor, stream=None) -> torch.Tensor:
    """a1: raw, gate bf16 [B][T][512] -> out bf16 [B][T/2][512] (may be a cache slice)."""
    B, T, _ = raw.shape
    for t, n in ((raw, "raw"), (gate, "gate"), (out, "out")):
        if t.dtype != torch.bfloat16 or t.stride(-1) != 1 or t.stride(-2) != D:
            raise ValueError(f"compress: {n} must be bf16 with contiguous 512-wide rows")
    check("csa2_compress", lib().csa2_compress(B, T, _p(raw), raw.stride(0), _p(gate), gate.stride(0),
                                               _p(out), out.stride(0), _stream(stream)))
    return out


def compress_nvfp4(raw: torch.Tensor, gate: torch.Tensor, codes: torch.Tensor,
                   scales: torch.Tensor, stream=None):
    """a1 with the NVFP4 epilogue: raw, gate bf16 [B][T][512] -> codes uint8
    [B][rows][256] and E4M3 scales uint8 [B][rows][32] for rows 0..T/2-1 (the
    tensors may be views of a larger cache with the same row stride)."""
    B, T, _ = raw.shape
    for t, n in ((raw, "raw"), (gate, "gate")):
        if t.dtype != torch.bfloat16 or t.stride(-1) != 1 or t.stride(-2) != D:
            raise ValueError(f"compress_nvfp4: {n} must be bf16 with contiguous 512-wide rows")
    sb = _fp4_rows(codes, scales, "compress_nvfp4")
    check("csa2_compress_nvfp4", lib().csa2_compress_nvfp4(
        B, T, _p(raw), raw.stride(0), _p(gate), gate.stride(0), _p(codes), _p(scales), sb,
        _stream(stream)))
    return codes, scales


def _fp4_rows(codes, scales, fn):
    if codes.dtype != torch.uint8 or scales.dtype != torch.uint8:
        raise ValueError(f"{fn}: codes and scales must be uint8")
    if codes.stride(-1) != 1 or codes.stride(-2) != D // 2 or scales.stride(-1) != 1 or \
            scales.stride(-2) != D // 16 or codes.stride(0) // (D // 2) != scales.stride(0) // (D // 16):
        raise ValueError(f"{fn}: codes [B][rows][256] / scales [B][rows][32] need one row stride")
    return codes.stride(0) // (D // 2)


def compress_step(kv: torch.Tensor, gate: torch.Tensor, pos: torch.Tensor, state: torch.Tensor,
                  cache, n_cache: int = None, stream=None):
    """One decode step of the compressor: kv, gate bf16 [B][512] at raw
    positions pos (int64 [B], device; negative = none); state bf16
    [B][2][512] carried between calls.  cache: a bf16 tensor [B][rows][512],
    or a (codes, scales) pair for the NVFP4 cache."""
    B = kv.shape[0]
    if state.dtype != torch.bfloat16 or tuple(state.shape) != (B, 2, D) or not state.is_contiguous():
        raise ValueError("compress_step: state must be contiguous bf16 [B][2][512]")
    if isinstance(cache, tuple):
        codes, scales = cache
        sb = _fp4_rows(codes, scales, "compress_step")
        rows = codes.shape[1] if n_cache is None else n_cache
        args = (NVFP4, _p(codes), _p(scales), sb, rows)
    else:
        if cache.dtype != torch.bfloat16 or cache.stride(-1) != 1 or cache.stride(-2) != D:
            raise ValueError("compress_step: bf16 cache needs contiguous 512-wide rows")
        rows = cache.shape[1] if n_cache is None else n_cache
        args = (BF16, _p(cache), None, cache.stride(0) // D, rows)
    check("csa2_compress_step", lib().csa2_compress_step(
        B, _p(kv), kv.stride(0), _p(gate), gate.stride(0), _p(pos), _p(state), *args,
        _stream(stream)))
    return cache


def quant_nvfp4(src: torch.Tensor, packed=None, scales=None, stream=None):
    """src bf16 or f32 [rows][cols] (contiguous, cols % 16 == 0) -> (packed
    uint8 [rows][cols/2], scales uint8 [rows][cols/16])."""
    rows, cols = src.shape
    if not src.is_contiguous() or src.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("quant_nvfp4: src must be contiguous bf16 or f32")
    if packed is None:
        packed = torch.empty((rows, cols // 2), dtype=torch.uint8, device=src.device)
    if scales is None:
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=src.device)
    dt = F32 if src.dtype == torch.float32 else BF16
    check("csa2_quant_nvfp4", lib().csa2_quant_nvfp4(_p(src), dt, rows, cols, _p(packed),
                                                     _p(scales), _stream(stream)))
    return packed, scales


def index_scan(q, w, k, q_pos, scores=None, block_max=None, k_scale=None, stream=None):
    """a2: indexer scores of every latent and/or per-block maxima.

    q bf16 [B][Tq][32][128], w f32 [B][Tq][32], k [B][N][128] (bf16 or E4M3
    bytes) or, with k_scale (E8M0 bytes [B][N][4]), MXFP4 codes [B][N][64];
    q_pos int64 [B][Tq]; scores f32 [B*Tq][>=N], block_max f32
    [B*Tq][>=ceil(N/8)]."""
    B, Tq = q.shape[:2]
    N = k.shape[1]
    assert q.is_contiguous() and w.is_contiguous() and q_pos.is_contiguous()
    if k_scale is not None:
        if k.dtype != torch.uint8 or k.shape[2] != DI // 2 or tuple(k_scale.shape) != (B, N, DI // 32) \
                or not k_scale.is_contiguous() or k.stride(0) != 16 * k_scale.stride(0):
            raise ValueError("index_scan: MXFP4 keys are uint8 codes [B][N][64] with E8M0 "
                             "scales [B][N][4], scale batch stride = code batch stride / 16")
        k_dt = MXFP4
    else:
        k_dt = _key_dtype(k)
    check("csa2_index_scores", lib().csa2_index_scores(
        SCORES_SCAN, B, Tq, _p(q), BF16, _p(w), _p(k), k_dt, _p(k_scale), _rows_contig(k, DI, "k"), N,
        _p(q_pos), None, 0, _p(scores), scores.stride(0) if scores is not None else 0, None,
        _p(block_max), block_max.stride(0) if block_max is not None else 0, _stream(stream)))
    return scores, block_max


def index_cand(q, w, k, q_pos, blocks, scores, ids, stream=None):
    """a4: scores of the latents of the chosen blocks (blocks int32 [B*Tq][K_b])."""
    B, Tq = q.shape[:2]
    N = k.shape[1]
    K_b = blocks.shape[1]
    assert q.is_contiguous() and w.is_contiguous() and q_pos.is_contiguous() and blocks.is_contiguous()
    assert scores.stride(0) == ids.stride(0)
    check("csa2_index_scores", lib().csa2_index_scores(
        SCORES_CAND, B, Tq, _p(q), BF16, _p(w), _p(k), _key_dtype(k), None, _rows_contig(k, DI, "k"), N,
        _p(q_pos), _p(blocks), K_b, _p(scores), scores.stride(0), _p(ids), None, 0, _stream(stream)))
    return scores, ids


def gather_scores(all_scores, q_pos, blocks, scores, ids, n_cache=None, stream=None):
    """a4 from stored scores: the candidates' entries of the scan's score
    matrix all_scores f32 [B*Tq][>=N] (same output as index_cand).  q_pos
    int64 [B][Tq], blocks int32 [B*Tq][K_b]."""
    B, Tq = q_pos.shape
    K_b = blocks.shape[1]
    N = all_scores.shape[1] if n_cache is None else n_cache
    assert blocks.is_contiguous() and q_pos.is_contiguous() and all_scores.stride(1) == 1
    check("csa2_gather_scores", lib().csa2_gather_scores(
        B, Tq, _p(all_scores), all_scores.stride(0), N, _p(q_pos), _p(blocks), K_b, _p(scores),
        _p(ids), scores.stride(0), _stream(stream)))
    return scores, ids

def gather_select(all_scores, q_pos, blocks, k: int, out, n_cache=None, stream=None):
    """a4 from stored scores and a5 in one pass: the position top-k of the
    candidates of ``blocks`` gathered from the scan's score matrix, equal to
    gather_scores followed by select_topk.  out int32 [B*Tq][>=k]."""
    B, Tq = q_pos.shape
    K_b = blocks.shape[1]
    N = all_scores.shape[1] if n_cache is None else n_cache
    assert blocks.is_contiguous() and q_pos.is_contiguous() and all_scores.stride(1) == 1
    assert out.stride(1) == 1
    check("csa2_gather_select", lib().csa2_gather_select(
        B, Tq, _p(all_scores), all_scores.stride(0), N, _p(q_pos), _p(blocks), K_b, k, _p(out),
        out.stride(0), _stream(stream)))
    return out


def select_topk(scores, k: int, out, ids=None, forced=None, force_last=False, ws=None,
                stream=None):
    """a3 / a5: top-k ids per row (ascending, -1 padded).  ``ws``: scratch of
    workspace_bytes(OP_SELECT, R, n, k) bytes (allocated here when None)."""
    R, n = scores.shape
    if ws is None:
        need = workspace_bytes(_lib.OP_SELECT, R, n, k)
        if need:
            ws = torch.empty((need + 63) // 64 * 8, dtype=torch.float64, device=scores.device)
    check("csa2_select_topk", lib().csa2_select_topk(
        R, n, _p(scores), scores.stride(0), _p(ids), ids.stride(0) if ids is not None else 0,
        _p(forced), 1 if force_last else 0, k, _p(out), out.stride(0), _p(ws),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))
    return out


def sparse_attn(q, lat, sel, win, q_pos, sink, W: int, scale: float, out, lat_scale=None,
                win_scale=None, lse=None, ws=None, stream=None):
    """a6: attention over the selected latents + the raw window with sinks.

    q bf16 [B][Tq][64][512]; lat bf16 [B][N][512] or NVFP4 uint8 [B][N][256]
    with lat_scale uint8 [B][N][32]; sel int32 [B*Tq][K]; win bf16
    [B][W_cap][512] or E4M3 uint8 with win_scale f32 [B][W_cap]; out bf16
    [B*Tq][64][512]; lse f32 [B*Tq][64] or None; ws from workspace_bytes."""
    B, Tq = q.shape[:2]
    N = lat.shape[1]
    W_cap = win.shape[1]
    K = sel.shape[1]
    lat_dt = BF16 if lat.dtype == torch.bfloat16 else NVFP4
    win_dt = BF16 if win.dtype == torch.bfloat16 else FP8_E4M3
    assert q.stride(-1) == 1 and q.stride(1) == HQ * D
    check("csa2_sparse_attn", lib().csa2_sparse_attn(
        B, Tq, _p(q), q.stride(0), _p(lat), lat_dt, _p(lat_scale), lat.stride(0) // lat.stride(1), N,
        _p(sel), K, sel.stride(0), _p(win), win_dt, _p(win_scale), W, W_cap,
        win.stride(0) // win.stride(1), _p(q_pos), _p(sink), float(scale), _p(out), out.stride(0),
        _p(lse), _p(ws), ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))
    return out, lse


def sparse_attn_noalloc(q, lat, sel, win, q_pos, sink, W: int, scale: float, out, lat_scale=None,
                        win_scale=None, lse=None, stream=None):
    """a6 as sparse_attn, with the split partials in the library's fixed
    per-device scratch instead of a caller workspace (nothing is allocated;
    calls that overlap on one GPU race)."""
    B, Tq = q.shape[:2]
    N = lat.shape[1]
    W_cap = win.shape[1]
    K = sel.shape[1]
    lat_dt = BF16 if lat.dtype == torch.bfloat16 else NVFP4
    win_dt = BF16 if win.dtype == torch.bfloat16 else FP8_E4M3
    assert q.stride(-1) == 1 and q.stride(1) == HQ * D
    check("csa2_sparse_attn_noalloc", lib().csa2_sparse_attn_noalloc(
        B, Tq, _p(q), q.stride(0), _p(lat), lat_dt, _p(lat_scale), lat.stride(0) // lat.stride(1), N,
        _p(sel), K, sel.stride(0), _p(win), win_dt, _p(win_scale), W, W_cap,
        win.stride(0) // win.stride(1), _p(q_pos), _p(sink), float(scale), _p(out), out.stride(0),
        _p(lse), _stream(stream)))
    return out, lse


def dequant_fp8(src, row_scale=None, dtype=torch.bfloat16, out=None, stream=None):
    rows, cols = src.shape
    if out is None:
        out = torch.empty((rows, cols), dtype=dtype, device=src.device)
    dt = F32 if out.dtype == torch.float32 else BF16
    check("csa2_dequant_fp8", lib().csa2_dequant_fp8(_p(src), _p(row_scale), rows, cols, _p(out), dt,
                                                     _stream(stream)))
    return out


def dequant_nvfp4(packed, scales, dtype=torch.bfloat16, out=None, stream=None):
    rows, half = packed.shape
    cols = half * 2
    if out is None:
        out = torch.empty((rows, cols), dtype=dtype, device=packed.device)
    dt = F32 if out.dtype == torch.float32 else BF16
    check("csa2_dequant_nvfp4", lib().csa2_dequant_nvfp4(_p(packed), _p(scales), rows, cols, _p(out),
                                                         dt, _stream(stream)))
    return out


class DecodePath:
    """Buffers and call order of one pass of the CSA2 hot path.

    The call order is the method's (NVFP4 article, section 3 call tree):
    [compressor] -> candidate-source scan + block max -> block top-K_b with
    the newest block kept -> current-layer indexer over the candidates ->
    position top-K -> sparse attention over Sel + window with sinks.

    one_indexer: the same indexer (q, w, k) serves both stages (the chunked
    prefill); the scan then also keeps every score and the candidate stage
    gathers them (csa2_gather_scores) instead of scoring again."""

    def __init__(self, B: int, Tq: int, N: int, K_b: int = 2048, K: int = 512, W: int = 128,
                 device="cuda", one_indexer: bool = False):
        self.B, self.Tq, self.N, self.K_b, self.K, self.W = B, Tq, N, K_b, K, W
        R = B * Tq
        nblk = (N + BLK - 1) // BLK
        dev = torch.device(device)
        self.one_indexer = one_indexer
        # one indexer: gather + position top-k in one call when a row of
        # 8 * K_b candidates fits one workgroup's registers
        R8 = K_b * BLK
        self.fused_gather = one_indexer and (R8 <= 16384 or (R >= 256 and R8 <= 32768))
        # row stride a multiple of 4 floats (16-byte rows for the gather)
        self.all_scores = (torch.empty((R, (N + 3) // 4 * 4), dtype=torch.float32, device=dev)
                           if one_indexer else None)
        self.block_max = torch.empty((R, nblk), dtype=torch.float32, device=dev)
        self.blocks = torch.empty((R, K_b), dtype=torch.int32, device=dev)
        self.cand_scores = torch.empty((R, K_b * BLK), dtype=torch.float32, device=dev)
        self.cand_ids = torch.empty((R, K_b * BLK), dtype=torch.int32, device=dev)
        self.sel = torch.empty((R, K), dtype=torch.int32, device=dev)
        self.out = torch.empty((R, HQ, D), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((R, HQ), dtype=torch.float32, device=dev)
        wsb = workspace_bytes(_lib.OP_SPARSE_ATTN, R, K, W)
        self.ws = torch.empty((max(wsb, 16) // 4 + 4,), dtype=torch.float32, device=dev)
        sel_b = max(workspace_bytes(_lib.OP_SELECT, R, nblk, K_b),
                    workspace_bytes(_lib.OP_SELECT, R, K_b * BLK, K))
        self.sel_ws = torch.empty(((max(sel_b, 64) + 63) // 64 * 8,), dtype=torch.float64, device=dev)

    def run(self, inp: dict, scale: float, compress_first: bool = True, stream=None, marks=None):
        """One pass.  ``marks``: optional 7 torch.cuda.Events recorded on the
        stream before the first step and after each of the six steps."""
        def mark(i):
            if marks is not None:
                marks[i].record(stream if stream is not None else torch.cuda.current_stream())
        mark(0)
        if compress_first and inp.get("raw") is not None:
            g0 = inp["cfg"].comp_pos0 // 2
            T = inp["raw"].shape[1]
            compress(inp["raw"], inp["gate"], inp["lat"][:, g0:g0 + T // 2], stream=stream)
        if inp.get("tok_kv") is not None:
            # the compressor's decode step: completes the pair ending at
            # step_pos and writes its latent (NVFP4 or bf16) into the cache
            cache = (inp["lat"], inp["lat_scale"]) if inp.get("lat_scale") is not None else inp["lat"]
            compress_step(inp["tok_kv"], inp["tok_gate"], inp["step_pos"], inp["state"], cache,
                          stream=stream)
        mark(1)
        index_scan(inp["qs"], inp["ws"], inp["ks"], inp["q_pos"], block_max=self.block_max,
                   scores=self.all_scores, k_scale=inp.get("ks_scale"), stream=stream)
        mark(2)
        select_topk(self.block_max, self.K_b, self.blocks, force_last=True, ws=self.sel_ws,
                    stream=stream)
        mark(3)
        if self.one_indexer:
            if not (inp["qi"] is inp["qs"] and inp["wi"] is inp["ws"] and inp["ki"] is inp["ks"]):
                raise ValueError("one_indexer path needs the same indexer for both stages")
            mark(4)
            if self.fused_gather:
                # the candidates gathered inside the position top-k (one pass)
                gather_select(self.all_scores, inp["q_pos"], self.blocks, self.K, self.sel,
                              n_cache=self.N, stream=stream)
            else:
                gather_scores(self.all_scores, inp["q_pos"], self.blocks, self.cand_scores,
                              self.cand_ids, n_cache=self.N, stream=stream)
                select_topk(self.cand_scores, self.K, self.sel, ids=self.cand_ids,
                            ws=self.sel_ws, stream=stream)
        else:
            index_cand(inp["qi"], inp["wi"], inp["ki"], inp["q_pos"], self.blocks,
                       self.cand_scores, self.cand_ids, stream=stream)
            mark(4)
            select_topk(self.cand_scores, self.K, self.sel, ids=self.cand_ids, ws=self.sel_ws,
                        stream=stream)
        mark(5)
        sparse_attn(inp["q"], inp["lat"], self.sel, inp["win"], inp["q_pos"], inp["sink"], self.W,
                    scale, self.out, lat_scale=inp.get("lat_scale"), win_scale=inp.get("win_scale"),
                    lse=self.lse, ws=self.ws, stream=stream)
        mark(6)
        return self.out


    def capture(self, inp: dict, scale: float, compress_first: bool = True):
        """Record one pass into a HIP graph (torch.cuda.CUDAGraph) for callers
        that replay work under graph capture; buffers and inputs are the ones
        given here.  Call run() once before, so that one-time kernel
        attributes are set outside the capture."""
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.run(inp, scale, compress_first=compress_first)
        return graph


def stack_route(layer: int, index_sources, kv_sources, window_only):
    """Which published Sel and which compressed cache a layer reads (NVFP4
    article, sections 3.3 and 4: index source layers publish their top-K,
    KV source layers store the cache the other layers share; section 3.2:
    window-only layers read neither).  A layer reads the most recent source
    at or before it; None for a window-only layer."""
    if layer in window_only:
        return None
    idx = max((s for s in index_sources if s <= layer), default=-1)
    kv = max((s for s in kv_sources if s <= layer), default=-1)
    return idx, kv


class LayerStackPath:
    """One decode step through a stack of layers that share index results and
    compressed caches (NVFP4 article, sections 3.3 and 4): the block stage
    once; the candidate indexer and the position top-K once per index source
    layer; sparse attention for every layer, reading the Sel of its index
    source layer and the latent cache of its KV source layer (window only for
    the window-only layers).  Layers run in order, one attention launch each,
    as a model's forward pass would.  Inputs from gen.make_stack_inputs."""

    def __init__(self, inp: dict, K_b: int = 2048, K: int = 512, W: int = 128):
        cfg = inp["cfg"]
        self.B, self.Tq, self.N, self.K_b, self.K, self.W = cfg.B, cfg.Tq, cfg.N, K_b, K, W
        self.layers = inp["layers"]
        self.window_only = inp["window_only"]
        self.index_sources = inp["index_sources"]
        self.kv_sources = inp["kv_sources"]
        R = cfg.B * cfg.Tq
        nblk = (cfg.N + BLK - 1) // BLK
        dev = inp["q_pos"].device
        self.block_max = torch.empty((R, nblk), dtype=torch.float32, device=dev)
        self.blocks = torch.empty((R, K_b), dtype=torch.int32, device=dev)
        self.cand_scores = torch.empty((R, K_b * BLK), dtype=torch.float32, device=dev)
        self.cand_ids = torch.empty((R, K_b * BLK), dtype=torch.int32, device=dev)
        self.sel = {s: torch.empty((R, K), dtype=torch.int32, device=dev) for s in self.index_sources}
        self.no_sel = torch.empty((R, 0), dtype=torch.int32, device=dev)
        self.out = [torch.empty((R, HQ, D), dtype=torch.bfloat16, device=dev)
                    for _ in range(self.layers)]
        self.lse = [torch.empty((R, HQ), dtype=torch.float32, device=dev) for _ in range(self.layers)]
        wsb = max(workspace_bytes(_lib.OP_SPARSE_ATTN, R, K, W),
                  workspace_bytes(_lib.OP_SPARSE_ATTN, R, 0, W))
        self.ws = torch.empty((max(wsb, 16) // 4 + 4,), dtype=torch.float32, device=dev)
        sel_b = max(workspace_bytes(_lib.OP_SELECT, R, nblk, K_b),
                    workspace_bytes(_lib.OP_SELECT, R, K_b * BLK, K))
        self.sel_ws = torch.empty(((max(sel_b, 64) + 63) // 64 * 8,), dtype=torch.float64, device=dev)

    def source_of(self, layer: int):
        """(index source, KV source) read by ``layer``; None for window-only layers."""
        return stack_route(layer, self.index_sources, self.kv_sources, self.window_only)

    def run(self, inp: dict, scale: float, stream=None):
        index_scan(inp["qs"], inp["ws"], inp["ks"], inp["q_pos"], block_max=self.block_max,
                   stream=stream)
        select_topk(self.block_max, self.K_b, self.blocks, force_last=True, ws=self.sel_ws,
                    stream=stream)
        any_lat = inp["lat"][self.kv_sources[0]]
        for layer in range(self.layers):
            if layer in self.index_sources:
                index_cand(inp["qi"][layer], inp["wi"][layer], inp["ki"][layer], inp["q_pos"],
                           self.blocks, self.cand_scores, self.cand_ids, stream=stream)
                select_topk(self.cand_scores, self.K, self.sel[layer], ids=self.cand_ids,
                            ws=self.sel_ws, stream=stream)
            src = self.source_of(layer)
            if src is None:
                lat, sel = any_lat, self.no_sel
            else:
                lat, sel = inp["lat"][src[1]], self.sel[src[0]]
            sparse_attn(inp["q"][layer], lat, sel, inp["win"][layer], inp["q_pos"],
                        inp["sink"][layer], self.W, scale, self.out[layer], lse=self.lse[layer],
                        ws=self.ws, stream=stream)
        return self.out


STAGES = ("compress", "index_scan", "select_blocks", "index_cand", "select_positions",
          "sparse_attn")
