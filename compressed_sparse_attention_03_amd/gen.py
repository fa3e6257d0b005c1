"""Seeded synthetic inputs for the CSA2 hot path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic, so both the device path and the CPU oracle can consume
exactly the same bytes.  Encodings into the cache formats are done by torch
dtype conversions (bf16, float8_e4m3fn) or by drawing the format's raw codes
directly (NVFP4 nibbles and E4M3 group-scale bytes).

Shapes follow the method's constants (NVFP4 article sections 3-3.4; oQ3e
config walkthrough section 2.1): 64 query heads x 512, one shared 512-wide
latent KV head, 32 index heads x 128, blocks of 8 latents, window 128.  The
workload sizes (1M context, 32 sequences, 8192-token prefill chunks) follow
the serving limits the NVFP4 article gives in its deployment section.

Layout of one input set (all torch tensors on ``device``):
  q      bf16 [B][Tq][64][512]   attention queries
  sink   f32  [64]               per-head sink logit
  qs/ws/ks   candidate-source indexer: bf16 [B][Tq][32][128], f32 [B][Tq][32],
             keys [B][N][128] (bf16, or uint8 E4M3 codes), or MXFP4 keys as
             uint8 E2M1 codes [B][N][64] with ks_scale E8M0 bytes [B][N][4]
             (ks_scale None otherwise; ki_scale likewise)
  qi/wi/ki   current-layer indexer, same shapes (the same tensors when the
             config uses one shared indexer)
  lat    latent cache: bf16 [B][N][512], or uint8 NVFP4 [B][N][256] with
         lat_scale uint8 E4M3 [B][N][32]
  win    window source [B][W_cap][512] (bf16, or uint8 E4M3 codes with
         win_scale f32 [B][W_cap]); row of raw position p sits at p % W_cap
  q_pos  int64 [B][Tq]           raw position of each query
  raw, gate  bf16 [B][T_c][512]  compressor input (raw KV latents and gate
             logits) for raw positions raw_pos0 .. raw_pos0+T_c-1; its
             output belongs in lat rows raw_pos0/2 ..
  tok_kv, tok_gate  bf16 [B][512]  (configs with a compressor decode step)
             the token at raw position step_pos[b] = t_last (odd), whose
             partner, token t_last - 1, is parked in state bf16 [B][2][512]
             (kv row, gate row); the step writes lat row t_last // 2
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import torch

D, HQ, HI, DI, BLK = 512, 64, 32, 128, 8


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    Tq: int
    N: int                 # compressed latents held in the cache
    t_last: int            # raw position of the last query of each sequence
    K_b: int = 2048
    K: int = 512
    W: int = 128
    W_cap: int = 128
    key_fmt: str = "bf16"  # "bf16" | "fp8" | "mxfp4"
    lat_fmt: str = "bf16"  # "bf16" | "nvfp4"
    win_fmt: str = "bf16"  # "bf16" | "fp8"
    shared_indexer: bool = False
    comp_T: int = 0        # compressor input tokens (0 = no compressor)
    comp_pos0: int = 0     # raw position of the first compressor token
    comp_from_win: bool = False  # compressor input is a slice of the window ring
    comp_step: bool = False  # one compressor decode step (pair completed at t_last)
    win_pos0: int = 0      # lowest raw position the window source must hold
    seed: int = 0
    scale: float = 512 ** -0.5
    desc: str = ""

    @property
    def R(self) -> int:
        return self.B * self.Tq

    @property
    def nblk(self) -> int:
        return (self.N + BLK - 1) // BLK


def _configs():
    c1 = Config(
        "tiny", B=1, Tq=4, N=2048, t_last=4095, K_b=64, K=512, W=128, W_cap=256,
        comp_T=4096, comp_pos0=0, win_pos0=4092 - 127, seed=0,
        desc="1 sequence, 4096 raw tokens -> 2048 latents, 4 queries at the end")
    c2 = Config(
        "128k", B=32, Tq=1, N=65536, t_last=131071, W_cap=128,
        comp_T=256, comp_pos0=131072 - 256, win_pos0=131071 - 127, seed=1,
        desc="32 sequences x 131072 raw tokens, 1 query each")
    c3 = Config(
        "prefill", B=1, Tq=8192, N=36864, t_last=73727, W_cap=16384,
        shared_indexer=True, comp_T=8192, comp_pos0=65536, comp_from_win=True,
        win_pos0=65536 - 127, seed=2,
        desc="8192-token chunk after 65536 raw tokens, causal, one indexer")
    c4 = Config(
        "1m", B=8, Tq=1, N=524288, t_last=1048575, W_cap=128, win_pos0=1048575 - 127,
        seed=3, desc="8 sequences x 1,048,576 raw tokens, bf16 caches (no compressor step)")
    c5 = Config(
        "1m_lowp", B=32, Tq=1, N=524288, t_last=1048575, W_cap=128,
        key_fmt="fp8", lat_fmt="nvfp4", win_fmt="fp8", win_pos0=1048575 - 127, comp_step=True,
        seed=4, desc="32 sequences x 1,048,576 raw tokens, NVFP4 latents, FP8 window/keys; "
                     "the compressor's decode step writes the newest latent first")
    c6 = Config(
        "1m_verify", B=8, Tq=5, N=524288, t_last=1048575, W_cap=256,
        win_pos0=1048575 - 4 - 127, seed=5,
        desc="speculative verification at 1M: 8 sequences x 5 draft tokens at the end of "
             "1,048,576 raw tokens, bf16 caches")
    c7 = replace(c3, name="prefill_fp8", key_fmt="fp8", seed=6,
                 desc="the chunked prefill with FP8 E4M3 index keys (integer-valued, exact)")
    c8 = replace(c3, name="prefill_mxfp4", key_fmt="mxfp4", seed=7,
                 desc="the chunked prefill with MXFP4 index keys (E2M1 x E8M0, exact scores)")
    return {c.name: c for c in (c1, c2, c3, c4, c5, c6, c7, c8)}


CONFIGS = _configs()


def shrink(cfg: Config, **kw) -> Config:
    """A smaller variant of a config (same structure, fewer sequences/latents)."""
    return replace(cfg, **kw)


def q_positions(cfg: Config) -> torch.Tensor:
    """Raw positions of the queries: the last Tq tokens of every sequence."""
    t = torch.arange(cfg.t_last - cfg.Tq + 1, cfg.t_last + 1, dtype=torch.int64)
    return t.unsqueeze(0).expand(cfg.B, cfg.Tq).contiguous()


def _normal_bf16(shape, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def _int_bf16(shape, g, device):
    return torch.randint(-3, 4, shape, generator=g, device=device, dtype=torch.int32).to(torch.bfloat16)


def _int_fp8(shape, g, device):
    x = torch.randint(-3, 4, shape, generator=g, device=device, dtype=torch.int32)
    return x.to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)


def _mx_keys(shape, g, device):
    """MXFP4 index keys: uniform random E2M1 codes (every code, values up to
    +-6) and E8M0 block scales 2^-1 or 2^0, so every key is a multiple of
    1/4 and every score stays exact in fp32.  Returns (codes [B][N][64],
    scales [B][N][4])."""
    B, N, _ = shape
    codes = torch.randint(0, 256, (B, N, DI // 2), generator=g, device=device,
                          dtype=torch.int32).to(torch.uint8)
    scales = torch.randint(126, 128, (B, N, DI // 32), generator=g, device=device,
                           dtype=torch.int32).to(torch.uint8)
    return codes, scales


def _head_weights(shape, g, device):
    return torch.randint(1, 17, shape, generator=g, device=device, dtype=torch.int32).to(torch.float32) / 16.0


def make_inputs(cfg: Config, device="cpu", seed: Optional[int] = None) -> dict:
    """Draw one seeded input set for ``cfg`` on ``device``."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed if seed is None else seed)
    B, Tq, N = cfg.B, cfg.Tq, cfg.N
    out = {"cfg": cfg}
    out["q_pos"] = q_positions(cfg).to(dev)
    out["q"] = _normal_bf16((B, Tq, HQ, D), g, dev)
    out["sink"] = torch.randn((HQ,), generator=g, device=dev, dtype=torch.float32)
    out["qs"] = _int_bf16((B, Tq, HI, DI), g, dev)
    out["ws"] = _head_weights((B, Tq, HI), g, dev)
    if cfg.key_fmt == "mxfp4":
        out["ks"], out["ks_scale"] = _mx_keys((B, N, DI), g, dev)
    else:
        out["ks"] = (_int_fp8 if cfg.key_fmt == "fp8" else _int_bf16)((B, N, DI), g, dev)
        out["ks_scale"] = None
    if cfg.shared_indexer:
        out["qi"], out["wi"], out["ki"], out["ki_scale"] = out["qs"], out["ws"], out["ks"], out["ks_scale"]
    else:
        assert cfg.key_fmt != "mxfp4", "MXFP4 keys serve the one-indexer prefill"
        kmake = _int_fp8 if cfg.key_fmt == "fp8" else _int_bf16
        out["qi"] = _int_bf16((B, Tq, HI, DI), g, dev)
        out["wi"] = _head_weights((B, Tq, HI), g, dev)
        out["ki"] = kmake((B, N, DI), g, dev)
        out["ki_scale"] = None
    if cfg.lat_fmt == "nvfp4":
        out["lat"] = torch.randint(0, 256, (B, N, D // 2), generator=g, device=dev,
                                   dtype=torch.int32).to(torch.uint8)
        # E4M3 group-scale codes 0x18..0x3F: magnitudes 2^-4 .. 1.875
        out["lat_scale"] = torch.randint(0x18, 0x40, (B, N, D // 16), generator=g, device=dev,
                                         dtype=torch.int32).to(torch.uint8)
    else:
        out["lat"] = _normal_bf16((B, N, D), g, dev)
        out["lat_scale"] = None
    if cfg.win_fmt == "fp8":
        x = torch.randn((B, cfg.W_cap, D), generator=g, device=dev, dtype=torch.float32)
        out["win"] = x.to(torch.float8_e4m3fn).view(torch.uint8)
        out["win_scale"] = torch.rand((B, cfg.W_cap), generator=g, device=dev,
                                      dtype=torch.float32) + 0.5
    else:
        out["win"] = _normal_bf16((B, cfg.W_cap, D), g, dev)
        out["win_scale"] = None
    if cfg.comp_T:
        gate = _normal_bf16((B, cfg.comp_T, D), g, dev)
        if cfg.comp_from_win:
            s0 = cfg.comp_pos0 % cfg.W_cap
            assert s0 + cfg.comp_T <= cfg.W_cap
            raw = out["win"][:, s0:s0 + cfg.comp_T]
        else:
            raw = _normal_bf16((B, cfg.comp_T, D), g, dev)
            # raw rows that fall inside the window are the window's rows
            lo = max(cfg.win_pos0, cfg.comp_pos0)
            for p in range(lo, cfg.comp_pos0 + cfg.comp_T):
                out["win"][:, p % cfg.W_cap] = raw[:, p - cfg.comp_pos0]
        out["raw"], out["gate"] = raw, gate
    else:
        out["raw"] = out["gate"] = None
    if cfg.comp_step:
        assert cfg.t_last % 2 == 1 and cfg.t_last // 2 < N
        out["tok_kv"] = _normal_bf16((B, D), g, dev)
        out["tok_gate"] = _normal_bf16((B, D), g, dev)
        out["state"] = _normal_bf16((B, 2, D), g, dev)
        out["step_pos"] = torch.full((B,), cfg.t_last, dtype=torch.int64, device=dev)
    return out


def to_numpy(t: torch.Tensor):
    """Host numpy view of a tensor; bf16 becomes its uint16 bit pattern."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()


# ---- a stack of layers sharing index results and compressed caches ----------
# Layout of the NVFP4 article (sections 3.3 and 4): 40 layers; layers 0 and 1
# attend to their sliding window only; 8 index source layers compute and
# publish their position top-K, every later layer reads the one of the most
# recent index source layer; 4 KV source layers store a compressed cache that
# the layers up to the next source read through a shared handle; the block
# stage runs once per token (at the candidate-source layer).
STACK_LAYERS = 40
STACK_WINDOW_ONLY = (0, 1)
STACK_INDEX_SOURCES = (2, 8, 14, 20, 24, 28, 32, 36)
STACK_KV_SOURCES = (2, 8, 14, 20)


def make_stack_inputs(cfg: Config, layers: int = STACK_LAYERS, window_only=STACK_WINDOW_ONLY,
                      index_sources=STACK_INDEX_SOURCES, kv_sources=STACK_KV_SOURCES,
                      device="cpu", seed: Optional[int] = None) -> dict:
    """Inputs of a layer stack: the candidate-source indexer (qs, ws, ks), per
    index source layer s an indexer (qi[s], wi[s], ki[s]), per KV source
    layer a latent cache lat[s], per layer an attention query q[l], window
    source win[l] and sink[l]; one set of query positions.  bf16 caches."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed if seed is None else seed)
    B, Tq, N = cfg.B, cfg.Tq, cfg.N
    out = {"cfg": cfg, "layers": layers, "window_only": tuple(window_only),
           "index_sources": tuple(index_sources), "kv_sources": tuple(kv_sources)}
    out["q_pos"] = q_positions(cfg).to(dev)
    out["qs"] = _int_bf16((B, Tq, HI, DI), g, dev)
    out["ws"] = _head_weights((B, Tq, HI), g, dev)
    out["ks"] = _int_bf16((B, N, DI), g, dev)
    out["qi"], out["wi"], out["ki"] = {}, {}, {}
    for s in index_sources:
        out["qi"][s] = _int_bf16((B, Tq, HI, DI), g, dev)
        out["wi"][s] = _head_weights((B, Tq, HI), g, dev)
        out["ki"][s] = _int_bf16((B, N, DI), g, dev)
    out["lat"] = {s: _normal_bf16((B, N, D), g, dev) for s in kv_sources}
    out["q"] = [_normal_bf16((B, Tq, HQ, D), g, dev) for _ in range(layers)]
    out["win"] = [_normal_bf16((B, cfg.W_cap, D), g, dev) for _ in range(layers)]
    out["sink"] = [torch.randn((HQ,), generator=g, device=dev, dtype=torch.float32)
                   for _ in range(layers)]
    return out
