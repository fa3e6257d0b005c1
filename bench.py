#!/usr/bin/env python3
"""Benchmark of the CSA2 hot path on one MI355X.

A step is one pass of the whole path over one batch: candidate-source
indexer scan with the fused block max -> block top-2048 (newest block kept)
-> current-layer indexer over the 16,384 candidates -> position top-512 ->
sparse attention over the 512 latents + 128-token window with sinks.  The
bf16 1M workload has no compressor step (its cache is given); the
compressor is timed in the low-precision 1M step (its decode step writes the
newest NVFP4 latent), in the prefill pass (which pools its 8192-token chunk)
and on its own over a whole 1M-token sequence.

The headline workload is 1M-context decode: 8 sequences x 1,048,576 raw
tokens (524,288 bf16 latents of 512, bf16 index keys), one query each.
Inputs are seeded synthetic tensors already resident in HBM when the timed
region starts.  Prints ONE JSON line: the headline metric with its roofline
(the scan kernel against the HBM peak), the CPU oracle's rate, and the
secondary workloads under "extra".

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                  [--only-main] [--calib] [--only CONFIG]

--only CONFIG times one workload's step alone and prints its stage times
instead (used for the counter runs behind the committed profiles).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA2 decode queries/s (64 heads) at 1M ctx; % HBM peak; prefill indexer MFMA %"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E peak
MFMA_BF16_PEAK_TFS = 2500.0
MFMA_FP8_PEAK_TFS = 5000.0  # MI355X dense fp8 MFMA peak
MFMA_FP4_PEAK_TFS = 10100.0  # MI355X dense fp4 MFMA peak
D, HQ, HI, DI, BLK = 512, 64, 32, 128, 8


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def n_vis(t, N):
    return min(N, (t + 1) // 2)


def step_bytes(cfg) -> dict:
    """Algorithmic HBM bytes of one step, per stage: every operand the method
    must read once and every result it must write once."""
    R, B, Tq = cfg.R, cfg.B, cfg.Tq
    kel = 1 if cfg.key_fmt == "fp8" else 2
    nblk = cfg.nblk
    lat_row = D // 2 + D // 16 if cfg.lat_fmt == "nvfp4" else 2 * D
    win_row = D + 4 if cfg.win_fmt == "fp8" else 2 * D
    t_hi = cfg.t_last
    keys_per_seq = n_vis(t_hi, cfg.N)  # one pass over the keys serves all queries of a sequence
    b = {}
    b["compress"] = B * (cfg.comp_T * D * 2 * 2 + (cfg.comp_T // 2) * D * 2) if cfg.comp_T else 0
    if cfg.comp_step:  # new token + parked token (kv and gate rows), position; one latent row out
        b["compress"] += B * (4 * D * 2 + 8 + lat_row)
    b["index_scan"] = B * keys_per_seq * DI * kel + R * (HI * DI * 2 + HI * 4 + nblk * 4 + 8)
    b["select_blocks"] = R * (nblk * 4 + cfg.K_b * 4)
    b["index_cand"] = R * (cfg.K_b * BLK * DI * kel + HI * DI * 2 + HI * 4 + cfg.K_b * 4 +
                           cfg.K_b * BLK * 8)
    b["select_positions"] = R * (cfg.K_b * BLK * 8 + cfg.K * 4)
    b["sparse_attn"] = R * (cfg.K * lat_row + cfg.W * win_row + HQ * D * 2 * 2 + cfg.K * 4 + HQ * 4)
    return b


def prefill_indexer_flops(cfg) -> float:
    pairs = sum(n_vis(t, cfg.N) for t in range(cfg.t_last - cfg.Tq + 1, cfg.t_last + 1))
    return float(pairs) * HI * DI * 2


SCAN_SOURCES = ("index_scan.hip", "indexer.h", "device_common.h")


def source_hash(paths):
    """Hash of the sources that define a kernel (None if one is missing)."""
    h = hashlib.sha256()
    for p in paths:
        if not os.path.exists(p):
            return None
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(kernel_src, workload: str):
    """HBM traffic of the dominant kernel from the committed rocprofv3 PMC
    summary, if it was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "index_scan_1m_pmc.md")
    if not os.path.exists(p):
        return None
    vals = {}
    for line in open(p):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256_16") != source_hash(kernel_src) or vals.get("workload") != workload:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def time_config(name, steps, warmup, torch, gen, api):
    """Whole-step time: `steps` passes launched back to back on one stream
    between two events (the host queues each pass while the GPU runs the
    previous one's scan, so no launch gaps open between kernels).  Plus a
    per-stage breakdown from a second, eager pass with events between the
    stages (those stage times include the host's launch latency)."""
    cfg = gen.CONFIGS[name]
    log(f"[bench] {name}: generating inputs (B={cfg.B}, N={cfg.N}, seed={cfg.seed})")
    inp = gen.make_inputs(cfg, device="cuda")
    path = api.DecodePath(cfg.B, cfg.Tq, cfg.N, cfg.K_b, cfg.K, cfg.W, one_indexer=cfg.shared_indexer)
    comp = cfg.comp_T > 0
    torch.cuda.synchronize()
    for _ in range(warmup):
        path.run(inp, cfg.scale, compress_first=comp)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        path.run(inp, cfg.scale, compress_first=comp)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(steps)]
    for i in range(steps):
        path.run(inp, cfg.scale, compress_first=comp, marks=marks[i])
        torch.cuda.synchronize()
    stage_ms = {}
    for si, sname in enumerate(api.STAGES):
        stage_ms[sname] = sum(m[si].elapsed_time(m[si + 1]) for m in marks) / steps
    log(f"[bench] {name}: {ms * 1e3:.1f} us/step;  eager stages: " +
        "  ".join(f"{k}={v * 1e3:.1f}us" for k, v in stage_ms.items()))
    return cfg, inp, path, ms, stage_ms


def time_layer_stack(steps, torch, gen, api):
    """One decode step through the pages' 40-layer stack on the 1M workload:
    the block stage once, the candidate indexer + position top-512 at each of
    the 8 index source layers, attention at every layer (window only at
    layers 0-1), 4 shared compressed caches.  Steps launched back to back."""
    cfg = gen.CONFIGS["1m"]
    log(f"[bench] layer stack: generating inputs ({gen.STACK_LAYERS} layers, B={cfg.B}, N={cfg.N})")
    inp = gen.make_stack_inputs(cfg, device="cuda")
    path = api.LayerStackPath(inp, cfg.K_b, cfg.K, cfg.W)
    for _ in range(2):
        path.run(inp, cfg.scale)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        path.run(inp, cfg.scale)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    L, R = gen.STACK_LAYERS, cfg.R
    n_idx, n_win = len(gen.STACK_INDEX_SOURCES), len(gen.STACK_WINDOW_ONLY)
    sb = step_bytes(cfg)
    win_row = 2 * D
    attn_win_only = R * (cfg.W * win_row + HQ * D * 2 * 2 + HQ * 4)
    total = (sb["index_scan"] + sb["select_blocks"] + n_idx * (sb["index_cand"] + sb["select_positions"])
             + (L - n_win) * sb["sparse_attn"] + n_win * attn_win_only)
    log(f"[bench] layer stack: {ms * 1e3:.1f} us/step ({ms * 1e3 / L:.1f} us per layer)")
    del path, inp
    return {
        "workload": f"{L}-layer decode step at 1M ctx (8 sequences x 1 query): block stage once, "
                    f"{n_idx} index source layers, 4 shared compressed caches, {n_win} window-only layers",
        "ms_per_step": round(ms, 4), "us_per_layer": round(ms * 1e3 / L, 2),
        "queries_per_s": round(R / (ms * 1e-3), 1),
        "step_hbm_frac": round(total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes": total,
    }


def time_compress_fp4(torch, api, launches=10):
    """The compressor writing the NVFP4 cache for a whole 1M-token sequence
    (1,048,576 raw tokens -> 524,288 latents): streaming, HBM-bound."""
    T = 1 << 20
    g = torch.Generator(device="cuda").manual_seed(7)
    raw = torch.randn((1, T, D), generator=g, device="cuda").bfloat16()
    gate = torch.randn((1, T, D), generator=g, device="cuda").bfloat16()
    codes = torch.empty((1, T // 2, D // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((1, T // 2, D // 16), dtype=torch.uint8, device="cuda")
    api.compress_nvfp4(raw, gate, codes, scales)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(launches):
        api.compress_nvfp4(raw, gate, codes, scales)
    end.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1e3 / launches
    nbytes = 2 * T * D * 2 + (T // 2) * (D // 2 + D // 16)
    gbs = nbytes / (us * 1e-6) / 1e9
    log(f"[bench] compress_nvfp4 1M tokens: {us:.1f} us/launch = {gbs:.0f} GB/s")
    del raw, gate, codes, scales
    return {"workload": "compressor with NVFP4 epilogue over one 1,048,576-token sequence "
                        "(524,288 latents)", "us_per_launch": round(us, 2),
            "algorithmic_bytes": nbytes, "GB/s": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def scan_launch_us(torch, api, path, inp, launches):
    """Average duration of the candidate-source scan kernel: `launches`
    back-to-back launches on the current stream between two events (each
    launch is long enough that the queue never runs dry)."""
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    api.index_scan(inp["qs"], inp["ws"], inp["ks"], inp["q_pos"], block_max=path.block_max)
    torch.cuda.synchronize()
    start.record()
    for _ in range(launches):
        api.index_scan(inp["qs"], inp["ws"], inp["ks"], inp["q_pos"], block_max=path.block_max)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / launches * 1e3


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_sequence(inp, gen, b, queries=None):
    """Host copy of sequence b's inputs (optionally only some of its queries)."""
    per_query = {"q", "qs", "ws", "qi", "wi", "q_pos"}
    host = {}
    for k, v in inp.items():
        if k == "cfg":
            continue
        if v is None:
            host[k] = None
            continue
        t = v if k == "sink" else v[b:b + 1]
        if queries is not None and k in per_query:
            t = t[:, queries]
        host[k] = gen.to_numpy(t)
    host["comp_pos0"] = inp["cfg"].comp_pos0
    return host


def cpu_baseline(cfg, inp, gen, budget_s=10.0, threads=None, max_seqs=8, what=None):
    """The oracle as it stands, on sequences of the same workload: each
    sequence's inputs are copied to the host once (at most max_seqs of
    them), then whole-sequence oracle decodes run round-robin until about
    budget_s of oracle time (the host copies are not counted).  threads:
    OpenMP threads for the oracle (default: as the environment sets)."""
    from oracle import csa2_ref as ref

    default = ref.threads()
    if threads:
        ref.set_threads(threads)
    used = ref.threads()
    hosts = [host_sequence(inp, gen, b) for b in range(min(cfg.B, max_seqs))]
    done, spent = 0, 0.0
    try:
        while spent < budget_s:
            host = hosts[done % len(hosts)]
            ts = time.perf_counter()
            ref.decode(host, cfg.K_b, cfg.K, cfg.W, cfg.scale, compress_first=cfg.comp_T > 0)
            spent += time.perf_counter() - ts
            done += 1
    finally:
        ref.set_threads(default)
    log(f"[cpu] oracle {cfg.name} ({used} threads): {done} sequence decodes in {spent:.1f} s")
    what = what or cfg.desc
    return {"value": round(done * cfg.Tq / spent, 4), "unit": "queries/s", "cores": used,
            "kind": "oracle",
            "sample": f"{done} whole-sequence decodes ({cfg.Tq} quer{'y' if cfg.Tq == 1 else 'ies'} "
                      f"each, round-robin over {len(hosts)} sequences of the {what} workload"
                      f"{', compressor included' if cfg.comp_T else ''}), {spent:.1f} s of oracle "
                      f"time on {used} threads; host copies of the inputs excluded"}


def cpu_baseline_prefill(cfg, inp, gen, budget_s=5.0):
    """The oracle on the chunked prefill, in tokens/s: the compressor over the
    whole chunk once, then groups of 32 queries spread over the chunk (each
    with its own causal horizon and window) until about budget_s; the rate
    is Tq / (compressor time + Tq x time per query)."""
    from oracle import csa2_ref as ref

    used = ref.threads()
    host = host_sequence(inp, gen, 0, queries=[0])
    ts = time.perf_counter()
    ref.compress(host["raw"], host["gate"])
    t_comp = time.perf_counter() - ts
    done, spent, g, group = 0, 0.0, 0, 0
    while spent < budget_s:
        qs = list(range(g % 256, cfg.Tq, 256))
        group = len(qs)
        h = host_sequence(inp, gen, 0, queries=qs)
        ts = time.perf_counter()
        ref.decode(h, cfg.K_b, cfg.K, cfg.W, cfg.scale, compress_first=False)
        spent += time.perf_counter() - ts
        done += len(qs)
        g += 97
    per_q = spent / done
    rate = cfg.Tq / (t_comp + cfg.Tq * per_q)
    log(f"[cpu] oracle prefill ({used} threads): compressor {t_comp:.2f} s, {done} queries in "
        f"{spent:.1f} s -> {rate:.1f} tokens/s")
    return {"value": round(rate, 3), "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"compressor over the whole {cfg.comp_T}-token chunk ({t_comp:.2f} s), then "
                      f"{done} of the chunk's {cfg.Tq} queries in groups of {group} spread over it "
                      f"({spent:.1f} s; each query scans, selects and attends over its own causal "
                      f"horizon); rate = {cfg.Tq} / (compressor + {cfg.Tq} x mean query time)"}


def time_config_evict(cfg, inp, path, steps, torch, evict_bytes=1 << 30):
    """The same step with a 1 GiB read between steps (four times the 256 MB
    last-level cache), so no step finds the previous step's bytes cached.
    A read, not a write: the write-back of a 1 GiB write would still be
    draining into HBM when the step starts and slow it down (random 2 KiB
    gathers measured at 2.3 TB/s right after such a write, 4.9 TB/s after a
    read).  Events around each step alone: the eviction read is not timed."""
    comp = cfg.comp_T > 0
    evict = torch.ones(evict_bytes // 4, dtype=torch.float32, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    sink = torch.empty((steps,), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    for i in range(steps):
        torch.sum(evict, dim=0, out=sink[i])
        ev[i][0].record()
        path.run(inp, cfg.scale, compress_first=comp)
        ev[i][1].record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    mean = sum(t) / len(t)
    del evict
    log(f"[bench] {cfg.name} with a 1 GiB eviction read between steps: {mean * 1e3:.1f} us/step "
        f"(median {t[len(t) // 2] * 1e3:.1f})")
    return {"workload": f"the headline step with a {evict_bytes >> 20} MiB read between steps "
                        "(untimed), so every step starts with a cold last-level cache",
            "ms_per_step_mean": round(mean, 4), "ms_per_step_median": round(t[len(t) // 2], 4),
            "queries_per_s": round(cfg.R / (mean * 1e-3), 1)}


def calib_copy(torch, nbytes=1 << 30):
    """A plain elementwise copy of known size (reads and writes nbytes), for
    scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.add(src, 0.0, out=dst)
    torch.cuda.synchronize()


def hbm_ceiling(torch, nbytes=1 << 30, iters=10):
    """Practical HBM ceiling for context (never the roofline's denominator):
    torch's own elementwise copy (reads and writes nbytes) and sum (reads
    nbytes) over 1 GiB, timed with events on the current stream."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    out = {}
    for name, fn, moved in (("copy", lambda: dst.copy_(src), 2 * nbytes),
                            ("sum", lambda: torch.sum(src), nbytes)):
        fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(iters):
            fn()
        e.record()
        torch.cuda.synchronize()
        out[f"torch_{name}_GBs"] = round(moved * iters / (s.elapsed_time(e) * 1e-3) / 1e9, 1)
    del src, dst
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-main", action="store_true", help="skip the low-precision and prefill extras")
    ap.add_argument("--calib", action="store_true", help="also run a 1 GiB plain copy (counter scaling)")
    ap.add_argument("--only", metavar="CONFIG", default=None,
                    help="time only this workload's step (e.g. prefill) and print its stage times "
                         "instead of the benchmark line (for counter runs)")
    ap.add_argument("--evict", action="store_true",
                    help="with --only: also time steps with a 1 GiB read between them")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the CSA2 path here is built and timed on a single "
              "MI355X (no collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from compressed_sparse_attention_03_amd import api, gen

    api.lib()  # fail loudly if the HIP library is not built
    if args.calib:
        calib_copy(torch)
    if args.only is not None:
        if args.only not in gen.CONFIGS:
            print(f"unknown workload {args.only!r}; one of {sorted(gen.CONFIGS)}", file=sys.stderr)
            sys.exit(2)
        ocfg, oinp, opath, oms, ost = time_config(args.only, args.steps, args.warmup, torch, gen, api)
        line = {"workload": args.only, "ms_per_step": round(oms, 4),
                "stages_us_eager": {k: round(v * 1e3, 2) for k, v in ost.items()}}
        if args.evict:
            line["evict"] = time_config_evict(ocfg, oinp, opath, args.steps, torch)
        print(json.dumps(line), flush=True)
        return

    cfg, inp, path, ms, stage_ms = time_config("1m", args.steps, args.warmup, torch, gen, api)
    sb = step_bytes(cfg)
    total_b = sum(sb.values())
    q_per_s = cfg.R / (ms * 1e-3)
    scan_us = scan_launch_us(torch, api, path, inp, args.steps)
    scan_s = scan_us * 1e-6
    scan_gbs = sb["index_scan"] / scan_s / 1e9
    log(f"[bench] 1m: scan kernel {scan_us:.1f} us/launch = {scan_gbs:.0f} GB/s")
    path_keep = path
    del path
    kernel_src = [os.path.join(ROOT, "compressed_sparse_attention_03_amd", "csrc", f) for f in SCAN_SOURCES]
    workload = "1m"
    traffic = stored_traffic(kernel_src, workload)
    result = {
        "metric": METRIC,
        "value": round(q_per_s, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded bf16 N(0,1) latents/queries, integer-valued bf16 index q/k in [-3,3]",
        "config": {
            "workload": "1M-context decode: 8 sequences x 1,048,576 raw tokens (524,288 bf16 latents "
                        "x 512), 1 query each; 64 heads x 512, 1 latent KV head; indexer 32 x 128; "
                        "top-2048 blocks of 8 -> top-512 positions; window 128",
            "sequences": cfg.B, "context_tokens": cfg.t_last + 1, "latents": cfg.N,
            "queries_per_step": cfg.R, "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": "index_scan (candidate-source indexer scan + fused block max)",
            "bound": "hbm",
            "achieved": round(scan_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(scan_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": sb["index_scan"],
            "avg_launch_us": round(scan_s * 1e6, 2),
        },
        "step_hbm": {
            "algorithmic_bytes": total_b,
            "GB/s": round(total_b / (ms * 1e-3) / 1e9, 1),
            "frac_of_peak": round(total_b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        },
        "stages_us_eager": {k: round(v * 1e3, 2) for k, v in stage_ms.items()},
    }

    extra = {}
    # secondary view: the stages a layer runs when it reuses the block stage
    # of an earlier layer (candidate indexer, position top-k, attention)
    amort = stage_ms["index_cand"] + stage_ms["select_positions"] + stage_ms["sparse_attn"]
    extra["amortized_layer_1m"] = {
        "workload": "the 1M decode's candidate indexer + position top-512 + sparse attention only "
                    "(eager stage times, launch gaps included); secondary",
        "us": round(amort * 1e3, 2), "queries_per_s": round(cfg.R / (amort * 1e-3), 1),
    }
    extra["evict_1m"] = time_config_evict(cfg, inp, path_keep, args.steps, torch)
    del path_keep
    extra["hbm_ceiling_context"] = hbm_ceiling(torch)
    cpu = {}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, inp, gen, budget_s=10.0,
                                              what="1M-context decode")
        result["cpu_baseline"]["cpu_model"] = cpu_model()
        result["cpu_baseline"]["affinity_cores"] = len(os.sched_getaffinity(0))
    else:
        result["cpu_baseline"] = None
    if not args.only_main:
        del inp
        torch.cuda.empty_cache()
        ccfg, cinp, cpath, cms, cst = time_config("128k", args.steps, args.warmup, torch, gen, api)
        del cpath
        csb = step_bytes(ccfg)
        ct = sum(csb.values())
        extra["decode_128k"] = {
            "workload": "128K batched decode: 32 sequences x 131,072 raw tokens (65,536 bf16 "
                        "latents), 1 query each; the step starts with the compressor pooling "
                        "each sequence's last 256 raw tokens",
            "queries_per_s": round(ccfg.R / (cms * 1e-3), 1), "ms_per_step": round(cms, 4),
            "algorithmic_bytes": ct,
            "step_hbm_frac": round(ct / (cms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "stages_us_eager": {k: round(v * 1e3, 2) for k, v in cst.items()},
        }
        if not args.no_cpu_baseline:
            cpu["128k"] = cpu_baseline(ccfg, cinp, gen, budget_s=4.0, max_seqs=4,
                                       what="128K batched decode")
            cpu["128k_1thread"] = cpu_baseline(ccfg, cinp, gen, budget_s=4.0, threads=1,
                                               max_seqs=2, what="128K batched decode")
        del cinp
        torch.cuda.empty_cache()
        lcfg, linp, lpath, lms, lst = time_config("1m_lowp", max(3, args.steps // 2), 2, torch, gen,
                                                  api)
        del lpath
        lsb = step_bytes(lcfg)
        lt = sum(lsb.values())
        extra["lowp_1m"] = {
            "workload": "32 sequences x 1M ctx, NVFP4 latents, FP8 E4M3 window + index keys; "
                        "the step starts with the compressor's decode step (NVFP4 write)",
            "queries_per_s": round(lcfg.R / (lms * 1e-3), 1), "ms_per_step": round(lms, 4),
            "step_hbm_frac": round(lt / (lms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "index_scan_GBs_eager_stage": round(lsb["index_scan"] / (lst["index_scan"] * 1e-3) / 1e9, 1),
            "stages_us_eager": {k: round(v * 1e3, 2) for k, v in lst.items()},
        }
        if not args.no_cpu_baseline:
            cpu["1m_lowp"] = cpu_baseline(lcfg, linp, gen, budget_s=4.0, max_seqs=4,
                                          what="low-precision 1M decode")
        del linp
        torch.cuda.empty_cache()
        vcfg, vinp, vpath, vms, vst = time_config("1m_verify", max(3, args.steps // 2), 2, torch, gen,
                                                  api)
        del vpath
        vsb = step_bytes(vcfg)
        vt = sum(vsb.values())
        extra["verify_1m"] = {
            "workload": "speculative verification: 8 sequences x 5 draft tokens at 1M ctx, bf16 caches",
            "queries_per_s": round(vcfg.R / (vms * 1e-3), 1), "ms_per_step": round(vms, 4),
            "step_hbm_frac": round(vt / (vms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "index_scan_GBs_eager_stage": round(vsb["index_scan"] / (vst["index_scan"] * 1e-3) / 1e9, 1),
            "stages_us_eager": {k: round(v * 1e3, 2) for k, v in vst.items()},
        }
        del vinp
        torch.cuda.empty_cache()
        extra["layer_stack_1m"] = time_layer_stack(max(3, args.steps // 4), torch, gen, api)
        torch.cuda.empty_cache()
        extra["compress_nvfp4_1m"] = time_compress_fp4(torch, api)
        torch.cuda.empty_cache()
        pcfg, pinp, ppath, pms, pst = time_config("prefill", 2, 1, torch, gen, api)
        del ppath
        flops = prefill_indexer_flops(pcfg)
        tfs = flops / (pst["index_scan"] * 1e-3) / 1e12
        extra["prefill"] = {
            "workload": "8192-token chunk after 65,536 raw tokens (36,864 latents), causal",
            "indexer_flops": flops, "indexer_TFLOPs": round(tfs, 2),
            "indexer_mfma_frac": round(tfs / MFMA_BF16_PEAK_TFS, 4),
            "tokens_per_s": round(pcfg.R / (pms * 1e-3), 1), "ms_per_step": round(pms, 3),
            "stages_us_eager": {k: round(v * 1e3, 2) for k, v in pst.items()},
        }
        if not args.no_cpu_baseline:
            cpu["prefill"] = cpu_baseline_prefill(pcfg, pinp, gen, budget_s=5.0)
        del pinp
        torch.cuda.empty_cache()
        fcfg, finp, fpath, fms, fst = time_config("prefill_fp8", 2, 1, torch, gen, api)
        del fpath
        ftfs = prefill_indexer_flops(fcfg) / (fst["index_scan"] * 1e-3) / 1e12
        extra["prefill_fp8"] = {
            "workload": "the same chunked prefill with FP8 E4M3 index keys (FP8 MFMA indexer)",
            "indexer_TFLOPs": round(ftfs, 2), "indexer_mfma_frac_fp8": round(ftfs / MFMA_FP8_PEAK_TFS, 4),
            "indexer_mfma_frac_of_bf16_peak": round(ftfs / MFMA_BF16_PEAK_TFS, 4),
            "tokens_per_s": round(fcfg.R / (fms * 1e-3), 1), "ms_per_step": round(fms, 3),
            "stages_us_eager": {k: round(v * 1e3, 2) for k, v in fst.items()},
        }
        del finp
        torch.cuda.empty_cache()
        xcfg, xinp, xpath, xms, xst = time_config("prefill_mxfp4", 2, 1, torch, gen, api)
        del xpath
        xtfs = prefill_indexer_flops(xcfg) / (xst["index_scan"] * 1e-3) / 1e12
        extra["prefill_mxfp4"] = {
            "workload": "the same chunked prefill with MXFP4 index keys (FP4 MFMA indexer)",
            "indexer_TFLOPs": round(xtfs, 2), "indexer_mfma_frac_fp4": round(xtfs / MFMA_FP4_PEAK_TFS, 4),
            "indexer_mfma_frac_of_bf16_peak": round(xtfs / MFMA_BF16_PEAK_TFS, 4),
            "tokens_per_s": round(xcfg.R / (xms * 1e-3), 1), "ms_per_step": round(xms, 3),
            "stages_us_eager": {k: round(v * 1e3, 2) for k, v in xst.items()},
        }
        del xinp
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        tcfg = gen.CONFIGS["tiny"]
        tinp = gen.make_inputs(tcfg, device="cpu")
        cpu["tiny_1thread"] = cpu_baseline(tcfg, tinp, gen, budget_s=3.0, threads=1,
                                           what="tiny decode")
        extra["cpu_baselines"] = dict(cpu, cpu_model=cpu_model(),
                                      affinity_cores=len(os.sched_getaffinity(0)))
    result["extra"] = extra
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
