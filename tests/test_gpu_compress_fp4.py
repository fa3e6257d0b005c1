"""GPU parity of the NVFP4 cache writers (NVFP4 article, section 3.2): the
standalone quantiser, the compressor with its quantising epilogue, and the
compressor's decode step with device-side state, all called through the
C ABI and compared with the CPU oracle on the same bytes.

Bar: the quantiser's codes and scales are bit-exact (both sides decide on
the same fp32 inputs, exactly); the compressor's rows are bit-exact except
where the exact pooled value sits within fp32 pooling error of a rounding
midpoint (checked, and counted); the decode step's rows are bit-identical to
the batch compressor's for the same tokens, in both cache formats."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_03_amd import api, gen
from oracle import csa2_ref as ref
from tests.gpu_util import BF16_TOL, bf16_to_np, check_close, check_fp4_pooling, say

pytestmark = pytest.mark.gpu

E4M3 = np.array([ref.e4m3(c) for c in range(0x7F)])


def _special_rows(rng, cols):
    """Rows that reach every branch of the quantiser: zeros, a scale that
    rounds to 0, saturation, exact E2M1 and E4M3 rounding ties, groups of
    representable values, negative zeros."""
    rows = []
    rows.append(np.zeros(cols))
    rows.append(np.full(cols, 1e-5) * rng.choice([-1, 1], cols))
    rows.append(rng.normal(size=cols) * 1e4)
    ties = np.zeros(cols)
    tmid = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for g in range(cols // 16):
        s = E4M3[rng.integers(1, 0x7F)]
        grp = [6.0 * s] + [t * s * rng.choice([-1, 1]) for t in rng.choice(tmid, 15)]
        ties[16 * g:16 * g + 16] = grp
    rows.append(ties)
    rep = np.zeros(cols)
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    for g in range(cols // 16):
        s = E4M3[rng.integers(0, 0x7F)]
        grp = [6.0 * s] + [mags[m] * s * rng.choice([-1, 1]) for m in rng.integers(0, 8, 15)]
        rep[16 * g:16 * g + 16] = grp
    rows.append(rep)
    smid = np.zeros(cols)
    for g in range(cols // 16):
        c = rng.integers(0, 0x7E)
        amax = 6 * (E4M3[c] + E4M3[c + 1]) / 2  # amax/6 exactly at an E4M3 midpoint
        grp = rng.uniform(-amax, amax, 16)
        grp[rng.integers(16)] = amax * rng.choice([-1, 1])
        smid[16 * g:16 * g + 16] = grp
    rows.append(smid)
    rows.append(np.copysign(np.where(rng.random(cols) < 0.1, 1.0, 0.0), rng.choice([-1.0, 1.0], cols)))
    return np.array(rows)


@pytest.mark.parametrize("rows,cols,src", [(1001, 512, "f32"), (333, 48, "bf16"), (7, 16, "f32")])
def test_quant_nvfp4_bit_exact(rows, cols, src):
    rng = np.random.default_rng(rows + cols)
    x = rng.normal(size=(rows, cols)) * rng.lognormal(0, 2.5, (rows, 1))
    sp = _special_rows(rng, cols)
    x[:len(sp)] = sp[:rows]
    xf = torch.from_numpy(x.astype(np.float32))
    if src == "bf16":
        xf = xf.bfloat16()
    say(f"[quant] {rows}x{cols} {src}")
    packed, scales = api.quant_nvfp4(xf.cuda())
    torch.cuda.synchronize()
    want_p, want_s = ref.quant_nvfp4(xf.float().numpy())
    assert np.array_equal(scales.cpu().numpy(), want_s), "scales"
    assert np.array_equal(packed.cpu().numpy(), want_p), "codes"
    # and the library's own dequantiser inverts it to the oracle's values
    dq = api.dequant_nvfp4(packed, scales, dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(dq.cpu().numpy().astype(np.float64), ref.dequant_nvfp4(want_p, want_s))
    say(f"  {rows * cols // 16} groups bit-exact")


@pytest.mark.parametrize("B,T,seed", [(3, 514, 80), (1, 2, 81), (2, 4096, 82)])
def test_compress_nvfp4_vs_oracle(B, T, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    raw = torch.randn((B, T, 512), generator=g, device="cuda").bfloat16()
    gate = torch.randn((B, T, 512), generator=g, device="cuda").bfloat16()
    say(f"[compress_nvfp4] B={B} T={T} seed={seed}")
    # write into the middle of a larger cache: rows outside must stay put
    rows = T // 2 + 10
    codes = torch.full((B, rows, 256), 0xA5, dtype=torch.uint8, device="cuda")
    scales = torch.full((B, rows, 32), 0x5A, dtype=torch.uint8, device="cuda")
    api.compress_nvfp4(raw, gate, codes[:, 5:5 + T // 2], scales[:, 5:5 + T // 2])
    torch.cuda.synchronize()
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    assert (c[:, :5] == 0xA5).all() and (c[:, 5 + T // 2:] == 0xA5).all()
    assert (s[:, :5] == 0x5A).all() and (s[:, 5 + T // 2:] == 0x5A).all()
    nd = check_fp4_pooling("compress_nvfp4", c[:, 5:5 + T // 2], s[:, 5:5 + T // 2],
                           gen.to_numpy(raw), gen.to_numpy(gate))
    assert sum(nd) <= max(1, B * T // 2 * 512 // 100000)


@pytest.mark.parametrize("fmt", ["bf16", "nvfp4"])
def test_compress_step_stream(fmt):
    """Tokens streamed one step at a time through the device state fill the
    cache exactly as the batch compressor does: sequences start at even and
    odd positions (an odd start finds its partner parked by the caller), end
    at different steps, and rows at or past n_cache are never written."""
    B, T, n_cache, rows = 6, 24, 10, 14
    g = torch.Generator(device="cuda").manual_seed(90 + (fmt == "nvfp4"))
    raw = torch.randn((B, T, 512), generator=g, device="cuda").bfloat16()
    gate = torch.randn((B, T, 512), generator=g, device="cuda").bfloat16()
    start = [0, 1, 4, 7, 2, 0]
    stop = [T, T, 15, T, 9, 0]          # exclusive; sequence 5 never gets a token
    state = torch.zeros((B, 2, 512), dtype=torch.bfloat16, device="cuda")
    for b in range(B):
        if start[b] % 2:
            state[b, 0], state[b, 1] = raw[b, start[b] - 1], gate[b, start[b] - 1]
    if fmt == "bf16":
        cache = torch.full((B, rows, 512), -9.0, dtype=torch.bfloat16, device="cuda")
    else:
        cache = (torch.full((B, rows, 256), 0xA5, dtype=torch.uint8, device="cuda"),
                 torch.full((B, rows, 32), 0x5A, dtype=torch.uint8, device="cuda"))
    say(f"[compress_step] {fmt}: B={B} T={T} n_cache={n_cache}")
    for step in range(T):
        p = [start[b] + step if start[b] + step < stop[b] else -1 for b in range(B)]
        idx = torch.tensor([min(max(v, 0), T - 1) for v in p], device="cuda")
        kv = raw[torch.arange(B, device="cuda"), idx].contiguous()
        gt = gate[torch.arange(B, device="cuda"), idx].contiguous()
        pos = torch.tensor(p, dtype=torch.int64, device="cuda")
        api.compress_step(kv, gt, pos, state, cache, n_cache=n_cache)
    torch.cuda.synchronize()
    # the batch kernels over the same tokens
    if fmt == "bf16":
        want = torch.empty((B, T // 2, 512), dtype=torch.bfloat16, device="cuda")
        api.compress(raw, gate, want)
    else:
        want = (torch.empty((B, T // 2, 256), dtype=torch.uint8, device="cuda"),
                torch.empty((B, T // 2, 32), dtype=torch.uint8, device="cuda"))
        api.compress_nvfp4(raw, gate, *want)
    torch.cuda.synchronize()
    parts = [(cache, want)] if fmt == "bf16" else list(zip(cache, want))
    for got_t, want_t in parts:
        got_t, want_t = got_t.cpu(), want_t.cpu()
        fill = got_t[0, rows - 1, 0].item()  # never written (row >= n_cache)
        for b in range(B):
            lo = (start[b] + 1) // 2 if start[b] % 2 == 0 else start[b] // 2
            hi = min(stop[b] // 2, n_cache)
            if hi > lo:
                assert torch.equal(got_t[b, lo:hi], want_t[b, lo:hi]), (b, lo, hi)
            untouched = torch.cat([got_t[b, :lo], got_t[b, max(hi, lo):]])
            assert (untouched == fill).all(), b
    # and against the oracle on the rows written
    r, gt_ = gen.to_numpy(raw), gen.to_numpy(gate)
    if fmt == "bf16":
        _, y64 = ref.compress(r, gt_)
        got = bf16_to_np(cache[:, :n_cache])
        m = np.zeros(got.shape[:2], bool)
        for b in range(B):
            m[b, (start[b] + 1) // 2 if start[b] % 2 == 0 else start[b] // 2:min(stop[b] // 2, n_cache)] = True
        check_close("compress_step bf16", got[m], y64[:, :n_cache][m], BF16_TOL)
        x = ref.bf16_array(r[:, :2 * n_cache]).reshape(B, n_cache, 2, 512)
        slack = 1e-6 * (np.abs(x[:, :, 0]) + np.abs(x[:, :, 1]))
        assert np.all(np.abs(got[m] - y64[:, :n_cache][m]) <= np.abs(y64[:, :n_cache][m]) * 2 ** -8 + slack[m])
    else:
        check_fp4_pooling("compress_step nvfp4", cache[0][1:2, 0:n_cache].cpu().numpy(),
                          cache[1][1:2, 0:n_cache].cpu().numpy(), r[1:2, :2 * n_cache],
                          gt_[1:2, :2 * n_cache])
    say("  stream == batch compressor, bit for bit")
