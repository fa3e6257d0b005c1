"""GPU parity of the index query's rounding to the key format, over every bf16
value, through csa2_index_scores.

With FP8 E4M3 or MXFP4 index keys the kernels round the bf16 index query to
the key's element format (E4M3, resp. E2M1) before the contraction, nearest
with ties to even and saturating (the oracle's reading of the NVFP4 article,
section 3.3, where index queries are FP4).  Here every one of the 65,536 bf16
bit patterns except the NaNs is a query element, and the indexer itself
reads the rounded value back: query row j has one-hot head weights (head
j % 32) and its 128 dims carry patterns 128 j .. 128 j + 127; the 256 keys
are +1 and -1 on one dim each, so score[2d] - score[2d+1] = ReLU(r) -
ReLU(-r) = r, the rounded element, exactly.  Both conversion sites run: the
prefill tile scan (512 queries of one sequence, FP8 and MXFP4 keys) and the
decode scan (512 sequences of one query, FP8 keys).  Expected values: the
oracle's rounding (round_e4m3 / round_e2m1) decoded by its format tables.
"""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_03_amd import api
from oracle import csa2_ref as ref
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

HI, DI = 32, 128
ROWS = 65536 // DI                   # 512 query rows of 128 patterns
NK = 2 * DI                          # keys: +1 and -1 on each dim


def _patterns():
    """[512][128] bf16 patterns 0..65535; NaN patterns replaced by 0."""
    p = np.arange(65536, dtype=np.uint32)
    nan = (p & 0x7fff) > 0x7f80
    return np.where(nan, 0, p).astype(np.uint16).reshape(ROWS, DI), nan.reshape(ROWS, DI)


def _expected(fmt, pats, nan):
    x = np.array([ref.bf16(b) for b in pats.reshape(-1)], np.float64)
    if fmt == "fp8":
        r = np.array([ref.e4m3(ref.round_e4m3(v)) for v in x])
    else:
        r = np.array([ref.e2m1(ref.round_e2m1(v)) for v in x])
    return r.reshape(ROWS, DI)


def _keys(fmt, B):
    d = np.arange(DI)
    if fmt == "fp8":
        k = np.zeros((NK, DI), np.uint8)
        k[2 * d, d] = 0x38          # E4M3 +1
        k[2 * d + 1, d] = 0xB8      # E4M3 -1
        return torch.from_numpy(np.broadcast_to(k, (B, NK, DI)).copy()).cuda(), None
    nib = np.zeros((NK, DI), np.uint8)
    nib[2 * d, d] = 0x2             # E2M1 +1
    nib[2 * d + 1, d] = 0xA         # E2M1 -1
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)   # dim 2i in the low nibble
    scales = np.full((NK, DI // 32), 127, np.uint8)                 # E8M0 2^0
    return (torch.from_numpy(np.broadcast_to(codes, (B, NK, DI // 2)).copy()).cuda(),
            torch.from_numpy(np.broadcast_to(scales, (B, NK, DI // 32)).copy()).cuda())


@pytest.mark.parametrize("fmt,decode", [("fp8", False), ("fp8", True), ("mxfp4", False)])
def test_index_query_rounding_every_bf16(fmt, decode):
    pats, nan = _patterns()
    B, Tq = (ROWS, 1) if decode else (1, ROWS)
    q = np.zeros((ROWS, HI, DI), np.uint16)
    w = np.zeros((ROWS, HI), np.float32)
    j = np.arange(ROWS)
    q[j, j % HI, :] = pats
    w[j, j % HI] = 1.0
    q_t = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).reshape(B, Tq, HI, DI).cuda()
    w_t = torch.from_numpy(w).reshape(B, Tq, HI).cuda()
    k, k_scale = _keys(fmt, B)
    q_pos = torch.full((B, Tq), 2 * NK - 1, dtype=torch.int64, device="cuda")   # all keys visible
    scores = torch.empty((ROWS, NK), dtype=torch.float32, device="cuda")
    say(f"[run] {fmt} query rounding, {'decode scan' if decode else 'prefill tile scan'}: "
        f"B={B} Tq={Tq}, {NK} one-hot keys")
    api.index_scan(q_t, w_t, k, q_pos, scores=scores, k_scale=k_scale)
    torch.cuda.synchronize()
    s = scores.cpu().numpy().astype(np.float64)
    got = s[:, 0::2] - s[:, 1::2]                 # ReLU(r) - ReLU(-r) = r
    want = _expected(fmt, pats, nan)
    bad = (got != want) & ~nan
    assert not bad.any(), (fmt, decode, [(int(pats[i]), got[i], want[i]) for i in zip(*np.nonzero(bad))][:8])
    say(f"  {fmt}: {int((~nan).sum())} bf16 values rounded as the oracle rounds them")
