"""The C-ABI library on the CPU: it loads, exports every entry point the
public header declares, and its host-side validation rejects bad arguments
with the documented status before anything would reach the GPU.  No compute
call is made here (fake device addresses are never dereferenced because
validation fails first)."""
import ctypes
import os
import re

import pytest

from compressed_sparse_attention_03_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")

FAKE = ctypes.c_void_p(0x10000)       # 16-byte aligned stand-in address
MISALIGNED = ctypes.c_void_p(0x10002)
NULL = None


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        from compressed_sparse_attention_03_amd import build
        build.build()
    return _lib.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", text)))


def test_header_and_exports_agree(L):
    decl = declared_functions()
    assert set(decl) == set(_lib.EXPORTS), decl
    for name in decl:
        assert hasattr(L, name), name


def test_status_strings_and_version(L):
    for st in (0, -1, -2, -3, -4, 7):
        assert L.csa2_status_string(st)
    assert L.csa2_version() >> 16 >= 1


def test_compress_validation(L):
    s = None
    assert L.csa2_compress(1, 3, FAKE, 0, FAKE, 0, FAKE, 0, s) == _lib.EINVAL        # odd T
    assert L.csa2_compress(-1, 2, FAKE, 0, FAKE, 0, FAKE, 0, s) == _lib.EINVAL
    assert L.csa2_compress(0, 2, NULL, 0, NULL, 0, NULL, 0, s) == _lib.OK            # empty
    assert L.csa2_compress(1, 0, NULL, 0, NULL, 0, NULL, 0, s) == _lib.OK
    assert L.csa2_compress(1, 2, NULL, 0, FAKE, 0, FAKE, 0, s) == _lib.EINVAL
    assert L.csa2_compress(1, 2, MISALIGNED, 0, FAKE, 0, ctypes.c_void_p(0x20000), 0, s) == _lib.EINVAL
    # batch stride smaller than a sequence
    assert L.csa2_compress(2, 4, FAKE, 100, ctypes.c_void_p(0x100000), 4096,
                           ctypes.c_void_p(0x200000), 2048, s) == _lib.EINVAL
    # output overlapping the input
    assert L.csa2_compress(1, 4, FAKE, 2048, ctypes.c_void_p(0x100000), 2048, FAKE, 1024, s) == _lib.EINVAL


def _scores(L, mode=0, B=1, Tq=1, q=FAKE, q_dt=_lib.BF16, w=FAKE, k=FAKE, k_dt=_lib.BF16,
            k_sb=0, n=64, qp=FAKE, blocks=NULL, K_b=0, sc=FAKE, s_stride=64, ids=NULL, bm=NULL,
            bm_stride=0, k_scale=NULL):
    return L.csa2_index_scores(mode, B, Tq, q, q_dt, w, k, k_dt, k_scale, k_sb, n, qp, blocks, K_b, sc,
                               s_stride, ids, bm, bm_stride, None)


def test_index_scores_validation(L):
    assert _scores(L, mode=5) == _lib.EINVAL
    assert _scores(L, q_dt=_lib.FP8_E4M3) == _lib.EUNSUPPORTED
    assert _scores(L, k_dt=_lib.NVFP4) == _lib.EUNSUPPORTED
    assert _scores(L, B=0) == _lib.OK
    assert _scores(L, q=NULL) == _lib.EINVAL
    assert _scores(L, q=MISALIGNED) == _lib.EINVAL
    assert _scores(L, k=NULL) == _lib.EINVAL
    assert _scores(L, sc=NULL, bm=NULL) == _lib.EINVAL                       # no output at all
    assert _scores(L, s_stride=10) == _lib.EINVAL                            # stride < n
    assert _scores(L, sc=NULL, bm=FAKE, bm_stride=7) == _lib.EINVAL          # < ceil(64/8)
    assert _scores(L, B=2, k_sb=64 * 128 - 8) == _lib.EINVAL                 # overlapping batches
    assert _scores(L, B=2, k_sb=64 * 128 + 4) == _lib.EINVAL                 # misaligned rows
    assert _scores(L, mode=1, blocks=NULL, K_b=4, ids=FAKE) == _lib.EINVAL
    assert _scores(L, mode=1, blocks=FAKE, K_b=0, ids=FAKE) == _lib.EINVAL
    assert _scores(L, mode=1, blocks=FAKE, K_b=16, ids=FAKE, s_stride=100) == _lib.EINVAL
    assert _scores(L, mode=1, blocks=FAKE, K_b=4, ids=NULL) == _lib.EINVAL
    # MXFP4 keys: the many-query scan only, with its scales
    mx = dict(k_dt=_lib.MXFP4, Tq=64, k_scale=ctypes.c_void_p(0x300000))
    assert _scores(L, k_dt=_lib.MXFP4, Tq=1, k_scale=FAKE) == _lib.EUNSUPPORTED   # decode scan
    assert _scores(L, mode=1, blocks=FAKE, K_b=4, ids=FAKE, **mx) == _lib.EUNSUPPORTED
    assert _scores(L, **dict(mx, k_scale=NULL)) == _lib.EINVAL
    assert _scores(L, **dict(mx, k_scale=ctypes.c_void_p(0x300002))) == _lib.EINVAL
    assert _scores(L, B=2, k_sb=64 * 64 - 16, **mx) == _lib.EINVAL              # overlapping batches
    assert _scores(L, B=2, k_sb=64 * 64 + 8, **mx) == _lib.EINVAL               # rows not 16-aligned


def _select(L, R=1, n=16, sc=FAKE, s_stride=16, ids=NULL, id_stride=0, forced=NULL, last=0, k=4,
            out=FAKE, o_stride=4):
    return L.csa2_select_topk(R, n, sc, s_stride, ids, id_stride, forced, last, k, out, o_stride,
                              None, 0, None)


def test_select_validation(L):
    assert _select(L, k=0) == _lib.EINVAL
    assert _select(L, n=0) == _lib.EINVAL
    assert _select(L, R=-1) == _lib.EINVAL
    assert _select(L, R=0) == _lib.OK
    assert _select(L, n=(1 << 24) + 1, s_stride=(1 << 24) + 1) == _lib.EUNSUPPORTED
    assert _select(L, sc=NULL) == _lib.EINVAL
    assert _select(L, s_stride=8) == _lib.EINVAL
    assert _select(L, o_stride=3) == _lib.EINVAL
    assert _select(L, ids=FAKE, id_stride=8) == _lib.EINVAL
    assert _select(L, forced=FAKE, last=1) == _lib.EINVAL
    assert _select(L, sc=ctypes.c_void_p(0x10001)) == _lib.EINVAL
    # a long row with few rows needs scratch
    assert _select(L, n=65536, s_stride=65536, k=2048, o_stride=2048) == _lib.EWORKSPACE


def _attn(L, B=1, Tq=1, q=FAKE, q_sb=0, lat=FAKE, lat_dt=_lib.BF16, lat_scale=NULL, lat_sb=0,
          n=1024, sel=FAKE, K=512, sel_sb=512, win=FAKE, win_dt=_lib.BF16, win_scale=NULL, W=128,
          W_cap=128, win_sb=0, qp=FAKE, sink=FAKE, out=FAKE, out_sb=64 * 512, lse=NULL, ws=NULL,
          ws_bytes=0):
    return L.csa2_sparse_attn(B, Tq, q, q_sb, lat, lat_dt, lat_scale, lat_sb, n, sel, K, sel_sb,
                              win, win_dt, win_scale, W, W_cap, win_sb, qp, sink, 0.044, out,
                              out_sb, lse, ws, ws_bytes, None)


def test_sparse_attn_validation(L):
    assert _attn(L, W=0) == _lib.EINVAL
    assert _attn(L, W_cap=64) == _lib.EINVAL
    assert _attn(L, K=-1) == _lib.EINVAL
    assert _attn(L, K=4096, sel_sb=4096) == _lib.EUNSUPPORTED
    assert _attn(L, lat_dt=_lib.FP8_E4M3) == _lib.EUNSUPPORTED
    assert _attn(L, win_dt=_lib.NVFP4) == _lib.EUNSUPPORTED
    assert _attn(L, B=0) == _lib.OK
    assert _attn(L, q=NULL) == _lib.EINVAL
    assert _attn(L, lat_dt=_lib.NVFP4, lat_scale=NULL) == _lib.EINVAL
    assert _attn(L, win_dt=_lib.FP8_E4M3, win_scale=NULL) == _lib.EINVAL
    assert _attn(L, sel_sb=100) == _lib.EINVAL
    assert _attn(L, out_sb=1000) == _lib.EINVAL
    assert _attn(L, out=ctypes.c_void_p(0x10008)) == _lib.EINVAL
    assert _attn(L, B=2, lat_sb=10, q_sb=64 * 512, win_sb=128) == _lib.EINVAL
    # one query row splits its 640 rows over several workgroups: needs scratch
    need = L.csa2_workspace_bytes(_lib.OP_SPARSE_ATTN, 1, 512, 128)
    assert need > 0
    assert _attn(L) == _lib.EWORKSPACE
    assert _attn(L, ws=FAKE, ws_bytes=need - 1) == _lib.EWORKSPACE
    assert _attn(L, ws=ctypes.c_void_p(0x10004), ws_bytes=need) == _lib.EWORKSPACE


def _attn_noalloc(L, B=1, Tq=1, q=FAKE, q_sb=0, lat=FAKE, lat_dt=_lib.BF16, lat_scale=NULL,
                  lat_sb=0, n=1024, sel=FAKE, K=512, sel_sb=512, win=FAKE, win_dt=_lib.BF16,
                  win_scale=NULL, W=128, W_cap=128, win_sb=0, qp=FAKE, sink=FAKE, out=FAKE,
                  out_sb=64 * 512, lse=NULL):
    return L.csa2_sparse_attn_noalloc(B, Tq, q, q_sb, lat, lat_dt, lat_scale, lat_sb, n, sel, K,
                                      sel_sb, win, win_dt, win_scale, W, W_cap, win_sb, qp, sink,
                                      0.044, out, out_sb, lse, None)


def test_sparse_attn_noalloc_validation(L):
    """The allocation-free variant checks its arguments as csa2_sparse_attn
    does and refuses, before touching any device, a call whose split
    partials would not fit the fixed scratch."""
    assert _attn_noalloc(L, W=0) == _lib.EINVAL
    assert _attn_noalloc(L, q=NULL) == _lib.EINVAL
    assert _attn_noalloc(L, lat_dt=_lib.FP8_E4M3) == _lib.EUNSUPPORTED
    assert _attn_noalloc(L, B=0) == _lib.OK
    assert _attn_noalloc(L, out=ctypes.c_void_p(0x10008)) == _lib.EINVAL
    big = 64 * 512 * 2
    # 40 NVFP4 queries of 512 + 128 rows: 7 splits each, 37 MB of partials
    need = 40 * 7 * 64 * 516 * 4
    assert need > _lib.ATTN_SCRATCH_BYTES
    assert _attn_noalloc(L, B=40, q_sb=big, lat_dt=_lib.NVFP4, lat_scale=FAKE, lat_sb=1024,
                         win_sb=128) == _lib.EWORKSPACE
    assert L.csa2_workspace_bytes(_lib.OP_SPARSE_ATTN, 40, 512, 128) >= need


def test_workspace_sizes(L):
    # many query rows (prefill): one workgroup per row, no merge, no scratch
    assert L.csa2_workspace_bytes(_lib.OP_SPARSE_ATTN, 8192, 512, 128) == 0
    # few long rows: the pass over each row is split over many workgroups
    assert L.csa2_workspace_bytes(_lib.OP_SELECT, 8, 65536, 2048) > 0
    # many rows, or short rows: one workgroup per row, no scratch
    assert L.csa2_workspace_bytes(_lib.OP_SELECT, 8192, 16384, 512) == 0
    assert L.csa2_workspace_bytes(_lib.OP_SELECT, 8, 1000, 512) == 0
    a = L.csa2_workspace_bytes(_lib.OP_SPARSE_ATTN, 8, 512, 128)
    b = L.csa2_workspace_bytes(_lib.OP_SPARSE_ATTN, 32, 512, 128)
    assert a > 0 and b > 0
    assert L.csa2_workspace_bytes(_lib.OP_SPARSE_ATTN, 0, 512, 128) == 0


def test_dequant_validation(L):
    assert L.csa2_dequant_fp8(FAKE, NULL, 4, 0, FAKE, _lib.BF16, None) == _lib.EINVAL
    assert L.csa2_dequant_fp8(FAKE, NULL, 4, 8, FAKE, _lib.NVFP4, None) == _lib.EUNSUPPORTED
    assert L.csa2_dequant_fp8(NULL, NULL, 4, 8, FAKE, _lib.F32, None) == _lib.EINVAL
    assert L.csa2_dequant_fp8(FAKE, NULL, 0, 8, FAKE, _lib.F32, None) == _lib.OK
    assert L.csa2_dequant_nvfp4(FAKE, FAKE, 4, 24, FAKE, _lib.F32, None) == _lib.EINVAL  # cols % 16
    assert L.csa2_dequant_nvfp4(FAKE, NULL, 4, 32, FAKE, _lib.F32, None) == _lib.EINVAL
    assert L.csa2_dequant_nvfp4(FAKE, FAKE, 4, 32, ctypes.c_void_p(0x10002), _lib.BF16, None) == _lib.EINVAL


def test_compress_nvfp4_validation(L):
    s = None
    A, G, C, S = (ctypes.c_void_p(a) for a in (0x100000, 0x200000, 0x300000, 0x400000))
    assert L.csa2_compress_nvfp4(1, 3, A, 0, G, 0, C, S, 0, s) == _lib.EINVAL        # odd T
    assert L.csa2_compress_nvfp4(0, 2, NULL, 0, NULL, 0, NULL, NULL, 0, s) == _lib.OK
    assert L.csa2_compress_nvfp4(1, 2, A, 0, G, 0, C, NULL, 0, s) == _lib.EINVAL     # no scales
    assert L.csa2_compress_nvfp4(1, 2, A, 0, G, 0, ctypes.c_void_p(0x300004), S, 0, s) == _lib.EINVAL
    # batch stride (rows) smaller than the T/2 rows a sequence writes
    assert L.csa2_compress_nvfp4(2, 8, A, 4096, G, 4096, C, S, 3, s) == _lib.EINVAL
    # codes overlapping the input
    assert L.csa2_compress_nvfp4(1, 4, A, 2048, G, 2048, ctypes.c_void_p(0x100100), S, 2, s) == _lib.EINVAL
    assert L.csa2_compress_nvfp4(1, 4, A, 2048, G, 2048, C, ctypes.c_void_p(0x300040), 2, s) == _lib.EINVAL


def test_compress_step_validation(L):
    s = None
    K, G, P, ST, O, SC = (ctypes.c_void_p(a) for a in
                          (0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 0x600000))
    ok = dict(B=2, kv=K, kv_sb=512, g=G, g_sb=512, pos=P, st=ST, dt=_lib.NVFP4, out=O, osc=SC,
              out_sb=16, n=16)

    def call(**kw):
        a = dict(ok, **kw)
        return L.csa2_compress_step(a["B"], a["kv"], a["kv_sb"], a["g"], a["g_sb"], a["pos"],
                                    a["st"], a["dt"], a["out"], a["osc"], a["out_sb"], a["n"], s)
    assert call(B=0, kv=NULL) == _lib.OK
    assert call(B=-1) == _lib.EINVAL
    assert call(n=-1) == _lib.EINVAL
    assert call(dt=_lib.FP8_E4M3) == _lib.EUNSUPPORTED
    assert call(osc=NULL) == _lib.EINVAL                     # NVFP4 needs the scale rows
    assert call(pos=ctypes.c_void_p(0x300004)) == _lib.EINVAL
    assert call(kv_sb=256) == _lib.EINVAL                    # rows overlap
    assert call(out_sb=8) == _lib.EINVAL                     # stride below n_cache
    assert call(st=ctypes.c_void_p(0x100200)) == _lib.EINVAL  # state overlaps kv
    assert call(out=ctypes.c_void_p(0x400100)) == _lib.EINVAL  # cache overlaps state
    assert call(dt=_lib.BF16, out=ctypes.c_void_p(0x500008)) == _lib.EINVAL  # bf16 rows 16-aligned


def test_quant_nvfp4_validation(L):
    s = None
    A, P, S = (ctypes.c_void_p(a) for a in (0x100000, 0x200000, 0x300000))
    assert L.csa2_quant_nvfp4(A, _lib.BF16, 4, 24, P, S, s) == _lib.EINVAL   # cols % 16
    assert L.csa2_quant_nvfp4(A, _lib.FP8_E4M3, 4, 32, P, S, s) == _lib.EUNSUPPORTED
    assert L.csa2_quant_nvfp4(A, _lib.F32, 0, 32, P, S, s) == _lib.OK
    assert L.csa2_quant_nvfp4(A, _lib.F32, 4, 32, NULL, S, s) == _lib.EINVAL
    assert L.csa2_quant_nvfp4(MISALIGNED, _lib.F32, 4, 32, P, S, s) == _lib.EINVAL
    assert L.csa2_quant_nvfp4(A, _lib.F32, 4, 32, ctypes.c_void_p(0x100010), S, s) == _lib.EINVAL


def test_gather_select_validation(L):
    s = None
    A, Q, BL, O = (ctypes.c_void_p(a) for a in (0x100000, 0x200000, 0x300000, 0x400000))
    assert L.csa2_gather_select(0, 4, NULL, 0, 10, NULL, NULL, 1, 5, NULL, 8, s) == _lib.OK   # no rows
    assert L.csa2_gather_select(1, 1, A, 64, 64, Q, BL, 0, 5, O, 8, s) == _lib.EINVAL         # K_b < 1
    assert L.csa2_gather_select(1, 1, A, 64, 64, Q, BL, 2, 0, O, 8, s) == _lib.EINVAL         # k < 1
    assert L.csa2_gather_select(1, 1, A, 64, 64, Q, BL, 2, 9, O, 8, s) == _lib.EINVAL         # o_stride < k
    assert L.csa2_gather_select(1, 1, A, 32, 64, Q, BL, 2, 5, O, 8, s) == _lib.EINVAL         # a_stride < n
    assert L.csa2_gather_select(1, 1, A, 64, 64, NULL, BL, 2, 5, O, 8, s) == _lib.EINVAL      # no q_pos
    assert L.csa2_gather_select(1, 1, A, 64, 64, Q, BL, 2, 5, ctypes.c_void_p(0x400002), 8, s) == _lib.EINVAL
    assert L.csa2_gather_select(1, 1, A, 64, 64, Q, BL, 2, 5, ctypes.c_void_p(0x100010), 8, s) == _lib.EINVAL  # overlap
    # rows longer than one workgroup's registers: the two-call path instead
    assert L.csa2_gather_select(1, 1, A, 64, 64, Q, BL, 2049, 5, O, 8, s) == _lib.EUNSUPPORTED
    assert L.csa2_gather_select(1, 255, A, 64, 64, Q, BL, 4096, 5, O, 8, s) == _lib.EUNSUPPORTED


def test_gather_scores_validation(L):
    s = None
    A, Q, BL, S, I = (ctypes.c_void_p(a) for a in (0x100000, 0x200000, 0x300000, 0x400000, 0x500000))
    assert L.csa2_gather_scores(0, 4, NULL, 0, 10, NULL, NULL, 1, NULL, NULL, 8, s) == _lib.OK
    assert L.csa2_gather_scores(1, 1, A, 64, 64, Q, BL, 0, S, I, 8, s) == _lib.EINVAL      # K_b < 1
    assert L.csa2_gather_scores(1, 1, A, 64, 64, Q, BL, 2, S, I, 8, s) == _lib.EINVAL      # s_stride < 16
    assert L.csa2_gather_scores(1, 1, A, 62, 62, Q, BL, 2, S, I, 16, s) == _lib.EINVAL     # a_stride % 4
    assert L.csa2_gather_scores(1, 1, A, 32, 64, Q, BL, 2, S, I, 16, s) == _lib.EINVAL     # a_stride < n
    assert L.csa2_gather_scores(1, 1, A, 64, 64, Q, BL, 2, ctypes.c_void_p(0x400004), I, 16, s) == _lib.EINVAL
    assert L.csa2_gather_scores(1, 1, A, 64, 64, Q, BL, 2, S, ctypes.c_void_p(0x400020), 16, s) == _lib.EINVAL
    assert L.csa2_gather_scores(1, 1, A, 64, 64, Q, BL, 2, ctypes.c_void_p(0x100040), I, 16, s) == _lib.EINVAL
