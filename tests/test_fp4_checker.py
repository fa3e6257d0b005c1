"""The NVFP4 row checker the GPU tests use, exercised on the CPU: it accepts
the oracle's own rows and rejects a planted wrong code or scale."""
import numpy as np
import pytest
import torch

from oracle import csa2_ref as ref
from tests.gpu_util import check_fp4_pooling


def _pair_inputs():
    g = torch.Generator().manual_seed(5)
    raw = torch.randn(2, 6, 512, generator=g).bfloat16().view(torch.uint16).numpy()
    gate = torch.randn(2, 6, 512, generator=g).bfloat16().view(torch.uint16).numpy()
    return raw, gate


def test_checker_accepts_oracle_rows():
    raw, gate = _pair_inputs()
    packed, scales, _ = ref.compress_nvfp4(raw, gate)
    assert check_fp4_pooling("self", packed, scales, raw, gate) == (0, 0)


def test_checker_rejects_planted_mistakes():
    raw, gate = _pair_inputs()
    packed, scales, _ = ref.compress_nvfp4(raw, gate)
    bad = packed.copy()
    bad[1, 2, 7] ^= 0x01  # one element one code off
    with pytest.raises(AssertionError):
        check_fp4_pooling("code", bad, scales, raw, gate)
    bad = scales.copy()
    bad[0, 1, 3] += 1     # one scale one code up
    with pytest.raises(AssertionError):
        check_fp4_pooling("scale", packed, bad, raw, gate)
