"""GPU parity of the fused FP8 block -> BF16 -> MXFP8 re-quantization against
the CPU oracle's composition, byte for byte."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import announce, assert_same, u8

pytestmark = pytest.mark.gpu


def check_requant(gpu, orc, q, S, name):
    announce(f"requant {name} {q.shape}")
    q8, s8 = gpu.blockfp8_to_mxfp8(torch.from_numpy(q).cuda(), torch.from_numpy(S).cuda())
    torch.cuda.synchronize()
    oq, os_ = orc.blockfp8_to_mxfp8(q, S)
    assert_same(f"{name} q8", u8(q8), oq)
    assert_same(f"{name} s8", u8(s8), os_)


def test_requant_square_8192_full(gpu, orc):
    """The [8192, 8192] block-FP8 tensor of the bench, every output byte."""
    q, S = orc.blockfp8_quantize(workloads.square_8192(), 128)
    check_requant(gpu, orc, q, S, "square_8192")


@pytest.mark.parametrize("shape", [(1, 32), (33, 160), (130, 544), (256, 384), (97, 7168)])
def test_requant_ragged(gpu, orc, shape):
    q, S = orc.blockfp8_quantize(workloads.random_bf16(shape, 3 * shape[0] + shape[1]), 128)
    check_requant(gpu, orc, q, S, f"ragged{shape}")


def test_requant_arbitrary_codes_and_scales(gpu, orc):
    """Every code (NaN codes included) under tile scales that are zero,
    subnormal, tiny, huge (products overflow bf16), NaN, Inf and ordinary."""
    rng = np.random.default_rng(12)
    rows, cols = 512, 1024
    q = rng.integers(0, 256, size=(rows, cols)).astype(np.uint8)
    q[:, :256] = np.tile(np.arange(256, dtype=np.uint8), (rows, 1))
    specials = np.array([0.0, 1e-45, 2.0 ** -140, 1e-30, 3.0e38, 1e38, np.inf, np.nan, -1.0,
                         0.375, 2.0 ** -6, 1.0, 3.5, 2.0 ** 20, 7.1e-3, 1e5,
                         -0.0, 2.0 ** 127, 5e-39, 42.0, 1.0 / 3.0, 448.0, 1e-3, 65504.0,
                         2.0 ** -100, 0.1, 9.0, 0.5, 1e10, 2.5e-7, 12.25, 1.5], np.float32)
    S = specials.reshape(4, 8)
    check_requant(gpu, orc, q, S, "arbitrary")


def test_requant_pow2_tiles(gpu, orc):
    rng = np.random.default_rng(9)
    rows, cols = 384, 640
    q = rng.integers(0, 256, size=(rows, cols)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x7E
    S = np.exp2(rng.integers(-30, 30, size=(3, 5)).astype(np.float64)).astype(np.float32)
    check_requant(gpu, orc, q, S, "pow2")
